// Internal launch entry points of the kernel translation units.  Arguments are
// validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "plx.h"

namespace plx {

// flags: PLX_UNIFORM_WEIGHTS | PLX_NO_INTERCEPT; cor may be NULL.
hipError_t launch_fwd(int dtype, const void* q, const void* k, const void* v, const void* rho,
                      float* o, float* lse, float* c_aux, float* vbar_aux, float* cor,
                      unsigned flags, int B, int Hq, int Hkv, int T, int d, float scale,
                      hipStream_t stream);

// Decode: key-split partial kernel followed by the merge kernel.
int decode_auto_splits(int B, int Hkv, int S_max);
int decode_chunk_keys(int S_max, int num_splits);
size_t decode_record_floats(int d);
int decode_balanced_ctas(int B, int Hkv, int S_max);
size_t decode_balanced_records(int B, int Hq, int Hkv, int S_max);
hipError_t launch_decode(int dtype, const void* q, const void* rho, const void* k_cache,
                         const void* v_cache, const int32_t* ctx_len, float* o, float* lse,
                         float* cor, unsigned flags, int B, int Hq, int Hkv, int S_max, int d,
                         float scale, int num_splits, float* partials, hipStream_t stream);

// Decode with the records in the library's own per-device scratch array
// (PLX_DECODE_SCRATCH_BYTES); the caller has checked the size.
hipError_t launch_decode_noalloc(int dtype, const void* q, const void* rho, const void* k_cache,
                                 const void* v_cache, const int32_t* ctx_len, float* o, float* lse,
                                 int B, int Hq, int Hkv, int S_max, int d, float scale,
                                 int num_splits, hipStream_t stream);

// Backward: workspace bytes (G and delta, then the fp16 input copies of the bf16 path).
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int d);
hipError_t launch_bwd(int dtype, const void* q, const void* k, const void* v, const void* rho,
                      const void* d_o, const float* o, const float* lse, const float* c_aux,
                      const float* vbar_aux, float* dq, float* dk, float* dv, float* drho, int B,
                      int Hq, int Hkv, int T, int d, float scale, float* ws, hipStream_t stream);

// Stacked projection [Q | K | V | rho] = X W^T into the [B, H, T, d] layout.
hipError_t launch_proj(const void* x, const void* w, void* q, void* k, void* v, void* rho, int B,
                       int T, int D, int Hq, int Hkv, int d, hipStream_t stream);

}  // namespace plx
