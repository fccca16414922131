// C-ABI layer: argument validation (before any HIP call) and dispatch.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "plx.h"
#include "plx_kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }  // NULL passes

bool flags_ok(unsigned f) { return (f & ~(PLX_UNIFORM_WEIGHTS | PLX_NO_INTERCEPT)) == 0; }

bool dtype_ok(plx_dtype dt) { return dt == PLX_F32 || dt == PLX_BF16; }

// d = 256 is served by the bf16 kernels (forward, decode, backward, projection);
// the fp32 kernels stop at d = 128.
plx_status check_heads(int B, int Hq, int Hkv, int d, plx_dtype dtype, bool allow256) {
  if (B < 1 || Hq < 1 || Hkv < 1) return PLX_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return PLX_ERR_INVALID_ARG;
  if (d == 256 && allow256 && dtype == PLX_BF16) return PLX_OK;
  if (d != 64 && d != 128) return PLX_ERR_UNSUPPORTED;
  return PLX_OK;
}

bool dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

plx_status from_hip(hipError_t e) { return e == hipSuccess ? PLX_OK : PLX_ERR_HIP; }

// Element counts must stay addressable with 32-bit row indices times d.
bool size_ok(long long rows, int d) { return rows > 0 && rows * (long long)d < (1LL << 40); }

}  // namespace

extern "C" {

int plx_abi_version(void) { return PLX_ABI_VERSION; }

const char* plx_status_string(plx_status s) {
  switch (s) {
    case PLX_OK: return "ok";
    case PLX_ERR_INVALID_ARG: return "invalid argument";
    case PLX_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PLX_ERR_WORKSPACE: return "workspace too small";
    case PLX_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

plx_status plx_fwd_prefill_ex(const void* q, const void* k, const void* v, const void* rho,
                              float* o, float* lse, float* c_aux, float* vbar_aux, float* cor,
                              int B, int Hq, int Hkv, int T, int d, float scale, unsigned flags,
                              plx_dtype dtype, plx_stream stream) {
  if (!q || !k || !v || !rho || !o) return PLX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || T < 1 || !scale_ok(scale) || !flags_ok(flags)) return PLX_ERR_INVALID_ARG;
  plx_status st = check_heads(B, Hq, Hkv, d, dtype, true);
  if (st != PLX_OK) return st;
  if (!size_ok((long long)B * Hq * T, d)) return PLX_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(rho) || !aligned16(o) ||
      (vbar_aux && !aligned16(vbar_aux)) || !aligned4(lse) || !aligned4(c_aux) || !aligned4(cor))
    return PLX_ERR_INVALID_ARG;
  return from_hip(plx::launch_fwd(dtype, q, k, v, rho, o, lse, c_aux, vbar_aux, cor, flags, B, Hq,
                                  Hkv, T, d, scale, (hipStream_t)stream));
}

plx_status plx_fwd_prefill(const void* q, const void* k, const void* v, const void* rho, float* o,
                           float* lse, float* c_aux, float* vbar_aux, int B, int Hq, int Hkv, int T,
                           int d, float scale, plx_dtype dtype, plx_stream stream) {
  return plx_fwd_prefill_ex(q, k, v, rho, o, lse, c_aux, vbar_aux, nullptr, B, Hq, Hkv, T, d, scale,
                            0u, dtype, stream);
}

size_t plx_decode_workspace_size(int B, int Hq, int Hkv, int S_max, int d, int num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S_max < 1 || num_splits < 0) return 0;
  if (!dim_ok(d)) return 0;
  int ns = num_splits > 0 ? num_splits : plx::decode_auto_splits(B, Hkv, S_max);
  if (ns > S_max) ns = S_max;
  const int chunk = plx::decode_chunk_keys(S_max, ns);
  ns = (S_max + chunk - 1) / chunk;
  size_t bytes = (size_t)B * Hq * ns * plx::decode_record_floats(d) * sizeof(float);
  if (num_splits == 0) {
    // automatic: bf16 runs the balanced schedule, fp32 the automatic split count
    const size_t bal =
        plx::decode_balanced_records(B, Hq, Hkv, S_max) * plx::decode_record_floats(d) * sizeof(float);
    if (bal > bytes) bytes = bal;
  }
  return bytes;
}

// Arguments of the decode entry points other than the workspace.
static plx_status check_decode(const void* q, const void* rho, const void* k_cache, const void* v_cache,
                        const int32_t* ctx_len, const float* o, const float* lse, const float* cor,
                        int B, int Hq, int Hkv, int S_max, int d, float scale, int num_splits,
                        unsigned flags, plx_dtype dtype) {
  if (!q || !rho || !k_cache || !v_cache || !ctx_len || !o) return PLX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || S_max < 1 || num_splits < 0 || !scale_ok(scale) || !flags_ok(flags))
    return PLX_ERR_INVALID_ARG;
  plx_status st = check_heads(B, Hq, Hkv, d, dtype, true);
  if (st != PLX_OK) return st;
  if (!size_ok((long long)B * Hkv * S_max, d)) return PLX_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(rho) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(o) || !aligned4(ctx_len) || !aligned4(lse) || !aligned4(cor))
    return PLX_ERR_INVALID_ARG;
  return PLX_OK;
}

plx_status plx_decode_ex(const void* q, const void* rho, const void* k_cache, const void* v_cache,
                         const int32_t* ctx_len, float* o, float* lse, float* cor, int B, int Hq,
                         int Hkv, int S_max, int d, float scale, int num_splits, unsigned flags,
                         void* workspace, size_t workspace_bytes, plx_dtype dtype,
                         plx_stream stream) {
  plx_status st = check_decode(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, B, Hq, Hkv, S_max, d,
                               scale, num_splits, flags, dtype);
  if (st != PLX_OK) return st;
  if (workspace && !aligned16(workspace)) return PLX_ERR_INVALID_ARG;
  const size_t need = plx_decode_workspace_size(B, Hq, Hkv, S_max, d, num_splits);
  if (!workspace || workspace_bytes < need) return PLX_ERR_WORKSPACE;
  return from_hip(plx::launch_decode(dtype, q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B,
                                     Hq, Hkv, S_max, d, scale, num_splits, (float*)workspace,
                                     (hipStream_t)stream));
}

plx_status plx_decode(const void* q, const void* rho, const void* k_cache, const void* v_cache,
                      const int32_t* ctx_len, float* o, float* lse, int B, int Hq, int Hkv,
                      int S_max, int d, float scale, int num_splits, void* workspace,
                      size_t workspace_bytes, plx_dtype dtype, plx_stream stream) {
  return plx_decode_ex(q, rho, k_cache, v_cache, ctx_len, o, lse, nullptr, B, Hq, Hkv, S_max, d,
                       scale, num_splits, 0u, workspace, workspace_bytes, dtype, stream);
}

plx_status plx_decode_noalloc(const void* q, const void* rho, const void* k_cache,
                              const void* v_cache, const int32_t* ctx_len, float* o, float* lse,
                              int B, int Hq, int Hkv, int S_max, int d, float scale, int num_splits,
                              plx_dtype dtype, plx_stream stream) {
  plx_status st = check_decode(q, rho, k_cache, v_cache, ctx_len, o, lse, nullptr, B, Hq, Hkv, S_max,
                               d, scale, num_splits, 0u, dtype);
  if (st != PLX_OK) return st;
  if (plx_decode_workspace_size(B, Hq, Hkv, S_max, d, num_splits) > PLX_DECODE_SCRATCH_BYTES)
    return PLX_ERR_WORKSPACE;
  return from_hip(plx::launch_decode_noalloc(dtype, q, rho, k_cache, v_cache, ctx_len, o, lse, B, Hq,
                                             Hkv, S_max, d, scale, num_splits, (hipStream_t)stream));
}

size_t plx_bwd_workspace_size(int B, int Hq, int Hkv, int T, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1) return 0;
  if (!dim_ok(d)) return 0;
  // G_i = dO_i . o_i and delta_i = dO_i . vbar_i (fp32 each), the dO scale
  // and its partial maxima, then the fp16 copies of q, rho, s dO and k that
  // the bf16 path's kernels read
  return plx::bwd_workspace_bytes(B, Hq, Hkv, T, d);
}

plx_status plx_bwd(const void* q, const void* k, const void* v, const void* rho, const void* d_o,
                   const float* o, const float* lse, const float* c_aux, const float* vbar_aux,
                   float* dq, float* dk, float* dv, float* drho, int B, int Hq, int Hkv, int T, int d,
                   float scale, void* workspace, size_t workspace_bytes, plx_dtype dtype,
                   plx_stream stream) {
  if (!q || !k || !v || !rho || !d_o || !o || !lse || !c_aux || !vbar_aux) return PLX_ERR_INVALID_ARG;
  if (!dq || !dk || !dv || !drho) return PLX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || T < 1 || !scale_ok(scale)) return PLX_ERR_INVALID_ARG;
  plx_status st = check_heads(B, Hq, Hkv, d, dtype, true);
  if (st != PLX_OK) return st;
  if (!size_ok((long long)B * Hq * T, d)) return PLX_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, rho, d_o, o, vbar_aux, dq, dk, dv, drho};
  for (const void* p : ptrs)
    if (!aligned16(p)) return PLX_ERR_INVALID_ARG;
  const size_t need = plx_bwd_workspace_size(B, Hq, Hkv, T, d);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PLX_ERR_WORKSPACE;
  return from_hip(plx::launch_bwd(dtype, q, k, v, rho, d_o, o, lse, c_aux, vbar_aux, dq, dk, dv,
                                  drho, B, Hq, Hkv, T, d, scale, (float*)workspace,
                                  (hipStream_t)stream));
}

plx_status plx_qkvr_proj(const void* x, const void* w, void* q, void* k, void* v, void* rho, int B,
                         int T, int D, int Hq, int Hkv, int d, plx_dtype dtype, plx_stream stream) {
  if (!x || !w || !q || !k || !v || !rho) return PLX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || T < 1 || D < 1) return PLX_ERR_INVALID_ARG;
  plx_status st = check_heads(B, Hq, Hkv, d, dtype, true);
  if (st != PLX_OK) return st;
  if (dtype != PLX_BF16 || D % 64 != 0) return PLX_ERR_UNSUPPORTED;
  const long long M = (long long)B * T, N = (2LL * Hq + 2LL * Hkv) * d;
  if (M * D >= (1LL << 40) || N * D >= (1LL << 40) || M * N >= (1LL << 40) || M >= (1LL << 31))
    return PLX_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w, q, k, v, rho};
  for (const void* p : ptrs)
    if (!aligned16(p)) return PLX_ERR_INVALID_ARG;
  return from_hip(plx::launch_proj(x, w, q, k, v, rho, B, T, D, Hq, Hkv, d, (hipStream_t)stream));
}

}  // extern "C"
