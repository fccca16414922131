// Measured ceilings of this GPU, for reading the kernels' roofline fractions
// beside the published peaks: the bf16 matrix-core rate the 16x16x32 MFMA
// sustains when nothing else is issued, and the rate at which a plain
// streaming kernel reads HBM.  Built into its own library (libplx_peak.so);
// nothing of the operator uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PK_CHAINS = 8;  // independent accumulator chains per wave

// Every wave runs PK_CHAINS independent chains of 16x16x32 bf16 MFMAs,
// iters deep; nothing else sits in the loop.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x4_t acc[PK_CHAINS];
#pragma unroll
  for (int i = 0; i < PK_CHAINS; ++i) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < PK_CHAINS; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PK_CHAINS; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  // a sum no input produces: the store is never taken, but the compiler
  // cannot drop the chains
  if (s == 1234567.0f) out[blockIdx.x] = s;
}

// Streaming read of n 16-byte chunks: the workgroups take 32 KB tiles in a
// grid-stride order, each thread keeping the eight loads of a tile in
// flight; the data only feed an XOR that decides a store that never happens.
constexpr int RD_UNROLL = 8;
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4_t* __restrict__ src, size_t n,
                                                       uint32_t* __restrict__ out) {
  constexpr size_t TILE = 256 * RD_UNROLL;
  const size_t ntiles = n / TILE;
  uint32_t x = 0;
  for (size_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const u32x4_t* p = src + t * TILE + threadIdx.x;
    u32x4_t v[RD_UNROLL];
#pragma unroll
    for (int j = 0; j < RD_UNROLL; ++j) v[j] = __builtin_nontemporal_load(p + 256 * j);
#pragma unroll
    for (int j = 0; j < RD_UNROLL; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // the tail past the last whole tile
  for (size_t i = ntiles * TILE + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const u32x4_t v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9E3779B9u) out[0] = x;
}

}  // namespace

extern "C" {

// Floating-point operations of one plx_peak_mfma_bf16 launch.
double plx_peak_mfma_flops(int blocks, int iters) {
  return (double)blocks * (256 / 64) * iters * PK_CHAINS * (2.0 * 16 * 16 * 32);
}

// Launches the MFMA loop on `stream`: `blocks` workgroups of four waves.
// `out` (device, >= blocks floats) is never written in practice.
int plx_peak_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned device memory) once on
// `stream`.  `out` (device, one uint32) is never written in practice.
int plx_peak_hbm_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  if (!src || !out || bytes % 16 || ((uintptr_t)src & 15) || blocks <= 0) return 1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4_t*)src,
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
