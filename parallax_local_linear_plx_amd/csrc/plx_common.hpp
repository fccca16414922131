// Shared device helpers for the Parallax kernels (CDNA4 / gfx950).
//
// MFMA conventions used by every kernel (wave64, 32x32 output tiles):
//   * A operand (32 x K): lane l holds row (l % 32) and the K-chunk picked by
//     the lane half h = l / 32.  B operand (K x 32): lane l holds column (l % 32)
//     and the same K-chunk.  A and B use the same chunk assignment, so a
//     contraction only needs both sides to agree on which key/dim sits in
//     (half, element); the kernels choose that assignment themselves.
//   * C/D (32 x 32, 16 fp32 per lane): acc[4*i + j] is row 8*i + 4*h + j,
//     column l % 32.
//   * 16x16 tiles (the bf16 prefill, decode and backward kernels): operands
//     give lane l row / column l % 16 and K-chunk l / 16; acc[j] is row
//     4 * (l / 16) + j, column l % 16.
// "Transposed" scoring (S^T = K Q^T) therefore puts one query per lane column
// and that query's keys along the accumulator, so row statistics (max, sums,
// rescale factors) stay inside a lane plus one exchange between lane halves,
// and the score accumulator feeds the next MFMA's B operand with no shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// bf16 -> fp16 conversion: exact for |x| in [2^-14, 65504] (every bf16 with
// 8 significant bits fits fp16's 11), rounded for smaller magnitudes.
__device__ __forceinline__ _Float16 bf16_bits_to_f16(uint16_t b) {
  return (_Float16)bf16_bits_to_f32(b);
}

// Operand policies.  `in_t` is the storage type of q, k, v, rho (and dO);
// `sop_t` is the MFMA operand of the score GEMMs (inputs exactly as stored);
// `vop_t` is the operand of the GEMMs whose other side is derived from the
// softmax weights (fp16 for the bf16 path: P in bf16 loses too much), with
// V / K / Q / rho / dO converted exactly to it when staged.
struct PolBF16 {
  using in_t = uint16_t;
  static constexpr int KW = 8;     // operand elements per lane per MFMA
  static constexpr int KSTEP = 16; // contraction depth per MFMA
  static constexpr int CW = 8;     // elements per 16-byte global chunk
  using sop_t = bf16x8;
  using vop_t = f16x8;
  using vel_t = _Float16;  // element type of value operands in LDS
  static __device__ __forceinline__ f32x16 mma_s(sop_t a, sop_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma_v(vop_t a, vop_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vel_t to_vel(in_t x) { return bf16_bits_to_f16(x); }
  static __device__ __forceinline__ float to_f32(in_t x) { return bf16_bits_to_f32(x); }
  static __device__ __forceinline__ vel_t round_v(float x) { return (_Float16)x; }
  static __device__ __forceinline__ float vel_to_f32(vel_t x) { return (float)x; }
};

struct PolF32 {
  using in_t = float;
  static constexpr int KW = 1;
  static constexpr int KSTEP = 2;
  static constexpr int CW = 4;
  using sop_t = float;
  using vop_t = float;
  using vel_t = float;
  static __device__ __forceinline__ f32x16 mma_s(sop_t a, sop_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mma_v(vop_t a, vop_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vel_t to_vel(in_t x) { return x; }
  static __device__ __forceinline__ float to_f32(in_t x) { return x; }
  static __device__ __forceinline__ vel_t round_v(float x) { return x; }
  static __device__ __forceinline__ float vel_to_f32(vel_t x) { return x; }
};

// Set element `e` of an operand vector (scalar policies have one element).
template <class V, class X>
__device__ __forceinline__ void set_elem(V& v, int e, X x) { v[e] = x; }
template <class X>
__device__ __forceinline__ void set_elem(float& v, int, X x) { v = x; }

// Key (row of a 32-row accumulator tile) held at accumulator slot a in lane
// half h: a = 4*i + j  ->  row 8*i + 4*h + j.
__device__ __forceinline__ int acc_row(int a, int h) { return 8 * (a >> 2) + 4 * h + (a & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Load one score operand (KW consecutive elements) from global memory.
template <class Pol>
__device__ __forceinline__ typename Pol::sop_t load_sop(const typename Pol::in_t* p);

template <>
__device__ __forceinline__ bf16x8 load_sop<PolBF16>(const uint16_t* p) {
  u32x4 raw = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, raw);
}
template <>
__device__ __forceinline__ float load_sop<PolF32>(const float* p) {
  return *p;
}

template <class Pol>
__device__ __forceinline__ typename Pol::sop_t zero_sop();
template <>
__device__ __forceinline__ bf16x8 zero_sop<PolBF16>() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}
template <>
__device__ __forceinline__ float zero_sop<PolF32>() {
  return 0.f;
}

// Exchange with the other lane half (lane ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Block order for a grid whose blocks enumerate (level, slot) with `slots`
// consecutive slots per level.  Consecutive block ids are dispatched round-
// robin to the 8 XCDs (each with its own L2), so without remapping every XCD
// sees every slot.  The remap gives XCD x the contiguous slot range
// [x*slots/8, (x+1)*slots/8) at every level (neighbouring heads share K/V),
// keeping each level's blocks in order.  Identity when slots or the grid is
// not a multiple of 8.
__device__ __forceinline__ int xcd_block_order(int id, int slots, int total) {
  if ((slots & 7) != 0 || (total & 7) != 0) return id;
  const int x = id & 7, m = id >> 3;
  const int per = slots >> 3;
  return (m / per) * slots + x * per + (m % per);
}

// Cooperative copy of ROWS rows of D elements (rows at or beyond `nvalid` read
// as zero) into a row-major LDS tile with row stride `ld` (elements).
template <class Pol, int D, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(typename Pol::in_t* dst, int ld,
                                           const typename Pol::in_t* src, int nvalid) {
  constexpr int CW = Pol::CW;
  constexpr int CPR = D / CW;
  for (int it = threadIdx.x; it < ROWS * CPR; it += NT) {
    const int r = it / CPR, c = (it % CPR) * CW;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < nvalid) val = *reinterpret_cast<const u32x4*>(src + (size_t)r * D + c);
    *reinterpret_cast<u32x4*>(dst + r * ld + c) = val;
  }
}

// Cooperative transposed copy: dst[d * ld + r] = to_vel(src[r][d]) for ROWS
// rows (zero at or beyond `nvalid`), two rows per work item so each LDS write
// stores a pair of adjacent rows.
template <class Pol, int D, int ROWS, int NT>
__device__ __forceinline__ void stage_rows_t(typename Pol::vel_t* dst, int ld,
                                             const typename Pol::in_t* src, int nvalid) {
  using in_t = typename Pol::in_t;
  constexpr int CW = Pol::CW;
  constexpr int CPR = D / CW;
  for (int it = threadIdx.x; it < (ROWS / 2) * CPR; it += NT) {
    const int rp = it / CPR, c = (it % CPR) * CW;
    const int r = 2 * rp;
    u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
    if (r < nvalid) va = *reinterpret_cast<const u32x4*>(src + (size_t)r * D + c);
    if (r + 1 < nvalid) vb = *reinterpret_cast<const u32x4*>(src + (size_t)(r + 1) * D + c);
    in_t a[CW], b[CW];
    __builtin_memcpy(a, &va, 16);
    __builtin_memcpy(b, &vb, 16);
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      typename Pol::vel_t* p = dst + (c + e) * ld + r;
      p[0] = Pol::to_vel(a[e]);
      p[1] = Pol::to_vel(b[e]);
    }
  }
}

// Value operand read from a transposed LDS tile: row `drow`, the 32-wide
// column block starting at `c0`, MFMA step `s`, lane half `h`; element e is
// column c0 + acc_row(KW*s + e, h), matching a score accumulator used as the
// other operand.
template <class Pol>
__device__ __forceinline__ typename Pol::vop_t load_t_op(const typename Pol::vel_t* tile, int ld,
                                                         int drow, int c0, int s, int h) {
  typename Pol::vop_t a;
  const typename Pol::vel_t* row = tile + drow * ld + c0;
#pragma unroll
  for (int e = 0; e < Pol::KW; ++e) set_elem(a, e, row[acc_row(Pol::KW * s + e, h)]);
  return a;
}

// LDS byte address of a shared-memory pointer, and transpose / 16-byte reads
// at such an address.  A base address the compiler cannot see through keeps
// every per-read displacement in the instruction's offset field.
typedef short lds_s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)((__attribute__((address_space(3))) const char*)p);
}
__device__ __forceinline__ f16x4 tr16_at(unsigned a) {
  lds_s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) lds_s16x4*)(size_t)a);
  return __builtin_bit_cast(f16x4, t);
}
__device__ __forceinline__ u32x4 ld128_at(unsigned a) {
  return *(__attribute__((address_space(3))) const u32x4*)(size_t)a;
}

}  // namespace plx
