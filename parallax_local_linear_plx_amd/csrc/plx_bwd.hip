// Backward of the causal Parallax prefill.
//
// The write-ups give no backward pass; these are the exact gradients of the
// forward with the probe rho an independent input.  Per query row i, with
// g = dO_i, the recomputed weights w_ij = exp(tau q_i.k_j - LSE_i),
// r_ij = rho_i . k_j, A_ij = g . v_j, G_i = g . o_i, delta_i = g . vbar_i and
// c_i = kbar_i . rho_i (so o_i = sum_j w_ij (1 + c_i - r_ij) v_j):
//   dV_j  = sum_i w_ij (1 + c_i - r_ij) g_i
//   dS_ij = w_ij [ (1 + c_i - r_ij) A_ij - G_i + delta_i (r_ij - c_i) ]
//   dR_ij = -w_ij (A_ij - delta_i)
//   dQ = tau dS K,  dK = tau dS^T Q + dR^T rho,  drho = dR K.
//
// Kernels, no atomics (the result is deterministic):
//   pre   : (fp32 inputs) G and delta per row.
//   cvt   : (bf16 inputs) an fp16 copy of k in the workspace.
//   dq    : query-outer, laid out like the forward (S^T = K Q^T, one query per
//           lane column): recomputes S, R and A^T = V dO^T per key tile, forms
//           dS, dR in registers and accumulates dQ^T = K^T dS^T, drho^T = K^T dR^T.
//           The bf16 kernel also forms G and delta of its rows and writes fp16
//           copies of q, rho and dO for the key-outer kernel.
//   dkdv  : key-outer: one key per lane column (S = Q K^T), loops over the
//           query tiles of every head that shares the KV head, accumulates
//           dV^T = dO^T Ptilde and dK^T = Q^T (tau dS) + rho^T dR.
// The bf16 dq and dkdv kernels run 16-row blocks on 16x16x32 fp16 MFMAs, two
// waves per SIMD; at d = 64 each wave carries two blocks (query rows in dq,
// keys in dkdv) so that one LDS operand read feeds both.  The fp32 kernels
// (the exact-parity path) run 32-row waves on fp32 MFMAs.
#include <algorithm>
#include <type_traits>

#include "plx_common.hpp"
#include "plx_kernels.hpp"

namespace plx {

namespace {

constexpr int BWD_THREADS = 256;

// ---------------------------------------------------------------- preprocess
template <class Pol, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const typename Pol::in_t* __restrict__ d_o,
                                                     const float* __restrict__ o,
                                                     const float* __restrict__ vbar,
                                                     float* __restrict__ G, float* __restrict__ delta,
                                                     long long rows) {
  constexpr int PER = D / 16;  // elements per thread, 16 threads per row
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  float g = 0.f, dl = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * D + t * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float x = Pol::to_f32(d_o[base + e]);
      g += x * o[base + e];
      dl += x * vbar[base + e];
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    g += __shfl_xor(g, off, 16);
    dl += __shfl_xor(dl, off, 16);
  }
  if (row < rows && t == 0) {
    G[row] = g;
    delta[row] = dl;
  }
}

// ------------------------------------------------------------- dQ and drho
constexpr int DQ_BR = 128;
constexpr int DQ_BC = 64;

template <class Pol, int D>
struct DqSmem {
  using in_t = typename Pol::in_t;
  using vel_t = typename Pol::vel_t;
  static constexpr int LD = D + 16 / sizeof(in_t);
  static constexpr int TLD = DQ_BC + 4;
  in_t k[DQ_BC * LD];
  in_t v[DQ_BC * LD];
  vel_t kt[D * TLD];
};

template <class Pol, int D>
__global__ __launch_bounds__(BWD_THREADS, 1) void bwd_dq_kernel(
    const typename Pol::in_t* __restrict__ q, const typename Pol::in_t* __restrict__ k,
    const typename Pol::in_t* __restrict__ v, const typename Pol::in_t* __restrict__ rho,
    const typename Pol::in_t* __restrict__ d_o, const float* __restrict__ lse,
    const float* __restrict__ c_aux, const float* __restrict__ Gv, const float* __restrict__ dlt,
    float* __restrict__ dq, float* __restrict__ drho, int B, int Hq, int Hkv, int T, float scale,
    float scale_log2) {
  using in_t = typename Pol::in_t;
  using sop_t = typename Pol::sop_t;
  using vop_t = typename Pol::vop_t;
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP;
  constexpr int NS = D / KSTEP, NV = 32 / KSTEP, ND = D / 32;
  using SM = DqSmem<Pol, D>;
  __shared__ SM sm;

  const int nqb = (T + DQ_BR - 1) / DQ_BR;
  const int bh_count = B * Hq;
  const int lin = xcd_block_order(blockIdx.x, bh_count, nqb * bh_count);
  const int qb = nqb - 1 - lin / bh_count;
  const int bh = lin % bh_count;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int q0 = qb * DQ_BR;
  const int qw = q0 + 32 * wave;
  const int my_q = qw + col;
  const bool qvalid = my_q < T;

  const size_t rowbase = (size_t)bh * T;
  sop_t qop[NS], rop[NS], gop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (qvalid) {
      const size_t off = (rowbase + my_q) * D + KSTEP * s + KW * half;
      qop[s] = load_sop<Pol>(q + off);
      rop[s] = load_sop<Pol>(rho + off);
      gop[s] = load_sop<Pol>(d_o + off);
    } else {
      qop[s] = rop[s] = gop[s] = zero_sop<Pol>();
    }
  }
  const float lse2 = qvalid ? lse[rowbase + my_q] * kLog2e : 0.f;
  const float ci = qvalid ? c_aux[rowbase + my_q] : 0.f;
  const float Gi = qvalid ? Gv[rowbase + my_q] : 0.f;
  const float di = qvalid ? dlt[rowbase + my_q] : 0.f;

  f32x16 dqa[ND], dra[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    dqa[i] = zero16();
    dra[i] = zero16();
  }

  const in_t* kp = k + ((size_t)(b * Hkv + hk) * T) * D;
  const in_t* vp = v + ((size_t)(b * Hkv + hk) * T) * D;
  const int kend = min(T, q0 + DQ_BR);
  const int ntiles = (kend + DQ_BC - 1) / DQ_BC;

  for (int j = 0; j < ntiles; ++j) {
    const int key0 = j * DQ_BC;
    const int nvalid = min(DQ_BC, T - key0);
    __syncthreads();
    stage_rows<Pol, D, DQ_BC, BWD_THREADS>(sm.k, SM::LD, kp + (size_t)key0 * D, nvalid);
    stage_rows<Pol, D, DQ_BC, BWD_THREADS>(sm.v, SM::LD, vp + (size_t)key0 * D, nvalid);
    stage_rows_t<Pol, D, DQ_BC, BWD_THREADS>(sm.kt, SM::TLD, kp + (size_t)key0 * D, nvalid);
    __syncthreads();
    if (key0 > qw + 31) continue;

    f32x16 sa[2], ra[2], aa[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sa[st] = ra[st] = aa[st] = zero16();
      const in_t* krow = &sm.k[(32 * st + col) * SM::LD + KW * half];
      const in_t* vrow = &sm.v[(32 * st + col) * SM::LD + KW * half];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const sop_t ak = load_sop<Pol>(krow + KSTEP * s);
        const sop_t av = load_sop<Pol>(vrow + KSTEP * s);
        sa[st] = Pol::mma_s(ak, qop[s], sa[st]);
        ra[st] = Pol::mma_s(ak, rop[s], ra[st]);
        aa[st] = Pol::mma_s(av, gop[s], aa[st]);
      }
    }
    // dS^T and dR^T in place of S^T and R^T
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = key0 + 32 * st + acc_row(a, half);
        float p = fast_exp2(__builtin_fmaf(sa[st][a], scale_log2, -lse2));
        if (key > my_q || !qvalid) p = 0.f;
        const float r = ra[st][a], A = aa[st][a];
        const float f = 1.f + ci - r;
        sa[st][a] = p * (f * A - Gi + di * (r - ci));
        ra[st][a] = -p * (A - di);
      }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int s = 0; s < NV; ++s) {
        vop_t dsop, drop;
#pragma unroll
        for (int e = 0; e < KW; ++e) {
          set_elem(dsop, e, Pol::round_v(sa[st][KW * s + e]));
          set_elem(drop, e, Pol::round_v(ra[st][KW * s + e]));
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const vop_t a = load_t_op<Pol>(sm.kt, SM::TLD, 32 * dt + col, 32 * st, s, half);
          dqa[dt] = Pol::mma_v(a, dsop, dqa[dt]);
          dra[dt] = Pol::mma_v(a, drop, dra[dt]);
        }
      }
  }

  if (qvalid) {
    float* dqr = dq + (rowbase + my_q) * D;
    float* drr = drho + (rowbase + my_q) * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * half;
        f32x4 x, y;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          x[jj] = scale * dqa[dt][4 * i + jj];
          y[jj] = dra[dt][4 * i + jj];
        }
        *reinterpret_cast<f32x4*>(dqr + d0) = x;
        *reinterpret_cast<f32x4*>(drr + d0) = y;
      }
  }
}

// --------------------------------------------------------------- dK and dV
constexpr int KV_BK = 128;  // keys per workgroup (32 per wave)

// Queries per LDS tile: 64 for 2-byte inputs; 32 for fp32 so that the six
// staged tiles of d = 128 stay within the 160 KB of LDS.
template <class Pol>
constexpr int kv_bq() {
  return sizeof(typename Pol::in_t) == 2 ? 64 : 32;
}

template <class Pol, int D>
struct DkvSmem {
  using in_t = typename Pol::in_t;
  using vel_t = typename Pol::vel_t;
  static constexpr int BQ = kv_bq<Pol>();
  static constexpr int LD = D + 16 / sizeof(in_t);
  static constexpr int TLD = BQ + 4;
  alignas(16) in_t q[BQ * LD];
  alignas(16) in_t r[BQ * LD];
  alignas(16) in_t g[BQ * LD];
  alignas(16) vel_t qt[D * TLD];
  alignas(16) vel_t rt[D * TLD];
  alignas(16) vel_t gt[D * TLD];
  alignas(16) float lse2[BQ];
  alignas(16) float c[BQ];
  alignas(16) float G[BQ];
  alignas(16) float dl[BQ];
};

template <class Pol, int D>
__global__ __launch_bounds__(BWD_THREADS, 1) void bwd_dkdv_kernel(
    const typename Pol::in_t* __restrict__ q, const typename Pol::in_t* __restrict__ k,
    const typename Pol::in_t* __restrict__ v, const typename Pol::in_t* __restrict__ rho,
    const typename Pol::in_t* __restrict__ d_o, const float* __restrict__ lse,
    const float* __restrict__ c_aux, const float* __restrict__ Gv, const float* __restrict__ dlt,
    float* __restrict__ dk, float* __restrict__ dv, int B, int Hq, int Hkv, int T, float scale,
    float scale_log2) {
  using in_t = typename Pol::in_t;
  using sop_t = typename Pol::sop_t;
  using vop_t = typename Pol::vop_t;
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP;
  constexpr int NS = D / KSTEP, NV = 32 / KSTEP, ND = D / 32;
  using SM = DkvSmem<Pol, D>;
  constexpr int KV_BQ = SM::BQ;
  __shared__ SM sm;

  const int bhk_count = B * Hkv;
  const int lin = blockIdx.x;
  const int kb = lin / bhk_count;  // ascending: early key blocks see the most queries
  const int bhk = lin % bhk_count;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int k0 = kb * KV_BK;
  const int kw = k0 + 32 * wave;
  const int my_k = kw + col;
  const bool kvalid = my_k < T;

  const size_t kvbase = (size_t)bhk * T;
  sop_t kop[NS], vop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (kvalid) {
      const size_t off = (kvbase + my_k) * D + KSTEP * s + KW * half;
      kop[s] = load_sop<Pol>(k + off);
      vop[s] = load_sop<Pol>(v + off);
    } else {
      kop[s] = vop[s] = zero_sop<Pol>();
    }
  }

  f32x16 dka[ND], dva[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    dka[i] = zero16();
    dva[i] = zero16();
  }

  for (int hh = 0; hh < G; ++hh) {
    const int h = hk * G + hh;
    const size_t rowbase = ((size_t)b * Hq + h) * T;
    for (int qt0 = k0; qt0 < T; qt0 += KV_BQ) {
      const int nvalid = min(KV_BQ, T - qt0);
      __syncthreads();
      stage_rows<Pol, D, KV_BQ, BWD_THREADS>(sm.q, SM::LD, q + (rowbase + qt0) * D, nvalid);
      stage_rows<Pol, D, KV_BQ, BWD_THREADS>(sm.r, SM::LD, rho + (rowbase + qt0) * D, nvalid);
      stage_rows<Pol, D, KV_BQ, BWD_THREADS>(sm.g, SM::LD, d_o + (rowbase + qt0) * D, nvalid);
      stage_rows_t<Pol, D, KV_BQ, BWD_THREADS>(sm.qt, SM::TLD, q + (rowbase + qt0) * D, nvalid);
      stage_rows_t<Pol, D, KV_BQ, BWD_THREADS>(sm.rt, SM::TLD, rho + (rowbase + qt0) * D, nvalid);
      stage_rows_t<Pol, D, KV_BQ, BWD_THREADS>(sm.gt, SM::TLD, d_o + (rowbase + qt0) * D, nvalid);
      if (threadIdx.x < KV_BQ) {
        const int i = threadIdx.x;
        const bool ok = i < nvalid;
        sm.lse2[i] = ok ? lse[rowbase + qt0 + i] * kLog2e : 0.f;
        sm.c[i] = ok ? c_aux[rowbase + qt0 + i] : 0.f;
        sm.G[i] = ok ? Gv[rowbase + qt0 + i] : 0.f;
        sm.dl[i] = ok ? dlt[rowbase + qt0 + i] : 0.f;
      }
      __syncthreads();

#pragma unroll
      for (int st = 0; st < KV_BQ / 32; ++st) {
        const int qs = qt0 + 32 * st;
        if (qs + 31 < kw) continue;  // every query of the sub-tile precedes every key of the wave
        f32x16 sa = zero16(), ra = zero16(), aa = zero16();
        const in_t* qrow = &sm.q[(32 * st + col) * SM::LD + KW * half];
        const in_t* rrow = &sm.r[(32 * st + col) * SM::LD + KW * half];
        const in_t* grow = &sm.g[(32 * st + col) * SM::LD + KW * half];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          sa = Pol::mma_s(load_sop<Pol>(qrow + KSTEP * s), kop[s], sa);
          ra = Pol::mma_s(load_sop<Pol>(rrow + KSTEP * s), kop[s], ra);
          aa = Pol::mma_s(load_sop<Pol>(grow + KSTEP * s), vop[s], aa);
        }
        // lane column = key my_k; accumulator slot a = query qs + acc_row(a, half)
        float pt[16], ds[16], dr[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = 32 * st + 8 * i4 + 4 * half;  // local query of slot 4*i4
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[r0]);
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(&sm.c[r0]);
          const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sm.G[r0]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dl[r0]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int a = 4 * i4 + jj;
            const int qi = qt0 + r0 + jj;
            float p = fast_exp2(__builtin_fmaf(sa[a], scale_log2, -l4[jj]));
            if (qi < my_k || qi >= T) p = 0.f;
            const float r = ra[a], A = aa[a];
            const float f = 1.f + c4[jj] - r;
            pt[a] = p * f;
            ds[a] = scale * p * (f * A - g4[jj] + d4[jj] * (r - c4[jj]));
            dr[a] = -p * (A - d4[jj]);
          }
        }
#pragma unroll
        for (int s = 0; s < NV; ++s) {
          vop_t pop, dsop, drop;
#pragma unroll
          for (int e = 0; e < KW; ++e) {
            set_elem(pop, e, Pol::round_v(pt[KW * s + e]));
            set_elem(dsop, e, Pol::round_v(ds[KW * s + e]));
            set_elem(drop, e, Pol::round_v(dr[KW * s + e]));
          }
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            const int drow = 32 * dt + col;
            const vop_t ag = load_t_op<Pol>(sm.gt, SM::TLD, drow, 32 * st, s, half);
            const vop_t aq = load_t_op<Pol>(sm.qt, SM::TLD, drow, 32 * st, s, half);
            const vop_t ar = load_t_op<Pol>(sm.rt, SM::TLD, drow, 32 * st, s, half);
            dva[dt] = Pol::mma_v(ag, pop, dva[dt]);
            dka[dt] = Pol::mma_v(aq, dsop, dka[dt]);
            dka[dt] = Pol::mma_v(ar, drop, dka[dt]);
          }
        }
      }
    }
  }

  if (kvalid) {
    float* dkr = dk + (kvbase + my_k) * D;
    float* dvr = dv + (kvbase + my_k) * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * half;
        f32x4 x, y;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          x[jj] = dka[dt][4 * i + jj];
          y[jj] = dva[dt][4 * i + jj];
        }
        *reinterpret_cast<f32x4*>(dkr + d0) = x;
        *reinterpret_cast<f32x4*>(dvr + d0) = y;
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 path.  Q, rho, dO, K and V enter every MFMA of the two main kernels as
// fp16: the bf16 -> fp16 conversion is exact over fp16's normal range, and
// fp16 operands let one row-major LDS tile serve both the score GEMMs (rows
// read with ds_read_b128) and the gradient GEMMs (transpose reads,
// ds_read_b64_tr_b16).  A conversion pass writes the fp16 copies once.
//
// Every gradient is linear in dO, and so are the fp16 operands formed from it
// (dO itself, dS, dR).  An upstream gradient far from unit scale (a loss
// averaged over many tokens gives |dO| ~ 1e-6) would put them on fp16's
// subnormal grid, or past its largest value.  The kernels therefore run on
// s dO, with s the power of two that brings max |dO| into [1, 2), and
// multiply the four gradients by 1 / s as they store them.  Both scalings are
// exact, so the result does not depend on the scale of dO except through
// fp32 underflow or overflow of the gradients themselves.
inline size_t bwd_ws_align(size_t n) { return (n + 255) & ~(size_t)255; }
// 16-key blocks per dK/dV wave and 16-row blocks per dQ wave at d = 64 (one
// block each at d = 128 and 256, where the registers hold no second block);
// 1 builds the one-block kernels, which give the same gradients bit for bit.
#ifndef PLX_KB64
#define PLX_KB64 2
#endif
#ifndef PLX_QB64
#define PLX_QB64 2
#endif

// Workgroups of the preparation pass: each reduces its part of dO to one
// partial maximum, which bounds the partials buffer in the workspace.
constexpr int kPrepBlocks = 2048;
inline size_t bwd_head_bytes(size_t rows) {
  return bwd_ws_align(2 * rows * sizeof(float)) + bwd_ws_align((4 + kPrepBlocks) * sizeof(unsigned));
}

__device__ __forceinline__ f16x8 cvt_bf16x8_f16(u32x4 raw) {
  const u16x8 b = __builtin_bit_cast(u16x8, raw);
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = bf16_bits_to_f16(b[e]);
  return h;
}

// Preparation pass, one grid-stride sweep per tensor:
//  - bf16 -> fp16 copy of K (nk8 chunks of 8 elements): the dQ kernel stages
//    its K tiles from this copy, so a tile read by every query block of a head
//    is not converted again by each of them;
//  - the largest |dO| of this workgroup's chunks (ng8 of them), as bf16 bits
//    (for non-negative bf16 values the bit patterns order as the values do).
__global__ __launch_bounds__(256) void bwd_prep16_kernel(const u32x4* __restrict__ k,
                                                        f16x8* __restrict__ k16, long long nk8,
                                                        const u32x4* __restrict__ d_o, long long ng8,
                                                        unsigned* __restrict__ part) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < nk8; i += stride)
    k16[i] = cvt_bf16x8_f16(k[i]);
  unsigned m = 0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < ng8; i += stride) {
    const u32x4 x = d_o[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max(m, max(x[e] & 0x7fffu, (x[e] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  __shared__ unsigned wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
}

// One workgroup: the largest of the n partial maxima gives the dO scale s (a
// power of two with s max|dO| in [1, 2)) and its inverse, written to sc[0..1].
// An all-zero dO, or one holding an infinity or NaN, keeps s = 1.
__global__ __launch_bounds__(256) void bwd_scale_kernel(const unsigned* __restrict__ part, int n,
                                                       float* __restrict__ sc) {
  unsigned m = 0;
  for (int i = threadIdx.x; i < n; i += 256) m = max(m, part[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  __shared__ unsigned wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
    // biased exponent of max|dO| (bf16 shares fp32's 8-bit exponent)
    const int ex = (int)(m >> 7);
    int e2 = 0;
    if (m != 0 && ex < 255) e2 = min(126, max(-126, 127 - max(ex, 1)));
    sc[0] = __builtin_ldexpf(1.f, e2);
    sc[1] = __builtin_ldexpf(1.f, -e2);
  }
}

// dQ and drho on 16x16x32 MFMA tiles, two waves per SIMD (bf16 inputs).  The
// layout follows the forward kernel: a wave owns 16 query rows (lane column
// c = lane % 16; the four 16-lane groups g split the keys of a score tile and
// the head dimension of the gradient tiles).  Per 32-key sub-tile:
//   S^T, R^T = K [Q; rho]^T (fp16 MFMAs: K from its fp16 copy, Q and rho
//     converted in registers) and A^T = V dO^T (bf16 MFMAs on the inputs as
//     stored), 32 keys x 16 queries, A = K / V rows from LDS, B from registers;
//   dS^T, dR^T in registers, rounded to the fp16 B operand of
//   [dQ | drho]^T += K^T [dS | dR]^T, A = K^T from transpose reads of the K tile.
// Workgroup: 8 waves, 128 query rows of one (b, h); 128-key K / V tiles
// double-buffered in LDS, one barrier per tile.
// The kernel also does the per-row preprocessing the key-outer kernel needs,
// for the rows it owns: G_i = dO_i . o_i, delta_i = dO_i . vbar_i, and fp16
// copies of q_i, rho_i and dO_i (the key-outer kernel's LDS tiles), so no
// separate pass reads dO, o and vbar.
// Shape per head dim (bwd16_shape): d <= 128 runs 8 waves (two per SIMD) on
// 128-key tiles; d = 256 runs 4 waves (one per SIMD: its doubled operands and
// accumulators need the whole register file) on 32-key tiles, which keeps the
// double-buffered tiles and their staging registers within LDS and registers.
template <int D, int BC>
struct DqbSmem {
  static constexpr int LD = D + 16;  // as the forward's tiles: conflict-free rows and transpose reads
  alignas(16) _Float16 k[2][BC * LD];
  alignas(16) uint16_t v[2][BC * LD];  // bf16, as stored
};

// QB: 16-row query blocks per wave; each K / V operand read from LDS feeds
// the MFMAs of all QB blocks (QB = 2 at d = 64, where the registers allow it).
template <int D, int NW, int BC, int QB>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq16b_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k16, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ rho, const uint16_t* __restrict__ d_o, const float* __restrict__ o,
    const float* __restrict__ vbar, const float* __restrict__ lse, const float* __restrict__ c_aux,
    float* __restrict__ Gv, float* __restrict__ dlt, _Float16* __restrict__ q16,
    _Float16* __restrict__ r16, _Float16* __restrict__ g16, const float* __restrict__ dsc,
    float* __restrict__ dq, float* __restrict__ drho, int B, int Hq, int Hkv, int T, float scale,
    float scale_log2) {
  constexpr int NT = 64 * NW, BR = 16 * NW * QB;
  constexpr int NS = D / 32, ND = D / 16, CPR = D / 8;
  constexpr int NCH = BC * CPR / NT;  // 16-byte chunks per thread per tile and tensor
  using SM = DqbSmem<D, BC>;
  __shared__ SM sm;

  const int nqb = (T + BR - 1) / BR;
  const int bh_count = B * Hq;
  const int lin = xcd_block_order(blockIdx.x, bh_count, nqb * bh_count);
  const int qb = nqb - 1 - lin / bh_count;
  const int bh = lin % bh_count;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int q0 = qb * BR;
  const int qw = q0 + 16 * QB * wave;  // first query of the wave; block qb2 starts at qw + 16 qb2

  const size_t rowbase = (size_t)bh * T;
  const uint16_t* kp = k16 + ((size_t)(b * Hkv + hk) * T) * D;
  const uint16_t* vp = v + ((size_t)(b * Hkv + hk) * T) * D;
  const int kend = min(T, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;
  const int nsub = (min(kend, qw + 16 * QB) + 31) / 32;

  // global -> register staging of one tile (rows past T read row T-1: finite,
  // and masked by the causal test since they follow every query)
  u32x4 pk[NCH], pv[NCH];
  auto gload = [&](int key0) {
    if (key0 + BC <= T) {
      // whole tile in range: a uniform tile base plus this thread's fixed offsets
      const uint16_t* kt = kp + (size_t)key0 * D;
      const uint16_t* vt = vp + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int off = (threadIdx.x + NT * i) * 8;  // row * D + column
        pk[i] = *reinterpret_cast<const u32x4*>(kt + off);
        pv[i] = *reinterpret_cast<const u32x4*>(vt + off);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int it = threadIdx.x + NT * i;
      const size_t off = (size_t)min(key0 + it / CPR, T - 1) * D + (it % CPR) * 8;
      pk[i] = *reinterpret_cast<const u32x4*>(kp + off);
      pv[i] = *reinterpret_cast<const u32x4*>(vp + off);
    }
  };
  auto lds_put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int it = threadIdx.x + NT * i;
      const int o = (it / CPR) * SM::LD + (it % CPR) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[buf][o]) = pk[i];
      *reinterpret_cast<u32x4*>(&sm.v[buf][o]) = pv[i];
    }
  };

  gload(0);
  // dO scale s and 1 / s (powers of two, from the preparation pass)
  const float gsc = dsc[0], ginv = dsc[1];
  // this lane's quarter of its query rows: elements 32 s + 8 g .. + 8
  f16x8 qop[QB][NS], rop[QB][NS];
  bf16x8 gop[QB][NS];
  // per query row: lse * log2e, delta, and (dS = p [A k1 + r (delta - A) - k2])
  // k1 = 1 + c, k2 = G + delta c
  float lse2[QB], di[QB], k1[QB], k2[QB];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    const int my_q = qw + 16 * qb2 + c;
    const bool qvalid = my_q < T;
    float Gi = 0.f, dd = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 qa = {0u, 0u, 0u, 0u}, ra = qa, ga = qa;
      if (qvalid) {
        const size_t off = (rowbase + my_q) * D + 32 * s + 8 * g;
        qa = *reinterpret_cast<const u32x4*>(q + off);
        ra = *reinterpret_cast<const u32x4*>(rho + off);
        ga = *reinterpret_cast<const u32x4*>(d_o + off);
        // s dO is exact in bf16 (a power of two moves only the exponent)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __builtin_bit_cast(float, ga[e] << 16) * gsc;
          const float hi = __builtin_bit_cast(float, ga[e] & 0xffff0000u) * gsc;
          ga[e] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xffff0000u);
        }
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(o + off);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(o + off + 4);
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(vbar + off);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(vbar + off + 4);
        const u16x8 gb = __builtin_bit_cast(u16x8, ga);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_bits_to_f32(gb[e]), x1 = bf16_bits_to_f32(gb[4 + e]);
          Gi = __builtin_fmaf(x0, o0[e], __builtin_fmaf(x1, o1[e], Gi));
          dd = __builtin_fmaf(x0, v0[e], __builtin_fmaf(x1, v1[e], dd));
        }
      }
      qop[qb2][s] = cvt_bf16x8_f16(qa);
      rop[qb2][s] = cvt_bf16x8_f16(ra);
      gop[qb2][s] = __builtin_bit_cast(bf16x8, ga);
      if (qvalid) {
        const size_t off = (rowbase + my_q) * D + 32 * s + 8 * g;
        *reinterpret_cast<f16x8*>(q16 + off) = qop[qb2][s];
        *reinterpret_cast<f16x8*>(r16 + off) = rop[qb2][s];
        *reinterpret_cast<f16x8*>(g16 + off) = cvt_bf16x8_f16(ga);
      }
    }
    // the four 16-lane groups hold disjoint quarters of the row
    Gi += __shfl_xor(Gi, 16, 64);
    Gi += __shfl_xor(Gi, 32, 64);
    dd += __shfl_xor(dd, 16, 64);
    dd += __shfl_xor(dd, 32, 64);
    if (qvalid && g == 0) {
      Gv[rowbase + my_q] = Gi;
      dlt[rowbase + my_q] = dd;
    }
    lse2[qb2] = qvalid ? lse[rowbase + my_q] * kLog2e : 0.f;
    const float ci = qvalid ? c_aux[rowbase + my_q] : 0.f;
    di[qb2] = dd;
    k1[qb2] = 1.f + ci;
    k2[qb2] = Gi + dd * ci;
  }  // query blocks
  lds_put(0);
  __syncthreads();

  f32x4 dqa[QB][ND], dra[QB][ND];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dqa[qb2][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dra[qb2][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

  auto subtile = [&](int buf, int st, int kbase) {
    // scores S^T, R^T and A^T = V dO^T for 32 keys
    unsigned kaddr = lds_addr(&sm.k[buf][(32 * st + c) * SM::LD + 8 * g]);
    unsigned vaddr = lds_addr(&sm.v[buf][(32 * st + c) * SM::LD + 8 * g]);
    asm volatile("" : "+v"(kaddr), "+v"(vaddr));
    f16x8 ka[2][NS];
    bf16x8 va[2][NS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        ka[t][s] = __builtin_bit_cast(f16x8, ld128_at(kaddr + 2 * (16 * t * SM::LD + 32 * s)));
        va[t][s] = __builtin_bit_cast(bf16x8, ld128_at(vaddr + 2 * (16 * t * SM::LD + 32 * s)));
      }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    f32x4 sacc[QB][2], racc[QB][2], aacc[QB][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          sacc[qb2][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[t][s], qop[qb2][s], s == 0 ? z : sacc[qb2][t], 0, 0, 0);
          racc[qb2][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[t][s], rop[qb2][s], s == 0 ? z : racc[qb2][t], 0, 0, 0);
          aacc[qb2][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[t][s], gop[qb2][s], s == 0 ? z : aacc[qb2][t], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    // K^T operands of the gradient MFMAs, in flight during the elementwise part
    unsigned taddr = lds_addr(&sm.k[buf][(32 * st + 4 * g + (c >> 2)) * SM::LD + 4 * (c & 3)]);
    asm volatile("" : "+v"(taddr));
    f16x8 kt[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      kt[dt] = __builtin_shufflevector(tr16_at(taddr + 2 * 16 * dt),
                                       tr16_at(taddr + 2 * (16 * dt + 16 * SM::LD)), 0, 1, 2, 3, 4, 5, 6, 7);
    __builtin_amdgcn_sched_barrier(0);
    // causal mask where the sub-tile reaches past the wave's first query (a
    // uniform branch: one code path for every sub-tile, so the accumulators
    // stay in place instead of being copied where two variants would join)
    if (kbase + 31 > qw) {
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kbase + 16 * t + 4 * g + j > qw + 16 * qb2 + c) sacc[qb2][t][j] = -INFINITY;
    }
    // dS^T, dR^T: element e of group g is key 16 (e / 4) + 4 g + e % 4, query c
    f16x8 dsop[QB], drop[QB];
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = e >> 2, j = e & 3;
        const float p = fast_exp2(__builtin_fmaf(sacc[qb2][t][j], scale_log2, -lse2[qb2]));
        const float r = racc[qb2][t][j], A = aacc[qb2][t][j];
        const float tt = di[qb2] - A;
        dsop[qb2][e] = (_Float16)(p * __builtin_fmaf(A, k1[qb2], __builtin_fmaf(r, tt, -k2[qb2])));
        drop[qb2][e] = (_Float16)(p * tt);
      }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) {
        dqa[qb2][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kt[dt], dsop[qb2], dqa[qb2][dt], 0, 0, 0);
        dra[qb2][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kt[dt], drop[qb2], dra[qb2][dt], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  auto iter = [&](int j, int buf) {
    const int key0 = j * BC;
    if (j + 1 < ntiles) gload(key0 + BC);
#pragma unroll
    for (int st = 0; st < BC / 32; ++st) {
      const int kbase = key0 + 32 * st;
      if ((BC / 32) * j + st < nsub) subtile(buf, st, kbase);
    }
    if (j + 1 < ntiles) lds_put(buf ^ 1);
    __syncthreads();
  };
  for (int j = 0; j < ntiles; j += 2) {
    iter(j, 0);
    if (j + 1 < ntiles) iter(j + 1, 1);
  }

  // dqa[qb2][dt][jj] is d = 16 dt + 4 g + jj of query qw + 16 qb2 + c
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    const int my_q = qw + 16 * qb2 + c;
    if (my_q < T) {
      float* dqr = dq + (rowbase + my_q) * D;
      float* drr = drho + (rowbase + my_q) * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        f32x4 x, y;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          x[jj] = (scale * ginv) * dqa[qb2][dt][jj];
          y[jj] = ginv * dra[qb2][dt][jj];
        }
        *reinterpret_cast<f32x4*>(dqr + 16 * dt + 4 * g) = x;
        *reinterpret_cast<f32x4*>(drr + 16 * dt + 4 * g) = y;
      }
    }
  }
}

// dK and dV on 16x16x32 MFMA tiles, two waves per SIMD (bf16 inputs, read
// from their fp16 copies).  A wave owns 16 keys (lane column c = lane % 16 is
// the key; the 16-lane groups g split the queries of a score tile and the head
// dimension of the gradient tiles).  Per 32-query sub-tile:
//   S, R = [Q; rho] K^T and A = dO V^T (32 queries x 16 keys), A operand = Q /
//     rho / dO rows from LDS, B = K / V from registers;
//   P (1 + c - r), tau dS and dR in registers, rounded to the fp16 B operands of
//   dV^T += dO^T [P (1 + c - r)],  dK^T += Q^T [tau dS] + rho^T dR,
//   A = Q^T / rho^T / dO^T from transpose reads of the query tiles.
// Workgroup: 8 waves, 128 keys of one KV head; the 64-row query tiles of all G
// query heads form one sequence, double-buffered in LDS, one barrier per tile.
template <int D, int BQ>
struct DkbSmem {
  static constexpr int LD = D + 16;
  alignas(16) _Float16 q[2][BQ * LD];
  alignas(16) _Float16 r[2][BQ * LD];
  alignas(16) _Float16 g[2][BQ * LD];
  alignas(16) float sc[2][BQ][4];  // per query row: lse * log2e, 1 + c, G + delta c, delta
};

// KB: 16-key blocks per wave; each query-tile operand read from LDS feeds
// the MFMAs of all KB blocks (KB = 2 at d = 64, where the registers allow it).
template <int D, int NW, int BQ, int KB>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv16b_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ rho, const uint16_t* __restrict__ d_o, const float* __restrict__ lse,
    const float* __restrict__ c_aux, const float* __restrict__ Gv, const float* __restrict__ dlt,
    const float* __restrict__ dsc, float* __restrict__ dk, float* __restrict__ dv, int B, int Hq,
    int Hkv, int T, float scale, float scale_log2) {
  constexpr int NT = 64 * NW, BK = 16 * NW * KB;
  constexpr int NS = D / 32, ND = D / 16, CPR = D / 8;
  constexpr int NCH = BQ * CPR / NT;  // 16-byte chunks per thread per tile and tensor
  using SM = DkbSmem<D, BQ>;
  __shared__ SM sm;

  const int bhk_count = B * Hkv;
  const int kb = blockIdx.x / bhk_count;
  const int bhk = blockIdx.x % bhk_count;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int k0 = kb * BK;
  const int kw = k0 + 16 * KB * wave;  // first key of the wave; block kb2 starts at kw + 16 kb2

  const size_t kvbase = (size_t)bhk * T;
  const float ginv = dsc[1];  // 1 / s of the dO scale
  const int nqt = (T - k0 + BQ - 1) / BQ;  // query tiles per head (queries >= k0)
  const int ntile = G * nqt;

  u32x4 pq[NCH], pr[NCH], pg[NCH];
  float psc[4];
  // Tiles are loaded, and then computed, in increasing order n = hh * nqt + i,
  // so each side keeps its (head, tile) pair as a cursor that advances by one
  // tile instead of dividing n by nqt.
  int ld_hh = 0, ld_i = 0, cp_hh = 0, cp_i = 0;
  auto advance = [&](int n, int& hh, int& i) {
    if (hh * nqt + i != n && ++i == nqt) {
      i = 0;
      ++hh;
    }
  };
  auto tile_rows = [&](int n, size_t& rowbase, int& qt0) {
    advance(n, ld_hh, ld_i);
    qt0 = k0 + ld_i * BQ;
    rowbase = ((size_t)b * Hq + hk * G + ld_hh) * T;
  };
  auto gload = [&](int n) {
    size_t rowbase;
    int qt0;
    tile_rows(n, rowbase, qt0);
    if (threadIdx.x < BQ) {
      const size_t r = rowbase + min(qt0 + (int)threadIdx.x, T - 1);
      psc[0] = lse[r];
      psc[1] = c_aux[r];
      psc[2] = Gv[r];
      psc[3] = dlt[r];
    }
    if (qt0 + BQ <= T) {
      // whole tile in range: a uniform tile base plus this thread's fixed offsets
      const size_t tb = (rowbase + qt0) * D;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int off = (threadIdx.x + NT * i) * 8;  // row * D + column
        pq[i] = *reinterpret_cast<const u32x4*>(q + tb + off);
        pr[i] = *reinterpret_cast<const u32x4*>(rho + tb + off);
        pg[i] = *reinterpret_cast<const u32x4*>(d_o + tb + off);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int it = threadIdx.x + NT * i;
      const size_t off = (rowbase + min(qt0 + it / CPR, T - 1)) * D + (it % CPR) * 8;
      pq[i] = *reinterpret_cast<const u32x4*>(q + off);
      pr[i] = *reinterpret_cast<const u32x4*>(rho + off);
      pg[i] = *reinterpret_cast<const u32x4*>(d_o + off);
    }
  };
  auto lds_put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int it = threadIdx.x + NT * i;
      const int o = (it / CPR) * SM::LD + (it % CPR) * 8;
      *reinterpret_cast<u32x4*>(&sm.q[buf][o]) = pq[i];
      *reinterpret_cast<u32x4*>(&sm.r[buf][o]) = pr[i];
      *reinterpret_cast<u32x4*>(&sm.g[buf][o]) = pg[i];
    }
    if (threadIdx.x < BQ)
      *reinterpret_cast<f32x4*>(&sm.sc[buf][threadIdx.x][0]) =
          (f32x4){psc[0] * kLog2e, 1.f + psc[1], psc[2] + psc[3] * psc[1], psc[3]};
  };

  gload(0);
  f16x8 kop[KB][NS], vop[KB][NS];
#pragma unroll
  for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int my_k = kw + 16 * kb2 + c;
      u32x4 ka = {0u, 0u, 0u, 0u}, va = ka;
      if (my_k < T) {
        const size_t off = (kvbase + my_k) * D + 32 * s + 8 * g;
        ka = *reinterpret_cast<const u32x4*>(k + off);
        va = *reinterpret_cast<const u32x4*>(v + off);
      }
      kop[kb2][s] = cvt_bf16x8_f16(ka);  // K and V as stored (bf16), converted once here
      vop[kb2][s] = cvt_bf16x8_f16(va);
    }
  lds_put(0);
  __syncthreads();

  f32x4 dka[KB][ND], dva[KB][ND];
#pragma unroll
  for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dka[kb2][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dva[kb2][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

  // one 32-query sub-tile st of the tile in buffer buf (first query qs)
  auto subtile = [&](int buf, int st, int qs) {
    f32x4 sacc[KB][2], racc[KB][2], aacc[KB][2];
    {
      unsigned qa = lds_addr(&sm.q[buf][(32 * st + c) * SM::LD + 8 * g]);
      unsigned ra = lds_addr(&sm.r[buf][(32 * st + c) * SM::LD + 8 * g]);
      unsigned ga = lds_addr(&sm.g[buf][(32 * st + c) * SM::LD + 8 * g]);
      asm volatile("" : "+v"(qa), "+v"(ra), "+v"(ga));
      // one 16-query tile at a time: its twelve operands are read before its MFMAs
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f16x8 qo[NS], ro[NS], go[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const unsigned off = 2 * (16 * t * SM::LD + 32 * s);
          qo[s] = __builtin_bit_cast(f16x8, ld128_at(qa + off));
          ro[s] = __builtin_bit_cast(f16x8, ld128_at(ra + off));
          go[s] = __builtin_bit_cast(f16x8, ld128_at(ga + off));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int kb2 = 0; kb2 < KB; ++kb2) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            sacc[kb2][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qo[s], kop[kb2][s], s == 0 ? z : sacc[kb2][t], 0, 0, 0);
            racc[kb2][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ro[s], kop[kb2][s], s == 0 ? z : racc[kb2][t], 0, 0, 0);
            aacc[kb2][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(go[s], vop[kb2][s], s == 0 ? z : aacc[kb2][t], 0, 0, 0);
          }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    // accumulator element j of key tile t: query qs + 16 t + 4 g + j, key c;
    // the same order as the K index of the transpose-read A operands below.
    // Causal mask (queries before the key) and rows past T, in a uniform
    // branch: one code path for every sub-tile (see the dQ kernel).
    if (qs < kw + 16 * KB - 1 || qs + 31 >= T) {
#pragma unroll
      for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int qi = qs + 16 * t + 4 * g + j;
            if (qi < kw + 16 * kb2 + c || qi >= T) sacc[kb2][t][j] = -INFINITY;
          }
    }
    f16x8 pop[KB], dsop[KB], drop[KB];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 32 * st + 16 * t + 4 * g;
      f32x4 rs[4];  // lse * log2e, 1 + c, G + delta c, delta of query r0 + j
#pragma unroll
      for (int j = 0; j < 4; ++j) rs[j] = *reinterpret_cast<const f32x4*>(&sm.sc[buf][r0 + j][0]);
#pragma unroll
      for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = fast_exp2(__builtin_fmaf(sacc[kb2][t][j], scale_log2, -rs[j][0]));
          const float r = racc[kb2][t][j], A = aacc[kb2][t][j];
          // with f = 1 + c - r:  dS = p [f A + delta r - (G + delta c)],  dR = p (delta - A)
          const float f = rs[j][1] - r;
          pop[kb2][4 * t + j] = (_Float16)(p * f);
          dsop[kb2][4 * t + j] = (_Float16)((scale * p) * __builtin_fmaf(A, f, __builtin_fmaf(r, rs[j][3], -rs[j][2])));
          drop[kb2][4 * t + j] = (_Float16)(p * (rs[j][3] - A));
        }
    }
    // gradient MFMAs: A = Q^T / rho^T / dO^T, 16 d rows x 32 queries each
    unsigned tq = lds_addr(&sm.q[buf][(32 * st + 4 * g + (c >> 2)) * SM::LD + 4 * (c & 3)]);
    unsigned tr = lds_addr(&sm.r[buf][(32 * st + 4 * g + (c >> 2)) * SM::LD + 4 * (c & 3)]);
    unsigned tg = lds_addr(&sm.g[buf][(32 * st + 4 * g + (c >> 2)) * SM::LD + 4 * (c & 3)]);
    asm volatile("" : "+v"(tq), "+v"(tr), "+v"(tg));
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const unsigned o0 = 2 * 16 * dt, o1 = 2 * (16 * dt + 16 * SM::LD);
      const f16x8 aq = __builtin_shufflevector(tr16_at(tq + o0), tr16_at(tq + o1), 0, 1, 2, 3, 4, 5, 6, 7);
      const f16x8 ar = __builtin_shufflevector(tr16_at(tr + o0), tr16_at(tr + o1), 0, 1, 2, 3, 4, 5, 6, 7);
      const f16x8 ag = __builtin_shufflevector(tr16_at(tg + o0), tr16_at(tg + o1), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int kb2 = 0; kb2 < KB; ++kb2) {
        dva[kb2][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ag, pop[kb2], dva[kb2][dt], 0, 0, 0);
        dka[kb2][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, dsop[kb2], dka[kb2][dt], 0, 0, 0);
        dka[kb2][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ar, drop[kb2], dka[kb2][dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto iter = [&](int n, int buf) {
    advance(n, cp_hh, cp_i);
    const int qt0 = k0 + cp_i * BQ;
    if (n + 1 < ntile) gload(n + 1);
#pragma unroll
    for (int st = 0; st < BQ / 32; ++st) {
      const int qs = qt0 + 32 * st;
      if (qs + 31 < kw) continue;  // every query of the sub-tile precedes every key of the wave
      subtile(buf, st, qs);
    }
    if (n + 1 < ntile) lds_put(buf ^ 1);  // buffer last read in iteration n-1
    __syncthreads();
  };
  for (int n = 0; n < ntile; n += 2) {
    iter(n, 0);
    if (n + 1 < ntile) iter(n + 1, 1);
  }

  // dka[kb2][dt][jj] is d = 16 dt + 4 g + jj of key kw + 16 kb2 + c; the sums ran on s dO
#pragma unroll
  for (int kb2 = 0; kb2 < KB; ++kb2) {
    const int my_k = kw + 16 * kb2 + c;
    if (my_k < T) {
      float* dkr = dk + (kvbase + my_k) * D;
      float* dvr = dv + (kvbase + my_k) * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        f32x4 x, y;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          x[jj] = ginv * dka[kb2][dt][jj];
          y[jj] = ginv * dva[kb2][dt][jj];
        }
        *reinterpret_cast<f32x4*>(dkr + 16 * dt + 4 * g) = x;
        *reinterpret_cast<f32x4*>(dvr + 16 * dt + 4 * g) = y;
      }
    }
  }
}

template <class Pol, int D>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* rho,
                        const void* d_o, const float* o, const float* lse, const float* c_aux,
                        const float* vbar, float* dq, float* dk, float* dv, float* drho, int B,
                        int Hq, int Hkv, int T, float scale, float* ws, hipStream_t stream) {
  using in_t = typename Pol::in_t;
  const long long rows = (long long)B * Hq * T;
  float* G = ws;
  float* dl = ws + rows;
  hipError_t e;
  const int nqb = (T + DQ_BR - 1) / DQ_BR;
  const int nkb = (T + KV_BK - 1) / KV_BK;
  if constexpr (sizeof(in_t) == 2) {
    // workspace after G and delta: fp16 copies of q, rho, dO (written by the
    // dQ kernel) and of K (written by the conversion pass)
    const size_t nq = (size_t)rows * D, nk = (size_t)B * Hkv * T * D;
    float* dsc = (float*)((char*)ws + bwd_ws_align(2 * rows * sizeof(float)));
    unsigned* part = (unsigned*)(dsc + 4);
    _Float16* q16 = (_Float16*)((char*)ws + bwd_head_bytes(rows));
    _Float16* r16 = q16 + nq;
    _Float16* g16 = r16 + nq;
    _Float16* k16 = g16 + nq;
    {
      const long long nk8 = (long long)nk / 8, ng8 = (long long)nq / 8;
      const unsigned blocks = (unsigned)std::min<long long>((std::max(nk8, ng8) + 255) / 256, kPrepBlocks);
      hipLaunchKernelGGL(bwd_prep16_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4*)k,
                         (f16x8*)k16, nk8, (const u32x4*)d_o, ng8, part);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_scale_kernel, dim3(1), dim3(256), 0, stream, (const unsigned*)part,
                         (int)blocks, dsc);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // waves per workgroup and tile sizes: see DqbSmem
    constexpr int NW = D > 128 ? 4 : 8, BC = D > 128 ? 32 : 128, BQ = D > 128 ? 32 : 64;
    constexpr int QB = D == 64 ? PLX_QB64 : 1;  // query blocks per dQ wave
    const int nqb16 = (T + 16 * NW * QB - 1) / (16 * NW * QB);
    constexpr int KB = D == 64 ? PLX_KB64 : 1;  // key blocks per dK/dV wave
    const int nkb16 = (T + 16 * NW * KB - 1) / (16 * NW * KB);
    hipLaunchKernelGGL((bwd_dq16b_kernel<D, NW, BC, QB>), dim3(nqb16 * B * Hq), dim3(64 * NW), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k16, (const uint16_t*)v,
                       (const uint16_t*)rho, (const uint16_t*)d_o, o, vbar, lse, c_aux, G, dl, q16,
                       r16, g16, dsc, dq, drho, B, Hq, Hkv, T, scale, scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv16b_kernel<D, NW, BQ, KB>), dim3(nkb16 * B * Hkv), dim3(64 * NW), 0, stream,
                       (const uint16_t*)q16, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)r16, (const uint16_t*)g16, lse, c_aux, G, dl, dsc, dk, dv, B,
                       Hq, Hkv, T, scale, scale * kLog2e);
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL((bwd_pre_kernel<Pol, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       stream, (const in_t*)d_o, o, vbar, G, dl, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<Pol, D>), dim3(nqb * B * Hq), dim3(BWD_THREADS), 0, stream,
                       (const in_t*)q, (const in_t*)k, (const in_t*)v, (const in_t*)rho,
                       (const in_t*)d_o, lse, c_aux, G, dl, dq, drho, B, Hq, Hkv, T, scale,
                       scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<Pol, D>), dim3(nkb * B * Hkv), dim3(BWD_THREADS), 0, stream,
                       (const in_t*)q, (const in_t*)k, (const in_t*)v, (const in_t*)rho,
                       (const in_t*)d_o, lse, c_aux, G, dl, dk, dv, B, Hq, Hkv, T, scale,
                       scale * kLog2e);
    return hipGetLastError();
  }
}

}  // namespace

// Workspace of the backward: G and delta (fp32 per query row); the dO scale,
// its inverse and the preparation pass's partial maxima; then, for bf16
// inputs, fp16 copies of q, rho, dO ([B, Hq, T, d]) and K ([B, Hkv, T, d]).
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int d) {
  const size_t rows = (size_t)B * Hq * T;
  return bwd_head_bytes(rows) + (3 * rows * d + (size_t)B * Hkv * T * d) * sizeof(uint16_t);
}

hipError_t launch_bwd(int dtype, const void* q, const void* k, const void* v, const void* rho,
                      const void* d_o, const float* o, const float* lse, const float* c_aux,
                      const float* vbar_aux, float* dq, float* dk, float* dv, float* drho, int B,
                      int Hq, int Hkv, int T, int d, float scale, float* ws, hipStream_t stream) {
  if (dtype == PLX_BF16) {
    if (d == 64)
      return launch_bwd_t<PolBF16, 64>(q, k, v, rho, d_o, o, lse, c_aux, vbar_aux, dq, dk, dv, drho, B, Hq, Hkv, T, scale, ws, stream);
    if (d == 256)
      return launch_bwd_t<PolBF16, 256>(q, k, v, rho, d_o, o, lse, c_aux, vbar_aux, dq, dk, dv, drho, B, Hq, Hkv, T, scale, ws, stream);
    return launch_bwd_t<PolBF16, 128>(q, k, v, rho, d_o, o, lse, c_aux, vbar_aux, dq, dk, dv, drho, B, Hq, Hkv, T, scale, ws, stream);
  }
  if (d == 64)
    return launch_bwd_t<PolF32, 64>(q, k, v, rho, d_o, o, lse, c_aux, vbar_aux, dq, dk, dv, drho, B, Hq, Hkv, T, scale, ws, stream);
  return launch_bwd_t<PolF32, 128>(q, k, v, rho, d_o, o, lse, c_aux, vbar_aux, dq, dk, dv, drho, B, Hq, Hkv, T, scale, ws, stream);
}

}  // namespace plx
