// Causal prefill forward of the Parallax operator.
//
// Output (technical summary "Riepilogo Tecnico: Parallax ...", section
// "Meccanismo Principale"; eta = 0 per its bullet on the boundary factor):
//     o_i = o_i^SA - Sigma_KV^(i) rho_i,
// with Sigma_KV^(i) the softmax-weighted KV covariance.  Expanding the
// covariance against the probe gives, with w_ij the softmax weights,
// r_ij = rho_i . k_j and c_i = sum_j w_ij r_ij (= kbar_i . rho_i):
//     Sigma_KV^(i) rho_i = sum_j w_ij r_ij v_j - vbar_i c_i,
//     o_i = vbar_i (1 + c_i) - sum_j w_ij r_ij v_j.
// One online-softmax pass over the key stream therefore carries the running
// max m and sum l plus O = sum p v, U = sum (p r) v and the scalar
// C = sum p r, and finishes with o = (O/l)(1 + C/l) - U/l.  The same key and
// value tiles serve both branches: the summary's kernel paragraph stresses
// that the softmax and covariance branches share one KV stream and that QK
// and RK are formed by the same matrix instructions; here the stacked
// [Q; rho] K^T is two MFMA chains sharing every K operand.
//
// Two kernels share this file:
//   * fwd16_kernel (bf16 inputs): 16x16x32 MFMA tiles, 16 query rows per
//     wave, 8 waves per workgroup, two waves per SIMD (described below);
//   * fwd_kernel (fp32 inputs, the exact-parity path): 32x32x2 fp32 MFMAs,
//     4 waves of 32 query rows; K rows and transposed V through double-
//     buffered LDS, one sub-tile at a time (scores, softmax, value MFMAs).
#include "plx_common.hpp"
#include "plx_kernels.hpp"

namespace plx {

namespace {

constexpr int FWD_BR = 128;
constexpr int FWD_BC = 64;
constexpr int FWD_THREADS = 256;
constexpr int FWD16_WAVES = 8;  // waves per workgroup of the bf16 kernel
constexpr int F16_BC = 128;     // keys per LDS tile of the bf16 kernel (d <= 128)

// bf16 kernel shape per head dim: d <= 128 runs 8 waves (two per SIMD) on
// 128-key tiles; d = 256 runs 4 waves (one per SIMD, whose 512 registers hold
// the doubled accumulators and operands) on 64-key tiles (LDS holds two
// double-buffered 64 x 256 K and V tiles).
template <int D>
constexpr int f16_bc() { return D > 128 ? 64 : F16_BC; }
template <int D>
constexpr int f16_waves() { return D > 128 ? 4 : FWD16_WAVES; }
// 16-row query blocks per wave: at d = 64 a wave's state leaves room for two,
// which share every K and V^T operand read from LDS (half the LDS traffic and
// half the softmax-independent instructions per MFMA).
#ifndef PLX_RB64
#define PLX_RB64 2
#endif
template <int D>
constexpr int f16_row_blocks() { return D == 64 ? PLX_RB64 : 1; }
// Lazy-rescale threshold (log2 units): p stays <= 16, so the fp16 operand
// p * r overflows only for |r| = |rho . k| > 4094.
constexpr float kRescaleLog2 = 4.f;

template <class Pol>
constexpr bool v_rowmajor() {
  return sizeof(typename Pol::in_t) == 2;  // bf16 inputs: transpose-read path
}

template <class Pol, int D>
struct FwdSmem {
  using in_t = typename Pol::in_t;
  using vel_t = typename Pol::vel_t;
  static constexpr int KLD = D + 16 / sizeof(in_t);  // K row stride (elements)
  // V row stride: row-major fp16 rows offset by 64 bytes mod 256 so that the
  // four rows one transpose read touches fall in distinct bank groups;
  // transposed fp32 rows padded by 4.
  static constexpr int VLD = v_rowmajor<Pol>() ? D + 32 : FWD_BC + 4;
  static constexpr int VSIZE = v_rowmajor<Pol>() ? FWD_BC * VLD : D * VLD;
  alignas(16) in_t k[2][FWD_BC * KLD];
  alignas(16) vel_t v[2][VSIZE];
};

// Per-thread prefetch registers for one K tile and one V tile.
template <class Pol, int D>
struct TileRegs {
  static constexpr int CPR = D / Pol::CW;                  // 16-byte chunks per row
  static constexpr int N = FWD_BC * CPR / FWD_THREADS;     // chunks per thread per tile
  u32x4 k[N];
  u32x4 v[N];
};

template <class Pol, int D>
__device__ __forceinline__ void gload_k(TileRegs<Pol, D>& r, const typename Pol::in_t* kb, int key0,
                                        int T) {
  constexpr int CPR = TileRegs<Pol, D>::CPR;
#pragma unroll
  for (int i = 0; i < TileRegs<Pol, D>::N; ++i) {
    const int it = threadIdx.x + FWD_THREADS * i;
    const int row = it / CPR, c = (it % CPR) * Pol::CW;
    // Rows past T load row T-1 instead (in bounds, finite).  Those keys are
    // after every valid query, so the causal mask gives them p = 0 and their
    // (finite) K and V contribute nothing; no select on the loaded value, so
    // the load's wait can stay at the LDS write.
    const int key = min(key0 + row, T - 1);
    r.k[i] = *reinterpret_cast<const u32x4*>(kb + (size_t)key * D + c);
  }
}

// V: row-major chunks for the transpose-read path; pairs of rows (same
// chunk) for the transposed fp32 layout.
template <class Pol, int D>
__device__ __forceinline__ void gload_v(TileRegs<Pol, D>& r, const typename Pol::in_t* vb, int key0,
                                        int T) {
  constexpr int CPR = TileRegs<Pol, D>::CPR;
  if constexpr (v_rowmajor<Pol>()) {
#pragma unroll
    for (int i = 0; i < TileRegs<Pol, D>::N; ++i) {
      const int it = threadIdx.x + FWD_THREADS * i;
      const int row = it / CPR, c = (it % CPR) * Pol::CW;
      const int key = min(key0 + row, T - 1);  // past T: row T-1, masked (see gload_k)
      r.v[i] = *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + c);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TileRegs<Pol, D>::N / 2; ++i) {
      const int it = threadIdx.x + FWD_THREADS * i;
      const int rp = it / CPR, c = (it % CPR) * Pol::CW;
      const int key = key0 + 2 * rp;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < T) a = *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + c);
      if (key + 1 < T) b = *reinterpret_cast<const u32x4*>(vb + (size_t)(key + 1) * D + c);
      r.v[2 * i] = a;
      r.v[2 * i + 1] = b;
    }
  }
}

template <class Pol, int D>
__device__ __forceinline__ void lds_put_k(FwdSmem<Pol, D>& sm, int buf, const TileRegs<Pol, D>& r) {
  constexpr int CPR = TileRegs<Pol, D>::CPR;
#pragma unroll
  for (int i = 0; i < TileRegs<Pol, D>::N; ++i) {
    const int it = threadIdx.x + FWD_THREADS * i;
    const int row = it / CPR, c = (it % CPR) * Pol::CW;
    *reinterpret_cast<u32x4*>(&sm.k[buf][row * FwdSmem<Pol, D>::KLD + c]) = r.k[i];
  }
}

template <class Pol, int D>
__device__ __forceinline__ void lds_put_v(FwdSmem<Pol, D>& sm, int buf, const TileRegs<Pol, D>& r) {
  using SM = FwdSmem<Pol, D>;
  constexpr int CPR = TileRegs<Pol, D>::CPR;
  if constexpr (v_rowmajor<Pol>()) {
#pragma unroll
    for (int i = 0; i < TileRegs<Pol, D>::N; ++i) {
      const int it = threadIdx.x + FWD_THREADS * i;
      const int row = it / CPR, c = (it % CPR) * Pol::CW;
      const u16x8 bits = __builtin_bit_cast(u16x8, r.v[i]);
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = bf16_bits_to_f16(bits[e]);
      *reinterpret_cast<f16x8*>(&sm.v[buf][row * SM::VLD + c]) = hv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < TileRegs<Pol, D>::N / 2; ++i) {
      const int it = threadIdx.x + FWD_THREADS * i;
      const int rp = it / CPR, c = (it % CPR) * Pol::CW;
      float a[4], b[4];
      __builtin_memcpy(a, &r.v[2 * i], 16);
      __builtin_memcpy(b, &r.v[2 * i + 1], 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        typename Pol::vel_t* dst = &sm.v[buf][(c + e) * SM::VLD + 2 * rp];
        dst[0] = a[e];
        dst[1] = b[e];
      }
    }
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x4 lds_read_tr16(const _Float16* p) {
  s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, t);
}

// A operand of O^T = V^T P^T for d sub-tile dt, key sub-tile st, MFMA step s.
// Element e of lane (row d, half h) is V[32 st + acc_row(KW s + e, h)][d].
template <class Pol, int D>
__device__ __forceinline__ typename Pol::vop_t load_v_op(const FwdSmem<Pol, D>& sm, int buf, int dt,
                                                         int st, int s, int lane) {
  using SM = FwdSmem<Pol, D>;
  if constexpr (v_rowmajor<Pol>()) {
    // ds_read_b64_tr_b16: within each 16-lane block, lane i receives element
    // i % 4 of the 4-element chunks addressed by lanes 4e + i / 4 (e = 0..3).
    // Lane L of a block therefore addresses row (row0 + L / 4), columns
    // (dbase + 4 (L % 4)), which hands lane i the four keys row0 .. row0+3 of
    // column dbase + i.
    const int h = lane >> 5, blk = (lane >> 4) & 1, li = lane & 15;
    const int row = 32 * st + 16 * s + 4 * h + (li >> 2);
    const int cv = 32 * dt + 16 * blk + 4 * (li & 3);
    const _Float16* base = &sm.v[buf][row * SM::VLD + cv];
    const f16x4 lo = lds_read_tr16(base);
    const f16x4 hi = lds_read_tr16(base + 8 * SM::VLD);
    f16x8 a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = lo[e];
      a[4 + e] = hi[e];
    }
    return a;
  } else {
    return load_t_op<Pol>(sm.v[buf], SM::VLD, 32 * dt + (lane & 31), 32 * st, s, lane >> 5);
  }
}

// Sum of the elements of a value operand, in fp32.
__device__ __forceinline__ float vop_sum(const f16x8& x) {
  const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 pr = {x[2 * i], x[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float vop_sum(float x) { return x; }

// Score MFMAs of one 32-key sub-tile: S^T and R^T (32 keys x 32 queries)
// from the K rows at LDS buffer `buf`, sub-tile `st`.
template <class Pol, int D>
__device__ __forceinline__ void score_sub(const FwdSmem<Pol, D>& sm, int buf, int st, int col,
                                          int half, const typename Pol::sop_t* qop,
                                          const typename Pol::sop_t* rop, f32x16& sacc,
                                          f32x16& racc) {
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP, NS = D / KSTEP;
  const typename Pol::in_t* krow = &sm.k[buf][(32 * st + col) * FwdSmem<Pol, D>::KLD + KW * half];
  {
    const typename Pol::sop_t a = load_sop<Pol>(krow);
    sacc = Pol::mma_s(a, qop[0], zero16());
    racc = Pol::mma_s(a, rop[0], zero16());
  }
#pragma unroll
  for (int s = 1; s < NS; ++s) {
    const typename Pol::sop_t a = load_sop<Pol>(krow + KSTEP * s);
    sacc = Pol::mma_s(a, qop[s], sacc);
    racc = Pol::mma_s(a, rop[s], racc);
  }
}

// Online-softmax state of one wave (one query per lane column).
template <class Pol, int D>
struct FwdState {
  static constexpr int ND = D / 32;
  f32x16 oacc[ND], uacc[ND];
  // l / c: sums of the rounded operands (normalise O, U, C consistently);
  // e: the unrounded sum, used only for the LSE.
  float m_run, l_part, c_part, e_part;
};

// Softmax statistics of one 32-key sub-tile whose first key is `kbase`
// (scores in sacc): causal mask, row max, and the rare lazy rescale.  Returns
// the reference max the probabilities of this sub-tile are taken against.
template <class Pol, int D>
__device__ __forceinline__ float softmax_stats(FwdState<Pol, D>& S, int kbase, int qw, int my_q,
                                               int half, float scale_log2, f32x16& sacc) {
  constexpr int ND = D / 32;
  // causal mask where the sub-tile reaches past the wave's first query
  if (kbase + 31 > qw) {
#pragma unroll
    for (int a = 0; a < 16; ++a)
      if (kbase + acc_row(a, half) > my_q) sacc[a] = -INFINITY;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int a = 0; a < 16; ++a) mt = fmaxf(mt, sacc[a]);
  mt = fmaxf(mt, xor32(mt)) * scale_log2;
  // Lazy rescale: the reference max m_run only moves when some row's max
  // exceeds it by more than kRescaleLog2 (so p <= 2^kRescaleLog2 in between);
  // the final normalisation uses the same m_run, so the result is unchanged.
  if (__any(mt > S.m_run + kRescaleLog2)) {
    const float m_new = fmaxf(S.m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(S.m_run - m_use);
    S.l_part *= alpha;
    S.c_part *= alpha;
    S.e_part *= alpha;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        S.oacc[i][a] *= alpha;
        S.uacc[i][a] *= alpha;
      }
    S.m_run = m_new;
  }
  return (S.m_run == -INFINITY) ? 0.f : S.m_run;
}

// Probabilities and value MFMAs of one 32-key sub-tile (straight-line code):
// p = exp2(s * scale_log2 - m); P and P.R rounded to the value operand with
// the row sums taken over exactly the rounded operands; then O^T += V^T P^T
// and U^T += V^T (P.R)^T with V rows from LDS buffer `buf`, sub-tile `st`.
// The V operand of step k+1 is read before the MFMAs of step k.
template <class Pol, int D>
__device__ __forceinline__ void softmax_pv_body(FwdState<Pol, D>& S, const FwdSmem<Pol, D>& sm,
                                                int buf, int st, int lane, float scale_log2,
                                                float m_use, const f32x16& sacc,
                                                const f32x16& racc) {
  using vop_t = typename Pol::vop_t;
  constexpr int KW = Pol::KW, NV = 32 / Pol::KSTEP, ND = D / 32;
  vop_t pop[NV], prop[NV];
#pragma unroll
  for (int s = 0; s < NV; ++s) {
#pragma unroll
    for (int e = 0; e < KW; ++e) {
      const int a = KW * s + e;
      const float p = fast_exp2(__builtin_fmaf(sacc[a], scale_log2, -m_use));
      S.e_part += p;
      set_elem(pop[s], e, Pol::round_v(p));
      set_elem(prop[s], e, Pol::round_v(p * racc[a]));
    }
    S.l_part += vop_sum(pop[s]);
    S.c_part += vop_sum(prop[s]);
  }
  vop_t av = load_v_op<Pol, D>(sm, buf, 0, st, 0, lane);
#pragma unroll
  for (int k = 0; k < NV * ND; ++k) {
    const int s = k / ND, dt = k % ND;
    vop_t an = av;
    if (k + 1 < NV * ND) an = load_v_op<Pol, D>(sm, buf, (k + 1) % ND, st, (k + 1) / ND, lane);
    S.oacc[dt] = Pol::mma_v(av, pop[s], S.oacc[dt]);
    S.uacc[dt] = Pol::mma_v(av, prop[s], S.uacc[dt]);
    av = an;
  }
}

template <class Pol, int D>
__global__ __launch_bounds__(FWD_THREADS, 1) void fwd_kernel(
    const typename Pol::in_t* __restrict__ q, const typename Pol::in_t* __restrict__ k,
    const typename Pol::in_t* __restrict__ v, const typename Pol::in_t* __restrict__ rho,
    float* __restrict__ o, float* __restrict__ lse, float* __restrict__ c_aux,
    float* __restrict__ vbar_aux, float* __restrict__ cor, unsigned flags, int B, int Hq, int Hkv,
    int T, float scale_log2) {
  using in_t = typename Pol::in_t;
  using sop_t = typename Pol::sop_t;
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP;
  constexpr int NS = D / KSTEP;  // score MFMA steps over d
  constexpr int ND = D / 32;     // 32-row d sub-tiles of O^T / U^T

  __shared__ FwdSmem<Pol, D> sm;

  // Longest causal rows first: block x enumerates (q-block descending, b*h).
  const int nqb = (T + FWD_BR - 1) / FWD_BR;
  const int bh_count = B * Hq;
  const int lin = xcd_block_order(blockIdx.x, bh_count, nqb * bh_count);
  const int qb = nqb - 1 - lin / bh_count;
  const int bh = lin % bh_count;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);

  const int lane = threadIdx.x & 63;
  // wave index as a scalar so that every per-wave tile condition below is a
  // uniform (scalar) branch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  const int q0 = qb * FWD_BR;
  const int qw = q0 + 32 * wave;  // first query of this wave
  const int my_q = qw + col;

  const in_t* qp = q + ((size_t)bh * T) * D;
  const in_t* rp = rho + ((size_t)bh * T) * D;
  const in_t* kp = k + ((size_t)(b * Hkv + hk) * T) * D;
  const in_t* vp = v + ((size_t)(b * Hkv + hk) * T) * D;

  const int kend = min(T, q0 + FWD_BR);
  const int ntiles = (kend + FWD_BC - 1) / FWD_BC;
  // 32-key sub-tiles this wave attends to: keys [0, min(kend, qw + 32))
  const int nsub = (min(kend, qw + 32) + 31) / 32;

  // prologue: K(0), K(1), V(0) into LDS
  TileRegs<Pol, D> pre;
  gload_k<Pol, D>(pre, kp, 0, T);
  gload_v<Pol, D>(pre, vp, 0, T);

  // Q and rho rows of this lane's query as B operands (uniform weights: a
  // zero Q operand, so every score is exactly 0 and every unmasked p is 1).
  const bool use_q = !(flags & PLX_UNIFORM_WEIGHTS);
  sop_t qop[NS], rop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (my_q < T) {
      qop[s] = use_q ? load_sop<Pol>(qp + (size_t)my_q * D + KSTEP * s + KW * half) : zero_sop<Pol>();
      rop[s] = load_sop<Pol>(rp + (size_t)my_q * D + KSTEP * s + KW * half);
    } else {
      qop[s] = zero_sop<Pol>();
      rop[s] = zero_sop<Pol>();
    }
  }
  lds_put_k<Pol, D>(sm, 0, pre);
  lds_put_v<Pol, D>(sm, 0, pre);
  if (ntiles > 1) {
    gload_k<Pol, D>(pre, kp, FWD_BC, T);
    lds_put_k<Pol, D>(sm, 1, pre);
  }
  __syncthreads();

  FwdState<Pol, D> S;
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    S.oacc[i] = zero16();
    S.uacc[i] = zero16();
  }
  S.m_run = -INFINITY;
  S.l_part = S.c_part = S.e_part = 0.f;

  f32x16 sa, ra;
  for (int j = 0; j < ntiles; ++j) {
    const int key0 = j * FWD_BC;
    const bool has_next_k = j + 2 < ntiles;
    const bool has_next_v = j + 1 < ntiles;
    if (has_next_k) gload_k<Pol, D>(pre, kp, key0 + 2 * FWD_BC, T);
    if (has_next_v) gload_v<Pol, D>(pre, vp, key0 + FWD_BC, T);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (2 * j + st < nsub) {
        score_sub<Pol, D>(sm, j & 1, st, col, half, qop, rop, sa, ra);
        const float m_use = softmax_stats<Pol, D>(S, key0 + 32 * st, qw, my_q, half, scale_log2, sa);
        softmax_pv_body<Pol, D>(S, sm, j & 1, st, lane, scale_log2, m_use, sa, ra);
      }
    }
    // every wave has read K buffer j&1 (refilled with K(j+2)) and V buffer
    // (j+1)&1 was last read in iteration j-1
    __syncthreads();
    if (has_next_k) lds_put_k<Pol, D>(sm, j & 1, pre);
    if (has_next_v) lds_put_v<Pol, D>(sm, (j + 1) & 1, pre);
    __syncthreads();
  }

  // epilogue: o = (O/l)(1 + C/l) - U/l (without an intercept: -U/l);
  // LSE = ln sum exp(scaled scores); COR = ||U/l - (O/l)(C/l)|| / ||o||
  // (without an intercept the correction is U/l).  The two lanes of one
  // query (same col, half = 0, 1) hold disjoint halves of its d values.
  const float l_tot = S.l_part + xor32(S.l_part);
  const float c_tot = S.c_part + xor32(S.c_part);
  const float e_tot = S.e_part + xor32(S.e_part);
  const float inv = 1.f / l_tot;
  const float cc = c_tot * inv;
  const bool no_icpt = flags & PLX_NO_INTERCEPT;
  float n_o = 0.f, n_c = 0.f;
  if (cor) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float vbar = S.oacc[dt][a] * inv;
        const float u = S.uacc[dt][a] * inv;
        const float ov = no_icpt ? -u : vbar * (1.f + cc) - u;
        const float corr = no_icpt ? u : u - vbar * cc;
        n_o = __builtin_fmaf(ov, ov, n_o);
        n_c = __builtin_fmaf(corr, corr, n_c);
      }
    n_o += xor32(n_o);
    n_c += xor32(n_c);
  }
  if (my_q < T) {
    float* orow = o + ((size_t)bh * T + my_q) * D;
    float* vrow = vbar_aux ? vbar_aux + ((size_t)bh * T + my_q) * D : nullptr;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * half;
        f32x4 ov, vv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float vbar = S.oacc[dt][4 * i + jj] * inv;
          const float u = S.uacc[dt][4 * i + jj] * inv;
          vv[jj] = vbar;
          ov[jj] = no_icpt ? -u : vbar * (1.f + cc) - u;
        }
        *reinterpret_cast<f32x4*>(orow + d0) = ov;
        if (vrow) *reinterpret_cast<f32x4*>(vrow + d0) = vv;
      }
    if (half == 0) {
      if (lse) lse[(size_t)bh * T + my_q] = (S.m_run + __log2f(e_tot)) * kLn2;
      if (c_aux) c_aux[(size_t)bh * T + my_q] = cc;
      if (cor) cor[(size_t)bh * T + my_q] = __builtin_sqrtf(n_c) / __builtin_sqrtf(n_o);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 forward on 16x16x32 MFMA tiles, two waves per SIMD.
//
// A wave owns 16 query rows (one per lane column c = lane % 16; the four
// 16-lane groups g = lane / 16 split the keys and the head dimension), so its
// state is half that of a 32-row wave: O^T and U^T (D x 16, fp32) take D/2
// registers each, the Q and rho B operands D/4 each.  The wave fits in 256
// registers and two waves share every SIMD: while one runs its softmax on the
// VALU the other feeds the matrix core (a wave raises its issue priority for
// its MFMA runs so that the matrix core is served first).
// Per 32-key sub-tile:
//   S^T, R^T (32 keys x 16 queries) = K [Q; rho]^T: 2 key tiles x D/32 steps,
//     A = K rows from LDS (ds_read_b128), B = Q / rho from registers;
//     acc[t][j] is key 16 t + 4 g + j, query c;
//   softmax in registers: 8 in-lane values per query, then the four 16-lane
//     groups through permlane swaps (no LDS round trip);
//   l and C as MFMAs against an all-ones A operand (every row of the result
//     is the column sum over the keys of the rounded P / P.R);
//   [O|U]^T += V^T [P | P.R]^T: D/16 d tiles, A = V^T from ds_read_b64_tr_b16,
//     element e of group g is key 16 (e / 4) + 4 g + e % 4, matching P's order.
// The K operands of a sub-tile are all read from LDS before its first score
// MFMA, and the V operands before its softmax, so that their latency is paid
// once per sub-tile and overlaps the softmax.
// Workgroup: 8 waves, 128 query rows of one (b, h).  Tiles of 128 keys are
// double-buffered in LDS (K bf16 rows, V fp16 rows); the global loads of tile
// j+1 are issued at the start of tile j and stored at its end, before the
// tile's single barrier.  At d = 256 the workgroup is 4 waves (64 rows, one
// wave per SIMD) and the tiles 64 keys (f16_bc, f16_waves).  At d = 64 a wave
// takes two 16-row blocks (RB = 2, 256 rows per workgroup): each K and V^T
// operand read from LDS feeds both blocks' MFMAs (f16_row_blocks).
template <int D>
struct Fwd16Smem {
  // row strides (elements), chosen so that the ds_read_b128 of K and the
  // transpose reads of V are free of bank conflicts (measured)
  static constexpr int KLD = D + 16;
  static constexpr int VLD = D + 16;
  alignas(16) uint16_t k[2][f16_bc<D>() * KLD];
  alignas(16) _Float16 v[2][f16_bc<D>() * VLD];
};


// AUX: the launch writes c_aux.  The probe mean c_i = kbar_i . rho_i handed to
// the backward is then taken from unrounded sums, sum_j p_j r_j / sum_j p_j,
// carried beside the rounded ones: the rounded C matches the fp16 operands the
// value MFMAs used (so o stays consistent with U), but its fp16 rounding of
// p r (|r| up to tens) shifts c by ~1e-2 on rows with few keys, and the
// backward's dV = sum_i w_ij (1 + c_i - r_ij) dO_i carries that shift
// straight through.
template <int D, int NW, int RB, bool AUX>
__global__ __launch_bounds__(64 * NW, (D > 128) ? 1 : 8 / NW) void fwd16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ rho, float* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ c_aux, float* __restrict__ vbar_aux, float* __restrict__ cor,
    unsigned flags, int B, int Hq, int Hkv, int T, float scale_log2) {
  constexpr int NT = 64 * NW;       // threads
  constexpr int BR = 16 * NW * RB;  // query rows per workgroup
  constexpr int NS = D / 32;        // score MFMA steps over d
  constexpr int ND = D / 16;        // 16-row d tiles of O^T / U^T
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int BC = f16_bc<D>();    // keys per LDS tile
  constexpr int NCH = BC * CPR / NT;  // chunks per thread per tile
  using SM = Fwd16Smem<D>;
  __shared__ SM sm;

  const int nqb = (T + BR - 1) / BR;
  const int bh_count = B * Hq;
  const int lin = xcd_block_order(blockIdx.x, bh_count, nqb * bh_count);
  const int qb = nqb - 1 - lin / bh_count;  // longest causal rows first
  const int bh = lin % bh_count;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int q0 = qb * BR;
  // the wave's RB blocks of 16 rows: block rb starts at qw + 16 rb
  const int qw = q0 + 16 * RB * wave;

  const uint16_t* qp = q + ((size_t)bh * T) * D;
  const uint16_t* rp = rho + ((size_t)bh * T) * D;
  const uint16_t* kp = k + ((size_t)(b * Hkv + hk) * T) * D;
  const uint16_t* vp = v + ((size_t)(b * Hkv + hk) * T) * D;

  const int kend = min(T, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;
  // 32-key sub-tiles this wave attends to: keys [0, min(kend, last row + 1))
  const int nsub = (min(kend, qw + 16 * RB) + 31) / 32;

  // global -> register prefetch of one K / V tile (rows past T read row T-1:
  // finite, and masked by the causal test since they follow every query)
  struct Pre { u32x4 k[NCH], v[NCH]; };
  Pre preA;
  auto gload = [&](Pre& p, int key0) {
    if (key0 + BC <= T) {
      // whole tile in range: scalar tile base plus this thread's fixed offsets
      const uint16_t* kt = kp + (size_t)key0 * D;
      const uint16_t* vt = vp + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int off = (threadIdx.x + NT * i) * 8;  // row * D + column
        p.k[i] = *reinterpret_cast<const u32x4*>(kt + off);
        p.v[i] = *reinterpret_cast<const u32x4*>(vt + off);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int it = threadIdx.x + NT * i;
      const int row = it / CPR, cc = (it % CPR) * 8;
      const size_t off = (size_t)min(key0 + row, T - 1) * D + cc;
      p.k[i] = *reinterpret_cast<const u32x4*>(kp + off);
      p.v[i] = *reinterpret_cast<const u32x4*>(vp + off);
    }
  };
  auto lds_put = [&](const Pre& p, int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int it = threadIdx.x + NT * i;
      const int row = it / CPR, cc = (it % CPR) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[buf][row * SM::KLD + cc]) = p.k[i];
      const u16x8 bits = __builtin_bit_cast(u16x8, p.v[i]);
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = bf16_bits_to_f16(bits[e]);
      *reinterpret_cast<f16x8*>(&sm.v[buf][row * SM::VLD + cc]) = hv;
    }
  };

  // prologue: tile 0 -> buffer 0
  gload(preA, 0);
  // Uniform weights: a zero query operand makes every score exactly 0, so
  // every unmasked key gets p = 1 and the running max stays 0.
  const bool use_q = !(flags & PLX_UNIFORM_WEIGHTS);
  bf16x8 qop[RB][NS], rop[RB][NS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int my_q = qw + 16 * rb + c;
      u32x4 qa = {0u, 0u, 0u, 0u}, ra = {0u, 0u, 0u, 0u};
      if (my_q < T) {
        if (use_q) qa = *reinterpret_cast<const u32x4*>(qp + (size_t)my_q * D + 32 * s + 8 * g);
        ra = *reinterpret_cast<const u32x4*>(rp + (size_t)my_q * D + 32 * s + 8 * g);
      }
      qop[rb][s] = __builtin_bit_cast(bf16x8, qa);
      rop[rb][s] = __builtin_bit_cast(bf16x8, ra);
    }
  lds_put(preA, 0);
  __syncthreads();

  f32x4 oacc[RB][ND], uacc[RB][ND];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      oacc[rb][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      uacc[rb][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  // l and C as MFMAs against an all-ones A operand: every row of lacc / cacc
  // holds the column (query) sum over the keys of the rounded P / P.R
  f32x4 lacc[RB], cacc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lacc[rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    cacc[rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.f;
  asm volatile("" : "+v"(ones));  // kept in registers, not rebuilt per sub-tile
  // e_part: this lane's unrounded sum of p (the LSE only); ce_part: the
  // unrounded sum of p r (c_aux only)
  float m_run[RB], e_part[RB], ce_part[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    e_part[rb] = 0.f;
    ce_part[rb] = 0.f;
  }

  auto subtile = [&](int kbuf, int vbuf, int st, int kbase) {
    // scores
    __builtin_amdgcn_s_setprio(1);
    f32x4 sacc[RB][2], racc[RB][2];
    unsigned kaddr = lds_addr(&sm.k[kbuf][(32 * st + c) * SM::KLD + 8 * g]);
    asm volatile("" : "+v"(kaddr));
    // every K operand of the sub-tile in flight before the first MFMA
    bf16x8 ka[2][NS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        ka[t][s] = __builtin_bit_cast(bf16x8, ld128_at(kaddr + 2 * (16 * t * SM::KLD + 32 * s)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = ka[t][s];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 zs = s == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : sacc[rb][t];
          const f32x4 zr = s == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : racc[rb][t];
          sacc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[rb][s], zs, 0, 0, 0);
          racc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, rop[rb][s], zr, 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // V^T operands of the value MFMAs, in flight during the softmax
    unsigned vaddr = lds_addr(&sm.v[vbuf][(32 * st + 4 * g + (c >> 2)) * SM::VLD + 4 * (c & 3)]);
    asm volatile("" : "+v"(vaddr));
    f16x4 va[ND][2];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      va[dt][0] = tr16_at(vaddr + 2 * 16 * dt);
      va[dt][1] = tr16_at(vaddr + 2 * (16 * dt + 16 * SM::VLD));
    }
    __builtin_amdgcn_sched_barrier(0);
    f16x8 pop[RB], prop[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qr = qw + 16 * rb;  // first query of this row block
      const int my_q = qr + c;
      // causal mask where the sub-tile reaches past the block's first query
      if (kbase + 31 > qr) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kbase + 16 * t + 4 * g + j > my_q) sacc[rb][t][j] = -INFINITY;
      }
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) mt = fmaxf(mt, sacc[rb][t][j]);
      {
        // max over the four 16-lane groups: permlane swaps, no LDS round trip
        // (NaN-propagating maximum: no canonicalising moves around the swaps)
        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = __builtin_elementwise_maximum(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = __builtin_elementwise_maximum(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
      }
      mt *= scale_log2;
      // lazy rescale: the reference max moves only when a row's max exceeds it
      // by more than kRescaleLog2, so p <= 2^kRescaleLog2 in between
      if (__any(mt > m_run[rb] + kRescaleLog2)) {
        const float m_new = fmaxf(m_run[rb], mt);
        const float m_u = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[rb] - m_u);
        e_part[rb] *= alpha;
        if constexpr (AUX) ce_part[rb] *= alpha;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          lacc[rb][jj] *= alpha;
          cacc[rb][jj] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            oacc[rb][i][j] *= alpha;
            uacc[rb][i][j] *= alpha;
          }
        m_run[rb] = m_new;
      }
      const float m_use = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float s0 = sacc[rb][e >> 2][e & 3], s1 = sacc[rb][e >> 2][(e & 3) + 1];
        const float p0 = fast_exp2(__builtin_fmaf(s0, scale_log2, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s1, scale_log2, -m_use));
        e_part[rb] += p0 + p1;
        const float pr0 = p0 * racc[rb][e >> 2][e & 3], pr1 = p1 * racc[rb][e >> 2][(e & 3) + 1];
        if constexpr (AUX) ce_part[rb] += pr0 + pr1;
        const f16x2 ph = {(_Float16)p0, (_Float16)p1};
        const f16x2 rh = {(_Float16)pr0, (_Float16)pr1};
        pop[rb][e] = ph[0];
        pop[rb][e + 1] = ph[1];
        prop[rb][e] = rh[0];
        prop[rb][e + 1] = rh[1];
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[rb], lacc[rb], 0, 0, 0);
      cacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, prop[rb], cacc[rb], 0, 0, 0);
    }
    // value MFMAs: every V^T operand feeds the RB row blocks
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const f16x4 v0 = va[dt][0], v1 = va[dt][1];
      f16x8 av;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = v0[e];
        av[4 + e] = v1[e];
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        oacc[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pop[rb], oacc[rb][dt], 0, 0, 0);
        uacc[rb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, prop[rb], uacc[rb][dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Tile j lives in buffer j % 2.  Iteration j issues the global loads of
  // tile j+1 and stores them into the other buffer, whose tile j-1 every wave
  // finished reading before the barrier that ended iteration j-1.
  auto iter = [&](int j, int buf) {
    const int key0 = j * BC;
    if (j + 1 < ntiles) gload(preA, key0 + BC);
#pragma unroll
    for (int st = 0; st < BC / 32; ++st)
      if ((BC / 32) * j + st < nsub) subtile(buf, buf, st, key0 + 32 * st);
    if (j + 1 < ntiles) lds_put(preA, buf ^ 1);
    __syncthreads();
  };
  for (int j = 0; j < ntiles; j += 2) {
    iter(j, 0);
    if (j + 1 < ntiles) iter(j + 1, 1);
  }

  // epilogue, per row block: o = (O/l)(1 + C/l) - U/l (without an intercept:
  // -U/l); LSE = ln sum exp(scaled scores); COR = ||U/l - (O/l)(C/l)|| / ||o||
  // (without an intercept the correction is U/l).  The lanes of one query
  // (same c, g = 0..3) hold disjoint quarters of its d values.
  const bool no_icpt = flags & PLX_NO_INTERCEPT;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int my_q = qw + 16 * rb + c;
    const float l_tot = lacc[rb][0], c_tot = cacc[rb][0];
    float e_tot = e_part[rb];
    e_tot += __shfl_xor(e_tot, 16, 64);
    e_tot += __shfl_xor(e_tot, 32, 64);
    float ce_tot = ce_part[rb];
    if constexpr (AUX) {
      ce_tot += __shfl_xor(ce_tot, 16, 64);
      ce_tot += __shfl_xor(ce_tot, 32, 64);
    }
    const float inv = 1.f / l_tot;
    const float cc = c_tot * inv;
    f32x4 ov[ND], vv[ND];
    float n_o = 0.f, n_c = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float vbar = oacc[rb][dt][jj] * inv;
        const float u = uacc[rb][dt][jj] * inv;
        vv[dt][jj] = vbar;
        ov[dt][jj] = no_icpt ? -u : vbar * (1.f + cc) - u;
        const float corr = no_icpt ? u : u - vbar * cc;
        n_o = __builtin_fmaf(ov[dt][jj], ov[dt][jj], n_o);
        n_c = __builtin_fmaf(corr, corr, n_c);
      }
    if (cor) {
      n_o += __shfl_xor(n_o, 16, 64);
      n_o += __shfl_xor(n_o, 32, 64);
      n_c += __shfl_xor(n_c, 16, 64);
      n_c += __shfl_xor(n_c, 32, 64);
    }
    if (my_q < T) {
      float* orow = o + ((size_t)bh * T + my_q) * D;
      float* vrow = vbar_aux ? vbar_aux + ((size_t)bh * T + my_q) * D : nullptr;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * g) = ov[dt];
        if (vrow) *reinterpret_cast<f32x4*>(vrow + 16 * dt + 4 * g) = vv[dt];
      }
      if (g == 0) {
        if (lse) lse[(size_t)bh * T + my_q] = (m_run[rb] + __log2f(e_tot)) * kLn2;
        if constexpr (AUX) c_aux[(size_t)bh * T + my_q] = ce_tot / e_tot;
        if (cor) cor[(size_t)bh * T + my_q] = __builtin_sqrtf(n_c) / __builtin_sqrtf(n_o);
      }
    }
  }
}

template <int D, int NW>
hipError_t launch_fwd16(const void* q, const void* k, const void* v, const void* rho, float* o,
                        float* lse, float* c_aux, float* vbar_aux, float* cor, unsigned flags, int B,
                        int Hq, int Hkv, int T, float scale, hipStream_t stream) {
  constexpr int RB = f16_row_blocks<D>();
  const int nqb = (T + 16 * NW * RB - 1) / (16 * NW * RB);
  if (c_aux)
    hipLaunchKernelGGL((fwd16_kernel<D, NW, RB, true>), dim3(nqb * B * Hq), dim3(64 * NW), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)rho,
                       o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale * kLog2e);
  else
    hipLaunchKernelGGL((fwd16_kernel<D, NW, RB, false>), dim3(nqb * B * Hq), dim3(64 * NW), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)rho,
                       o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale * kLog2e);
  return hipGetLastError();
}

template <class Pol, int D>
hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const void* rho, float* o,
                        float* lse, float* c_aux, float* vbar_aux, float* cor, unsigned flags, int B,
                        int Hq, int Hkv, int T, float scale, hipStream_t stream) {
  using in_t = typename Pol::in_t;
  const int nqb = (T + FWD_BR - 1) / FWD_BR;
  dim3 grid(nqb * B * Hq);
  hipLaunchKernelGGL((fwd_kernel<Pol, D>), grid, dim3(FWD_THREADS), 0, stream,
                     (const in_t*)q, (const in_t*)k, (const in_t*)v, (const in_t*)rho, o, lse, c_aux,
                     vbar_aux, cor, flags, B, Hq, Hkv, T, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(int dtype, const void* q, const void* k, const void* v, const void* rho,
                      float* o, float* lse, float* c_aux, float* vbar_aux, float* cor,
                      unsigned flags, int B, int Hq, int Hkv, int T, int d, float scale,
                      hipStream_t stream) {
  if (dtype == PLX_BF16) {
    if (d == 64)
      return launch_fwd16<64, f16_waves<64>()>(q, k, v, rho, o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale, stream);
    if (d == 256)
      return launch_fwd16<256, f16_waves<256>()>(q, k, v, rho, o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale, stream);
    return launch_fwd16<128, f16_waves<128>()>(q, k, v, rho, o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale, stream);
  }
  if (d == 64)
    return launch_fwd_t<PolF32, 64>(q, k, v, rho, o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale, stream);
  return launch_fwd_t<PolF32, 128>(q, k, v, rho, o, lse, c_aux, vbar_aux, cor, flags, B, Hq, Hkv, T, scale, stream);
}

}  // namespace plx
