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
// Work split: a workgroup (4 waves) owns 128 query rows of one (b, h);
// each wave owns 32 rows.  Keys stream in tiles of 64 through LDS:
//   K tile   row-major  [64][D + pad]   (A operand of S^T = K Q^T, R^T = K rho^T)
//   V tile   transposed [D][64 + pad]   (A operand of O^T = V^T P^T, U^T = V^T (P.R)^T)
// Q and rho stay in registers as B operands for the whole pass.
#include "plx_common.hpp"
#include "plx_kernels.hpp"

namespace plx {

namespace {

constexpr int FWD_BR = 128;
constexpr int FWD_BC = 64;
constexpr int FWD_THREADS = 256;

template <class Pol, int D>
struct FwdSmem {
  using in_t = typename Pol::in_t;
  using vel_t = typename Pol::vel_t;
  static constexpr int KPAD = 16 / sizeof(in_t);
  static constexpr int KLD = D + KPAD;       // K row stride (elements)
  static constexpr int VLD = FWD_BC + 4;     // V^T row stride (elements)
  in_t k[FWD_BC * KLD];
  vel_t vt[D * VLD];
};

// Cooperative global -> LDS staging of one 64-key tile.  K is copied as is;
// V is converted to the value-operand type and written transposed.  Rows at
// or beyond T read as zero.
template <class Pol, int D>
__device__ __forceinline__ void stage_kv_tile(FwdSmem<Pol, D>& sm, const typename Pol::in_t* kb,
                                              const typename Pol::in_t* vb, int key0, int T) {
  using in_t = typename Pol::in_t;
  constexpr int CW = Pol::CW;
  constexpr int CPR = D / CW;  // 16-byte chunks per row
  const int tid = threadIdx.x;
  // K: one chunk per item
  for (int it = tid; it < FWD_BC * CPR; it += FWD_THREADS) {
    const int r = it / CPR, c = (it % CPR) * CW;
    const int key = key0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < T) val = *reinterpret_cast<const u32x4*>(kb + (size_t)key * D + c);
    *reinterpret_cast<u32x4*>(&sm.k[r * FwdSmem<Pol, D>::KLD + c]) = val;
  }
  // V: two rows x one chunk per item, written as key pairs of the transpose
  for (int it = tid; it < (FWD_BC / 2) * CPR; it += FWD_THREADS) {
    const int rp = it / CPR, c = (it % CPR) * CW;
    const int key = key0 + 2 * rp;
    in_t a[CW], b[CW];
    u32x4 va = {0u, 0u, 0u, 0u}, vb2 = {0u, 0u, 0u, 0u};
    if (key < T) va = *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + c);
    if (key + 1 < T) vb2 = *reinterpret_cast<const u32x4*>(vb + (size_t)(key + 1) * D + c);
    __builtin_memcpy(a, &va, 16);
    __builtin_memcpy(b, &vb2, 16);
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      typename Pol::vel_t* dst = &sm.vt[(c + e) * FwdSmem<Pol, D>::VLD + 2 * rp];
      dst[0] = Pol::to_vel(a[e]);
      dst[1] = Pol::to_vel(b[e]);
    }
  }
}

// Value-operand (A of O^T = V^T P^T) for d-row `drow`, key sub-tile `st`,
// MFMA step `s`, lane half `h`.
template <class Pol, int D>
__device__ __forceinline__ typename Pol::vop_t load_vt_op(const FwdSmem<Pol, D>& sm, int drow, int st,
                                                          int s, int h) {
  typename Pol::vop_t a;
  const typename Pol::vel_t* row = &sm.vt[drow * FwdSmem<Pol, D>::VLD + 32 * st];
#pragma unroll
  for (int e = 0; e < Pol::KW; ++e) set_elem(a, e, row[acc_row(Pol::KW * s + e, h)]);
  return a;
}

template <class Pol, int D>
__global__ __launch_bounds__(FWD_THREADS, 1) void fwd_kernel(
    const typename Pol::in_t* __restrict__ q, const typename Pol::in_t* __restrict__ k,
    const typename Pol::in_t* __restrict__ v, const typename Pol::in_t* __restrict__ rho,
    float* __restrict__ o, float* __restrict__ lse, float* __restrict__ c_aux,
    float* __restrict__ vbar_aux, int B, int Hq, int Hkv, int T, float scale_log2) {
  using in_t = typename Pol::in_t;
  using sop_t = typename Pol::sop_t;
  using vop_t = typename Pol::vop_t;
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP;
  constexpr int NS = D / KSTEP;     // score MFMA steps over d
  constexpr int NV = 32 / KSTEP;    // value MFMA steps per 32-key sub-tile
  constexpr int ND = D / 32;        // 32-row d sub-tiles of O^T / U^T

  __shared__ FwdSmem<Pol, D> sm;

  // Longest causal rows first: block x enumerates (q-block descending, b*h).
  const int nqb = (T + FWD_BR - 1) / FWD_BR;
  const int bh_count = B * Hq;
  const int lin = blockIdx.x;
  const int qb = nqb - 1 - lin / bh_count;
  const int bh = lin % bh_count;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int q0 = qb * FWD_BR;
  const int qw = q0 + 32 * wave;  // first query of this wave
  const int my_q = qw + col;

  const in_t* qp = q + ((size_t)bh * T) * D;
  const in_t* rp = rho + ((size_t)bh * T) * D;
  const in_t* kp = k + ((size_t)(b * Hkv + hk) * T) * D;
  const in_t* vp = v + ((size_t)(b * Hkv + hk) * T) * D;

  // Q and rho rows of this lane's query as B operands.
  sop_t qop[NS], rop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (my_q < T) {
      qop[s] = load_sop<Pol>(qp + (size_t)my_q * D + KSTEP * s + KW * half);
      rop[s] = load_sop<Pol>(rp + (size_t)my_q * D + KSTEP * s + KW * half);
    } else {
      qop[s] = zero_sop<Pol>();
      rop[s] = zero_sop<Pol>();
    }
  }

  f32x16 oacc[ND], uacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    oacc[i] = zero16();
    uacc[i] = zero16();
  }
  // l_part / c_part: sums of the rounded operands (normalise O, U, C
  // consistently); e_part: the unrounded sum, used only for the LSE.
  float m_run = -INFINITY, l_part = 0.f, c_part = 0.f, e_part = 0.f;

  const int kend = min(T, q0 + FWD_BR);
  const int ntiles = (kend + FWD_BC - 1) / FWD_BC;

  for (int j = 0; j < ntiles; ++j) {
    const int key0 = j * FWD_BC;
    __syncthreads();
    stage_kv_tile<Pol, D>(sm, kp, vp, key0, T);
    __syncthreads();
    if (key0 > qw + 31) continue;  // every key of the tile is after every query of the wave

    f32x16 sacc[2], racc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = zero16();
      racc[st] = zero16();
      const in_t* krow = &sm.k[(32 * st + col) * FwdSmem<Pol, D>::KLD + KW * half];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sop_t a = load_sop<Pol>(krow + KSTEP * s);
        sacc[st] = Pol::mma_s(a, qop[s], sacc[st]);
        racc[st] = Pol::mma_s(a, rop[s], racc[st]);
      }
    }

    // causal mask on the tiles that reach past the wave's first query
    if (key0 + FWD_BC - 1 > qw) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = key0 + 32 * st + acc_row(a, half);
          if (key > my_q) sacc[st][a] = -INFINITY;
        }
    }

    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) mt = fmaxf(mt, sacc[st][a]);
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    // p = exp2(s * scale_log2 - m); P and P.R rounded to the value operand,
    // and the row sums taken over exactly the rounded operands.
    float lsum = 0.f, csum = 0.f, esum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float p = fast_exp2(__builtin_fmaf(sacc[st][a], scale_log2, -m_use));
        esum += p;
        const auto pv = Pol::round_v(p);
        const auto prv = Pol::round_v(p * racc[st][a]);
        lsum += Pol::vel_to_f32(pv);
        csum += Pol::vel_to_f32(prv);
        sacc[st][a] = Pol::vel_to_f32(pv);
        racc[st][a] = Pol::vel_to_f32(prv);
      }
    l_part = alpha * l_part + lsum;
    c_part = alpha * c_part + csum;
    e_part = alpha * e_part + esum;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        oacc[i][a] *= alpha;
        uacc[i][a] *= alpha;
      }

#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int s = 0; s < NV; ++s) {
        vop_t pop, prop;
#pragma unroll
        for (int e = 0; e < KW; ++e) {
          set_elem(pop, e, Pol::round_v(sacc[st][KW * s + e]));
          set_elem(prop, e, Pol::round_v(racc[st][KW * s + e]));
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          vop_t a = load_vt_op<Pol, D>(sm, 32 * dt + col, st, s, half);
          oacc[dt] = Pol::mma_v(a, pop, oacc[dt]);
          uacc[dt] = Pol::mma_v(a, prop, uacc[dt]);
        }
      }
  }

  // epilogue: o = (O/l)(1 + C/l) - U/l ; LSE = ln sum exp(scaled scores)
  const float l_tot = l_part + xor32(l_part);
  const float c_tot = c_part + xor32(c_part);
  const float e_tot = e_part + xor32(e_part);
  const float inv = 1.f / l_tot;
  const float cc = c_tot * inv;
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
          const float vbar = oacc[dt][4 * i + jj] * inv;
          vv[jj] = vbar;
          ov[jj] = vbar * (1.f + cc) - uacc[dt][4 * i + jj] * inv;
        }
        *reinterpret_cast<f32x4*>(orow + d0) = ov;
        if (vrow) *reinterpret_cast<f32x4*>(vrow + d0) = vv;
      }
    if (half == 0) {
      if (lse) lse[(size_t)bh * T + my_q] = (m_run + __log2f(e_tot)) * kLn2;
      if (c_aux) c_aux[(size_t)bh * T + my_q] = cc;
    }
  }
}

template <class Pol, int D>
hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const void* rho, float* o,
                        float* lse, float* c_aux, float* vbar_aux, int B, int Hq, int Hkv, int T,
                        float scale, hipStream_t stream) {
  using in_t = typename Pol::in_t;
  const int nqb = (T + FWD_BR - 1) / FWD_BR;
  dim3 grid(nqb * B * Hq);
  hipLaunchKernelGGL((fwd_kernel<Pol, D>), grid, dim3(FWD_THREADS), 0, stream,
                     (const in_t*)q, (const in_t*)k, (const in_t*)v, (const in_t*)rho, o, lse, c_aux,
                     vbar_aux, B, Hq, Hkv, T, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(int dtype, const void* q, const void* k, const void* v, const void* rho,
                      float* o, float* lse, float* c_aux, float* vbar_aux, int B, int Hq, int Hkv,
                      int T, int d, float scale, hipStream_t stream) {
  if (dtype == PLX_BF16) {
    if (d == 64) return launch_fwd_t<PolBF16, 64>(q, k, v, rho, o, lse, c_aux, vbar_aux, B, Hq, Hkv, T, scale, stream);
    return launch_fwd_t<PolBF16, 128>(q, k, v, rho, o, lse, c_aux, vbar_aux, B, Hq, Hkv, T, scale, stream);
  }
  if (d == 64) return launch_fwd_t<PolF32, 64>(q, k, v, rho, o, lse, c_aux, vbar_aux, B, Hq, Hkv, T, scale, stream);
  return launch_fwd_t<PolF32, 128>(q, k, v, rho, o, lse, c_aux, vbar_aux, B, Hq, Hkv, T, scale, stream);
}

}  // namespace plx
