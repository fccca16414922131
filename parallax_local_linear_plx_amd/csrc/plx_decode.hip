// Split-K decode of the Parallax operator over a ragged KV cache.
//
// Every sequence b attends with one query per head to cache rows
// [0, ctx_len[b]).  The decode kernel of the write-ups streams the KV cache
// once for both the softmax branch and the covariance branch (technical
// summary "Riepilogo Tecnico: Parallax ...", section "Algoritmo Consapevole
// dell'Hardware": same KV stream, QK and RK in the same matrix instructions);
// the Russian write-up's caption contrasts a variant tuned for parallel
// decoding, read here as splitting each sequence's keys over workgroups.
//
// Kernel 1 (partial): workgroup = (split, kv head, b).  The query heads that
// share the KV head are stacked with their probes as the 2G columns
// [q_0, rho_0, q_1, rho_1, ...] of one MFMA B operand, so each K row is read
// once for all of them:  S^T = K [q;rho]^T  gives scores (even columns) and
// r = rho . k (odd columns) in one MFMA chain.  Per split it accumulates
//   m, l = sum p, O = sum p v, U = sum (p r) v, Kbar = sum p k
// and writes one partial record per query head.
// Kernel 2 (merge): per (b, h) rescales the records to a common max and
// finishes  o = (O/l)(1 + (Kbar . rho)/l) - U/l,  LSE = M + ln l.
#include "plx_common.hpp"
#include "plx_kernels.hpp"

namespace plx {

namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = 4;
constexpr int DEC_SUB = 32;                       // keys per wave sub-tile
constexpr int DEC_GROUP_KEYS = DEC_SUB * DEC_WAVES;  // keys per workgroup step
constexpr int DEC_TLD = DEC_SUB + 4;              // transposed tile row stride

template <class Pol, int D>
struct DecSmem {
  using vel_t = typename Pol::vel_t;
  static constexpr int MLD = D + 1;  // merge buffer row stride (floats)
  static constexpr size_t TILE_BYTES = (size_t)DEC_WAVES * 2 * D * DEC_TLD * sizeof(vel_t);
  static constexpr size_t MERGE_BYTES = (size_t)2 * 32 * MLD * sizeof(float);
  static constexpr size_t BYTES = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
  union {
    vel_t tiles[DEC_WAVES][2][D * DEC_TLD];  // per wave: K^T then V^T
    float merge[2][32 * MLD];                // [O/U, Kbar] x column x d
  };
  float mw[DEC_WAVES][32];
  float lsum[32];
  float esum[32];
};

__device__ __forceinline__ float dpp_even_partner(float x) {
  // quad_perm [0,0,2,2]: lanes 2k and 2k+1 both read lane 2k
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xA0, 0xF, 0xF, false));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <class Pol, int D, int G>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode_partial_kernel(
    const typename Pol::in_t* __restrict__ q, const typename Pol::in_t* __restrict__ rho,
    const typename Pol::in_t* __restrict__ kc, const typename Pol::in_t* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, float* __restrict__ part, int Hkv, int S_max, int chunk,
    int nsplit, float scale_log2) {
  using in_t = typename Pol::in_t;
  using sop_t = typename Pol::sop_t;
  using vop_t = typename Pol::vop_t;
  using vel_t = typename Pol::vel_t;
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP;
  constexpr int NS = D / KSTEP;
  constexpr int NV = DEC_SUB / KSTEP;
  constexpr int ND = D / 32;
  constexpr int REC = 3 * D + 4;

  __shared__ DecSmem<Pol, D> sm;

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int ctx = ctx_len[b];
  if (ctx < 1 || ctx > S_max) return;  // the merge writes NaN for this sequence
  const int k_begin = split * chunk;
  if (k_begin >= ctx) return;  // the merge reads only splits below ctx
  const int k_end = min(ctx, k_begin + chunk);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int Hq = Hkv * G;

  // B operand: column c -> q (even) or rho (odd) of head hk*G + c/2
  sop_t bop[NS];
  {
    const int hq = hk * G + (col >> 1);
    const in_t* src = (col & 1) ? rho : q;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      bop[s] = (col < 2 * G) ? load_sop<Pol>(src + ((size_t)b * Hq + hq) * D + KSTEP * s + KW * half)
                             : zero_sop<Pol>();
  }

  const in_t* kbase = kc + ((size_t)(b * Hkv + hk) * S_max) * D;
  const in_t* vbase = vc + ((size_t)(b * Hkv + hk) * S_max) * D;
  vel_t* kt = sm.tiles[wave][0];
  vel_t* vt = sm.tiles[wave][1];

  f32x16 ou[ND], kb[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    ou[i] = zero16();
    kb[i] = zero16();
  }
  // l_part: sum of the rounded operands (normalises O, U, Kbar);
  // e_part: the unrounded sum, used only for the LSE.
  float m_run = -INFINITY, l_part = 0.f, e_part = 0.f;

  for (int g0 = k_begin; g0 < k_end; g0 += DEC_GROUP_KEYS) {
    const int key0 = g0 + DEC_SUB * wave;
    if (key0 >= k_end) break;  // wave-uniform: nothing left for this wave
    const int my_key = key0 + col;
    const bool kvalid = my_key < k_end;

    sop_t kop[NS], vop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kvalid) {
        kop[s] = load_sop<Pol>(kbase + (size_t)my_key * D + KSTEP * s + KW * half);
        vop[s] = load_sop<Pol>(vbase + (size_t)my_key * D + KSTEP * s + KW * half);
      } else {
        kop[s] = zero_sop<Pol>();
        vop[s] = zero_sop<Pol>();
      }
    }

    f32x16 sacc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) sacc = Pol::mma_s(kop[s], bop[s], sacc);

    // K and V rows -> transposed per-wave tiles (value-operand type)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < KW; ++e) {
        const int d = KSTEP * s + KW * half + e;
        in_t kx, vx;
        if constexpr (KW == 1) {
          kx = kop[s];
          vx = vop[s];
        } else {
          kx = __builtin_bit_cast(u16x8, kop[s])[e];
          vx = __builtin_bit_cast(u16x8, vop[s])[e];
        }
        kt[d * DEC_TLD + col] = Pol::to_vel(kx);
        vt[d * DEC_TLD + col] = Pol::to_vel(vx);
      }

    // softmax over this sub-tile: even columns hold scores, odd columns r
    float sv[16];
    float mt = -INFINITY;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      float se = dpp_even_partner(sacc[a]);
      if (key0 + acc_row(a, half) >= k_end) se = -INFINITY;
      sv[a] = se;
      mt = fmaxf(mt, se);
    }
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    const bool used = col < 2 * G;
    const bool odd = col & 1;
    float lsum = 0.f, esum = 0.f;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const float p = used ? fast_exp2(__builtin_fmaf(sv[a], scale_log2, -m_use)) : 0.f;
      esum += p;
      const float val = odd ? p * sacc[a] : p;
      const float rv = Pol::vel_to_f32(Pol::round_v(val));
      lsum += rv;
      sv[a] = rv;
    }
    l_part = alpha * l_part + lsum;
    e_part = alpha * e_part + esum;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        ou[i][a] *= alpha;
        kb[i][a] *= alpha;
      }

    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      vop_t pop;
#pragma unroll
      for (int e = 0; e < KW; ++e) set_elem(pop, e, Pol::round_v(sv[KW * s + e]));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        vop_t av, ak;
        const int drow = (32 * dt + col) * DEC_TLD;
#pragma unroll
        for (int e = 0; e < KW; ++e) {
          const int key = acc_row(KW * s + e, half);
          set_elem(av, e, vt[drow + key]);
          set_elem(ak, e, kt[drow + key]);
        }
        ou[dt] = Pol::mma_v(av, pop, ou[dt]);
        kb[dt] = Pol::mma_v(ak, pop, kb[dt]);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four waves' states through LDS ----
  __syncthreads();
  if (half == 0) sm.mw[wave][col] = m_run;
  for (int i = threadIdx.x; i < 2 * 32 * DecSmem<Pol, D>::MLD; i += DEC_THREADS)
    (&sm.merge[0][0])[i] = 0.f;
  if (threadIdx.x < 32) {
    sm.lsum[threadIdx.x] = 0.f;
    sm.esum[threadIdx.x] = 0.f;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, sm.mw[w][col]);
  const float sc = (M == -INFINITY) ? 0.f : fast_exp2(m_run - M);
  const float l_tot = (l_part + xor32(l_part)) * sc;
  const float e_tot = (e_part + xor32(e_part)) * sc;
  if (half == 0) {
    atomicAdd(&sm.lsum[col], l_tot);
    atomicAdd(&sm.esum[col], e_tot);
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int d = 32 * dt + acc_row(a, half);
      atomicAdd(&sm.merge[0][col * DecSmem<Pol, D>::MLD + d], ou[dt][a] * sc);
      atomicAdd(&sm.merge[1][col * DecSmem<Pol, D>::MLD + d], kb[dt][a] * sc);
    }
  __syncthreads();

  // record of head g: [m, l, e, 0, O[D], U[D], Kbar[D]]  (m in log2 units;
  // l the rounded-operand sum, e the unrounded sum)
  for (int g = 0; g < G; ++g) {
    float* rec = part + (((size_t)b * Hq + hk * G + g) * nsplit + split) * REC;
    const int c0 = 2 * g;
    if (threadIdx.x == 0) {
      float M0 = -INFINITY;
      for (int w = 0; w < DEC_WAVES; ++w) M0 = fmaxf(M0, sm.mw[w][c0]);
      rec[0] = M0;
      rec[1] = sm.lsum[c0];
      rec[2] = sm.esum[c0];
      rec[3] = 0.f;
    }
    for (int d = threadIdx.x; d < D; d += DEC_THREADS) {
      rec[4 + d] = sm.merge[0][c0 * DecSmem<Pol, D>::MLD + d];
      rec[4 + D + d] = sm.merge[0][(c0 + 1) * DecSmem<Pol, D>::MLD + d];
      rec[4 + 2 * D + d] = sm.merge[1][c0 * DecSmem<Pol, D>::MLD + d];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 partial kernel on 16x16x32 MFMA tiles.
//
// Per wave and 32-key sub-tile: the K rows (loaded straight into A-operand
// registers, bf16) give S^T = K [q;rho]^T over 16 columns (2 per head, up to 8
// heads); K and V are then staged in the wave's LDS tile as fp16 rows and
// read back transposed (ds_read_b64_tr_b16) as the A operands of
//   [O|U]^T += V^T [p | p.r]^T   and   Kbar^T += K^T [p | p.r]^T.
// The next sub-tile's loads are issued as soon as the current one is staged.
// Lane layout of a 16x16 accumulator: acc[j] is row 4*g + j, column l % 16,
// with g = l / 16 the 16-lane group.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct Dec16Smem {
  static constexpr int LD = D + 16;  // fp16 row stride: 8 rows of one transpose read hit 8 bank groups
  static constexpr size_t TILE = (size_t)32 * LD;
  static constexpr int MLD = D + 1;
  union {
    _Float16 tiles[DEC_WAVES][2][TILE];  // per wave: K rows, V rows
    float merge[2][16 * MLD];            // [O/U, Kbar] x column x d
  };
  float mw[DEC_WAVES][16];
  float lsum[16];
  float esum[16];
};

__device__ __forceinline__ f16x4 tr16(const _Float16* p) {
  s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(f16x4, t);
}

__device__ __forceinline__ f16x8 cvt8(u32x4 raw) {
  const u16x8 b = __builtin_bit_cast(u16x8, raw);
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = bf16_bits_to_f16(b[e]);
  return h;
}

template <int D, int G>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode16_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rho, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len, float* __restrict__ part,
    int Hq, int Hkv, int S_max, int chunk, int nsplit, int hoff, float scale_log2) {
  constexpr int NS = D / 32;   // 32-deep score steps
  constexpr int ND = D / 16;   // 16-row d tiles of the value / Kbar accumulators
  constexpr int REC = 3 * D + 4;
  using SM = Dec16Smem<D>;
  __shared__ SM sm;

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int ctx = ctx_len[b];
  if (ctx < 1 || ctx > S_max) return;  // the merge writes NaN for this sequence
  const int k_begin = split * chunk;
  if (k_begin >= ctx) return;          // the merge reads only splits below ctx
  const int k_end = min(ctx, k_begin + chunk);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int hq0 = hk * (Hq / Hkv) + hoff;  // first query head of these columns

  // B operand of the score MFMAs: column c -> q (even) / rho (odd) of head hq0 + c/2
  bf16x8_t bop[NS];
  {
    const uint16_t* src = (c & 1) ? rho : q;
    const size_t row = ((size_t)b * Hq + hq0 + (c >> 1)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (c < 2 * G) raw = *reinterpret_cast<const u32x4*>(src + row + 32 * s + 8 * g);
      bop[s] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }
  const uint16_t* kbase = kc + ((size_t)(b * Hkv + hk) * S_max) * D;
  const uint16_t* vbase = vc + ((size_t)(b * Hkv + hk) * S_max) * D;
  _Float16* kt = sm.tiles[wave][0];
  _Float16* vt = sm.tiles[wave][1];

  f32x4 ou[ND], kb[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    ou[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    kb[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY, l_part = 0.f, e_part = 0.f;
  const bool used = c < 2 * G;
  const bool odd = c & 1;

  // raw bf16 K and V of one sub-tile: [key tile t][d step s]
  u32x4 kr[2][NS], vr[2][NS];
  auto load_sub = [&](int key0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // rows past k_end load row k_end-1 (valid, finite); they are masked below
      const int key = min(key0 + 16 * t + c, k_end - 1);
      const uint16_t* kp = kbase + (size_t)key * D + 8 * g;
      const uint16_t* vp = vbase + (size_t)key * D + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kr[t][s] = *reinterpret_cast<const u32x4*>(kp + 32 * s);
        vr[t][s] = *reinterpret_cast<const u32x4*>(vp + 32 * s);
      }
    }
  };

  int key0 = k_begin + DEC_SUB * wave;
  if (key0 < k_end) load_sub(key0);
  for (; key0 < k_end; key0 += DEC_GROUP_KEYS) {
    // scores of the two 16-key tiles
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[t][s]), bop[s],
                                                          sacc[t], 0, 0, 0);
    }
    // stage K and V rows (fp16) in this wave's LDS tiles
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = (16 * t + c) * SM::LD + 32 * s + 8 * g;
        *reinterpret_cast<f16x8*>(kt + off) = cvt8(kr[t][s]);
        *reinterpret_cast<f16x8*>(vt + off) = cvt8(vr[t][s]);
      }
    // next sub-tile's loads go out now (registers are free again)
    const int next = key0 + DEC_GROUP_KEYS;
    if (next < k_end) load_sub(next);
    wave_lds_sync();

    // softmax: even columns hold scores, odd columns r
    float sv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float se = dpp_even_partner(sacc[t][j]);
        if (key0 + 16 * t + 4 * g + j >= k_end) se = -INFINITY;
        sv[4 * t + j] = se;
        mt = fmaxf(mt, se);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    mt *= scale_log2;
    if (__any(mt > m_run + 4.f)) {
      // lazy rescale (p <= 16 in between; exact after the final normalisation)
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      l_part *= alpha;
      e_part *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ou[i][j] *= alpha;
          kb[i][j] *= alpha;
        }
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    f16x8 pop;
    float lsum = 0.f, esum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = used ? fast_exp2(__builtin_fmaf(sv[e], scale_log2, -m_use)) : 0.f;
      esum += p;
      const float val = odd ? p * sacc[e >> 2][e & 3] : p;
      const _Float16 h = (_Float16)val;
      lsum += (float)h;
      pop[e] = h;
    }
    l_part += lsum;
    e_part += esum;

    // value and Kbar MFMAs: A operands V^T and K^T from the transpose reads;
    // element e of group g is key 16*(e/4) + 4*g + e%4, matching pop
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int off = (4 * g + (c >> 2)) * SM::LD + 16 * dt + 4 * (c & 3);
      const f16x4 v0 = tr16(vt + off), v1 = tr16(vt + off + 16 * SM::LD);
      const f16x4 k0 = tr16(kt + off), k1 = tr16(kt + off + 16 * SM::LD);
      f16x8 av, ak;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = v0[e];
        av[4 + e] = v1[e];
        ak[e] = k0[e];
        ak[4 + e] = k1[e];
      }
      ou[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pop, ou[dt], 0, 0, 0);
      kb[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, pop, kb[dt], 0, 0, 0);
    }
    wave_lds_sync();
  }

  // ---- merge the four waves' states through LDS ----
  __syncthreads();
  if (g == 0) sm.mw[wave][c] = m_run;
  for (int i = threadIdx.x; i < 2 * 16 * SM::MLD; i += DEC_THREADS) (&sm.merge[0][0])[i] = 0.f;
  if (threadIdx.x < 16) {
    sm.lsum[threadIdx.x] = 0.f;
    sm.esum[threadIdx.x] = 0.f;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, sm.mw[w][c]);
  const float sc = (M == -INFINITY) ? 0.f : fast_exp2(m_run - M);
  float lt = l_part, et = e_part;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  et += __shfl_xor(et, 16, 64);
  et += __shfl_xor(et, 32, 64);
  if (g == 0) {
    atomicAdd(&sm.lsum[c], lt * sc);
    atomicAdd(&sm.esum[c], et * sc);
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 16 * dt + 4 * g + j;
      atomicAdd(&sm.merge[0][c * SM::MLD + d], ou[dt][j] * sc);
      atomicAdd(&sm.merge[1][c * SM::MLD + d], kb[dt][j] * sc);
    }
  __syncthreads();

  // record of head g: [m, l, e, 0, O[D], U[D], Kbar[D]]  (m in log2 units)
  for (int hh = 0; hh < G; ++hh) {
    float* rec = part + (((size_t)b * Hq + hq0 + hh) * nsplit + split) * REC;
    const int c0 = 2 * hh;
    if (threadIdx.x == 0) {
      float M0 = -INFINITY;
      for (int w = 0; w < DEC_WAVES; ++w) M0 = fmaxf(M0, sm.mw[w][c0]);
      rec[0] = M0;
      rec[1] = sm.lsum[c0];
      rec[2] = sm.esum[c0];
      rec[3] = 0.f;
    }
    for (int d = threadIdx.x; d < D; d += DEC_THREADS) {
      rec[4 + d] = sm.merge[0][c0 * SM::MLD + d];
      rec[4 + D + d] = sm.merge[0][(c0 + 1) * SM::MLD + d];
      rec[4 + 2 * D + d] = sm.merge[1][c0 * SM::MLD + d];
    }
  }
}

template <int D, int G>
hipError_t launch_partial16(const void* q, const void* rho, const void* kc, const void* vc,
                            const int32_t* ctx_len, float* part, int B, int Hq, int Hkv, int S_max,
                            int chunk, int nsplit, int hoff, float scale, hipStream_t stream) {
  dim3 grid(nsplit, Hkv, B);
  hipLaunchKernelGGL((decode16_partial_kernel<D, G>), grid, dim3(DEC_THREADS), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)rho, (const uint16_t*)kc, (const uint16_t*)vc,
                     ctx_len, part, Hq, Hkv, S_max, chunk, nsplit, hoff, scale * kLog2e);
  return hipGetLastError();
}

template <class Pol, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part,
                                                         const typename Pol::in_t* __restrict__ rho,
                                                         const int32_t* __restrict__ ctx_len,
                                                         float* __restrict__ o, float* __restrict__ lse,
                                                         int Hq, int S_max, int chunk, int nsplit) {
  constexpr int REC = 3 * D + 4;
  __shared__ float red[D / 64];
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int t = threadIdx.x;
  const int ctx = ctx_len[b];
  float* orow = o + (size_t)bh * D;
  if (ctx < 1 || ctx > S_max) {
    orow[t] = __builtin_nanf("");
    if (lse && t == 0) lse[bh] = __builtin_nanf("");
    return;
  }
  const int n = (ctx + chunk - 1) / chunk;
  const float* recs = part + (size_t)bh * nsplit * REC;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, recs[(size_t)s * REC]);
  float l = 0.f, le = 0.f, O = 0.f, U = 0.f, Kb = 0.f;
  for (int s = 0; s < n; ++s) {
    const float* r = recs + (size_t)s * REC;
    const float a = fast_exp2(r[0] - M);
    l += a * r[1];
    le += a * r[2];
    O += a * r[4 + t];
    U += a * r[4 + D + t];
    Kb += a * r[4 + 2 * D + t];
  }
  // c = (Kbar . rho) / l
  float x = Kb * Pol::to_f32(rho[(size_t)bh * D + t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  if ((t & 63) == 0) red[t >> 6] = x;
  __syncthreads();
  float dot = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) dot += red[w];
  const float inv = 1.f / l;
  const float c = dot * inv;
  orow[t] = O * inv * (1.f + c) - U * inv;
  if (lse && t == 0) lse[bh] = (M + __log2f(le)) * kLn2;
}

template <class Pol, int D, int G>
hipError_t launch_partial(const void* q, const void* rho, const void* kc, const void* vc,
                          const int32_t* ctx_len, float* part, int B, int Hkv, int S_max, int chunk,
                          int nsplit, float scale, hipStream_t stream) {
  using in_t = typename Pol::in_t;
  dim3 grid(nsplit, Hkv, B);
  hipLaunchKernelGGL((decode_partial_kernel<Pol, D, G>), grid, dim3(DEC_THREADS), 0, stream,
                     (const in_t*)q, (const in_t*)rho, (const in_t*)kc, (const in_t*)vc, ctx_len, part,
                     Hkv, S_max, chunk, nsplit, scale * kLog2e);
  return hipGetLastError();
}

template <class Pol, int D>
hipError_t launch_decode_t(const void* q, const void* rho, const void* kc, const void* vc,
                           const int32_t* ctx_len, float* o, float* lse, int B, int Hq, int Hkv,
                           int S_max, float scale, int chunk, int nsplit, float* part,
                           hipStream_t stream) {
  using in_t = typename Pol::in_t;
  const int G = Hq / Hkv;
  hipError_t e;
  if constexpr (sizeof(typename Pol::in_t) == 2) {
    // bf16: 16-column kernel; 16 heads per KV head take two column groups
    switch (G) {
      case 1: e = launch_partial16<D, 1>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, 0, scale, stream); break;
      case 2: e = launch_partial16<D, 2>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, 0, scale, stream); break;
      case 4: e = launch_partial16<D, 4>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, 0, scale, stream); break;
      case 8: e = launch_partial16<D, 8>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, 0, scale, stream); break;
      default:
        e = launch_partial16<D, 8>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, 0, scale, stream);
        if (e == hipSuccess)
          e = launch_partial16<D, 8>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, 8, scale, stream);
        break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<Pol, D>), dim3(B * Hq), dim3(D), 0, stream, part,
                       (const in_t*)rho, ctx_len, o, lse, Hq, S_max, chunk, nsplit);
    return hipGetLastError();
  }
  switch (G) {
    case 1: e = launch_partial<Pol, D, 1>(q, rho, kc, vc, ctx_len, part, B, Hkv, S_max, chunk, nsplit, scale, stream); break;
    case 2: e = launch_partial<Pol, D, 2>(q, rho, kc, vc, ctx_len, part, B, Hkv, S_max, chunk, nsplit, scale, stream); break;
    case 4: e = launch_partial<Pol, D, 4>(q, rho, kc, vc, ctx_len, part, B, Hkv, S_max, chunk, nsplit, scale, stream); break;
    case 8: e = launch_partial<Pol, D, 8>(q, rho, kc, vc, ctx_len, part, B, Hkv, S_max, chunk, nsplit, scale, stream); break;
    default: e = launch_partial<Pol, D, 16>(q, rho, kc, vc, ctx_len, part, B, Hkv, S_max, chunk, nsplit, scale, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<Pol, D>), dim3(B * Hq), dim3(D), 0, stream, part,
                     (const in_t*)rho, ctx_len, o, lse, Hq, S_max, chunk, nsplit);
  return hipGetLastError();
}

}  // namespace

// Split count: as few splits as give two workgroups per compute unit.  The
// partial kernel is bound by the loads each wave keeps in flight, and a long
// chunk keeps every wave streaming; more splits only add merge traffic and
// per-workgroup start-up.  Chunks stay at least 256 keys long.
int decode_auto_splits(int B, int Hkv, int S_max) {
  const long long slots = (long long)B * Hkv;
  long long ns = (512 + slots - 1) / slots;
  const long long max_ns = (S_max + 255) / 256;
  if (ns > max_ns) ns = max_ns;
  return ns < 1 ? 1 : (int)ns;
}

// Keys per split: S_max / num_splits rounded up to whole workgroup steps.
int decode_chunk_keys(int S_max, int num_splits) {
  int c = (S_max + num_splits - 1) / num_splits;
  c = ((c + DEC_GROUP_KEYS - 1) / DEC_GROUP_KEYS) * DEC_GROUP_KEYS;
  return c;
}

size_t decode_record_floats(int d) { return 3 * (size_t)d + 4; }

hipError_t launch_decode(int dtype, const void* q, const void* rho, const void* k_cache,
                         const void* v_cache, const int32_t* ctx_len, float* o, float* lse, int B,
                         int Hq, int Hkv, int S_max, int d, float scale, int num_splits,
                         float* partials, hipStream_t stream) {
  int ns = num_splits > 0 ? num_splits : decode_auto_splits(B, Hkv, S_max);
  if (ns > S_max) ns = S_max;
  const int chunk = decode_chunk_keys(S_max, ns);
  const int nsplit = (S_max + chunk - 1) / chunk;
  if (dtype == PLX_BF16) {
    if (d == 64)
      return launch_decode_t<PolBF16, 64>(q, rho, k_cache, v_cache, ctx_len, o, lse, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
    return launch_decode_t<PolBF16, 128>(q, rho, k_cache, v_cache, ctx_len, o, lse, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
  }
  if (d == 64)
    return launch_decode_t<PolF32, 64>(q, rho, k_cache, v_cache, ctx_len, o, lse, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
  return launch_decode_t<PolF32, 128>(q, rho, k_cache, v_cache, ctx_len, o, lse, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
}

}  // namespace plx
