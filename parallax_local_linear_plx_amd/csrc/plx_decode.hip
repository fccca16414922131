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
// Kernel 1 (partial): a workgroup takes a range of one sequence's keys.  The
// query heads that share the KV head are stacked with their probes as the 2G
// columns [q_0, rho_0, q_1, rho_1, ...] of one MFMA B operand, so each K row is
// read once for all of them:  S^T = K [q;rho]^T  gives scores (even columns)
// and r = rho . k (odd columns) in one MFMA chain.  Per range it accumulates
//   m, l = sum p, C = sum p r, O = sum p v, U = sum (p r) v
// and writes one partial record per query head.  C / l equals kbar . rho
// exactly (kbar = sum_j w_j k_j), so the scalar C carries everything of the
// mean key the output needs, and it merges across ranges like l.
// Kernel 2 (merge): per (b, h) rescales the records to a common max and
// finishes  o = (O/l)(1 + C/l) - U/l,  LSE = M + ln e  (and, on request, the
// no-intercept output -U/l and the correction-to-output ratio).
#include <atomic>
#include <mutex>

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
  union {
    vel_t tiles[DEC_WAVES][D * DEC_TLD];  // per wave: V^T
    float merge[DEC_WAVES][32 * MLD];     // per wave: [O | U] x column x d
  };
  float mw[DEC_WAVES][32];
  float wl[DEC_WAVES][32];  // per wave: l (even columns) / C (odd columns)
  float we[DEC_WAVES][32];  // per wave: e
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

// The launch covers the nh <= 16 heads hoff .. hoff+nh-1 of every KV head's
// group of Hq / Hkv (2 nh of the 32 B-operand columns).
template <class Pol, int D>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode_partial_kernel(
    const typename Pol::in_t* __restrict__ q, const typename Pol::in_t* __restrict__ rho,
    const typename Pol::in_t* __restrict__ kc, const typename Pol::in_t* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, float* __restrict__ part, int Hq, int Hkv, int S_max,
    int chunk, int nsplit, int hoff, int nh, unsigned flags, float scale_log2) {
  using in_t = typename Pol::in_t;
  using sop_t = typename Pol::sop_t;
  using vop_t = typename Pol::vop_t;
  using vel_t = typename Pol::vel_t;
  constexpr int KW = Pol::KW, KSTEP = Pol::KSTEP;
  constexpr int NS = D / KSTEP;
  constexpr int NV = DEC_SUB / KSTEP;
  constexpr int ND = D / 32;
  constexpr int REC = 2 * D + 4;

  __shared__ DecSmem<Pol, D> sm;

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int ctx = ctx_len[b];
  if (ctx < 1 || ctx > S_max) return;  // the merge writes NaN for this sequence
  const int k_begin = split * chunk;
  if (k_begin >= ctx) return;  // the merge reads only splits below ctx
  const int k_end = min(ctx, k_begin + chunk);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int hq0 = hk * (Hq / Hkv) + hoff;  // first query head of this launch's share

  // B operand: column c -> q (even) or rho (odd) of head hq0 + c/2; with
  // uniform weights the q columns are zero (every score exactly 0, p = 1)
  sop_t bop[NS];
  {
    const int hq = hq0 + (col >> 1);
    const in_t* src = (col & 1) ? rho : q;
    const bool load = col < 2 * nh && ((col & 1) || !(flags & PLX_UNIFORM_WEIGHTS));
#pragma unroll
    for (int s = 0; s < NS; ++s)
      bop[s] = load ? load_sop<Pol>(src + ((size_t)b * Hq + hq) * D + KSTEP * s + KW * half)
                    : zero_sop<Pol>();
  }

  const in_t* kbase = kc + ((size_t)(b * Hkv + hk) * S_max) * D;
  const in_t* vbase = vc + ((size_t)(b * Hkv + hk) * S_max) * D;
  vel_t* vt = sm.tiles[wave];

  f32x16 ou[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) ou[i] = zero16();
  // l_part: sum of the rounded operands (normalises O and U; in the odd
  // columns it is C); e_part: the unrounded sum, used only for the LSE.
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

    // V rows -> transposed per-wave tile (value-operand type)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < KW; ++e) {
        const int d = KSTEP * s + KW * half + e;
        in_t vx;
        if constexpr (KW == 1)
          vx = vop[s];
        else
          vx = __builtin_bit_cast(u16x8, vop[s])[e];
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
    const bool used = col < 2 * nh;
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
      for (int a = 0; a < 16; ++a) ou[i][a] *= alpha;

    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      vop_t pop;
#pragma unroll
      for (int e = 0; e < KW; ++e) set_elem(pop, e, Pol::round_v(sv[KW * s + e]));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        vop_t av;
        const int drow = (32 * dt + col) * DEC_TLD;
#pragma unroll
        for (int e = 0; e < KW; ++e) set_elem(av, e, vt[drow + acc_row(KW * s + e, half)]);
        ou[dt] = Pol::mma_v(av, pop, ou[dt]);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four waves' states through LDS: each wave stores its
  // rescaled state in its own slot and the record sums the slots in wave
  // order, so the result does not depend on timing ----
  constexpr int MLD = DecSmem<Pol, D>::MLD;
  __syncthreads();
  if (half == 0) sm.mw[wave][col] = m_run;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, sm.mw[w][col]);
  const float sc = (M == -INFINITY) ? 0.f : fast_exp2(m_run - M);
  const float l_tot = (l_part + xor32(l_part)) * sc;
  const float e_tot = (e_part + xor32(e_part)) * sc;
  if (half == 0) {
    sm.wl[wave][col] = l_tot;
    sm.we[wave][col] = e_tot;
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int d = 32 * dt + acc_row(a, half);
      sm.merge[wave][col * MLD + d] = ou[dt][a] * sc;
    }
  __syncthreads();

  // record of head g: [m, l, e, C, O[D], U[D]]  (m in log2 units; l the
  // rounded-operand sum, e the unrounded sum; C the odd column's rounded sum)
  for (int g = 0; g < nh; ++g) {
    float* rec = part + (((size_t)b * Hq + hq0 + g) * nsplit + split) * REC;
    const int c0 = 2 * g;
    if (threadIdx.x == 0) {
      float M0 = -INFINITY, l0 = 0.f, e0 = 0.f, C0 = 0.f;
      for (int w = 0; w < DEC_WAVES; ++w) {
        M0 = fmaxf(M0, sm.mw[w][c0]);
        l0 += sm.wl[w][c0];
        e0 += sm.we[w][c0];
        C0 += sm.wl[w][c0 + 1];
      }
      rec[0] = M0;
      rec[1] = l0;
      rec[2] = e0;
      rec[3] = C0;
    }
    for (int d = threadIdx.x; d < D; d += DEC_THREADS) {
      float od = 0.f, ud = 0.f;
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) {
        od += sm.merge[w][c0 * MLD + d];
        ud += sm.merge[w][(c0 + 1) * MLD + d];
      }
      rec[4 + d] = od;
      rec[4 + D + d] = ud;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 partial kernels on 16x16x32 MFMA tiles.
//
// Per wave and 32-key sub-tile: the K rows (loaded straight into A-operand
// registers, bf16) give S^T = K [q;rho]^T over 16 columns (2 per head, up to 8
// heads); the raw V rows are then staged in the wave's LDS tile and read
// back transposed (ds_read_b64_tr_b16), converted to fp16, as the A operand of
//   [O|U]^T += V^T [p | p.r]^T.
// Since V passes through LDS anyway, its loads need not follow the MFMA
// layout: each V load instruction reads whole rows (1 KB contiguous), and as
// non-temporal loads, since every row is read once.  Measured on the 2 GB
// cache of the batched decode: 364 -> 320 us; the same loads for K (whose
// MFMA layout reads 64-byte pieces of 16 rows per instruction) were no
// faster as non-temporal loads, nor when K too was staged through LDS.
// DEC_NSET register sets of loads rotate: a set's next loads go out as soon
// as it has been staged, so a sub-tile's loads are in flight while the
// previous one is computed.
// Lane layout of a 16x16 accumulator: acc[j] is row 4*g + j, column l % 16,
// with g = l / 16 the 16-lane group.
//
// Two schedules share the per-range body:
//   chunked  : workgroup (split, kv head, b) takes keys [split*chunk, ...)
//              of one sequence (the caller's explicit split count);
//   balanced : the (b, kv head, key) space of all valid sequences, laid end to
//              end, is cut into DEC_BAL_CTAS equal contiguous ranges, one per
//              workgroup.  A range may span several (b, kv head) segments and
//              writes one record set per segment piece, at slot = workgroup +
//              segment index (unique, since pieces are ordered by both).  Every
//              workgroup streams the same number of keys whatever the mix of
//              context lengths.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Register sets of loads in flight per wave.  One set (16 KB per wave, eight
// waves per compute unit) already streams at the rate this grid reaches with
// loads alone; a second set measured no faster and needs the registers the
// occupancy of two workgroups per compute unit depends on.
constexpr int DEC_NSET = 1;
constexpr int DEC_BAL_CTAS = 512;  // balanced schedule: at most two workgroups per compute unit

// NCG column groups of 16: one for up to 8 query heads per KV head, two for 16.
template <int D, int NCG>
struct Dec16Smem {
  static constexpr int LD = D + 16;  // row stride: 8 rows of one transpose read hit 8 bank groups
  static constexpr size_t TILE = (size_t)32 * LD;
  static constexpr int MLD = D + 1;
  union {
    uint16_t tiles[DEC_WAVES][TILE];  // per wave: raw bf16 V rows
    float merge[DEC_WAVES][16 * MLD]; // per wave: [O | U] x column x d (one column group at a time)
  };
  uint16_t bq[NCG][16 * D];  // score B operands: [column group][column][d]
  float mw[DEC_WAVES][16];
  float wl[DEC_WAVES][16];  // per wave: l (even columns) / C (odd columns)
  float we[DEC_WAVES][16];  // per wave: e
};

__device__ __forceinline__ s16x4_t tr16raw(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
}

// Valid context length of sequence b (0 for a length outside [1, S_max]).
__device__ __forceinline__ int dec_len(const int32_t* __restrict__ ctx_len, int b, int S_max) {
  const int c = ctx_len[b];
  return (c >= 1 && c <= S_max) ? c : 0;
}

// Wave-uniform value into scalar registers (the caller guarantees uniformity).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uni(long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(x & 0xffffffffll));
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Start of the balanced range of workgroup w of P, in keys of the flattened space.
__device__ __forceinline__ long long bal_lo(long long w, long long W, int P) { return w * W / P; }

// Workgroup whose range holds key x of the flattened space: the largest w with
// bal_lo(w) <= x, i.e. w W < (x + 1) P.
__device__ __forceinline__ long long bal_wg(long long x, long long W, int P) {
  const long long w = ((x + 1) * P - 1) / W;
  return w < P - 1 ? w : P - 1;
}

// Total keys of the flattened space: Hkv * sum of valid lengths (every lane).
__device__ long long bal_total(const int32_t* __restrict__ ctx_len, int B, int Hkv, int S_max) {
  const int lane = threadIdx.x & 63;
  long long s = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    s += wave_sum_ll(b < B ? dec_len(ctx_len, b, S_max) : 0);
  }
  return s * Hkv;
}

// One workgroup's pass over keys [k_begin, k_end) of (b, hk) for the nh <= G
// heads hq0 .. hq0+nh-1 (G: the column capacity in heads); writes record hh
// at rec + hh * rec_stride:
//   [m (log2 units), l, e, C, O[D], U[D]].
// G = 16 takes two column groups: both B operands are multiplied by every K
// operand and both sets of value MFMAs share every V operand, so up to sixteen
// heads of a KV head read its cache once.
template <int D, int G>
__device__ __forceinline__ void dec16_range(Dec16Smem<D, (G > 8 ? 2 : 1)>& sm,
                                            const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ rho,
                                            const uint16_t* __restrict__ kc,
                                            const uint16_t* __restrict__ vc, int b, int hk, int hq0,
                                            int Hq, int Hkv, int S_max, int k_begin, int k_end,
                                            int nh, unsigned flags, float scale_log2,
                                            float* __restrict__ rec, size_t rec_stride) {
  constexpr int NS = D / 32;  // 32-deep score steps
  constexpr int ND = D / 16;  // 16-row d tiles of the value accumulators
  constexpr int NCG = G > 8 ? 2 : 1;  // column groups of 16 (8 heads each)
  using SM = Dec16Smem<D, NCG>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // B operands of the score MFMAs, staged once in LDS: column cc of group cg
  // holds q (even) or rho (odd) of head hq0 + 8 cg + cc/2 (zero for unused
  // columns, and for the q columns with uniform weights: every score is then
  // exactly 0, p = 1)
  const bool use_q = !(flags & PLX_UNIFORM_WEIGHTS);
  for (int i = threadIdx.x; i < NCG * 16 * D / 8; i += DEC_THREADS) {
    const int cg = i / (16 * D / 8), cc = (i / (D / 8)) % 16, d0 = (i % (D / 8)) * 8;
    const int head = 8 * cg + (cc >> 1);
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (head < nh && ((cc & 1) || use_q)) {
      const uint16_t* src = (cc & 1) ? rho : q;
      raw = *reinterpret_cast<const u32x4*>(src + ((size_t)b * Hq + hq0 + head) * D + d0);
    }
    *reinterpret_cast<u32x4*>(&sm.bq[cg][cc * D + d0]) = raw;
  }
  __syncthreads();
  const uint16_t* kbase = kc + ((size_t)(b * Hkv + hk) * S_max) * D;
  const uint16_t* vbase = vc + ((size_t)(b * Hkv + hk) * S_max) * D;
  uint16_t* vt = sm.tiles[wave];

  f32x4 ou[NCG][ND];
  float m_run[NCG], l_part[NCG], e_part[NCG];
  bool used[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
    for (int i = 0; i < ND; ++i) ou[cg][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    m_run[cg] = -INFINITY;
    l_part[cg] = e_part[cg] = 0.f;
    used[cg] = 8 * cg + (c >> 1) < nh;
  }
  const bool odd = c & 1;

  // raw bf16 K and V of one sub-tile: [key tile t][d step s]
  u32x4 kr[DEC_NSET][2][NS], vr[DEC_NSET][2][NS];
  // V rows are loaded whole: V load (t, s) of a sub-tile covers its rows
  // VRPI (t NS + s) .. + VRPI - 1, lane l holding chunk l % VCPR of row l / VCPR
  constexpr int VCPR = D / 8, VRPI = 64 / VCPR;
  static_assert(2 * NS * VRPI == DEC_SUB, "V sub-tile load coverage");
  const int vrow = lane / VCPR, vch = lane % VCPR;
  auto load_sub = [&](u32x4 (&kx)[2][NS], u32x4 (&vx)[2][NS], int key0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // rows past k_end load row k_end-1 (valid, finite); they are masked below
      const int key = min(key0 + 16 * t + c, k_end - 1);
      const uint16_t* kp = kbase + (size_t)key * D + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kx[t][s] = *reinterpret_cast<const u32x4*>(kp + 32 * s);
        const int vkey = min(key0 + VRPI * (t * NS + s) + vrow, k_end - 1);
        vx[t][s] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vbase + (size_t)vkey * D + 8 * vch));
      }
    }
  };

  auto process = [&](u32x4 (&kx)[2][NS], u32x4 (&vx)[2][NS], int key0) {
    f32x4 sacc[NCG][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) sacc[cg][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          sacc[cg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, kx[t][s]),
              *reinterpret_cast<const bf16x8_t*>(&sm.bq[cg][c * D + 32 * s + 8 * g]), sacc[cg][t],
              0, 0, 0);
    }
    // stage the raw V rows; the loaded registers feed only this write and the
    // score MFMAs
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        *reinterpret_cast<u32x4*>(vt + (VRPI * (t * NS + s) + vrow) * SM::LD + 8 * vch) = vx[t][s];
    // this set's next loads, unconditionally: past the end the rows clamp to
    // k_end-1, so every sub-tile issues the same loads and the waits stay exact
    load_sub(kx, vx, key0 + DEC_NSET * DEC_GROUP_KEYS);
    wave_lds_sync();

    // softmax per column group: even columns hold scores, odd columns r
    f16x8 pop[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float sv[8];
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float se = dpp_even_partner(sacc[cg][t][j]);
          if (key0 + 16 * t + 4 * g + j >= k_end) se = -INFINITY;
          sv[4 * t + j] = se;
          mt = fmaxf(mt, se);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      mt *= scale_log2;
      if (__any(mt > m_run[cg] + 4.f)) {
        // lazy rescale (p <= 16 in between; exact after the final normalisation)
        const float m_new = fmaxf(m_run[cg], mt);
        const float alpha = fast_exp2(m_run[cg] - m_new);
        l_part[cg] *= alpha;
        e_part[cg] *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) ou[cg][i][j] *= alpha;
        m_run[cg] = m_new;
      }
      const float m_use = (m_run[cg] == -INFINITY) ? 0.f : m_run[cg];
      float lsum = 0.f, esum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = used[cg] ? fast_exp2(__builtin_fmaf(sv[e], scale_log2, -m_use)) : 0.f;
        esum += p;
        const float val = odd ? p * sacc[cg][e >> 2][e & 3] : p;
        const _Float16 h = (_Float16)val;
        lsum += (float)h;
        pop[cg][e] = h;
      }
      l_part[cg] += lsum;
      e_part[cg] += esum;
    }

    // value MFMAs: A operand V^T from the transpose reads; element e of
    // group g is key 16*(e/4) + 4*g + e%4, matching pop
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int off = (4 * g + (c >> 2)) * SM::LD + 16 * dt + 4 * (c & 3);
      const s16x4_t v0 = tr16raw(vt + off), v1 = tr16raw(vt + off + 16 * SM::LD);
      f16x8 av;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = bf16_bits_to_f16((uint16_t)v0[e]);
        av[4 + e] = bf16_bits_to_f16((uint16_t)v1[e]);
      }
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
        ou[cg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pop[cg], ou[cg][dt], 0, 0, 0);
    }
    wave_lds_sync();
  };

  // Sub-tiles past k_end (at most DEC_NSET-1 per wave, at the end) are
  // processed too: every key is masked (p = 0), so they add nothing.
  int key0 = k_begin + DEC_SUB * wave;
#pragma unroll
  for (int i = 0; i < DEC_NSET; ++i) {
    // issue the sets oldest-first so each wait in the loop covers one set only
    load_sub(kr[i], vr[i], key0 + i * DEC_GROUP_KEYS);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; key0 < k_end; key0 += DEC_NSET * DEC_GROUP_KEYS) {
#pragma unroll
    for (int i = 0; i < DEC_NSET; ++i) process(kr[i], vr[i], key0 + i * DEC_GROUP_KEYS);
  }

  // ---- merge the four waves' states through LDS (each wave its own slot,
  // summed in wave order: the record does not depend on timing), one column
  // group at a time ----
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    __syncthreads();
    if (g == 0) sm.mw[wave][c] = m_run[cg];
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, sm.mw[w][c]);
    const float sc = (M == -INFINITY) ? 0.f : fast_exp2(m_run[cg] - M);
    float lt = l_part[cg], et = e_part[cg];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    et += __shfl_xor(et, 16, 64);
    et += __shfl_xor(et, 32, 64);
    if (g == 0) {
      sm.wl[wave][c] = lt * sc;
      sm.we[wave][c] = et * sc;
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 16 * dt + 4 * g + j;
        sm.merge[wave][c * SM::MLD + d] = ou[cg][dt][j] * sc;
      }
    __syncthreads();

    for (int hl = 0; hl < 8 && 8 * cg + hl < nh; ++hl) {
      float* r = rec + (8 * cg + hl) * rec_stride;
      const int c0 = 2 * hl;
      if (threadIdx.x == 0) {
        float M0 = -INFINITY, l0 = 0.f, e0 = 0.f, C0 = 0.f;
        for (int w = 0; w < DEC_WAVES; ++w) {
          M0 = fmaxf(M0, sm.mw[w][c0]);
          l0 += sm.wl[w][c0];
          e0 += sm.we[w][c0];
          C0 += sm.wl[w][c0 + 1];
        }
        r[0] = M0;
        r[1] = l0;
        r[2] = e0;
        r[3] = C0;
      }
      for (int d = threadIdx.x; d < D; d += DEC_THREADS) {
        float od = 0.f, ud = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) {
          od += sm.merge[w][c0 * SM::MLD + d];
          ud += sm.merge[w][(c0 + 1) * SM::MLD + d];
        }
        r[4 + d] = od;
        r[4 + D + d] = ud;
      }
    }
  }
  __syncthreads();  // the next range reuses the LDS tiles that alias the merge buffer
}

template <int D, int G>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode16_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rho, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len, float* __restrict__ part,
    int Hq, int Hkv, int S_max, int chunk, int nsplit, int hoff, int nh, unsigned flags,
    float scale_log2) {
  constexpr int REC = 2 * D + 4;
  __shared__ Dec16Smem<D, (G > 8 ? 2 : 1)> sm;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int ctx = dec_len(ctx_len, b, S_max);
  const int k_begin = split * chunk;
  if (k_begin >= ctx) return;  // the merge reads only splits below ctx (none if ctx is invalid)
  const int k_end = min(ctx, k_begin + chunk);
  const int hq0 = hk * (Hq / Hkv) + hoff;
  float* rec = part + (((size_t)b * Hq + hq0) * nsplit + split) * REC;
  dec16_range<D, G>(sm, q, rho, kc, vc, b, hk, hq0, Hq, Hkv, S_max, k_begin, k_end, nh, flags,
                    scale_log2, rec, (size_t)nsplit * REC);
}

// One wave merges the n records of one head (record i at rec0 + i * stride;
// a record with valid(i) false was never written and is skipped) into
//   o = (O/l)(1 + C/l) - U/l   (without an intercept: o = -U/l),
//   LSE = M + ln e   (natural log),
//   COR = ||U/l - (O/l)(C/l)|| / ||o||   (without an intercept: ||U/l|| / ||o||).
// Lane j holds elements j * D/64 ..; every record's O and U loads are issued
// unconditionally (the slots lie inside the workspace) so that they overlap.
template <int D, class Valid>
__device__ __forceinline__ void wave_merge(const float* __restrict__ rec0, size_t stride, int n,
                                           Valid valid, unsigned flags, float* __restrict__ orow,
                                           float* __restrict__ lse_out, float* __restrict__ cor_out) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  // O and U rows of eight records, loaded together; past the end the last
  // record is read again (it gets weight zero)
  auto load8 = [&](int first, float (&ov)[8][EPL], float (&uv)[8][EPL]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* r = rec0 + (size_t)min(first + j, n - 1) * stride + 4 + lane * EPL;
      if constexpr (EPL == 4) {
        const float4 o4 = *reinterpret_cast<const float4*>(r);
        const float4 u4 = *reinterpret_cast<const float4*>(r + D);
        ov[j][0] = o4.x, ov[j][1] = o4.y, ov[j][2] = o4.z, ov[j][3] = o4.w;
        uv[j][0] = u4.x, uv[j][1] = u4.y, uv[j][2] = u4.z, uv[j][3] = u4.w;
      } else if constexpr (EPL == 2) {
        const float2 o2 = *reinterpret_cast<const float2*>(r);
        const float2 u2 = *reinterpret_cast<const float2*>(r + D);
        ov[j][0] = o2.x, ov[j][1] = o2.y, uv[j][0] = u2.x, uv[j][1] = u2.y;
      } else {
        ov[j][0] = r[0], uv[j][0] = r[D];
      }
    }
  };
  float l = 0.f, e = 0.f, C = 0.f, O[EPL], U[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) O[j] = U[j] = 0.f;
  // a record that was never written (weight 0) may hold anything: selects,
  // not products, keep it out
  auto accum8 = [&](float a, int k0, int cnt, const float (&ov)[8][EPL], const float (&uv)[8][EPL]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j;
      const float ak = k < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), k & 63)) : 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        O[i] = ak != 0.f ? __builtin_fmaf(ak, ov[j][i], O[i]) : O[i];
        U[i] = ak != 0.f ? __builtin_fmaf(ak, uv[j][i], U[i]) : U[i];
      }
    }
  };

  // Records 0..63: one header per lane, and the rows of records 0..7, all
  // requested before the max is known (one round trip for most heads).
  float4 hdr = {-INFINITY, 0.f, 0.f, 0.f};
  const bool mine = lane < n && valid(lane);
  if (lane < n) hdr = *reinterpret_cast<const float4*>(rec0 + (size_t)lane * stride);
  float ov[8][EPL], uv[8][EPL];
  load8(0, ov, uv);
  float M = mine ? hdr.x : -INFINITY;
  for (int i = lane + 64; i < n; i += 64)
    if (valid(i)) M = fmaxf(M, rec0[(size_t)i * stride]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    float a = 0.f;
    if (base == 0) {
      if (mine) {
        a = fast_exp2(hdr.x - M);
        l += a * hdr.y;
        e += a * hdr.z;
        C += a * hdr.w;
      }
    } else if (i < n && valid(i)) {
      const float* r = rec0 + (size_t)i * stride;
      a = fast_exp2(r[0] - M);
      l += a * r[1];
      e += a * r[2];
      C += a * r[3];
    }
    const int cnt = min(64, n - base);
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      if (base != 0 || k0 != 0) load8(base + k0, ov, uv);
      accum8(a, k0, cnt, ov, uv);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    l += __shfl_xor(l, off, 64);
    e += __shfl_xor(e, off, 64);
    C += __shfl_xor(C, off, 64);
  }
  const float inv = 1.f / l;
  const float cc = C * inv;
  const bool no_icpt = flags & PLX_NO_INTERCEPT;
  float n_o = 0.f, n_c = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const float vbar = O[j] * inv, u = U[j] * inv;
    const float ov = no_icpt ? -u : vbar * (1.f + cc) - u;
    const float corr = no_icpt ? u : u - vbar * cc;
    orow[lane * EPL + j] = ov;
    n_o = __builtin_fmaf(ov, ov, n_o);
    n_c = __builtin_fmaf(corr, corr, n_c);
  }
  if (lse_out && lane == 0) *lse_out = (M + __log2f(e)) * kLn2;
  if (cor_out) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      n_o += __shfl_xor(n_o, off, 64);
      n_c += __shfl_xor(n_c, off, 64);
    }
    if (lane == 0) *cor_out = __builtin_sqrtf(n_c) / __builtin_sqrtf(n_o);
  }
}

template <int D, int G>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode16_balanced_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rho, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ ctx_len, float* __restrict__ part,
    int B, int Hq, int Hkv, int S_max, int hoff, int nh, unsigned flags, float scale_log2) {
  constexpr int REC = 2 * D + 4;
  __shared__ Dec16Smem<D, (G > 8 ? 2 : 1)> sm;
  const int lane = threadIdx.x & 63;
  const int Gfull = Hq / Hkv;
  const int P = gridDim.x;
  const long long W = uni(bal_total(ctx_len, B, Hkv, S_max));
  const long long lo = bal_lo(blockIdx.x, W, P), hi = bal_lo(blockIdx.x + 1, W, P);
  if (lo >= hi) return;

  // first sequence whose segments reach past lo: Hkv * (keys before b + len b) > lo
  int b = 0;
  long long before = 0;  // Hkv * (valid keys of sequences before b)
  {
    long long base = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int bb = b0 + lane;
      const long long len = bb < B ? dec_len(ctx_len, bb, S_max) : 0;
      long long incl = len;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const long long t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
      }
      const unsigned long long hit = __ballot(bb < B && (base + incl) * Hkv > lo);
      if (hit) {
        const int first = __ffsll(hit) - 1;
        b = b0 + first;
        before = __shfl(base + incl - len, first, 64) * Hkv;
        break;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  b = uni(b);
  before = uni(before);
  int len = uni(dec_len(ctx_len, b, S_max));
  int hk = (int)((lo - before) / len);
  int key = (int)((lo - before) % len);
  long long pos = lo;
  while (true) {
    const int k_end = (int)min((long long)len, key + (hi - pos));
    const int hq0 = hk * Gfull + hoff;
    const long long seg = (long long)b * Hkv + hk;
    float* rec = part + ((size_t)(blockIdx.x + seg) * Gfull + hoff) * REC;
    dec16_range<D, G>(sm, q, rho, kc, vc, b, hk, hq0, Hq, Hkv, S_max, key, k_end, nh, flags,
                      scale_log2, rec, REC);
    pos += k_end - key;
    if (pos >= hi) break;
    key = 0;
    if (++hk == Hkv) {
      hk = 0;
      do {
        ++b;
        len = uni(dec_len(ctx_len, b, S_max));
      } while (len == 0);  // pos < hi <= W guarantees a later non-empty sequence
    }
  }
}

template <int D, int G>
hipError_t launch_partial16(const void* q, const void* rho, const void* kc, const void* vc,
                            const int32_t* ctx_len, float* part, int B, int Hq, int Hkv, int S_max,
                            int chunk, int nsplit, int hoff, int nh, unsigned flags, float scale,
                            hipStream_t stream) {
  if (chunk <= 0) {
    hipLaunchKernelGGL((decode16_balanced_kernel<D, G>), dim3(nsplit), dim3(DEC_THREADS), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)rho, (const uint16_t*)kc, (const uint16_t*)vc,
                       ctx_len, part, B, Hq, Hkv, S_max, hoff, nh, flags, scale * kLog2e);
  } else {
    dim3 grid(nsplit, Hkv, B);
    hipLaunchKernelGGL((decode16_chunk_kernel<D, G>), grid, dim3(DEC_THREADS), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)rho, (const uint16_t*)kc, (const uint16_t*)vc,
                       ctx_len, part, Hq, Hkv, S_max, chunk, nsplit, hoff, nh, flags, scale * kLog2e);
  }
  return hipGetLastError();
}

// Chunked schedule: the records of (b, h) are splits 0 .. ceil(ctx/chunk)-1.
// A wave per head, four heads per block.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_chunk_kernel(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ ctx_len,
                                                                 float* __restrict__ o, float* __restrict__ lse,
                                                                 float* __restrict__ cor, unsigned flags,
                                                                 int B, int Hq, int S_max, int chunk, int nsplit) {
  constexpr int REC = 2 * D + 4;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= B * Hq) return;
  const int ctx = dec_len(ctx_len, bh / Hq, S_max);
  float* orow = o + (size_t)bh * D;
  float* lse_out = lse ? lse + bh : nullptr;
  float* cor_out = cor ? cor + bh : nullptr;
  if (ctx == 0) {
    for (int i = lane; i < D; i += 64) orow[i] = __builtin_nanf("");
    if (lane == 0) {
      if (lse_out) *lse_out = __builtin_nanf("");
      if (cor_out) *cor_out = __builtin_nanf("");
    }
    return;
  }
  const int n = (ctx + chunk - 1) / chunk;
  wave_merge<D>(part + (size_t)bh * nsplit * REC, REC, n, [](int) { return true; }, flags, orow,
                lse_out, cor_out);
}

// Balanced schedule: segment s = b * Hkv + h / G covers keys [start, end) of
// the flattened space; its records sit at slots w + s for the workgroups
// w = bal_wg(start) .. bal_wg(end - 1).  With fewer keys than workgroups
// (W < P) some of those ranges are empty and wrote no record.  A wave per head.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_balanced_kernel(const float* __restrict__ part,
                                                                    const int32_t* __restrict__ ctx_len,
                                                                    float* __restrict__ o, float* __restrict__ lse,
                                                                    float* __restrict__ cor, unsigned flags,
                                                                    int B, int Hq, int Hkv, int S_max, int P) {
  constexpr int REC = 2 * D + 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= B * Hq) return;
  const int b = bh / Hq, h = bh % Hq, Gfull = Hq / Hkv, hk = h / Gfull;
  const int len = dec_len(ctx_len, b, S_max);
  float* orow = o + (size_t)bh * D;
  float* lse_out = lse ? lse + bh : nullptr;
  float* cor_out = cor ? cor + bh : nullptr;
  if (len == 0) {
    for (int i = lane; i < D; i += 64) orow[i] = __builtin_nanf("");
    if (lane == 0) {
      if (lse_out) *lse_out = __builtin_nanf("");
      if (cor_out) *cor_out = __builtin_nanf("");
    }
    return;
  }
  long long tot = 0, pre = 0;
  for (int bb = lane; bb < B; bb += 64) {
    const int l = dec_len(ctx_len, bb, S_max);
    tot += l;
    if (bb < b) pre += l;
  }
  tot = wave_sum_ll(tot);
  pre = wave_sum_ll(pre);
  const long long W = tot * Hkv;
  const long long start = pre * Hkv + (long long)hk * len, end = start + len;
  const long long w0 = bal_wg(start, W, P);
  const int n = (int)(bal_wg(end - 1, W, P) - w0 + 1);
  const long long seg = (long long)b * Hkv + hk;
  wave_merge<D>(part + ((size_t)(w0 + seg) * Gfull + (h % Gfull)) * REC, (size_t)Gfull * REC, n,
                [&](int i) { return W >= P || bal_lo(w0 + i, W, P) < bal_lo(w0 + i + 1, W, P); },
                flags, orow, lse_out, cor_out);
}

template <class Pol, int D>
hipError_t launch_partial(const void* q, const void* rho, const void* kc, const void* vc,
                          const int32_t* ctx_len, float* part, int B, int Hq, int Hkv, int S_max,
                          int chunk, int nsplit, int hoff, int nh, unsigned flags, float scale,
                          hipStream_t stream) {
  using in_t = typename Pol::in_t;
  dim3 grid(nsplit, Hkv, B);
  hipLaunchKernelGGL((decode_partial_kernel<Pol, D>), grid, dim3(DEC_THREADS), 0, stream,
                     (const in_t*)q, (const in_t*)rho, (const in_t*)kc, (const in_t*)vc, ctx_len, part,
                     Hq, Hkv, S_max, chunk, nsplit, hoff, nh, flags, scale * kLog2e);
  return hipGetLastError();
}

template <class Pol, int D>
hipError_t launch_decode_t(const void* q, const void* rho, const void* kc, const void* vc,
                           const int32_t* ctx_len, float* o, float* lse, float* cor,
                           unsigned flags, int B, int Hq, int Hkv, int S_max, float scale, int chunk,
                           int nsplit, float* part, hipStream_t stream) {
  const int G = Hq / Hkv;
  hipError_t e = hipSuccess;
  // Every group of G = Hq / Hkv query heads is covered by launches of at most
  // 16 heads (hoff .. hoff + nh - 1 of each group), each on the smallest
  // kernel whose column capacity holds nh heads; a group of up to 16 heads
  // thus reads its KV head's cache once.
  auto cap_of = [](int nh) { return nh <= 1 ? 1 : nh <= 2 ? 2 : nh <= 4 ? 4 : nh <= 8 ? 8 : 16; };
  if constexpr (sizeof(typename Pol::in_t) == 2) {
    // bf16: 16-column kernel; more than 8 heads take two column groups of the
    // same launch
    for (int hoff = 0; hoff < G && e == hipSuccess; hoff += 16) {
      const int nh = min(16, G - hoff);
#define PLX_P16(GG)                                                                                \
  launch_partial16<D, GG>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit, hoff,  \
                          nh, flags, scale, stream)
      switch (cap_of(nh)) {
        case 1: e = PLX_P16(1); break;
        case 2: e = PLX_P16(2); break;
        case 4: e = PLX_P16(4); break;
        case 8: e = PLX_P16(8); break;
        default: e = PLX_P16(16); break;
      }
#undef PLX_P16
    }
    if (e != hipSuccess) return e;
    if (chunk <= 0)
      hipLaunchKernelGGL((decode_merge_balanced_kernel<D>), dim3((B * Hq + 3) / 4), dim3(256), 0, stream,
                         part, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, nsplit);
    else
      hipLaunchKernelGGL((decode_merge_chunk_kernel<D>), dim3((B * Hq + 3) / 4), dim3(256), 0, stream,
                         part, ctx_len, o, lse, cor, flags, B, Hq, S_max, chunk, nsplit);
    return hipGetLastError();
  } else {
    // fp32: the generic 32-column kernel (chunked schedule only), up to 16
    // heads per launch
    for (int hoff = 0; hoff < G && e == hipSuccess; hoff += 16)
      e = launch_partial<Pol, D>(q, rho, kc, vc, ctx_len, part, B, Hq, Hkv, S_max, chunk, nsplit,
                                 hoff, min(16, G - hoff), flags, scale, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_chunk_kernel<D>), dim3((B * Hq + 3) / 4), dim3(256), 0, stream,
                       part, ctx_len, o, lse, cor, flags, B, Hq, S_max, chunk, nsplit);
    return hipGetLastError();
  }
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

size_t decode_record_floats(int d) { return 2 * (size_t)d + 4; }

// Workgroups of the balanced schedule: two per compute unit, fewer when the
// cache holds under ~512 keys per workgroup.  Small caches are latency-bound
// (each 128-key step of a workgroup waits for its loads), so they take short
// ranges: 512 keys per workgroup measured 16-20 us per call where 1024 took
// 22-24 us (B = 1..16, 1K-4K keys); 256 was no better overall.
int decode_balanced_ctas(int B, int Hkv, int S_max) {
  const long long keys = (long long)B * Hkv * S_max;
  long long p = (keys + 511) / 512;
  if (p > DEC_BAL_CTAS) p = DEC_BAL_CTAS;
  return p < 1 ? 1 : (int)p;
}

// Record slots of the balanced schedule: one per (workgroup, segment) piece,
// at most P + B * Hkv.
size_t decode_balanced_records(int B, int Hq, int Hkv, int S_max) {
  return ((size_t)decode_balanced_ctas(B, Hkv, S_max) + (size_t)B * Hkv) * (size_t)(Hq / Hkv);
}

hipError_t launch_decode(int dtype, const void* q, const void* rho, const void* k_cache,
                         const void* v_cache, const int32_t* ctx_len, float* o, float* lse,
                         float* cor, unsigned flags, int B, int Hq, int Hkv, int S_max, int d,
                         float scale, int num_splits, float* partials, hipStream_t stream) {
  if (dtype == PLX_BF16 && num_splits == 0) {
    // balanced schedule (chunk 0); nsplit carries the workgroup count
    const int P = decode_balanced_ctas(B, Hkv, S_max);
    if (d == 64)
      return launch_decode_t<PolBF16, 64>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, 0, P, partials, stream);
    if (d == 256)
      return launch_decode_t<PolBF16, 256>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, 0, P, partials, stream);
    return launch_decode_t<PolBF16, 128>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, 0, P, partials, stream);
  }
  int ns = num_splits > 0 ? num_splits : decode_auto_splits(B, Hkv, S_max);
  if (ns > S_max) ns = S_max;
  const int chunk = decode_chunk_keys(S_max, ns);
  const int nsplit = (S_max + chunk - 1) / chunk;
  if (dtype == PLX_BF16) {
    if (d == 64)
      return launch_decode_t<PolBF16, 64>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
    if (d == 256)
      return launch_decode_t<PolBF16, 256>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
    return launch_decode_t<PolBF16, 128>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
  }
  if (d == 64)
    return launch_decode_t<PolF32, 64>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
  return launch_decode_t<PolF32, 128>(q, rho, k_cache, v_cache, ctx_len, o, lse, cor, flags, B, Hq, Hkv, S_max, scale, chunk, nsplit, partials, stream);
}

// ---------------------------------------------------------------------------
// Records for plx_decode_noalloc: a static device array, one per GPU (each GPU
// the library runs on holds its own copy until the process ends).  In host
// code `decode_scratch` names a host-side stand-in, not the device array, so
// its device address is asked for once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to the kernels.
static __device__ __align__(256) float decode_scratch[PLX_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_for_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(decode_scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<float*>(addr);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc(int dtype, const void* q, const void* rho, const void* k_cache,
                                 const void* v_cache, const int32_t* ctx_len, float* o, float* lse,
                                 int B, int Hq, int Hkv, int S_max, int d, float scale,
                                 int num_splits, hipStream_t stream) {
  float* part = nullptr;
  const hipError_t e = scratch_for_current_device(&part);
  if (e != hipSuccess) return e;
  // the records need no clearing: the merge reads only records this call's
  // partial kernel writes (contents on entry are ignored, as for plx_decode)
  return launch_decode(dtype, q, rho, k_cache, v_cache, ctx_len, o, lse, nullptr, 0u, B, Hq, Hkv,
                       S_max, d, scale, num_splits, part, stream);
}

}  // namespace plx
