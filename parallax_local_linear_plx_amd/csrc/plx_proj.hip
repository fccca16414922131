// The projection in front of the operator: one GEMM that forms the query,
// key, value and probe of every token, written straight into the head-major
// [B, H, T, d] layout the attention kernels read.
//
// The probe is a learned linear map of the layer input, rho_i = W_R x_i
// ("当注意力学会追问...", section 1.3; "Riepilogo Tecnico: Parallax ...",
// section "Meccanismo Principale"), a fourth projection beside W_Q, W_K and
// W_V.  Stacking the four weights as W = [W_Q; W_K; W_V; W_R] (N = (2 Hq +
// 2 Hkv) d rows, D columns) turns them into one GEMM  Y = X W^T  over the
// M = B T tokens, so the layer input is read once for all four.
//
// Kernel: 256 x 256 output tiles (tokens x features), eight waves, two per
// SIMD, each owning 128 features x 64 tokens of the tile as 8 x 4
// accumulators of the 16x16x32 bf16 MFMA (fp32; on gfx950 the 16x16x32 form
// sustains about 15% more of the matrix-core peak than 32x32x16).  64-deep W
// and X tiles are double-buffered in LDS and loaded straight into it
// (global_load_lds, no register staging) in an XOR-swizzled layout that keeps
// the operand reads free of bank conflicts; tile t+1 is requested at the
// start of tile t.  The operands of each 32-deep step are read from LDS while
// the previous step's MFMAs run, in two groups between them (the tile loads
// likewise); at a tile boundary the barrier and the first reads of the next
// tile sit before the last step's MFMAs.  The epilogue rounds to bf16 (round
// to nearest even) and stores straight from the accumulators: two permlane16
// swaps per pair of 16-feature blocks give each lane 8 adjacent features of
// one token, so the four lanes of a token write 64 contiguous bytes of one
// head's d-row (no LDS round trip, no barrier).
#include "plx_common.hpp"
#include "plx_kernels.hpp"

namespace plx {

namespace {

constexpr int PJ_BM = 256;      // tokens per workgroup
constexpr int PJ_BN = 256;      // output features per workgroup
constexpr int PJ_BK = 64;       // reduction depth of one LDS tile
constexpr int PJ_THREADS = 512;
constexpr int PJ_LD = PJ_BK;  // LDS row stride (elements): 128 B, chunks XOR-swizzled
// the loads cover a tile as 8 waves x 4 instructions x 8 rows
static_assert(PJ_THREADS / 64 * 4 * 8 == PJ_BM && PJ_BM == PJ_BN, "tile load coverage");

struct ProjSmem {
  uint16_t w[2][PJ_BN * PJ_LD];
  uint16_t x[2][PJ_BM * PJ_LD];
};

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const __bf16 ha = static_cast<__bf16>(a), hb = static_cast<__bf16>(b);
  return (unsigned)__builtin_bit_cast(uint16_t, ha) | ((unsigned)__builtin_bit_cast(uint16_t, hb) << 16);
}

__global__ __launch_bounds__(PJ_THREADS, 1) void proj_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ q,
    uint16_t* __restrict__ k, uint16_t* __restrict__ v, uint16_t* __restrict__ rho, int T, int K,
    int Hq, int Hkv, int d, int M, int N) {
  __shared__ ProjSmem sm;
  const int nmb = (M + PJ_BM - 1) / PJ_BM;
  const int nnb = (N + PJ_BN - 1) / PJ_BN;
  // tiles of one feature block are consecutive, and consecutive tiles share an
  // XCD, so the eight that run together on one XCD read the same W tile
  const int lin = xcd_block_order(blockIdx.x, nmb, nmb * nnb);
  const int m0 = (lin % nmb) * PJ_BM;
  const int n0 = (lin / nmb) * PJ_BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;  // wave tile: features wn*128.., tokens wm*64..

  // Global -> LDS without registers: each wave's load instruction fills 8
  // rows (1 KB) of a tile; lane l writes 16-byte chunk l % 8 of row l / 8.
  // Physical chunk p of row r holds logical chunk p ^ ((r >> 1) & 7), which
  // spreads the 16 rows one operand read touches over all 64 banks.
  auto gload = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = wave * 4 + j;           // 8-row block of the 256-row tile
      const int row = blk * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ ((row >> 1) & 7);
      const uint16_t* gw = w + (size_t)min(n0 + row, N - 1) * K + k0 + 8 * lc;
      const uint16_t* gx = x + (size_t)min(m0 + row, M - 1) * K + k0 + 8 * lc;
      __builtin_amdgcn_global_load_lds((const void*)gw,
          (__attribute__((address_space(3))) void*)&sm.w[buf][blk * 8 * PJ_LD], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)gx,
          (__attribute__((address_space(3))) void*)&sm.x[buf][blk * 8 * PJ_LD], 16, 0, 0);
    }
  };
  // operands of one 32-deep step: A = W rows (features), B = X rows (tokens);
  // lane (c, g) supplies row c of each 16-row block and depth 8g .. 8g+7 of
  // the step (logical chunk 4 ks + g; the swizzle depends only on the row)
  struct Ops { bf16x8 a[8], b[4]; };
  const int c16 = lane & 15, g4 = lane >> 4;
  const int swz = (c16 >> 1) & 7;
  auto read_ops = [&](Ops& o, int buf, int ks) {
    const int pc = (4 * ks + g4) ^ swz;
    const uint16_t* wr = &sm.w[buf][(wn * 128 + c16) * PJ_LD + 8 * pc];
    const uint16_t* xr = &sm.x[buf][(wm * 64 + c16) * PJ_LD + 8 * pc];
#pragma unroll
    for (int i = 0; i < 8; ++i) o.a[i] = *reinterpret_cast<const bf16x8*>(wr + 16 * i * PJ_LD);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.b[i] = *reinterpret_cast<const bf16x8*>(xr + 16 * i * PJ_LD);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto mfmas = [&](const Ops& o) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
  };

  const int ntiles = K / PJ_BK;
  gload(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  Ops cur, nxt;
  read_ops(cur, 0, 0);
  static_assert(PJ_BK == 64, "two 32-deep steps per tile");
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // step 0: tile t+1 into the other buffer (whose tile t-1 every wave
    // finished reading before the barrier that ended tile t-1; the last tile
    // reloads itself there, which keeps the block free of branches) and the
    // operands of step 1, issued in two groups between the MFMAs
    __builtin_amdgcn_sched_barrier(0);
    gload(buf ^ 1, min(t + 1, ntiles - 1) * PJ_BK);
    read_ops(nxt, buf, 1);
    mfmas(cur);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);   // global loads
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
    // step 1: wait for tile t+1, make it visible, read its first operands
    // between this step's MFMAs
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    read_ops(nxt, buf ^ 1, 0);
    mfmas(cur);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  }
  __builtin_amdgcn_s_waitcnt(0);
  // epilogue from registers: acc[i][j][r] is feature wn*128 + 16 i + 4 g + r
  // of token wm*64 + 16 j + c; two permlane16 swaps per pair of feature
  // blocks (2p, 2p+1) leave in lane (c, g) the 8 adjacent features
  // 16 (2p + g % 2) + 8 (g / 2) .. + 7 of token c: 64 contiguous bytes of
  // one head's d-row per token and store
  const int nq = Hq * d, nk = nq + Hkv * d, nv = nk + Hkv * d;
  int bj[4];
  size_t tok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = min(m0 + wm * 64 + 16 * j + c16, M - 1);
    bj[j] = m / T;
    tok[j] = (size_t)(m - bj[j] * T) * d;
  }
  const int lf = 16 * (g4 & 1) + 8 * (g4 >> 1);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int nb = n0 + wn * 128 + 32 * p;  // one tensor and head for these 32 features
    if (nb >= N) continue;
    uint16_t* base;
    int H, loc;
    if (nb < nq) {
      base = q, H = Hq, loc = nb;
    } else if (nb < nk) {
      base = k, H = Hkv, loc = nb - nq;
    } else if (nb < nv) {
      base = v, H = Hkv, loc = nb - nk;
    } else {
      base = rho, H = Hq, loc = nb - nv;
    }
    const int head = loc / d, dd = loc - head * d;
    uint16_t* hb = base + (size_t)head * T * d + dd + lf;
    const size_t bstride = (size_t)H * T * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 ea = acc[2 * p][j], eb = acc[2 * p + 1][j];
      const unsigned a0 = pack_bf16x2(ea[0], ea[1]), a1 = pack_bf16x2(ea[2], ea[3]);
      const unsigned b0 = pack_bf16x2(eb[0], eb[1]), b1 = pack_bf16x2(eb[2], eb[3]);
      const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
      u32x4 val;
      val[0] = s0[0];
      val[1] = s1[0];
      val[2] = s0[1];
      val[3] = s1[1];
      if (m0 + wm * 64 + 16 * j + c16 < M)
        *reinterpret_cast<u32x4*>(hb + bj[j] * bstride + tok[j]) = val;
    }
  }
}

}  // namespace

hipError_t launch_proj(const void* x, const void* w, void* q, void* k, void* v, void* rho, int B,
                       int T, int D, int Hq, int Hkv, int d, hipStream_t stream) {
  const int M = B * T, N = (2 * Hq + 2 * Hkv) * d;
  const int tiles = ((M + PJ_BM - 1) / PJ_BM) * ((N + PJ_BN - 1) / PJ_BN);
  hipLaunchKernelGGL(proj_kernel, dim3(tiles), dim3(PJ_THREADS), 0, stream, (const uint16_t*)x,
                     (const uint16_t*)w, (uint16_t*)q, (uint16_t*)k, (uint16_t*)v, (uint16_t*)rho, T, D,
                     Hq, Hkv, d, M, N);
  return hipGetLastError();
}

}  // namespace plx
