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
// tile sit before the last step's MFMAs.  The epilogue
// rounds to bf16 (round to nearest even), transposes each wave's tile through
// LDS and stores whole rows of d, one head per 16-lane group.
#include "plx_common.hpp"
#include "plx_kernels.hpp"

namespace plx {

namespace {

constexpr int PJ_BM = 256;      // tokens per workgroup
constexpr int PJ_BN = 256;      // output features per workgroup
constexpr int PJ_BK = 64;       // reduction depth of one LDS tile
constexpr int PJ_THREADS = 512;
constexpr int PJ_LD = PJ_BK;  // LDS row stride (elements): 128 B, chunks XOR-swizzled
constexpr int PJ_OLD = 128 + 8;   // epilogue row stride (elements)
// the loads cover a tile as 8 waves x 4 instructions x 8 rows
static_assert(PJ_THREADS / 64 * 4 * 8 == PJ_BM && PJ_BM == PJ_BN, "tile load coverage");

struct ProjSmem {
  union {
    struct {
      uint16_t w[2][PJ_BN * PJ_LD];
      uint16_t x[2][PJ_BM * PJ_LD];
    } in;
    uint16_t out[8][64 * PJ_OLD];  // one 64 x 128 bf16 tile per wave
  };
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
          (__attribute__((address_space(3))) void*)&sm.in.w[buf][blk * 8 * PJ_LD], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)gx,
          (__attribute__((address_space(3))) void*)&sm.in.x[buf][blk * 8 * PJ_LD], 16, 0, 0);
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
    const uint16_t* wr = &sm.in.w[buf][(wn * 128 + c16) * PJ_LD + 8 * pc];
    const uint16_t* xr = &sm.in.x[buf][(wm * 64 + c16) * PJ_LD + 8 * pc];
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
  __syncthreads();  // every wave is done with the operand buffers

  // epilogue: acc[i][j][r] is feature wn*128 + 16 i + 4 g + r and token
  // wm*64 + 16 j + c; round to bf16 and transpose through LDS
  uint16_t* ot = sm.out[wave];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nl = 16 * i + 4 * g4, ml = 16 * j + c16;
      uint2 pk;
      pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
      pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      *reinterpret_cast<uint2*>(&ot[ml * PJ_OLD + nl]) = pk;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 16 lanes per token row, 8 features each: a head's whole d-row per group
  const int nq = Hq * d, nk = nq + Hkv * d, nv = nk + Hkv * d;
#pragma unroll 4
  for (int i = 0; i < 64 * 16 / 64; ++i) {
    const int it = 64 * i + lane;
    const int row = it >> 4, c = (it & 15) * 8;
    const int m = m0 + wm * 64 + row, n = n0 + wn * 128 + c;
    if (m >= M || n >= N) continue;
    const u32x4 val = *reinterpret_cast<const u32x4*>(&ot[row * PJ_OLD + c]);
    uint16_t* base;
    int H, loc;
    if (n < nq) {
      base = q, H = Hq, loc = n;
    } else if (n < nk) {
      base = k, H = Hkv, loc = n - nq;
    } else if (n < nv) {
      base = v, H = Hkv, loc = n - nk;
    } else {
      base = rho, H = Hq, loc = n - nv;
    }
    const int b = m / T, tt = m - b * T;
    const int head = loc / d, dd = loc - head * d;
    *reinterpret_cast<u32x4*>(base + (((size_t)b * H + head) * T + tt) * d + dd) = val;
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
