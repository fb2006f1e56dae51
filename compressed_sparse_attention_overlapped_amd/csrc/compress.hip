// Gated overlapping compressor for gfx950.
//
// Two launches (migration notes section 3.2: linear_wkv + linear_wgate, then
// a softmax over the overlapping window; DS-V4 analysis section 1.3):
//  1. proj: PG[s][row][c] = sum_{k in split s} x[row][k] * W[c][k] for the
//     stacked weight [W_kv; W_gate] (c < E: value channel, c >= E: gate
//     logit).  bf16 uses MFMA 32x32x16 tiles staged through LDS; fp32 uses a
//     plain VALU dot product.  Calls with few output tiles split K so that
//     enough workgroups run; the pool sums the split partials.
//  2. pool: one workgroup per emitted entry: per channel, a softmax of
//     G + ape over the window tokens (taken from this call's rows or from the
//     carried state), the weighted sum of P, then the storage rounding (fp32,
//     bf16 RNE, or e4m3 with a per-row amax/448 scale).  Extra workgroups
//     write the carried state for the next call.
#include <algorithm>
#include <cmath>

#include "common.h"

namespace csa {

// ---------------------------------------------------------------- proj (bf16)
// Tile 128 x 128 x 64, 512 threads = 8 waves in a 2 x 4 grid of 64 x 32
// (2 x 1 MFMA 32x32x16 per 16-deep k step; two waves per SIMD, so that one
// wave's products overlap another's loads and barrier).  The LDS tiles are
// double buffered; two more k tiles are in flight in two register stages (k tile
// t + 2 is requested as soon as k tile t has moved to LDS), so the load
// latency is hidden behind two tiles of products.  Loads are unconditional
// (rows past M and columns past N read row 0 and are dropped at the store;
// k tiles past the end re-read the last one) so that every wait counts them
// exactly.  LDS rows are padded to 72 bf16 (36 dwords) so that the 16-byte
// fragment reads of 16 consecutive rows hit all 64 banks once.  K % 64 == 0
// (checked by the host).
constexpr int PJ_BM = 128, PJ_BN = 128, PJ_BK = 64;
constexpr int PJ_LDS_STRIDE = PJ_BK + 8;
constexpr int PJ_TILE = PJ_BM * PJ_LDS_STRIDE;  // bf16 per operand tile

// The k loop of one 128 x 128 tile: arow[u] / brow[u] point at the k0 = 0
// element of the A row / B row that thread chunk u (of two) stages; acc gets
// the wave's 64 x 32 block (wave w: rows 64 (w / 4), columns 32 (w % 4)).
__device__ __forceinline__ void pj_mainloop(uint16_t* As, uint16_t* Bs,
                                            const uint16_t* const (&arow)[2],
                                            const uint16_t* const (&brow)[2], int nk,
                                            f32x16 (&acc)[2]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 2) * 64, wn = (wave & 3) * 32;
  u32x4 ra[2][2], rb[2][2];
  auto load = [&](int kt, u32x4(&a)[2], u32x4(&bq)[2]) {
    const int k0 = min(kt, nk - 1) * PJ_BK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      a[u] = *(const u32x4*)(arow[u] + k0);
      bq[u] = *(const u32x4*)(brow[u] + k0);
    }
  };
  auto store = [&](int buf, const u32x4(&a)[2], const u32x4(&bq)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = u * 512 + tid, r = c >> 3, q = c & 7;
      *(u32x4*)(&As[buf * PJ_TILE + r * PJ_LDS_STRIDE + q * 8]) = a[u];
      *(u32x4*)(&Bs[buf * PJ_TILE + r * PJ_LDS_STRIDE + q * 8]) = bq[u];
    }
  };
  for (int i = 0; i < 2; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  auto compute = [&](int buf) {
    // four k steps of 16; lane holds 8 consecutive k of one row (A) / column (B)
#pragma unroll
    for (int ks = 0; ks < PJ_BK / 16; ++ks) {
      bf16x8 a[2];
      for (int i = 0; i < 2; ++i)
        a[i] = *(const bf16x8*)(&As[buf * PJ_TILE +
                                    (wm + i * 32 + (lane & 31)) * PJ_LDS_STRIDE + ks * 16 +
                                    (lane >> 5) * 8]);
      const bf16x8 b = *(const bf16x8*)(&Bs[buf * PJ_TILE + (wn + (lane & 31)) * PJ_LDS_STRIDE +
                                            ks * 16 + (lane >> 5) * 8]);
      for (int i = 0; i < 2; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i], 0, 0, 0);
    }
  };
  // step kt: multiply k tile kt (LDS buffer kt & 1), move k tile kt + 1 from
  // its register stage to the other buffer, refill that stage with k tile
  // kt + 3
  auto step = [&](int kt, u32x4(&a)[2], u32x4(&bq)[2]) {
    compute(kt & 1);
    store((kt + 1) & 1, a, bq);
    load(kt + 3, a, bq);
    __syncthreads();
  };
  if (nk > 0) {
    load(0, ra[0], rb[0]);
    store(0, ra[0], rb[0]);
    load(1, ra[1], rb[1]);
    load(2, ra[0], rb[0]);
    __syncthreads();
    int kt = 0;
    // stage (kt + 1) & 1 holds k tile kt + 1
    for (; kt + 2 < nk; kt += 2) {
      step(kt, ra[1], rb[1]);
      step(kt + 1, ra[0], rb[0]);
    }
    for (; kt < nk; ++kt) {  // the last one or two k tiles
      compute(kt & 1);
      if (kt + 1 < nk) store((kt + 1) & 1, (kt & 1) ? ra[0] : ra[1], (kt & 1) ? rb[0] : rb[1]);
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(512) proj_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_kv,
    const uint16_t* __restrict__ w_gate, float* __restrict__ pg, int M, int E, int K,
    int k_per_split) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * PJ_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * PJ_TILE];
  const int N = 2 * E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.x * PJ_BM, n0 = blockIdx.y * PJ_BN;
  const int split = blockIdx.z;
  const int kb = split * k_per_split, ke = min(K, kb + k_per_split);
  const int nk = (ke - kb) / PJ_BK;
  const int wm = (wave >> 2) * 64, wn = (wave & 3) * 32;

  // global -> LDS: a tile row is 64 bf16 = 8 chunks of 16 B; 128 rows x 8 =
  // 1024 chunks per operand, 2 per thread (rows r = c / 8, chunk q = c % 8)
  const uint16_t* arow[2];
  const uint16_t* brow[2];
  for (int u = 0; u < 2; ++u) {
    const int c = u * 512 + tid, r = c >> 3, q = c & 7;
    const int gm = m0 + r < M ? m0 + r : 0, gn = n0 + r < N ? n0 + r : 0;
    arow[u] = x + (size_t)gm * K + kb + q * 8;
    brow[u] = (gn < E ? w_kv + (size_t)gn * K : w_gate + (size_t)(gn - E) * K) + kb + q * 8;
  }
  f32x16 acc[2];
  pj_mainloop(As, Bs, arow, brow, nk, acc);
  // accumulator layout (32x32): lane holds column (lane & 31), rows
  // 8 (r / 4) + 4 (lane / 32) + (r % 4)
  float* out = pg + (size_t)split * M * N;
  const int col = n0 + wn + (lane & 31);
  if (col < N)
    for (int i = 0; i < 2; ++i)
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) out[(size_t)row * N + col] = acc[i][r];
      }
}

// ------------------------------------------- fused projection + pool (bf16)
// The compressor of a prefill chunk (bf16 input, m = 4 with overlap, so that
// an entry pools the 8 tokens of blocks i - 1 and i; fp32 or bf16 output; no
// step that mixes channels) with the overlapping windows pooled out of LDS.
// Workgroup (t, c, b): the 32 blocks i0 + 32 t .. i0 + 32 t + 31 of sequence
// b (128 token positions from 4 (i0 + 32 t), i0 the call's first entry), and
// channels [64 c, 64 c + 64) of P and the same of G as the tile's 128
// columns; tiles of whole blocks, so that an 8K chunk with 256 channels is
// 64 x 4 workgroups, one per compute unit.  After the k loop the fp32 P and
// G tiles go to LDS (over the operand buffers) and each thread pools entries
// of one channel: the tile's entries i0 + 32 t + k, k = 1 .. 31, have both
// of their blocks in it.  The first block of every tile and the last block
// of every tile go to the workspace, and the seam kernel pools the entries
// i0 + 32 t from them (t = 0: the previous block from the carried state).
// Tokens before the call come from the carried state (absent without it);
// tile positions among the call's last 7 tokens go to the next call's state.
// GEMM rows for positions outside the call read row 0 of the sequence and
// are not used.
constexpr int FU_BLK = 32, FU_CH = 64, FU_PS = FU_CH + 8;  // fp32 LDS row stride

// One token of the workspace's seam buffer: [B][n_tiles][2 (first, last
// block)][4 tokens][2 (P, G)][E] fp32.
__device__ __forceinline__ size_t fu_seam_at(int b, int n_tiles, int t, int which, int u, int pg,
                                            int E, int e) {
  return ((((((size_t)b * n_tiles + t) * 2 + which) * 4 + u) * 2 + pg) * E) + e;
}

// P and G of one window token (absent: G = -inf; P = 0 wherever G = -inf)
struct FuTok {
  float p, g;
};

template <int OUT_DT>
__device__ __forceinline__ void fu_store(void* out, int64_t orow, int E, int e, float v) {
  if (OUT_DT == CSA_DT_F32) ((float*)out)[(size_t)orow * E + e] = v;
  else ((uint16_t*)out)[(size_t)orow * E + e] = f32_to_bf16(v);
}

// the gated pool of one 8-token window (the same arithmetic as pool_kernel)
__device__ __forceinline__ float fu_pool(const FuTok (&tk)[8], const float (&av)[8]) {
  float gv[8], cm = -INFINITY;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    gv[u] = tk[u].g == -INFINITY ? -INFINITY : tk[u].g + av[u];
    cm = fmaxf(cm, gv[u]);
  }
  float den = 0.0f, num = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float w = __expf(gv[u] - cm);
    den += w;
    num = fmaf(w, tk[u].g == -INFINITY ? 0.0f : tk[u].p, num);
  }
  return num / den;
}

template <int OUT_DT>
__global__ void __launch_bounds__(512) compress_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_kv,
    const uint16_t* __restrict__ w_gate, const int64_t* __restrict__ pos0, int L, int E, int K,
    const float* __restrict__ ape, const float* __restrict__ state_in,
    float* __restrict__ state_out, void* __restrict__ out, int Nc_cap, PageTable pt,
    float* __restrict__ seam, int n_tiles) {
  constexpr int m = 4, NS = 7;  // window 2m, carried tokens 2m - 1
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * PJ_TILE];  // 73728 B
  uint16_t* const As = smem;
  uint16_t* const Bs = smem + 2 * PJ_TILE;
  float* const Pl = (float*)smem;       // [128][FU_PS]
  float* const Gl = Pl + PJ_BM * FU_PS;  // [128][FU_PS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x, c0 = blockIdx.y * FU_CH, b = blockIdx.z;
  const int64_t p0 = pos0[b];
  const int64_t i0 = p0 / m;  // first entry whose last token is >= p0
  const int64_t tp0 = (int64_t)m * (i0 + (int64_t)FU_BLK * t);  // position of tile row 0
  if (tp0 >= p0 + L) return;  // uniform: nothing of this call in the tile
  const uint16_t* xb = x + (size_t)b * L * K;

  const uint16_t* arow[2];
  const uint16_t* brow[2];
  for (int u = 0; u < 2; ++u) {
    const int c = u * 512 + tid, r = c >> 3, q = c & 7;
    const int64_t rr = tp0 + r - p0;  // row of the call
    arow[u] = xb + (size_t)(rr >= 0 && rr < L ? rr : 0) * K + q * 8;
    brow[u] = (r < FU_CH ? w_kv + (size_t)(c0 + r) * K : w_gate + (size_t)(c0 + r - FU_CH) * K) +
              q * 8;
  }
  f32x16 acc[2];
  pj_mainloop(As, Bs, arow, brow, K / PJ_BK, acc);
  // (the main loop ends with a barrier: the operand buffers are free)
  {
    const int wm = (wave >> 2) * 64, wn = (wave & 3) * 32;
    const int col = wn + (lane & 31);
    float* const dst = col < FU_CH ? Pl + col : Gl + (col - FU_CH);
    for (int i = 0; i < 2; ++i)
      for (int r = 0; r < 16; ++r) {
        const int row = wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        dst[row * FU_PS] = acc[i][r];
      }
  }
  __syncthreads();
  const int ch = lane, e = c0 + ch;
  auto token = [&](int r) -> FuTok {
    const int64_t pos = tp0 + r;
    FuTok tk{0.0f, -INFINITY};
    if (pos >= p0) {
      tk.p = Pl[r * FU_PS + ch];
      tk.g = Gl[r * FU_PS + ch];
    } else if (state_in && pos >= 0 && pos >= p0 - NS) {
      const float* sr = state_in + (((size_t)b * NS + (size_t)(pos - (p0 - NS))) * 2) * E;
      tk.p = sr[e];
      tk.g = sr[E + e];
    }
    if (tk.g == -INFINITY) tk.p = 0.0f;
    return tk;
  };
  float av[2 * m];
#pragma unroll
  for (int u = 0; u < 2 * m; ++u) av[u] = ape ? ape[(size_t)u * E + e] : 0.0f;
  // entries i0 + 32 t + k, k = 1 .. 31: blocks k - 1 and k of the tile
  for (int k = 1 + wave; k < FU_BLK; k += 8) {
    const int64_t i = i0 + (int64_t)FU_BLK * t + k;
    if (i >= Nc_cap || (int64_t)m * (i + 1) - 1 >= p0 + L) continue;  // uniform per wave
    const int64_t orow = pt.block_table ? paged_row(pt, b, (int)i) : (int64_t)b * Nc_cap + i;
    if (orow < 0) continue;  // an absent page: not stored
    FuTok tk[2 * m];
#pragma unroll
    for (int u = 0; u < 2 * m; ++u) tk[u] = token(m * (k - 1) + u);
    fu_store<OUT_DT>(out, orow, E, e, fu_pool(tk, av));
  }
  // the tile's first and last blocks for the seam kernel (waves 0 and 1)
  if (wave < 2) {
    const int r0 = wave == 0 ? 0 : PJ_BM - m;
#pragma unroll
    for (int u = 0; u < m; ++u) {
      const FuTok tk = token(r0 + u);
      seam[fu_seam_at(b, n_tiles, t, wave, u, 0, E, e)] = tk.p;
      seam[fu_seam_at(b, n_tiles, t, wave, u, 1, E, e)] = tk.g;
    }
  }
  // the next call's state: positions p0 + L - 7 .. p0 + L - 1 in this tile
  // (L >= 7: all of them are rows of this call)
  if (state_out) {  // (uniform)
    for (int s = wave; s < NS; s += 8) {
      const int64_t r = p0 + L - NS + s - tp0;
      if (r < 0 || r >= PJ_BM) continue;
      const FuTok tk = token((int)r);
      state_out[(((size_t)b * NS + s) * 2 + 0) * E + e] = tk.p;
      state_out[(((size_t)b * NS + s) * 2 + 1) * E + e] = tk.g;
    }
  }
}

// The entries i0 + 32 t whose windows straddle two tiles: the last block of
// tile t - 1 (for t = 0, the block before the call, from the carried state)
// and the first block of tile t.  Grid (tiles, E / 64, B), 64 threads: one
// channel each.  Reads state_in, never state_out, so that the two may not
// alias as in every compressor call.
template <int OUT_DT>
__global__ void __launch_bounds__(64) compress_seam_kernel(
    const int64_t* __restrict__ pos0, int L, int E, const float* __restrict__ ape,
    const float* __restrict__ state_in, void* __restrict__ out, int Nc_cap, PageTable pt,
    const float* __restrict__ seam, int n_tiles) {
  constexpr int m = 4, NS = 7;
  const int t = blockIdx.x, e = blockIdx.y * FU_CH + threadIdx.x, b = blockIdx.z;
  const int64_t p0 = pos0[b];
  const int64_t i0 = p0 / m;
  const int64_t i = i0 + (int64_t)FU_BLK * t;
  if (i >= Nc_cap || (int64_t)m * (i + 1) - 1 >= p0 + L) return;
  const int64_t orow = pt.block_table ? paged_row(pt, b, (int)i) : (int64_t)b * Nc_cap + i;
  if (orow < 0) return;
  FuTok tk[2 * m];
#pragma unroll
  for (int u = 0; u < m; ++u) {
    if (t > 0) {
      tk[u].p = seam[fu_seam_at(b, n_tiles, t - 1, 1, u, 0, E, e)];
      tk[u].g = seam[fu_seam_at(b, n_tiles, t - 1, 1, u, 1, E, e)];
    } else {
      const int64_t pos = (int64_t)m * (i - 1) + u;  // before the call
      tk[u] = FuTok{0.0f, -INFINITY};
      if (state_in && pos >= 0 && pos >= p0 - NS) {
        const float* sr = state_in + (((size_t)b * NS + (size_t)(pos - (p0 - NS))) * 2) * E;
        tk[u].p = sr[e];
        tk[u].g = sr[E + e];
      }
      if (tk[u].g == -INFINITY) tk[u].p = 0.0f;
    }
    tk[m + u].p = seam[fu_seam_at(b, n_tiles, t, 0, u, 0, E, e)];
    tk[m + u].g = seam[fu_seam_at(b, n_tiles, t, 0, u, 1, E, e)];
  }
  float av[2 * m];
#pragma unroll
  for (int u = 0; u < 2 * m; ++u) av[u] = ape ? ape[(size_t)u * E + e] : 0.0f;
  fu_store<OUT_DT>(out, orow, E, e, fu_pool(tk, av));
}

// ------------------------------------------------------- proj (bf16, few rows)
// Decode steps and short chunks (M <= 16 rows): a workgroup per 16 output
// columns and K split (grid y, at most four split partials, so that the
// grid covers the chip), its 8 waves taking an eighth of its K range each,
// with all of a wave's loads in flight at once (batches of eight k steps,
// the last one clamped and masked); MFMA 16x16x32 with the rows as M (rows
// past M read row M - 1 and are dropped) and 16 columns of the stacked
// weight as N.  Each weight byte is read once; the few x rows stay in L2.
// The waves' partial sums are added in wave order through LDS, the splits'
// by the pool, in split order.  K % (256 splits) == 0 (checked by the host).
constexpr int PS_COLS = 16, PS_UNROLL = 8, PS_WAVES = 8;

__global__ void __launch_bounds__(64 * PS_WAVES) proj_small_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_kv,
    const uint16_t* __restrict__ w_gate, float* __restrict__ pg, int M, int E, int K) {
  __shared__ float red[PS_WAVES][16 * PS_COLS];
  const int N = 2 * E;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * PS_COLS;
  const int kq = K / (PS_WAVES * (int)gridDim.y);
  const int k0 = ((int)blockIdx.y * PS_WAVES + wave) * kq;
  // operand lanes: row / column lane % 16, k chunk 8 (lane / 16) of each
  // 32-deep step (the same k order for both operands)
  const int arow = min(lane & 15, M - 1);
  const uint16_t* ap = x + (size_t)arow * K + k0 + 8 * (lane >> 4);
  const int gn = min(n0 + (lane & 15), N - 1);
  const uint16_t* bp =
      (gn < E ? w_kv + (size_t)gn * K : w_gate + (size_t)(gn - E) * K) + k0 + 8 * (lane >> 4);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < kq; k += 32 * PS_UNROLL) {
    bf16x8 a[PS_UNROLL], bv[PS_UNROLL];
#pragma unroll
    for (int u = 0; u < PS_UNROLL; ++u) {
      const int kk = min(k + 32 * u, kq - 32);  // in range; masked below
      a[u] = *(const bf16x8*)(ap + kk);
      bv[u] = *(const bf16x8*)(bp + kk);
    }
#pragma unroll
    for (int u = 0; u < PS_UNROLL; ++u)
      if (k + 32 * u < kq)  // uniform
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bv[u], acc, 0, 0, 0);
  }
  // accumulator: lane holds column lane % 16, rows 4 (lane / 16) + i
  for (int i = 0; i < 4; ++i) red[wave][(4 * (lane >> 4) + i) * PS_COLS + (lane & 15)] = acc[i];
  __syncthreads();
  if (tid < 16 * PS_COLS) {
    const int row = tid / PS_COLS, col = n0 + tid % PS_COLS;
    float sum = red[0][tid];
    for (int w = 1; w < PS_WAVES; ++w) sum += red[w][tid];
    if (row < M && col < N) pg[((size_t)blockIdx.y * M + row) * N + col] = sum;
  }
}

static bool use_proj_small(int M, int K, csa_dtype_t dt) {
  return dt == CSA_DT_BF16 && M <= 16 && K % (32 * PS_WAVES) == 0;
}

// K splits of the few-row projection: up to four, while the grid has fewer
// than 256 workgroups and every wave keeps whole 32-deep k steps
static int proj_small_splits(int E, int K) {
  const int groups = (2 * E + PS_COLS - 1) / PS_COLS;
  int s = 1;
  while (s < 4 && groups * s < 256 && K % (32 * PS_WAVES * 2 * s) == 0) s *= 2;
  return s;
}

// ---------------------------------------------------------------- proj (fp32)
__global__ void __launch_bounds__(256) proj_f32_kernel(const float* __restrict__ x,
                                                       const float* __restrict__ w_kv,
                                                       const float* __restrict__ w_gate,
                                                       float* __restrict__ pg, int M, int E,
                                                       int K) {
  const int N = 2 * E;
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (size_t)M * N) return;
  const int row = (int)(id / N), col = (int)(id % N);
  const float* w = col < E ? (w_kv + (size_t)col * K) : (w_gate + (size_t)(col - E) * K);
  const float* xr = x + (size_t)row * K;
  float s = 0.0f;
  for (int k = 0; k < K; ++k) s = fmaf(xr[k], w[k], s);
  pg[id] = s;
}

// ---------------------------------------------------------------- MXFP4 store
// OCP MXFP4: a block of 32 values shares the exponent X = floor(log2(amax))
// - 2 (2: the largest E2M1 exponent), clamped to [-127, 127] and 0 for an
// all-zero block; stored as the E8M0 byte X + 127.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int ef = (int)((__float_as_uint(amax) >> 23) & 255u);
  return ef == 0 ? -127 : max(ef - 129, -127);  // subnormal amax: below 2^-126
}

// E2M1 code of y (sign in bit 3): the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6,
// a tie going to the even mantissa bit, beyond 6 saturating.  The decision
// points are the midpoints, and a midpoint belongs to its even neighbour.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const uint32_t sgn = (__float_as_uint(y) >> 31) << 3;
  const float a = fabsf(y);
  const uint32_t mag = a <= 0.25f ? 0u
                     : a < 0.75f  ? 1u
                     : a <= 1.25f ? 2u
                     : a < 1.75f  ? 3u
                     : a <= 2.5f  ? 4u
                     : a < 3.5f   ? 5u
                     : a <= 5.0f  ? 6u
                                  : 7u;
  return sgn | mag;
}

// ---------------------------------------------------------------- pool
// Grid (n_slots + 1, B).  Slot q < n_slots handles entry i_lo(b) + q; the last
// slot writes state_out.  Each thread owns channels e = tid, tid + blockDim.x,
// ... (64, 128 or 256 threads by E, at most four channels each)
// WIN > 0: the window is WIN tokens and, with at most NSP projection
// partials, every entry takes a path whose loads are all issued before the
// softmax; WIN = 0: the general path only.
template <int OUT_DT, int WIN, int NSP>
__global__ void __launch_bounds__(256) pool_kernel(
    const float* __restrict__ pg, const int64_t* __restrict__ pos0, int B, int L,
    int E, int m, int overlap, const float* __restrict__ ape, const float* __restrict__ state_in,
    float* __restrict__ state_out, void* __restrict__ out, void* __restrict__ out_scale,
    int Nc_cap, int n_slots, int n_split, bool rotate, float rot_scale, PageTable pt,
    csa_host::EntryOpts opt, Varlen vl) {
  const int b = blockIdx.y, q = blockIdx.x, tid = threadIdx.x;
  const int ns = (1 + overlap) * m - 1;
  // this sequence's rows of the call: [rb, rb + L) of the projection output
  // (packed sequences: the sequence's own length, from position 0)
  const int M = vl.cu_q ? vl.cu_q[B] : B * L;
  const size_t rb = vl.cu_q ? (size_t)vl.cu_q[b] : (size_t)b * L;
  if (vl.cu_q) {
    L = vl.cu_q[b + 1] - vl.cu_q[b];
    Nc_cap = vl.cu_k[b + 1] - vl.cu_k[b];
  }
  const int64_t p0 = vl.cu_q ? 0 : pos0[b];
  const size_t N = 2 * (size_t)E;

  // P and G of the token at absolute position j, channel e; the caller
  // guarantees pos0 - ns <= j < pos0 + L.  Absent tokens get G = -inf.
  auto fetch = [&](int64_t j, int e, float& pv, float& gv) {
    pv = 0.0f;
    gv = -INFINITY;
    if (j < 0) return;
    if (j >= p0) {
      // the projection's split-K partials are summed here, in split order
      const float* r = pg + (rb + (size_t)(j - p0)) * N;
      const size_t stride = (size_t)M * N;
      pv = r[e];
      gv = r[E + e];
      for (int s0 = 1; s0 < n_split; s0 += 8) {  // eight splits' loads in flight
        float a[8], c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool ok = s0 + u < n_split;
          a[u] = ok ? r[(s0 + u) * stride + e] : 0.0f;
          c[u] = ok ? r[(s0 + u) * stride + E + e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          pv += a[u];
          gv += c[u];
        }
      }
      return;
    }
    if (!state_in) return;
    const int slot = (int)(j - (p0 - ns));
    const float* r = state_in + (((size_t)b * ns + slot) * 2) * E;
    pv = r[e];
    gv = r[E + e];
    if (gv == -INFINITY) pv = 0.0f;
  };

  if (q == n_slots) {  // carried state for the next call
    if (!state_out) return;
    const int total = ns * E;
    if (n_split == 1) {
      // four elements per thread with every load issued first (from a
      // readable stand-in for absent tokens)
      for (int i0 = 0; i0 < total; i0 += 4 * (int)blockDim.x) {
        float pv[4], gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = min(i0 + u * (int)blockDim.x + tid, total - 1);
          const int slot = idx / E, e = idx - slot * E;
          const int64_t j = p0 + L - ns + slot;
          const bool in_call = j >= p0;
          const bool in_state = !in_call && state_in && j >= 0;
          const float* src =
              in_call ? pg + (rb + (size_t)(j - p0)) * N
                      : (in_state ? state_in + ((size_t)b * ns + (size_t)(j - (p0 - ns))) * 2 * E : pg);
          pv[u] = src[e];
          gv[u] = src[E + e];
          if (!(in_call || in_state)) gv[u] = -INFINITY;
          if (gv[u] == -INFINITY) pv[u] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = i0 + u * (int)blockDim.x + tid;
          if (idx < total) {
            const int slot = idx / E, e = idx - slot * E;
            state_out[(((size_t)b * ns + slot) * 2 + 0) * E + e] = pv[u];
            state_out[(((size_t)b * ns + slot) * 2 + 1) * E + e] = gv[u];
          }
        }
      }
      return;
    }
    for (int idx = tid; idx < total; idx += blockDim.x) {
      int slot = idx / E, e = idx % E;
      int64_t j = p0 + L - ns + slot;
      float pv, gv;
      fetch(j, e, pv, gv);
      state_out[(((size_t)b * ns + slot) * 2 + 0) * E + e] = pv;
      state_out[(((size_t)b * ns + slot) * 2 + 1) * E + e] = gv;
    }
    return;
  }

  const int64_t i_lo = (p0 + m) / m - 1;  // first entry whose last token is >= p0
  const int64_t i = i_lo + q;
  if (i < 0 || i >= Nc_cap) return;
  const int64_t last = (int64_t)m * (i + 1) - 1;
  if (last >= p0 + L) return;
  const int64_t first = (int64_t)m * (i - overlap);
  // paged output: an entry whose page is absent is not stored (uniform)
  const int64_t orow64 = pt.block_table ? paged_row(pt, b, (int)i)
                         : (vl.cu_k ? (int64_t)vl.cu_k[b] : (int64_t)b * Nc_cap) + i;
  if (orow64 < 0) return;

  __shared__ float red[256];
  float vals[4];  // E <= 1024 supported (checked by the host)
  float amax = 0.0f;
  int nv = 0;
  bool done = false;
  if constexpr (WIN > 0) {
    if (n_split <= NSP) {  // uniform
      // Window token u is a row of this call (with n_split partials), a
      // carried-state slot, or absent; the choice depends on u only
      // (scalar), and every load is issued before the softmax, which repeats
      // one chunk of the general path below (the same arithmetic, partials
      // summed in split order).
      const float* src[WIN];
      bool present[WIN], in_call[WIN];
#pragma unroll
      for (int u = 0; u < WIN; ++u) {
        const int64_t j = first + u;
        in_call[u] = j >= p0;
        if (j >= p0) {
          src[u] = pg + (rb + (size_t)(j - p0)) * N;
          present[u] = true;
        } else if (state_in && j >= 0 && j >= p0 - ns) {
          src[u] = state_in + ((size_t)b * ns + (size_t)(j - (p0 - ns))) * 2 * E;
          present[u] = true;
        } else {
          src[u] = pg;  // a readable stand-in; the token is absent
          present[u] = false;
        }
      }
      const size_t sstride = (size_t)M * N;  // between split partials
      const float* ap = ape ? ape : pg;  // a readable stand-in when there is no ape
      for (int e = tid; e < E; e += blockDim.x, ++nv) {
        float pv[WIN], gv[WIN], av[WIN];
        float pe[NSP > 1 ? NSP - 1 : 1][WIN], ge[NSP > 1 ? NSP - 1 : 1][WIN];
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
          pv[u] = src[u][e];
          gv[u] = src[u][E + e];
          av[u] = ap[(size_t)u * E + e];
        }
#pragma unroll
        for (int sp = 1; sp < NSP; ++sp)
#pragma unroll
          for (int u = 0; u < WIN; ++u) {
            const float* r = src[u] + (in_call[u] ? (size_t)min(sp, n_split - 1) * sstride : 0);
            pe[sp - 1][u] = r[e];
            ge[sp - 1][u] = r[E + e];
          }
#pragma unroll
        for (int sp = 1; sp < NSP; ++sp)
#pragma unroll
          for (int u = 0; u < WIN; ++u)
            if (sp < n_split && in_call[u]) {
              pv[u] += pe[sp - 1][u];
              gv[u] += ge[sp - 1][u];
            }
        float cm = -INFINITY;
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
          if (!present[u]) gv[u] = -INFINITY;
          if (gv[u] == -INFINITY) pv[u] = 0.0f;
          else if (ape) gv[u] += av[u];
          cm = fmaxf(cm, gv[u]);
        }
        float den = 0.0f, num = 0.0f;
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
          const float w = __expf(gv[u] - cm);
          den += w;
          num = fmaf(w, pv[u], num);
        }
        const float c = num / den;
        vals[nv] = c;
        amax = fmaxf(amax, fabsf(c));
      }
      done = true;
    }
  }
  if (!done) for (int e = tid; e < E; e += blockDim.x, ++nv) {
    // online softmax over the window in chunks of 8 tokens; every chunk's
    // loads are independent of each other
    float mx = -INFINITY, den = 0.0f, num = 0.0f;
    for (int64_t j0 = first; j0 <= last; j0 += 8) {
      float pv[8], gv[8];
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + u;
        if (j <= last) {
          fetch(j, e, pv[u], gv[u]);
          if (gv[u] != -INFINITY && ape) gv[u] += ape[(size_t)(j - first) * E + e];
        } else {
          pv[u] = 0.0f;
          gv[u] = -INFINITY;
        }
      }
      float cm = mx;
      for (int u = 0; u < 8; ++u) cm = fmaxf(cm, gv[u]);
      if (cm == -INFINITY) continue;
      const float corr = __expf(mx - cm);  // mx = -inf -> 0
      den *= corr;
      num *= corr;
      for (int u = 0; u < 8; ++u) {
        const float w = __expf(gv[u] - cm);
        den += w;
        num = fmaf(w, pv[u], num);
      }
      mx = cm;
    }
    float c = num / den;
    vals[nv] = c;
    amax = fmaxf(amax, fabsf(c));
  }
  // Post-processing of the entry, in this order (each branch uniform): RMS
  // norm over the E channels, the rotary embedding of the channel slice
  // [rope_off, rope_off + rope_dim) at the entry's position m i, and the
  // Hadamard rotation.  The angles are formed in double precision (positions
  // reach 2^20 and beyond), then rounded to fp32 sines and cosines.
  __shared__ float hb[1024];
  if (opt.norm_w) {
    float ss = 0.0f;
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) ss = fmaf(vals[nv], vals[nv], ss);
    red[tid] = ss;
    __syncthreads();
    for (int o = (int)blockDim.x / 2; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    const float r = 1.0f / sqrtf(red[0] / (float)E + opt.norm_eps);
    __syncthreads();  // red is reused by the fp8 store
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) vals[nv] = vals[nv] * r * opt.norm_w[e];
  }
  if (opt.rope_dim) {
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) hb[e] = vals[nv];
    __syncthreads();
    const int R = opt.rope_dim, half = R / 2;
    const double pos = (double)m * (double)i;
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) {
      const int c = e - opt.rope_off;
      if (c < 0 || c >= R) continue;
      const int k = opt.rope_interleaved ? c >> 1 : (c < half ? c : c - half);
      const bool first = opt.rope_interleaved ? (c & 1) == 0 : c < half;
      const int partner = opt.rope_interleaved ? (first ? e + 1 : e - 1) : (first ? e + half : e - half);
      const double ang = pos * pow((double)opt.rope_base, -2.0 * k / R);
      const float cs = (float)cos(ang), sn = (float)sin(ang);
      const float pv = hb[partner];
      vals[nv] = fmaf(vals[nv], cs, (first ? -pv : pv) * sn);
    }
    __syncthreads();  // hb is reused by the Hadamard step
  }
  if (opt.norm_w || opt.rope_dim) {
    amax = 0.0f;
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) amax = fmaxf(amax, fabsf(vals[nv]));
  }
  if (rotate) {  // uniform: the entry times H_E / sqrt(E) (Sylvester order)
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) hb[e] = vals[nv];
    __syncthreads();
    for (int len = 1; len < E; len <<= 1) {
      for (int k = tid; k < E / 2; k += blockDim.x) {
        const int j = (k / len) * 2 * len + (k % len);
        const float a = hb[j], c = hb[j + len];
        hb[j] = a + c;
        hb[j + len] = a - c;
      }
      __syncthreads();
    }
    amax = 0.0f;
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) {
      vals[nv] = hb[e] * rot_scale;
      amax = fmaxf(amax, fabsf(vals[nv]));
    }
  }
  const size_t orow = (size_t)orow64;
  if (OUT_DT == CSA_DT_F32) {
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) ((float*)out)[orow * E + e] = vals[nv];
  } else if (OUT_DT == CSA_DT_BF16) {
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv)
      ((uint16_t*)out)[orow * E + e] = f32_to_bf16(vals[nv]);
  } else if (OUT_DT == CSA_DT_MXFP4) {
    // per 32 channels (32 consecutive lanes: E and the block size are
    // multiples of 32) one E8M0 exponent and E2M1 codes, two per byte
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv) {
      const float v = vals[nv];
      float am = fabsf(v);
      for (int o = 16; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
      const int x = mx_block_exponent(am);
      const uint32_t c = e2m1_code(v * __builtin_ldexpf(1.0f, -x));
      const uint32_t c_next = (uint32_t)__shfl_xor((int)c, 1, 64);
      if ((e & 1) == 0) ((uint8_t*)out)[orow * (E / 2) + e / 2] = (uint8_t)(c | (c_next << 4));
      if ((e & 31) == 0) ((uint8_t*)out_scale)[orow * (E / 32) + e / 32] = (uint8_t)(x + 127);
    }
  } else {
    red[tid] = amax;
    __syncthreads();
    for (int o = (int)blockDim.x / 2; o > 0; o >>= 1) {
      if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
      __syncthreads();
    }
    float s = red[0] > 0.0f ? red[0] / 448.0f : 1.0f;
    if (tid == 0) ((float*)out_scale)[orow] = s;
    nv = 0;
    for (int e = tid; e < E; e += blockDim.x, ++nv)
      ((uint8_t*)out)[orow * E + e] = (uint8_t)(f32x2_to_e4m3x2(vals[nv] / s, 0.0f) & 0xff);
  }
}

// ------------------------------------------------ packed sequence offsets
// cmp_cu[0] = 0, cmp_cu[b + 1] = cmp_cu[b] + floor((cu[b + 1] - cu[b]) / m):
// the compressed entries of packed sequences.  One workgroup of 1024 threads,
// an inclusive block scan per chunk of 1024 sequences.
__global__ void __launch_bounds__(1024) cmp_cu_kernel(int n, const int32_t* __restrict__ cu, int m,
                                                      int32_t* __restrict__ cmp_cu) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    carry = 0;
    cmp_cu[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    const int v = i < n ? (cu[i + 1] - cu[i]) / m : 0;
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (i < n) cmp_cu[i + 1] = before + x;
    __syncthreads();
    if (tid == 1023) carry = before + x;
    __syncthreads();
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

hipError_t launch_cmp_cu(int n, const int32_t* cu, int m, int32_t* cmp_cu, hipStream_t st) {
  cmp_cu_kernel<<<1, 1024, 0, st>>>(n, cu, m, cmp_cu);
  return hipGetLastError();
}

static int proj_splits(int M, int E, int K, csa_dtype_t dt) {
  if (use_proj_small(M, K, dt)) return proj_small_splits(E, K);
  if (dt != CSA_DT_BF16) return 1;
  int tiles = ((M + PJ_BM - 1) / PJ_BM) * ((2 * E + PJ_BN - 1) / PJ_BN);
  int s = 1;
  // split K while the grid holds fewer than one workgroup per CU (two for
  // the few rows of a decode step); every split keeps whole k tiles - at
  // least four when the pool has many rows to re-read the partials for, and
  // then at most four splits (the pool's batched path)
  const int min_k = M <= PJ_BM ? 2 * PJ_BK : 4 * PJ_BK;
  const int target = M <= PJ_BM ? 512 : 256;
  while (tiles * s < target && K / (2 * s) >= min_k && (K / (2 * s)) % PJ_BK == 0 &&
         (M <= PJ_BM || s < 4))
    s *= 2;
  return s;
}

size_t compress_ws_bytes(int B, int L, int d_model, int E, int m, int overlap,
                         csa_dtype_t in_dt) {
  (void)m;
  (void)overlap;
  int M = B * L;
  int s = proj_splits(M, E, d_model, in_dt);
  return (size_t)s * M * 2 * E * sizeof(float);
}

// The fused kernel takes prefill chunks of bf16 tokens with m = 4 and
// overlap, stored as fp32 or bf16 with no step that mixes channels, and at
// least 128 channels: it cannot split K, so narrower entries (the indexer's
// 64: one channel block, a quarter of the 8K chunk's workgroups) keep the
// split-K projection and the pool.
static bool use_fused(const CompressArgs& a) {
  return a.in_dt == CSA_DT_BF16 && (a.out_dt == CSA_DT_F32 || a.out_dt == CSA_DT_BF16) &&
         !a.rotate && !a.opt.norm_w && !a.opt.rope_dim && a.m == 4 && a.overlap == 1 &&
         a.E % FU_CH == 0 && a.E >= 128 && !a.vl.cu_q && a.L >= PJ_BM &&
         a.d_model % PJ_BK == 0;
}

// Tiles of 32 blocks from block floor(pos0 / 4), whose first position is at
// most 3 before pos0: enough for any pos0 (the tiles past the call return at
// once).  Their seam buffer (2 blocks of P and G per tile and channel) fits
// the projection workspace the call is given.
static int fused_tiles(int L) { return (L + 3 + 4 * FU_BLK - 1) / (4 * FU_BLK); }

hipError_t launch_proj_pg(const void* x, const void* w_kv, const void* w_gate, int M, int E, int K,
                          float* pg, hipStream_t st) {
  dim3 grid((M + PJ_BM - 1) / PJ_BM, (2 * E + PJ_BN - 1) / PJ_BN, 1);
  proj_bf16_kernel<<<grid, 512, 0, st>>>((const uint16_t*)x, (const uint16_t*)w_kv,
                                         (const uint16_t*)w_gate, pg, M, E, K, K);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  if (use_fused(a)) {
    const int n_tiles = fused_tiles(a.L);
    dim3 grid(n_tiles, a.E / FU_CH, a.B);
    float* seam = (float*)a.ws;
#define CSA_LAUNCH_FUSED(DT)                                                                   \
  compress_fused_kernel<DT><<<grid, 512, 0, st>>>(                                             \
      (const uint16_t*)a.x, (const uint16_t*)a.w_kv, (const uint16_t*)a.w_gate, a.pos0, a.L,   \
      a.E, a.d_model, a.ape, a.state_in, a.state_out, a.out, a.Nc_cap, a.pages, seam, n_tiles); \
  compress_seam_kernel<DT><<<grid, FU_CH, 0, st>>>(a.pos0, a.L, a.E, a.ape, a.state_in, a.out, \
                                                   a.Nc_cap, a.pages, seam, n_tiles)
    if (a.out_dt == CSA_DT_F32) {
      CSA_LAUNCH_FUSED(CSA_DT_F32);
    } else {
      CSA_LAUNCH_FUSED(CSA_DT_BF16);
    }
#undef CSA_LAUNCH_FUSED
    return hipGetLastError();
  }
  // rows of the projection: every token of the call (packed sequences:
  // a.total_rows, the sum of their lengths)
  const int M = a.vl.cu_q ? a.total_rows : a.B * a.L, K = a.d_model, E = a.E;
  const int splits = proj_splits(M, E, K, a.in_dt);
  float* pg = (float*)a.ws;
  if (use_proj_small(M, K, a.in_dt)) {
    proj_small_kernel<<<dim3((2 * E + PS_COLS - 1) / PS_COLS, splits), 64 * PS_WAVES, 0, st>>>(
        (const uint16_t*)a.x, (const uint16_t*)a.w_kv, (const uint16_t*)a.w_gate, pg, M, E, K);
  } else if (a.in_dt == CSA_DT_BF16) {
    dim3 grid((M + PJ_BM - 1) / PJ_BM, (2 * E + PJ_BN - 1) / PJ_BN, splits);
    proj_bf16_kernel<<<grid, 512, 0, st>>>((const uint16_t*)a.x, (const uint16_t*)a.w_kv,
                                           (const uint16_t*)a.w_gate, pg, M, E, K, K / splits);
  } else {
    size_t n = (size_t)M * 2 * E;
    proj_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        (const float*)a.x, (const float*)a.w_kv, (const float*)a.w_gate, pg, M, E, K);
  }
  // packed sequences: a.L is the longest sequence (the grid covers its
  // entries; shorter sequences' extra slots return at once)
  const int n_slots = (a.L + a.m - 1) / a.m + 1;
  dim3 pgrid(n_slots + 1, a.B);
  // the common gated window (m = 4 with overlap: 8 tokens) has a batched path
  // (for up to four projection partials)
  const int w8 = (1 + a.overlap) * a.m == 8 ? (splits == 1 ? 1 : (splits <= 4 ? 4 : 0)) : 0;
  // a thread per channel (at most four per thread): narrow entries take
  // narrower workgroups
  const int pthreads = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
#define CSA_LAUNCH_POOL(DT, W, NS)                                                              \
  pool_kernel<DT, W, NS><<<pgrid, pthreads, 0, st>>>(                                           \
      pg, a.pos0, a.B, a.L, E, a.m, a.overlap, a.ape, a.state_in, a.state_out, a.out,           \
      a.out_scale, a.Nc_cap, n_slots, splits, a.rotate != 0, (float)(1.0 / std::sqrt((double)E)), \
      a.pages, a.opt, a.vl)
#define CSA_POOL_DT(DT)                            \
  if (w8 == 1) CSA_LAUNCH_POOL(DT, 8, 1);          \
  else if (w8 == 4) CSA_LAUNCH_POOL(DT, 8, 4);     \
  else CSA_LAUNCH_POOL(DT, 0, 1);
  switch (a.out_dt) {
    case CSA_DT_F32:
      CSA_POOL_DT(CSA_DT_F32);
      break;
    case CSA_DT_BF16:
      CSA_POOL_DT(CSA_DT_BF16);
      break;
    case CSA_DT_MXFP4:
      CSA_POOL_DT(CSA_DT_MXFP4);
      break;
    default:
      CSA_POOL_DT(CSA_DT_FP8E4M3);
  }
#undef CSA_POOL_DT
#undef CSA_LAUNCH_POOL
  return hipGetLastError();
}

}  // namespace csa_host
