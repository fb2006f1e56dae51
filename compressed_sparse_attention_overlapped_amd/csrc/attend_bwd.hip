// Attention backward for gfx950: gradients of the sparse (CSA) and dense
// (HCA) MQA attention with respect to the queries, the compressed and raw KV
// rows and the per-head sink, plus the main attention's probability mass per
// selected slot (CSA) or per visible entry (HCA form), the indexer loss's
// target in its sparse and dense forms.
//
// Math, per query token and head over the forward's key set J (DS-V4 analysis
// section 1.2; Notion copy section 1.1: one shared KV head, 1/sqrt(D) scale):
//   P_j = exp(l_j - lse) with the forward's lse,  dP_j = dO . V_j,
//   delta = dO . out,  dS_j = P_j (dP_j - delta),
//   dq = scale sum_j dS_j K_j,  dK_j += scale sum dS_j q,  dV_j += sum P_j dO,
//   dsink = -sum exp(sink - lse) delta.
//
// Launches: zero fills of the summed outputs; for CSA a bitmap kernel (the
// selected entries of each row as bits, with the rank of each word); a
// query-major dq kernel (the forward's tile walk: gathered or dense
// compressed tiles, then the window, 32 keys per tile in LDS), which also
// computes delta = sum_j P_j dP_j exactly (a first sweep over the row's tiles,
// so delta does not inherit the rounding of a stored output) and hands delta
// and lse to the next kernels; a reduction of the sink gradient; and a
// key-major dK/dV kernel (a workgroup owns 128 keys and walks the query rows
// that see them, each row's Q and dO staged in LDS) that leaves one partial
// per row chunk, summed in slot order by a reduction kernel (deterministic).
// The per-key sums need no atomics between query rows (MFMA reduces over
// heads and rows inside the workgroup); an fp32 atomic costs about as much as
// eight plain stores here, so the query-major form that scatters every
// (row, key) contribution is avoided.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace csa {

constexpr int BW_KT = 32;                   // keys per tile (dq kernel)
constexpr int BW_ROWB = 512;                // bytes of one [K | V] row (D = 128, bf16)
constexpr int BW_TILEB = BW_KT * BW_ROWB;   // 16 KB
constexpr int BW_IDX_MAX = 4096;            // index slots per row staged in LDS
constexpr int BW_KV_KEYS = 128;             // keys per workgroup (dK/dV kernel)
constexpr int BW_RC = 64;                   // query rows per dK/dV workgroup

// 16-byte chunk c of row r of an LDS tile sits at slot c ^ bw_swz(r): 16
// consecutive rows read at one chunk (the MFMA operand reads) and the 4 x 4
// row/chunk blocks of the transposing reads both spread over all banks.
__device__ __forceinline__ int bw_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// LDS transpose read: lane i of each 16-lane group receives element i % 4 of
// the 8-byte chunks whose addresses lanes i / 4 + 4 v (v = 0..3) supplied.
typedef __attribute__((ext_vector_type(4))) short bw_s16x4;
__device__ __forceinline__ bw_s16x4 bw_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bw_s16x4*)p);
}

// one 16-byte global -> LDS copy per lane: lane l fills dst + 16 l
__device__ __forceinline__ void bw_dma(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void bw_wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------- sink
// dsink[h] = sum over rows of dz[row][h] (the dq kernel's per-row terms):
// each workgroup sums a slice of rows per head, then one atomic per head.
template <int H>
__global__ void __launch_bounds__(256) bwd_sink_kernel(const float* __restrict__ dz, int rows,
                                                       float* __restrict__ dsink) {
  constexpr int RPS = 256 / H;  // rows per step
  __shared__ float part[256];
  const int tid = threadIdx.x, h = tid % H, r0 = tid / H;
  float s = 0.0f;
  for (int r = blockIdx.x * RPS + r0; r < rows; r += gridDim.x * RPS) s += dz[(size_t)r * H + h];
  part[tid] = s;
  __syncthreads();
  if (tid < H) {
    float t = 0.0f;
    for (int k = 0; k < RPS; ++k) t += part[k * H + tid];
    atomicAdd(dsink + tid, t);
  }
}

// ---------------------------------------------------------------- bitmap
// One wave per query row, BM_ROWS rows per workgroup: bit j of words[row] is
// set when entry j is selected (0 <= idx < Nc_cap); rank[row][w] = selected
// entries in words < w, so an entry's slot in an ascending index row is its
// rank.  Every step is the wave's own, with no workgroup barrier: a wave's LDS
// operations complete in issue order.  nw <= 2048 (Nc_cap <= 65536).
constexpr int BM_ROWS = 4;
__global__ void __launch_bounds__(64 * BM_ROWS) bwd_bitmap_kernel(const int32_t* __restrict__ idx,
                                                                  int rows, int topk, int Nc_cap,
                                                                  int nw, uint32_t* __restrict__ bm,
                                                                  uint32_t* __restrict__ rank) {
  __shared__ uint32_t words[BM_ROWS][2048];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * BM_ROWS + wave;
  if (row >= rows) return;  // the whole wave (no barrier follows)
  uint32_t* wd = words[wave];
  for (int w = lane; w < nw; w += 64) wd[w] = 0;
  // the row's index slots, eight loads per lane in flight at a time
  const int32_t* ir = idx + (size_t)row * topk;
  for (int k0 = 0; k0 < topk; k0 += 8 * 64) {
    int32_t jv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 64 * u + lane;
      jv[u] = k < topk ? ir[k] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (jv[u] >= 0 && jv[u] < Nc_cap) atomicOr(&wd[jv[u] >> 5], 1u << (jv[u] & 31));
  }
  // lane l owns words [l per, l per + per); exclusive prefix of their counts
  const int per = (nw + 63) / 64;
  const int w0 = min(nw, lane * per), w1 = min(nw, w0 + per);
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(wd[w]);
  uint32_t x = c;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  uint32_t r = x - c;
  uint32_t* brow = bm + (size_t)row * nw;
  uint32_t* rrow = rank + (size_t)row * nw;
  for (int w = w0; w < w1; ++w) {
    const uint32_t v = wd[w];
    brow[w] = v;
    rrow[w] = r;
    r += __popc(v);
  }
}

// ---------------------------------------------------------------- zero fill
__global__ void bwd_zero_kernel(float* __restrict__ p, size_t n) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    *(f32x4*)(p + 4 * i) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (size_t i = 4 * n4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// ---------------------------------------------------------------- dq
// One workgroup per query row, NHH waves (wave w: heads 32 w .. 32 w + 31).
// Tiles of 32 keys in the forward's order: the compressed segment (CSA: the
// row's index slots; HCA: entries [0, n_vis)), then the window's raw rows.
// Per tile and wave (keys on MFMA rows, heads on columns):
//   S^T = K Q^T, dP^T = V dO^T (16 MFMAs), P and dS in registers,
//   dq^T += K^T dS^T (8 MFMAs; K^T through transposing LDS reads).
template <int NHH, bool DENSE>
__global__ void __launch_bounds__(64 * NHH, 2) attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ sink,
    const uint16_t* __restrict__ kv_cmp,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw,
    const int64_t* __restrict__ q_pos, const int64_t* __restrict__ raw_base,
    const int32_t* __restrict__ n_cmp, int T, int Nc_cap, int R_cap, int topk, int window, int m,
    float scale, float* __restrict__ dq, float* __restrict__ ldw, float* __restrict__ dz) {
  constexpr int H = 32 * NHH;
  constexpr int NI = 16 / NHH;  // load instructions per wave per tile
  // two distinct buffers, each named at compile time in the loop below, so the
  // compiler sees that a tile's reads do not touch the buffer being loaded
  __shared__ __attribute__((aligned(1024))) uint8_t tile0[BW_TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t tile1[BW_TILEB];
  extern __shared__ int32_t idx_s[];  // [topk] (CSA form; sized at launch, so that four
                                      // workgroups fit one CU's LDS at topk 512)
  __shared__ int32_t sh_last;
  const int row = blockIdx.x, b = row / T, t = row - b * T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int head = 32 * wave + l32;
  const int64_t pos = q_pos[b] + t;
  const float lse_n = lse[(size_t)row * H + head];
  const float lse2 = lse_n * kLog2e;
  const float sc2 = scale * kLog2e;
  float dlt = 0.0f;  // delta of this lane's head (first sweep)

  // compressed segment: n_a tiles
  int nv = 0, n_a;
  if constexpr (DENSE) {
    nv = n_visible(pos, n_cmp[b], m, Nc_cap);
    n_a = (nv + BW_KT - 1) / BW_KT;
  } else {
    if (tid == 0) sh_last = -1;
    __syncthreads();
    int last = -1;
    const int32_t* ir = idx + (size_t)row * topk;
    for (int k = tid; k < topk; k += 64 * NHH) {
      const int32_t v = ir[k];
      const bool ok = v >= 0 && v < Nc_cap;
      idx_s[k] = ok ? v : -1;
      if (ok) last = k;
    }
    if (last >= 0) atomicMax(&sh_last, last);
    __syncthreads();
    n_a = (sh_last + 1 + BW_KT - 1) / BW_KT;
  }
  // window segment: raw rows [ra, rb]
  int64_t ra = 0, rb = -1;
  if (window > 0 && R_cap > 0) {
    const int64_t rbase = raw_base[b];
    int64_t wlo = pos - window + 1;
    if (wlo < 0) wlo = 0;
    ra = wlo - rbase;
    rb = pos - rbase;
    if (ra < 0) ra = 0;
    if (rb > R_cap - 1) rb = R_cap - 1;
  }
  const int n_w = rb >= ra ? (int)((rb - ra + BW_KT) / BW_KT) : 0;
  // (window rows are cache rows, below 2^23: 32-bit from here on)
  const int ra32 = (int)ra, rb32 = (int)rb;
  const int ntiles = n_a + n_w;

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;

  if (ntiles > 0) {
    // B operands: Q^T and dO^T, head `head`, dims 16 s + 8 h2 ..
    bf16x8 qf[8], of[8];
    {
      const uint16_t* qr = q + ((size_t)row * H + head) * 128 + 8 * h2;
      const uint16_t* orr = dout + ((size_t)row * H + head) * 128 + 8 * h2;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        qf[s] = *(const bf16x8*)(qr + 16 * s);
        of[s] = *(const bf16x8*)(orr + 16 * s);
      }
    }
    // K^T transposing reads: key rows 4 h2 + jj / 4 + 8 e, dims 32 dt +
    // 16 (gg & 1) + 4 (jj & 3), for lane jj of 16-lane group gg
    uint32_t tofs[4][2];
    const uint32_t krow = (uint32_t)(l32 * BW_ROWB), kx = (uint32_t)(h2 ^ bw_swz(l32));
    {
      const int gg = lane >> 4, jj = lane & 15;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 4 * (gg >> 1) + (jj >> 2) + 8 * e;
        const int fr = bw_swz(r);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int c = 4 * dt + 2 * (gg & 1) + ((jj & 3) >> 1);
          tofs[dt][e] = (uint32_t)(r * BW_ROWB + 16 * (c ^ fr) + 8 * (jj & 1));
        }
      }
    }
    const char* cmp_b = (const char*)(kv_cmp + (size_t)b * Nc_cap * 256);
    const char* raw_b = (const char*)(kv_raw + (size_t)b * R_cap * 256);
    // tile ti into dst: load instruction i = wave + NHH k covers tile rows
    // 2 i, 2 i + 1 (lane half h2); the lane's source is a 32-bit byte offset
    // from the segment's uniform base (cache rows are below 2^23), and the
    // index slots of a gathered tile are read before the first load
    auto issue = [&](int ti, uint8_t* dst) {
      const char* base = ti < n_a ? cmp_b : raw_b;
      // groups of (at most) eight instructions: offsets, then the loads
#pragma unroll
      for (int k0 = 0; k0 < NI; k0 += 8) {
        constexpr int NG = NI < 8 ? NI : 8;
        uint32_t off[NG];
        if (ti < n_a) {  // uniform: compressed entries
#pragma unroll
          for (int u = 0; u < NG; ++u) {
            const int r = 2 * (wave + NHH * (k0 + u)) + h2;
            const int kk = ti * BW_KT + r;
            uint32_t grow;
            if constexpr (DENSE) {
              grow = kk < nv ? (uint32_t)kk : 0u;
            } else {
              // (n_a > 0: some slot is valid, so topk >= 1)
              const int v = idx_s[min(kk, topk - 1)];
              grow = kk < topk && v >= 0 ? (uint32_t)v : 0u;
            }
            off[u] = grow * (uint32_t)BW_ROWB + 16u * (uint32_t)(l32 ^ bw_swz(r));
          }
        } else {  // window rows
#pragma unroll
          for (int u = 0; u < NG; ++u) {
            const int r = 2 * (wave + NHH * (k0 + u)) + h2;
            const int rr = ra32 + (ti - n_a) * BW_KT + r;
            const uint32_t grow = rr <= rb32 ? (uint32_t)rr : 0u;
            off[u] = grow * (uint32_t)BW_ROWB + 16u * (uint32_t)(l32 ^ bw_swz(r));
          }
        }
#pragma unroll
        for (int u = 0; u < NG; ++u) bw_dma(base + off[u], dst + 1024 * (wave + NHH * (k0 + u)));
      }
    };
    auto vmask = [&](int ti) -> uint32_t {
      bool ok;
      if (ti < n_a) {
        const int kk = ti * BW_KT + l32;
        if constexpr (DENSE) ok = kk < nv;
        else ok = kk < topk && idx_s[kk] >= 0;
      } else {
        ok = ra32 + (ti - n_a) * BW_KT + l32 <= rb32;
      }
      return (uint32_t)__ballot(ok);
    };
    // PASS 0: delta += sum_j P_j dP_j; PASS 1: dq^T += K^T dS^T
    float dacc = 0.0f;
    auto compute = [&](const uint8_t* tb, uint32_t vm, auto pass_tag) {
      constexpr int PASS = decltype(pass_tag)::value;
      f32x16 s_acc, p_acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) s_acc[r] = p_acc[r] = 0.0f;
      // K / V rows: key l32, chunk 2 s + h2 (+ 16 for V) at slot chunk ^ bw_swz(l32);
      // (2 s + h2) ^ f = 2 s ^ (h2 ^ f) since 2 s is even
#pragma unroll
      for (int s0 = 0; s0 < 8; s0 += 4) {
        bf16x8 kf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kf[u] = *(const bf16x8*)(tb + krow + 16 * ((uint32_t)(2 * (s0 + u)) ^ kx));
#pragma unroll
        for (int u = 0; u < 4; ++u)
          s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[u], qf[s0 + u], s_acc, 0, 0, 0);
      }
#pragma unroll
      for (int s0 = 0; s0 < 8; s0 += 4) {
        bf16x8 vf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          vf[u] = *(const bf16x8*)(tb + krow + 16 * ((uint32_t)(16 + 2 * (s0 + u)) ^ kx));
#pragma unroll
        for (int u = 0; u < 4; ++u)
          p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u], of[s0 + u], p_acc, 0, 0, 0);
      }
      // keys of register r: 8 (r / 4) + 4 h2 + r % 4
      // partial tiles zero the probabilities of absent keys; full tiles
      // (uniform test) skip the per-key selects
      const uint32_t mv = vm >> (4 * h2);
      const bool full = vm == 0xffffffffu;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[r], sc2, -lse2));
      if (!full)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((mv >> (8 * (r >> 2) + (r & 3))) & 1u)) p[r] = 0.0f;
      if constexpr (PASS == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dacc = __builtin_fmaf(p[r], p_acc[r], dacc);
      } else {
        bf16x8 dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) dsb[r >> 3][r & 7] = (__bf16)(p[r] * (p_acc[r] - dlt));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const uint32_t ko = (uint32_t)ks * 16 * BW_ROWB;
            const u32x2 v1 = __builtin_bit_cast(u32x2, bw_read_tr16(tb + tofs[dt][0] + ko));
            const u32x2 v2 = __builtin_bit_cast(u32x2, bw_read_tr16(tb + tofs[dt][1] + ko));
            const bf16x8 kt = __builtin_bit_cast(bf16x8, u32x4{v1[0], v1[1], v2[0], v2[1]});
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsb[ks], acc[dt], 0, 0, 0);
          }
      }
    };
    // step of tile ti in buffer BUF: publish it, start tile ti + 1 in the
    // other buffer (every wave finished tile ti - 1 before the barrier)
    auto step = [&](auto buf_tag, int ti, auto pass_tag) {
      constexpr int BUF = decltype(buf_tag)::value;
      bw_wait_loads();
      __syncthreads();
      if (ti + 1 < ntiles) issue(ti + 1, BUF ? tile0 : tile1);
      const uint32_t vm = vmask(ti);
      if (vm) compute(BUF ? tile1 : tile0, vm, pass_tag);
    };
    auto sweep = [&](auto pass_tag) {
      issue(0, tile0);
      for (int ti = 0; ti < ntiles; ti += 2) {
        step(std::integral_constant<int, 0>{}, ti, pass_tag);
        if (ti + 1 < ntiles) step(std::integral_constant<int, 1>{}, ti + 1, pass_tag);
      }
      __syncthreads();  // every wave is done with both buffers
    };
    sweep(std::integral_constant<int, 0>{});
    dlt = dacc + lane_xor32(dacc);  // the other half of the keys
    sweep(std::integral_constant<int, 1>{});
  }
  // delta and lse (log2 units) for the dK / dV kernel; the sink term
  if (h2 == 0) {
    ldw[(size_t)row * 2 * H + head] = lse2;
    ldw[(size_t)row * 2 * H + H + head] = dlt;
    if (dz) {
      const float z = sink[head];
      dz[(size_t)row * H + head] =
          (z > -INFINITY && lse_n > -INFINITY) ? -__builtin_amdgcn_exp2f((z - lse_n) * kLog2e) * dlt
                                               : 0.0f;
    }
  }
  // dq^T: head `head` on columns, dims 32 dt + 8 (r / 4) + 4 h2 + r % 4
  float* o = dq + ((size_t)row * H + head) * 128 + 4 * h2;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(o + 32 * dt + 8 * g) =
          f32x4{scale * acc[dt][4 * g], scale * acc[dt][4 * g + 1], scale * acc[dt][4 * g + 2],
                scale * acc[dt][4 * g + 3]};
}

// ---------------------------------------------------------------- dK / dV
// KIND: 0 compressed entries of the CSA form (a row attends entry j when bit
// j of its bitmap is set), 1 compressed entries of the HCA form (j < n_vis),
// 2 raw window rows.  Workgroup (kt, chunk, b): keys [128 kt, 128 kt + 128)
// of the cache and up to 64 query rows from the first row that can see the
// tile.  Eight waves: key group g = wave % 4 (the 32 keys from 128 kt + 32 g)
// is shared by two waves of different roles, so that each holds one set of
// key fragments and one set of accumulators (two waves per SIMD):
//   role 0: S = Q K^T (16 MFMAs), P = exp(S - lse) into LDS and registers,
//           the mass per slot (CSA) or per entry (HCA), dV^T += dO^T P
//           (16 MFMAs);
//   role 1: dP = dO V^T (16 MFMAs), after a barrier P from LDS,
//           dS = P (dP - delta), dK^T += Q^T dS (16 MFMAs)
// (heads on MFMA rows, keys on columns; dO^T and Q^T through transposing LDS
// reads).  Per row, every wave reads its Q and dO staged in LDS.
template <int NHH, int KIND>
__global__ void __launch_bounds__(512, 1) attn_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
    const float* __restrict__ ldw, const uint16_t* __restrict__ kv, int rows_cap,
    const uint32_t* __restrict__ bm, const uint32_t* __restrict__ rank, int nw,
    const int64_t* __restrict__ q_pos, const int64_t* __restrict__ raw_base,
    const int32_t* __restrict__ n_cmp, int T, int topk, int window, int m, float scale,
    int nslot, float* __restrict__ part, uint32_t* __restrict__ pflag,
    float* __restrict__ attn_mass) {
  constexpr int H = 32 * NHH;
  constexpr int QB = H * 256;             // bytes of one row's Q (or dO)
  constexpr int SB0 = 2 * QB + 8 * H;     // Q | dO | lse2 | delta
  constexpr int SB = SB0 > 2 * 32 * 129 * 4 ? SB0 : 2 * 32 * 129 * 4;  // (the epilogue's rows)
  constexpr int NQI = QB / 1024;          // load instructions for Q (and for dO)
  __shared__ __attribute__((aligned(1024))) uint8_t st0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[SB];
  // P of the current row for each key group: [group][head half][register][lane]
  __shared__ __attribute__((aligned(16))) float pex[4 * NHH * 16 * 64];
  __shared__ int32_t rows_s[BW_RC];
  __shared__ uint32_t rows_w[KIND == 0 ? BW_RC : 1][4];   // the row's bitmap words of the tile
  __shared__ uint32_t rows_r[KIND == 0 ? BW_RC : 1][4];   // and their ranks
  __shared__ uint32_t sh[32];
  // Workgroup order: consecutive workgroups go to the 8 XCDs in turn, so each
  // XCD takes a contiguous range of the logical order (key tile fastest for
  // compressed entries, whose tiles all read the same query rows; row chunk
  // fastest for window tiles, whose neighbours share rows), and workgroups
  // reading the same Q / dO rows share one L2.
  const int ntl = gridDim.x, nwg = ntl * nslot * gridDim.z;
  const int lin = blockIdx.x + ntl * (blockIdx.y + nslot * blockIdx.z);
  const int xcd = lin & 7, xq = nwg >> 3, xr = nwg & 7;
  const int lg = xcd * xq + min(xcd, xr) + (lin >> 3);
  int kt, chunk, b;
  if (KIND == 2) {
    chunk = lg % nslot;
    kt = (lg / nslot) % ntl;
  } else {
    kt = lg % ntl;
    chunk = (lg / ntl) % nslot;
  }
  b = lg / (ntl * nslot);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & 3, role = wave >> 2;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int j0 = BW_KV_KEYS * kt;
  const int jw = j0 + 32 * grp + l32;  // this lane's key (MFMA column)
  const int64_t qp = q_pos[b];
  const int64_t rbase = KIND == 2 ? raw_base[b] : 0;
  const int ncb = KIND == 1 ? n_cmp[b] : 0;

  // rows that can see the tile: [t_lo, t_hi]; this workgroup takes the
  // 64-row chunks slot, slot + nslot, ... of them and leaves one partial
  // [128 keys][2 D] (with a flag: 0 if it saw no row) for the reduction
  const size_t slot = ((size_t)b * gridDim.x + kt) * nslot + chunk;
  float* pdst = part + slot * (BW_KV_KEYS * 256);
  int64_t t_lo = 0, t_hi = T - 1;
  if (KIND == 2) {
    const int64_t p0 = rbase + j0, p1 = rbase + min(j0 + BW_KV_KEYS, rows_cap) - 1;
    t_lo = p0 - qp;
    t_hi = p1 + window - 1 - qp;
  } else if (KIND == 1) {
    if (ncb <= j0) t_hi = -1;  // no visible entry in the tile
    t_lo = (int64_t)m * (j0 + 1) - 1 - qp;
  }
  if (t_lo < 0) t_lo = 0;
  if (t_hi > T - 1) t_hi = T - 1;
  if (t_lo + (int64_t)chunk * BW_RC > t_hi) {  // uniform, before any barrier
    if (tid == 0) pflag[slot] = 0u;
    return;
  }

  // B operands: role 0 K^T, role 1 V^T of this lane's key (dims 16 s + 8 h2
  // ..); keys past the cache read row 0 and are masked
  const bool key_in = jw < rows_cap;
  bf16x8 kvf[8];
  {
    const uint16_t* kr = kv + ((size_t)b * rows_cap + (key_in ? jw : 0)) * 256 + 128 * role + 8 * h2;
#pragma unroll
    for (int s = 0; s < 8; ++s) kvf[s] = *(const bf16x8*)(kr + 16 * s);
  }
  // LDS offsets: A operands Q / dO (head l32 of each 32-head half, chunk
  // 2 s + h2); the transposing reads of Q^T / dO^T (head rows 4 (gg >> 1) +
  // jj / 4 + 8 e, dims 32 dt + 16 (gg & 1) + 4 (jj & 3))
  uint32_t aofs[8], tofs[4][2];
  {
    const int fa = bw_swz(l32);
#pragma unroll
    for (int s = 0; s < 8; ++s) aofs[s] = (uint32_t)(l32 * 256 + 16 * ((2 * s + h2) ^ fa));
    const int gg = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * (gg >> 1) + (jj >> 2) + 8 * e;
      const int fr = bw_swz(r);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int c = 4 * dt + 2 * (gg & 1) + ((jj & 3) >> 1);
        tofs[dt][e] = (uint32_t)(r * 256 + 16 * (c ^ fr) + 8 * (jj & 1));
      }
    }
  }
  // role 0 reads Q (A of S) then dO^T (A of dV); role 1 dO (A of dP) then
  // Q^T (A of dK)
  const uint32_t a_base = role ? (uint32_t)QB : 0u, t_base = role ? 0u : (uint32_t)QB;
  // stage row t into dst: Q and dO rows of 4 heads per load instruction
  // (lane l: head 4 i + l / 16, chunk l % 16 at slot chunk ^ bw_swz(head)),
  // instructions i = wave, wave + 8, ... of each; then lse2 | delta (8 H
  // bytes) by the lanes of wave 0 that cover it.  Sources are 32-bit byte
  // offsets from the row's uniform base.
  static_assert(NQI % 8 == 0, "Q load instructions split evenly over 8 waves");
  auto stage = [&](int t_row, uint8_t* dst) {
    const int t = __builtin_amdgcn_readfirstlane(t_row);  // (one row per workgroup step)
    const size_t rq = ((size_t)b * T + t) * H;
    const char* qrow = (const char*)(q + rq * 128);
    const char* orow = (const char*)(dout + rq * 128);
    const int hh = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int u = 0; u < NQI / 8; ++u) {
      const int qi = wave + 8 * u;
      const int hd = 4 * qi + hh;
      const uint32_t off = (uint32_t)(hd * 256 + 16 * (cc ^ bw_swz(hd)));
      bw_dma(qrow + off, dst + 1024 * qi);
      bw_dma(orow + off, dst + QB + 1024 * qi);
    }
    if (wave == 0 && lane < H / 2)
      bw_dma((const char*)(ldw + ((size_t)b * T + t) * 2 * H) + 16u * (uint32_t)lane, dst + 2 * QB);
  };

  // role 0: dV^T, role 1: dK^T (key jw on columns, dims 32 dt + 8 (r / 4) +
  // 4 h2 + r % 4)
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
  const float sc2 = scale * kLog2e;
  float* pexw = pex + grp * (NHH * 16 * 64) + lane;

  // one row: the waves of both roles meet at the barrier between the halves
  auto compute = [&](const uint8_t* sb, int ri) {
    const int t = rows_s[ri];
    const int64_t pos = qp + t;
    bool ok = key_in;
    uint32_t word = 0u;
    if (KIND == 0) {
      word = rows_w[ri][grp];  // zero past the cache's words
      ok = ok && ((word >> l32) & 1u);
    } else if (KIND == 1) {
      ok = ok && jw < n_visible(pos, ncb, m, rows_cap);
    } else {
      const int64_t p = rbase + jw;
      ok = ok && p <= pos && p > pos - window;
    }
    const bool any = __ballot(ok) != 0;  // uniform; the same in both roles of the group
    const float* lw = (const float*)(sb + 2 * QB);
    f32x16 x_acc[NHH];  // role 0: S, role 1: dP
    if (any) {
#pragma unroll
      for (int hf = 0; hf < NHH; ++hf) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x_acc[hf][r] = 0.0f;
        bf16x8 af[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) af[s] = *(const bf16x8*)(sb + a_base + hf * 32 * 256 + aofs[s]);
#pragma unroll
        for (int s = 0; s < 8; ++s)
          x_acc[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], kvf[s], x_acc[hf], 0, 0, 0);
      }
    }
    // heads of register r: 32 hf + 8 (r / 4) + 4 h2 + r % 4
    bf16x8 bop[NHH][2];
    if (any && role == 0) {
      float msum = 0.0f;
#pragma unroll
      for (int hf = 0; hf < NHH; ++hf)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4*)(lw + 32 * hf + 8 * g + 4 * h2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(x_acc[hf][r], sc2, -l4[e]))
                               : 0.0f;
            msum += p;
            pexw[(hf * 16 + r) * 64] = p;
            bop[hf][r >> 3][r & 7] = (__bf16)p;
          }
        }
      if (KIND != 2 && attn_mass) {
        msum += lane_xor32(msum);
        if (KIND == 0 && ok && h2 == 0) {
          const uint32_t sl = rows_r[ri][grp] + __popc(word & ((1u << l32) - 1u));
          if (sl < (uint32_t)topk) attn_mass[((size_t)b * T + t) * topk + sl] = msum;
        }
        if (KIND == 1 && ok && h2 == 0) attn_mass[((size_t)b * T + t) * rows_cap + jw] = msum;
      }
    }
    __syncthreads();  // P of every group is in LDS
    if (any) {
      if (role == 1) {
#pragma unroll
        for (int hf = 0; hf < NHH; ++hf)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 d4 = *(const f32x4*)(lw + H + 32 * hf + 8 * g + 4 * h2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g + e;
              const float p = pexw[(hf * 16 + r) * 64];
              bop[hf][r >> 3][r & 7] = (__bf16)(p * (x_acc[hf][r] - d4[e]));
            }
          }
      }
#pragma unroll
      for (int hf = 0; hf < NHH; ++hf)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t ho = (uint32_t)(32 * hf + 16 * ks) * 256;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const u32x2 o1 = __builtin_bit_cast(u32x2, bw_read_tr16(sb + t_base + ho + tofs[dt][0]));
            const u32x2 o2 = __builtin_bit_cast(u32x2, bw_read_tr16(sb + t_base + ho + tofs[dt][1]));
            const bf16x8 at = __builtin_bit_cast(bf16x8, u32x4{o1[0], o1[1], o2[0], o2[1]});
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, bop[hf][ks], acc[dt], 0, 0, 0);
          }
        }
    }
  };

  for (int64_t c0 = t_lo + (int64_t)chunk * BW_RC; c0 <= t_hi; c0 += (int64_t)nslot * BW_RC) {
    const int nc = (int)min((int64_t)BW_RC, t_hi - c0 + 1);
    // the chunk's rows that see any key of the tile (CSA: a selected entry)
    {
      bool act = false;
      uint32_t wv[4] = {0u, 0u, 0u, 0u}, rv[4] = {0u, 0u, 0u, 0u};
      if (tid < nc) {
        act = true;
        if (KIND == 0) {
          const size_t wi = ((size_t)b * T + c0 + tid) * nw + (j0 >> 5);
          uint32_t anyw = 0;
          for (int k = 0; k < 4; ++k)
            if ((j0 >> 5) + k < nw) {
              wv[k] = bm[wi + k];
              rv[k] = rank[wi + k];
              anyw |= wv[k];
            }
          act = anyw != 0;
        }
      }
      uint32_t tot;
      const uint32_t at = block_excl_scan(act ? 1u : 0u, sh, tot);
      if (act) {
        rows_s[at] = (int)(c0 + tid);
        if (KIND == 0)
          for (int k = 0; k < 4; ++k) {
            rows_w[at][k] = wv[k];
            rows_r[at][k] = rv[k];
          }
      }
      sh[24] = tot;  // read after the next barrier
    }
    __syncthreads();
    const int n_rows = (int)sh[24];
    if (n_rows > 0) {  // uniform
      stage(rows_s[0], st0);
      for (int i = 0; i < n_rows; i += 2) {
        bw_wait_loads();
        __syncthreads();
        if (i + 1 < n_rows) stage(rows_s[i + 1], st1);
        compute(st0, i);
        if (i + 1 >= n_rows) break;
        bw_wait_loads();
        __syncthreads();
        if (i + 2 < n_rows) stage(rows_s[i + 2], st0);
        compute(st1, i + 1);
      }
    }
    __syncthreads();  // the staging buffers, P and rows_s are free again
  }
  // dK^T (role 1) then dV^T (role 0) through LDS into key rows (stride 129
  // floats: the 32 keys of one store hit 32 banks), then stored as the
  // workgroup's partial in whole rows (64 consecutive floats per store);
  // groups 0-1 use st0, groups 2-3 st1.
  float* red = (float*)((grp < 2 ? st0 : st1)) + (grp & 1) * 32 * 129;
  float* prow = pdst + (size_t)(32 * grp) * 256;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const bool mine = role == (half ? 0 : 1);  // uniform
    if (mine)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * dt + 8 * (r >> 2) + 4 * h2 + (r & 3);
          red[l32 * 129 + d] = half ? acc[dt][r] : scale * acc[dt][r];
        }
    __syncthreads();
    if (mine)
      for (int k = 0; k < 32; ++k) {
        prow[(size_t)k * 256 + 128 * half + lane] = red[k * 129 + lane];
        prow[(size_t)k * 256 + 128 * half + 64 + lane] = red[k * 129 + 64 + lane];
      }
    __syncthreads();
  }
  if (tid == 0) pflag[slot] = 1u;
}

// dkv[b, key] = the sum, in slot order, of the valid partials of the key's
// tile.  Workgroup (8-key group g, b): keys 8 (g % 16) .. of tile g / 16;
// thread d: element d of each row.
__global__ void __launch_bounds__(256) bwd_dkv_reduce_kernel(const float* __restrict__ part,
                                                             const uint32_t* __restrict__ pflag,
                                                             int n_tiles, int nslot, int rows_cap,
                                                             float* __restrict__ dkv) {
  const int g = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int kt = g / 16, kl0 = 8 * (g % 16);
  const size_t s0 = ((size_t)b * n_tiles + kt) * nslot;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
  for (int p = 0; p < nslot; ++p) {
    if (!pflag[s0 + p]) continue;  // uniform
    const float* ps = part + (s0 + p) * (BW_KV_KEYS * 256) + (size_t)kl0 * 256 + d;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += ps[(size_t)k * 256];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int key = BW_KV_KEYS * kt + kl0 + k;
    if (key < rows_cap) dkv[((size_t)b * rows_cap + key) * 256 + d] = acc[k];
  }
}

}  // namespace csa

// ---------------------------------------------------------------- host side
namespace csa_host {
using namespace csa;

// workspace: ldw [rows][2 H] (lse in log2 units | delta), dz [rows][H] (the
// per-row sink terms), and for CSA the bitmap and word ranks [rows][nw]
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// row-chunk slots per key tile of the dK / dV kernel: compressed tiles take
// enough workgroups to fill the chip about twice (each looping over several
// 64-row chunks), window tiles one per chunk of the rows that can see them
static int dkv_slots_cmp(int B, int T, int Nc_cap) {
  const int tiles = (Nc_cap + BW_KV_KEYS - 1) / BW_KV_KEYS, ch = (T + BW_RC - 1) / BW_RC;
  if (tiles == 0) return 0;
  return std::max(1, std::min(ch, (512 + tiles * B - 1) / (tiles * B)));
}
static int dkv_slots_raw(int T, int window) {
  const int ch = (T + BW_RC - 1) / BW_RC;
  return std::max(1, std::min(ch, (BW_KV_KEYS + window - 1 + BW_RC - 1) / BW_RC));
}
static size_t dkv_part_floats(int B, int T, int Nc_cap, int R_cap, int window) {
  const size_t tc = (Nc_cap + BW_KV_KEYS - 1) / BW_KV_KEYS, tr = (R_cap + BW_KV_KEYS - 1) / BW_KV_KEYS;
  size_t slots = tc * dkv_slots_cmp(B, T, Nc_cap);
  if (window > 0) slots += tr * dkv_slots_raw(T, window);
  return (size_t)B * slots * BW_KV_KEYS * 256;
}

size_t attn_bwd_ws_bytes(int B, int T, int H, int Nc_cap, int R_cap, int window, bool sparse) {
  const size_t rows = (size_t)B * T;
  size_t n = al256(rows * 2 * H * sizeof(float)) + al256(rows * H * sizeof(float));
  if (sparse) n += 2 * al256(rows * (((size_t)Nc_cap + 31) / 32) * sizeof(uint32_t));
  const size_t pf = dkv_part_floats(B, T, Nc_cap, R_cap, window);
  n += al256(pf * sizeof(float)) + al256(pf / (BW_KV_KEYS * 256) * sizeof(uint32_t));
  return n;
}

static int zero_grid(size_t n) {
  const size_t g = (n / 4 + 255) / 256;
  return (int)std::min<size_t>(std::max<size_t>(g, 1), 2048);
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
  if (n) bwd_zero_kernel<<<zero_grid(n), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_sel_bitmap(const int32_t* idx, int rows, int topk, int Nc_cap, uint32_t* bm,
                             uint32_t* rank, hipStream_t s) {
  bwd_bitmap_kernel<<<(rows + BM_ROWS - 1) / BM_ROWS, 64 * BM_ROWS, 0, s>>>(
      idx, rows, topk, Nc_cap, (Nc_cap + 31) / 32, bm, rank);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
  const int rows = a.B * a.T;
  const bool sparse = !a.dense;
  // the dq kernel stages a row's index slots in LDS (4 bytes each)
  if (sparse && a.topk > BW_IDX_MAX) return hipErrorInvalidValue;
  const int nw = (a.Nc_cap + 31) / 32;
  char* ws = (char*)a.ws;
  float* ldw = (float*)ws;
  ws += al256((size_t)rows * 2 * a.H * sizeof(float));
  float* dz = (float*)ws;
  ws += al256((size_t)rows * a.H * sizeof(float));
  uint32_t* bm = nullptr;
  uint32_t* rank = nullptr;
  if (sparse) {
    bm = (uint32_t*)ws;
    rank = (uint32_t*)(ws + al256((size_t)rows * nw * sizeof(uint32_t)));
    ws += 2 * al256((size_t)rows * nw * sizeof(uint32_t));
  }
  const size_t pfl = dkv_part_floats(a.B, a.T, a.Nc_cap, a.R_cap, a.window);
  float* part = (float*)ws;
  uint32_t* pflag = (uint32_t*)(ws + al256(pfl * sizeof(float)));
  const int tc = (a.Nc_cap + BW_KV_KEYS - 1) / BW_KV_KEYS;
  const int sc = dkv_slots_cmp(a.B, a.T, a.Nc_cap);
  float* part_r = part + (size_t)a.B * tc * sc * BW_KV_KEYS * 256;
  uint32_t* pflag_r = pflag + (size_t)a.B * tc * sc;
  const size_t nc = (size_t)a.B * a.Nc_cap * 256, nr = (size_t)a.B * a.R_cap * 256;
  // rows with no partial (no compressed tile attended, no window) are zero
  if (nc && !(a.dense || a.topk > 0)) bwd_zero_kernel<<<zero_grid(nc), 256, 0, s>>>(a.dkv_cmp, nc);
  if (nr && a.window <= 0) bwd_zero_kernel<<<zero_grid(nr), 256, 0, s>>>(a.dkv_raw, nr);
  if (a.dsink) bwd_zero_kernel<<<1, 256, 0, s>>>(a.dsink, (size_t)a.H);
  // mass of the slots (CSA) or entries (HCA) no row attends stays zero
  const size_t nmass = (size_t)rows * (sparse ? a.topk : a.Nc_cap);
  if (a.attn_mass && nmass)
    bwd_zero_kernel<<<zero_grid(nmass), 256, 0, s>>>(a.attn_mass, nmass);
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* dout = (const uint16_t*)a.dout;
  const uint16_t* kvc = (const uint16_t*)a.kv_cmp;
  const uint16_t* kvr = (const uint16_t*)a.kv_raw;
  float* dzp = a.dsink ? dz : nullptr;
  if (sparse && a.topk > 0 && a.Nc_cap > 0)
    bwd_bitmap_kernel<<<(rows + BM_ROWS - 1) / BM_ROWS, 64 * BM_ROWS, 0, s>>>(
        a.idx, rows, a.topk, a.Nc_cap, nw, bm, rank);

#define CSA_BWD_DQ(NHH_, DENSE_)                                                              \
  attn_bwd_dq_kernel<NHH_, DENSE_><<<rows, 64 * NHH_, DENSE_ ? 0 : sizeof(int32_t) * a.topk,  \
                                     s>>>(                                                    \
      q, dout, a.lse, a.sink, kvc, a.idx, kvr, a.q_pos, a.raw_base, a.n_cmp, a.T, a.Nc_cap,   \
      a.R_cap, sparse ? a.topk : 0, a.window, a.m, a.scale, a.dq, ldw, dzp)
  if (a.H == 64) {
    if (a.dense) CSA_BWD_DQ(2, true);
    else CSA_BWD_DQ(2, false);
  } else {
    if (a.dense) CSA_BWD_DQ(1, true);
    else CSA_BWD_DQ(1, false);
  }
#undef CSA_BWD_DQ
  if (a.dsink) {
    const int g = std::min(64, std::max(1, rows / 64));
    if (a.H == 64) bwd_sink_kernel<64><<<g, 256, 0, s>>>(dz, rows, a.dsink);
    else bwd_sink_kernel<32><<<g, 256, 0, s>>>(dz, rows, a.dsink);
  }

#define CSA_BWD_KV(NHH_, KIND_, KV_, CAP_, NSL_, PART_, FLAG_)                                \
  attn_bwd_dkv_kernel<NHH_, KIND_><<<dim3((CAP_ + BW_KV_KEYS - 1) / BW_KV_KEYS, NSL_, a.B),  \
                                     512, 0, s>>>(                                            \
      q, dout, ldw, KV_, CAP_, bm, rank, nw, a.q_pos, a.raw_base, a.n_cmp, a.T, a.topk,       \
      a.window, a.m, a.scale, NSL_, PART_, FLAG_, a.attn_mass)
  if (a.Nc_cap > 0 && (a.dense || (a.topk > 0))) {
    if (a.H == 64) {
      if (a.dense) CSA_BWD_KV(2, 1, kvc, a.Nc_cap, sc, part, pflag);
      else CSA_BWD_KV(2, 0, kvc, a.Nc_cap, sc, part, pflag);
    } else {
      if (a.dense) CSA_BWD_KV(1, 1, kvc, a.Nc_cap, sc, part, pflag);
      else CSA_BWD_KV(1, 0, kvc, a.Nc_cap, sc, part, pflag);
    }
    bwd_dkv_reduce_kernel<<<dim3(tc * 16, a.B), 256, 0, s>>>(part, pflag, tc, sc, a.Nc_cap,
                                                            a.dkv_cmp);
  }
  if (a.R_cap > 0 && a.window > 0) {
    const int sr = dkv_slots_raw(a.T, a.window), tr = (a.R_cap + BW_KV_KEYS - 1) / BW_KV_KEYS;
    if (a.H == 64) CSA_BWD_KV(2, 2, kvr, a.R_cap, sr, part_r, pflag_r);
    else CSA_BWD_KV(1, 2, kvr, a.R_cap, sr, part_r, pflag_r);
    bwd_dkv_reduce_kernel<<<dim3(tr * 16, a.B), 256, 0, s>>>(part_r, pflag_r, tr, sr, a.R_cap,
                                                            a.dkv_raw);
  }
#undef CSA_BWD_KV
  return hipGetLastError();
}

}  // namespace csa_host
