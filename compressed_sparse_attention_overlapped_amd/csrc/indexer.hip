// Lightning Indexer scores and per-row top-k for gfx950.
//
// Score (DS-V4 analysis section 1.2; article section 3.2, here with the
// multi-head ReLU form of the DeepSeek lightning indexer):
//     s(t, j) = sum_h w[t, h] ReLU(sq[t, h] sk[j] q[t, h] . k[j])
// for visible entries j < n_vis(t).  Scores go to an fp32 workspace row.
//
// Selection keeps the min(topk, n_vis) best scores under (score desc, index
// asc) and writes them in ascending index order, -1 padded.  Scores map to
// order-preserving 32-bit keys.
//  * short rows (Nc_cap <= kShortMax): one wave per row; the keys sit in LDS,
//    an MSB-first radix select (8-bit digits) finds the k-th key, and an
//    ordered pass writes the selected indices, taking equal keys in index
//    order.
//  * long rows: the score kernel also builds a per-row histogram of the top
//    11 key bits; "collect" workgroups (one per 2048-entry chunk) find the
//    bin holding the k-th key, mark the chunk's entries above it (certainly
//    selected) in a bitmap of the row and pack those inside it (candidates)
//    into the chunk's segment; "finalize" (one workgroup per row) picks the
//    missing entries among the candidates by an exact radix select on (key,
//    then index), adds them to the bitmap and writes the selection in
//    ascending order from it.  The score workgroup must own one query row
//    (a histogram per row), and the histogram starts at zero.
//  * long rows the histogram path cannot take (bf16 prefill rows, packed
//    sequences): exact selection over 8192-entry segments and merge levels
//    of their candidates, with no workspace that must start at zero.
#include <algorithm>

#include <type_traits>

#include "common.h"

namespace csa {

constexpr int kHistBins = 2048, kHistShift = 21;
constexpr int kShortMax = 8192;
constexpr int kChunk = 2048;
constexpr int kFinalCandLds = 8192;  // candidates held in LDS by finalize

__device__ __forceinline__ void hist_flush(const uint32_t* lhist, uint32_t* ghist) {
  for (int bin = threadIdx.x; bin < kHistBins; bin += blockDim.x) {
    uint32_t c = lhist[bin];
    if (c) atomicAdd(ghist + bin, c);
  }
}

// Threshold bin of a row from its histogram: the bin where the count from the
// top first reaches `need` (1 <= need <= total).  256 threads; each owns 8
// consecutive bins from the top.  Returns the bin in every thread.
__device__ uint32_t threshold_bin(const uint32_t* __restrict__ hist, uint32_t need, uint32_t* sh) {
  const int tid = threadIdx.x;
  uint32_t c[8], s = 0;
  for (int i = 0; i < 8; ++i) {
    c[i] = hist[kHistBins - 1 - (tid * 8 + i)];
    s += c[i];
  }
  uint32_t tot;
  const uint32_t base = block_excl_scan(s, sh, tot);
  if (base < need && base + s >= need) {
    uint32_t cum = base;
    for (int i = 0; i < 8; ++i) {
      if (cum + c[i] >= need) {
        sh[20] = (uint32_t)(kHistBins - 1 - (tid * 8 + i));
        break;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  return sh[20];
}

// ---------------------------------------------------------------- scores: fp32
// One thread per (row, entry); any H_I, d_I.  Grid (ceil(Nc_cap / 256), rows).
template <bool HIST>
__global__ void __launch_bounds__(256) score_f32_kernel(
    const float* __restrict__ q_idx, const float* __restrict__ w_idx,
    const float* __restrict__ k_idx, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int T, int H_I, int d_I, int Nc_cap, int m,
    float* __restrict__ scores, uint32_t* __restrict__ ghist, Varlen vl) {
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];
  const int row = blockIdx.y;
  const int b = vl.cu_q ? varlen_seq(vl, row) : row / T;
  const int t = vl.cu_q ? row - vl.cu_q[b] : row % T;
  const size_t kb0 = vl.cu_q ? (size_t)vl.cu_k[b] : (size_t)b * Nc_cap;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int nv = vl.cu_q ? n_visible(t, vl.cu_k[b + 1] - vl.cu_k[b], m, Nc_cap)
                         : n_visible(q_pos[b] + t, n_cmp[b], m, Nc_cap);
  if (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lhist[i] = 0;
    __syncthreads();
  }
  if (j < nv) {
    const float* qr = q_idx + (size_t)row * H_I * d_I;
    const float* kr = k_idx + (kb0 + j) * d_I;
    float s = 0.0f;
    for (int h = 0; h < H_I; ++h) {
      float dot = 0.0f;
      for (int e = 0; e < d_I; ++e) dot = fmaf(qr[h * d_I + e], kr[e], dot);
      s = fmaf(w_idx[(size_t)row * H_I + h], fmaxf(dot, 0.0f), s);
    }
    scores[(size_t)row * Nc_cap + j] = s;
    if (HIST) atomicAdd(&lhist[score_key(s) >> kHistShift], 1u);
  }
  if (HIST) {
    __syncthreads();
    hist_flush(lhist, ghist + (size_t)row * kHistBins);
  }
}

// max(x, 0) on the bit pattern: a float with its sign bit set is a negative
// integer, so the signed integer maximum with 0 is the ReLU of every finite
// value in one instruction (fmaxf also quiets NaN inputs first)
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ---------------------------------------------------------------- scores: bf16
// H_I = 16, d_I = 64.  A workgroup (4 waves) owns 16 consecutive query rows of
// one sequence (4 per wave: two 32-row MFMA tiles of 2 rows x 16 heads) and a
// chunk of entries; 64-entry key tiles are staged in LDS for all waves.
constexpr int SB_ROWS = 16, SB_KT = 64, SB_KSTRIDE = 64 + 8;  // bf16 per LDS key row

template <bool HIST, bool PAGED>
__global__ void __launch_bounds__(256) score_bf16_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int T, int Nc_cap, int m, int key_chunk,
    float* __restrict__ scores, uint32_t* __restrict__ ghist, PageTable pt, Varlen vl) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][SB_KT * SB_KSTRIDE];
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];
  // paged caches: the chunk's page ids (pages of at least 16 entries)
  __shared__ int32_t pg_s[PAGED ? kChunk / 16 + 1 : 1];
  // later rows see more entries: they are dispatched first
  const int b = blockIdx.z, t0 = (gridDim.x - 1 - blockIdx.x) * SB_ROWS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this sequence's first query row and key row (packed sequences: their
  // offsets, positions from 0; the grid covers the longest sequence)
  const size_t qrow0 = vl.cu_q ? (size_t)vl.cu_q[b] : (size_t)b * T;
  const size_t kb0 = vl.cu_q ? (size_t)vl.cu_k[b] : (size_t)b * Nc_cap;
  if (vl.cu_q) T = vl.cu_q[b + 1] - vl.cu_q[b];
  if (t0 >= T) return;  // uniform, before any barrier
  const int64_t p0 = vl.cu_q ? 0 : q_pos[b];
  const int ncb = vl.cu_q ? vl.cu_k[b + 1] - vl.cu_k[b] : n_cmp[b];
  const int jb = blockIdx.y * key_chunk;
  // entries this workgroup must score: up to the largest n_vis of its rows
  const int t_last = min(T - 1, t0 + SB_ROWS - 1);
  const int nv_max = n_visible(p0 + t_last, ncb, m, Nc_cap);
  const int je = min(nv_max, jb + key_chunk);

  if (HIST) {
    for (int i = tid; i < kHistBins; i += blockDim.x) lhist[i] = 0;
  }
  const int p_first = PAGED ? jb >> pt.page_log2 : 0;
  if (PAGED && jb < Nc_cap) {
    const int n_pg = ((min(jb + key_chunk, Nc_cap) - 1) >> pt.page_log2) - p_first + 1;
    for (int i = tid; i < n_pg; i += blockDim.x) pg_s[i] = page_or_absent(pt, b, p_first + i);
  }
  // A operands: rows (token, head) -> lane row (lane & 31) of tile mt:
  // token = wave*4 + mt*2 + (lane&31)/16, head = lane & 15; k-step s covers
  // dims 16 s + 8 (lane / 32) .. + 8.
  bf16x8 a[2][4];
  int trow[2];
  for (int mt = 0; mt < 2; ++mt) {
    int tt = t0 + wave * 4 + mt * 2 + ((lane & 31) >> 4);
    trow[mt] = tt;
    int h = lane & 15;
    // rows past T read row T - 1 (loads stay unconditional, so that the
    // waits in the key loop count loads exactly); their scores are not stored
    const int tq = min(tt, T - 1);
    for (int s = 0; s < 4; ++s)
      a[mt][s] = *(const bf16x8*)(q_idx + ((qrow0 + tq) * 16 + h) * 64 + 16 * s +
                                  8 * (lane >> 5));
  }
  // head weights for the accumulator rows: tile mt, register r -> token
  // wave*4 + mt*2 + r/8, head 8 ((r%8)/4) + 4 (lane/32) + r%4
  float wv[2][16];
  int nvis[2][2];
  for (int mt = 0; mt < 2; ++mt) {
    for (int r = 0; r < 16; ++r) {
      int tt = t0 + wave * 4 + mt * 2 + (r >> 3);
      int h = 8 * ((r & 7) >> 2) + 4 * (lane >> 5) + (r & 3);
      wv[mt][r] = w_idx[(qrow0 + min(tt, T - 1)) * 16 + h];
    }
    for (int u = 0; u < 2; ++u) {
      int tt = t0 + wave * 4 + mt * 2 + u;
      nvis[mt][u] = tt < T ? n_visible(p0 + tt, ncb, m, Nc_cap) : 0;
    }
  }
  __syncthreads();

  // 64-key tiles, LDS double-buffered; the next tile's 512 chunks of 16 B
  // (2 per thread) load into registers while the current one multiplies.
  // Rows past je re-read row je - 1 (valid) and their scores are not stored.
  u32x4 pk[2];
  auto loadk = [&](int j0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * 256 + tid, r = c >> 3, q8 = c & 7;
      const int row = min(j0 + r, je - 1);
      size_t at = kb0 + row;
      if constexpr (PAGED) {
        // an absent page reads pool row 0 (its scores are replaced below)
        const int pg = pg_s[(row >> pt.page_log2) - p_first];
        at = pg < 0 ? 0
                    : ((size_t)pg << pt.page_log2) | (size_t)(row & ((1 << pt.page_log2) - 1));
      }
      pk[i] = *(const u32x4*)(k_idx + at * 64 + q8 * 8);
    }
  };
  auto storek = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * 256 + tid, r = c >> 3, q8 = c & 7;
      *(u32x4*)(Ks[buf] + r * SB_KSTRIDE + q8 * 8) = pk[i];
    }
  };
  if (jb < je) {
    loadk(jb);
    storek(0);
    loadk(jb + SB_KT);
  }
  __syncthreads();
  for (int j0 = jb, it = 0; j0 < je; j0 += SB_KT, ++it) {
    const uint16_t* kt = Ks[it & 1];
    for (int nt = 0; nt < 2; ++nt) {
      bf16x8 bk[4];
      for (int s = 0; s < 4; ++s)
        bk[s] = *(const bf16x8*)(kt + (nt * 32 + (lane & 31)) * SB_KSTRIDE + 16 * s + 8 * (lane >> 5));
      const int j = j0 + nt * 32 + (lane & 31);
      // the two row tiles' products interleaved: consecutive MFMAs independent
      f32x16 acc[2];
      for (int mt = 0; mt < 2; ++mt)
        for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
      for (int s = 0; s < 4; ++s)
        for (int mt = 0; mt < 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][s], bk[s], acc[mt], 0, 0, 0);
      for (int mt = 0; mt < 2; ++mt) {
        float s0 = 0.0f, s1 = 0.0f;
        for (int r = 0; r < 8; ++r) s0 = fmaf(wv[mt][r], relu_bits(acc[mt][r]), s0);
        for (int r = 8; r < 16; ++r) s1 = fmaf(wv[mt][r], relu_bits(acc[mt][r]), s1);
        s0 = sum_xor32(s0);
        s1 = sum_xor32(s1);
        const int u = lane >> 5;  // lanes < 32 write token 0 of the pair, others token 1
        float sc = u ? s1 : s0;
        const int tt = trow[mt] - ((lane & 31) >> 4) + u;
        if (tt < T && j < je && j < nvis[mt][u]) {
          // an entry of an absent page has no key: the lowest score
          if constexpr (PAGED)
            if (pg_s[(j >> pt.page_log2) - p_first] < 0) sc = -INFINITY;
          scores[(qrow0 + tt) * Nc_cap + j] = sc;
          if (HIST) atomicAdd(&lhist[score_key(sc) >> kHistShift], 1u);
        }
      }
    }
    if (j0 + SB_KT < je) {
      // buffer (it + 1) & 1 was last read for tile it - 1, before the
      // previous barrier
      storek((it + 1) & 1);
      loadk(j0 + 2 * SB_KT);
    }
    __syncthreads();
  }
  if (HIST) {
    // one histogram per query row: rows of this workgroup share the LDS
    // histogram, so long rows run with T == 1 (row = b)
    __syncthreads();
    hist_flush(lhist, ghist + (qrow0 + t0) * kHistBins);
  }
}

// ---------------------------------------------------------------- scores: fp8
// H_I = 16, d_I = 64, e4m3 codes with positive row scales.  One query row per
// workgroup, a chunk of kChunk entries split over 4 waves.  The codes are
// widened to bf16 (exact: e4m3 values are bf16 values) and multiplied on the
// bf16 16x16x32 MFMA, whose fp32 accumulation is exact to fp32 rounding; the
// fp8 MFMA accumulates with fewer bits, which would move scores by more than
// the top-k tie tolerance.  Each 16-entry group is two MFMAs (heads x
// entries).  Lane l loads 16 contiguous bytes of entry (l % 16) at byte
// offset 16 (l / 16); the first 8 codes feed the first MFMA and the next 8
// the second (the query uses the same k order).
constexpr int SF_UNROLL = 8;

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// MXFP4 (OCP): eight E2M1 codes of one 32-bit word (element 2i in the low
// nibble of byte i) to bf16 times the block scale; exact, E2M1 values having
// at most two significant bits.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}
// E8M0 scale byte to its value 2^(code - 127) (code 0: the subnormal 2^-127)
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  return __uint_as_float(code ? code << 23 : 0x00400000u);
}

// QK = CSA_DT_FP8E4M3: rows of 64 e4m3 codes with fp32 row scales (q_scale
// per head row, k_scale per entry).  QK = CSA_DT_MXFP4: rows of 32 bytes of
// E2M1 codes with two E8M0 block scales each; lane l then loads 8 bytes (the
// same 16 dims as above) and its block's scale byte.
template <bool HIST, int QK, bool PAGED>
__global__ void __launch_bounds__(256) score_fp8_kernel(
    const uint8_t* __restrict__ q_idx, const void* __restrict__ q_scale,
    const float* __restrict__ w_idx, const uint8_t* __restrict__ k_idx,
    const void* __restrict__ k_scale, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int T, int Nc_cap, int m, float* __restrict__ scores,
    uint32_t* __restrict__ ghist, PageTable pt) {
  constexpr bool FP4 = QK == CSA_DT_MXFP4;
  constexpr int KB = FP4 ? 32 : 64;  // code bytes per row of 64 values
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];
  // paged caches: the chunk's page ids (pages of at least 16 entries), read
  // once so that a key load waits on LDS rather than on the block table
  __shared__ int32_t pg_s[PAGED ? kChunk / 16 + 1 : 1];
  const int row = blockIdx.y, b = row / T, t = row % T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = n_visible(q_pos[b] + t, n_cmp[b], m, Nc_cap);
  const int jb = blockIdx.x * kChunk;
  const int p_first = PAGED ? jb >> pt.page_log2 : 0;
  if (PAGED) {
    const int n_pg = ((min(jb + kChunk, Nc_cap) - 1) >> pt.page_log2) - p_first + 1;
    for (int i = tid; i < n_pg; i += blockDim.x) pg_s[i] = page_or_absent(pt, b, p_first + i);
  }
  if (HIST) {
    for (int i = tid; i < kHistBins; i += blockDim.x) lhist[i] = 0;
  }
  if (HIST || PAGED) __syncthreads();
  const int je = min(nv, jb + kChunk);
  // this wave's entries: [wb, we), in SF_ITERS steps of 16 * SF_UNROLL
  constexpr int kPerWave = kChunk / 4, kStep = 16 * SF_UNROLL, SF_ITERS = kPerWave / kStep;
  const int wb = jb + wave * kPerWave;
  const int we = min(je, wb + kPerWave);
  if (wb < we) {
    const int h = lane & 15, g = lane >> 4;
    bf16x8 qa0, qa1;
    if constexpr (FP4) {
      const u32x2 qw = *(const u32x2*)(q_idx + ((size_t)row * 16 + h) * 32 + 8 * g);
      const float qs = e8m0_value(((const uint8_t*)q_scale)[((size_t)row * 16 + h) * 2 + (g >> 1)]);
      qa0 = fp4x8_to_bf16x8(qw[0], qs);
      qa1 = fp4x8_to_bf16x8(qw[1], qs);
    } else {
      const u32x4 qv = *(const u32x4*)(q_idx + ((size_t)row * 16 + h) * 64 + 16 * g);
      qa0 = e4m3x8_to_bf16x8(qv[0], qv[1]);
      qa1 = e4m3x8_to_bf16x8(qv[2], qv[3]);
    }
    float wq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int hh = 4 * g + i;
      wq[i] = w_idx[(size_t)row * 16 + hh] *
              (FP4 ? 1.0f : ((const float*)q_scale)[(size_t)row * 16 + hh]);
    }
    // paged caches: the rows sit in a shared pool (16 consecutive entries,
    // one load group, never straddle a page)
    const size_t kbase = PAGED ? 0 : (size_t)b * Nc_cap;
    // (an absent page reads pool row 0; its scores are replaced below)
    auto krow = [&](int j) -> size_t {
      if constexpr (PAGED) {
        const int pg = pg_s[(j >> pt.page_log2) - p_first];
        return pg < 0 ? 0 : ((size_t)pg << pt.page_log2) | (size_t)(j & ((1 << pt.page_log2) - 1));
      }
      return (size_t)j;
    };
    const uint8_t* kb = k_idx + kbase * KB;
    const float* ks = FP4 ? nullptr : (const float*)k_scale + kbase;
    const uint8_t* ks8 = FP4 ? (const uint8_t*)k_scale + kbase * 2 : nullptr;
    float* srow = scores + (size_t)row * Nc_cap;
    // two register stages: the codes of step i + 2 load while step i computes
    u32x4 kv[2][SF_UNROLL];
    float ksc[2][SF_UNROLL / 4];  // scale of the entry this lane writes, per 64-entry half
    // (MXFP4: words 0-1 the 16 codes, word 2 the block's scale byte)
    auto load = [&](int it, int st) {
#pragma unroll
      for (int u = 0; u < SF_UNROLL; ++u) {
        const int j = wb + it * kStep + 16 * u + (lane & 15);
        if constexpr (FP4) {
          const size_t r = j < we ? krow(j) : 0;
          const u32x2 w = j < we ? __builtin_nontemporal_load((const u32x2*)(kb + r * 32 + 8 * g))
                                 : u32x2{0, 0};
          kv[st][u] = u32x4{w[0], w[1], j < we ? (uint32_t)ks8[r * 2 + (g >> 1)] : 127u, 0u};
        } else {
          const size_t r = j < we ? krow(j) : 0;
          kv[st][u] = j < we ? __builtin_nontemporal_load((const u32x4*)(kb + r * 64 + 16 * g))
                             : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int hf = 0; hf < SF_UNROLL / 4; ++hf) {
        const int j = wb + it * kStep + 64 * hf + lane;
        ksc[st][hf] = FP4 ? 1.0f : (j < we ? ks[krow(j)] : 0.0f);
      }
    };
    load(0, 0);
    load(1, 1);
    const bool b5 = (lane >> 5) & 1, b4 = (lane >> 4) & 1;
#pragma unroll
    for (int it = 0; it < SF_ITERS; ++it) {
      const int st = it & 1;
      const int j0 = wb + it * kStep;
      float part[SF_UNROLL];
#pragma unroll
      for (int u = 0; u < SF_UNROLL; ++u) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        bf16x8 k0, k1;
        if constexpr (FP4) {
          const float sc_blk = e8m0_value(kv[st][u][2]);
          k0 = fp4x8_to_bf16x8(kv[st][u][0], sc_blk);
          k1 = fp4x8_to_bf16x8(kv[st][u][1], sc_blk);
        } else {
          k0 = e4m3x8_to_bf16x8(kv[st][u][0], kv[st][u][1]);
          k1 = e4m3x8_to_bf16x8(kv[st][u][2], kv[st][u][3]);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, k0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, k1, acc, 0, 0, 0);
        // acc[i]: head 4 (lane / 16) + i, entry lane % 16 of group u
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) p = fmaf(wq[i], relu_bits(acc[i]), p);
        part[u] = p;
      }
      float sc[SF_UNROLL / 4];
      sc[0] = ksc[st][0];
      sc[1] = ksc[st][1];
      if (it + 2 < SF_ITERS) load(it + 2, st);
      // Reduce-scatter over the four 16-lane head groups: afterwards lane l
      // holds the full score of entry l % 16 of group 4 half + l / 16, i.e.
      // entry j0 + 64 half + l.  Exchange across lane bit 5, then bit 4.
#pragma unroll
      for (int half = 0; half < SF_UNROLL / 4; ++half) {
        const float* q = part + 4 * half;
        const float s0 = b5 ? q[0] : q[2], s1 = b5 ? q[1] : q[3];
        const float k0 = b5 ? q[2] : q[0], k1 = b5 ? q[3] : q[1];
        const float r0 = k0 + lane_xor32(s0), r1 = k1 + lane_xor32(s1);
        float v = ((b4 ? r1 : r0) + lane_xor16(b4 ? r0 : r1)) * sc[half];
        const int j = j0 + 64 * half + lane;
        if (j < we) {
          // an entry of an absent page has no key: the lowest score
          if constexpr (PAGED)
            if (pg_s[(j >> pt.page_log2) - p_first] < 0) v = -INFINITY;
          srow[j] = v;
          if (HIST) atomicAdd(&lhist[score_key(v) >> kHistShift], 1u);
        }
      }
    }
  }
  if (HIST) {
    __syncthreads();
    hist_flush(lhist, ghist + (size_t)row * kHistBins);
  }
}

// Result of an MSB-first radix select of the `need` largest of n keys: with
// all_eq the selected set is {x : (x & mask) >= prefix}; otherwise the key
// width got fully resolved and the set is {x > prefix} plus `remaining` keys
// equal to prefix.
struct RadixResult {
  uint32_t prefix, mask, remaining;
  bool all_eq;
};

// ---------------------------------------------------------------- short rows
// One wave per row (4 rows per workgroup), Nc_cap <= KMAX: the row's keys sit
// in the wave's LDS slice, an MSB-first radix select (8-bit digits, a
// wave-private 256-bin histogram) finds the k-th key, and one ordered pass
// over 64-key groups (ballots) writes the selected indices ascending, taking
// keys equal to the k-th in index order.  No workgroup barrier: every step
// is the wave's own, and a wave's LDS operations complete in issue order.
template <int KMAX>
__global__ void __launch_bounds__(256) select_short_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int rows, int T, int Nc_cap, int m, int topk,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out, Varlen vl) {
  // rows of up to 2048 keys keep them in registers (lane l: keys l, l + 64,
  // ...), longer ones in the wave's LDS slice
  constexpr bool REG = KMAX <= 2048;
  constexpr int KPL = KMAX / 64;  // keys per lane
  __shared__ uint32_t keys_all[REG ? 1 : 4][REG ? 1 : KMAX];
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][2048];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const int b = vl.cu_q ? varlen_seq(vl, row) : row / T;
  const int t = vl.cu_q ? row - vl.cu_q[b] : row % T;
  uint32_t* keys = keys_all[REG ? 0 : wave];
  uint32_t* hist = hist_all[wave];
  const int nv = vl.cu_q ? n_visible(t, vl.cu_k[b + 1] - vl.cu_k[b], m, Nc_cap)
                         : n_visible(q_pos[b] + t, n_cmp[b], m, Nc_cap);
  const float* srow = scores + (size_t)row * Nc_cap;
  int32_t* orow = idx_out + (size_t)row * topk;
  float* sorow = score_out ? score_out + (size_t)row * topk : nullptr;
  const int nsel = min(topk, nv);
  for (int k = nsel + lane; k < topk; k += 64) {
    orow[k] = -1;
    if (sorow) sorow[k] = __uint_as_float(0x7fc00000u);
  }
  if (nsel == 0) return;
  if (nsel == nv) {  // everything visible is selected
    for (int j = lane; j < nv; j += 64) {
      orow[j] = j;
      if (sorow) sorow[j] = srow[j];
    }
    return;
  }
  const int ng = (nv + 63) / 64;  // 64-key groups
  // keys (order-preserving u32 of the scores), sixteen loads in flight per
  // lane from clamped addresses, and the row's smallest and largest key
  uint32_t kr[REG ? KPL : 1];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int g0 = 0; g0 < (REG ? KPL : ng); g0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = srow[min(64 * (g0 + u) + lane, nv - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = 64 * (g0 + u) + lane;
      const uint32_t x = score_key(v[u]);
      if (REG) kr[g0 + u] = x;
      else if (g0 + u < ng) keys[min(j, KMAX - 1)] = x;
      if (j < nv) {
        kmin = min(kmin, x);
        kmax = max(kmax, x);
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  // the histogram of one digit over the keys still matching the prefix; the
  // atomics of a batch are issued back to back
  // bin b lives at word b, or with swz at b ^ (((b >> 6) & 7) << 2): the
  // 16-byte groups of each 32-bin lane range are permuted by the range's
  // index, so that the lanes' 16-byte reads of their ranges hit distinct banks
  auto count = [&](uint32_t mask, uint32_t prefix, int shift, uint32_t dmask, bool swz) {
    auto bin_at = [&](uint32_t x) {
      const uint32_t bn = (x >> shift) & dmask;
      return swz ? bn ^ (((bn >> 6) & 7u) << 2) : bn;
    };
    if constexpr (REG) {
#pragma unroll
      for (int u = 0; u < KPL; ++u) {
        const int j = 64 * u + lane;
        if (j < nv && (kr[u] & mask) == prefix) atomicAdd(&hist[bin_at(kr[u])], 1u);
      }
    } else {
      for (int g0 = 0; g0 < ng; g0 += 8) {
        uint32_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = keys[min(64 * (g0 + u) + lane, KMAX - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = 64 * (g0 + u) + lane;
          if (j < nv && (x[u] & mask) == prefix) atomicAdd(&hist[bin_at(x[u])], 1u);
        }
      }
    }
  };
  // radix select over the bits below the keys' common prefix.  The first
  // digit is up to 11 bits wide (2048 bins, 32 per lane), so that the LDS
  // atomics of the full pass spread over many bins and few keys share the
  // threshold bin; later digits are up to 8 bits (256 bins, 4 per lane).
  // Lane l owns bins NB - 1 - (BPL l + i), i = 0 .. BPL - 1 (top bins first).
  // (Every key equal: the mask covers all bits, and the output pass takes the
  // first nsel entries.)
  const uint32_t diff = kmin ^ kmax;
  int hi = diff ? 31 - __clz((int)diff) : -1;  // highest bit where keys differ
  // the bits above hi (all of them when every key is equal, hi = -1), as one
  // 64-bit shift rather than nested selects
  uint32_t mask = (uint32_t)(0xffffffffull << (hi + 1));
  uint32_t prefix = kmax & mask, remaining = (uint32_t)nsel;
  bool all_eq = false;
  auto radix_pass = [&](auto bpl_tag) {
    constexpr int BPL = decltype(bpl_tag)::value, NB = 64 * BPL;
    constexpr int WMAX = BPL == 32 ? 11 : 8;
    const int width = min(WMAX, hi + 1), shift = hi - width + 1;
    const uint32_t dmask = (1u << width) - 1u;
    const int base = NB - BPL * (lane + 1);  // lowest bin of this lane
    constexpr bool SWZ = BPL == 32;          // 2048 bins: swizzled groups
#pragma unroll
    for (int i = 0; i < BPL; i += 4) *(u32x4*)&hist[4 * lane + 64 * i] = u32x4{0u, 0u, 0u, 0u};
    count(mask, prefix, shift, dmask, SWZ);
    uint32_t c[BPL], sum = 0u;
#pragma unroll
    for (int i = 0; i < BPL; i += 4) {
      const int at = SWZ ? base + (i ^ ((((base >> 6) & 7) << 2))) : base + i;
      const u32x4 v = *(const u32x4*)&hist[at];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[BPL - 1 - (i + e)] = v[e];
    }
#pragma unroll
    for (int i = 0; i < BPL; ++i) sum += c[i];
    uint32_t incl = sum;  // inclusive prefix over lanes (lane 0 = top bins)
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    uint32_t above = incl - sum;
    int dsel = -1;
    uint32_t cum_sel = 0u, cnt_sel = 0u;
    if (above < remaining && above + sum >= remaining) {
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        if (dsel < 0 && above + c[i] >= remaining) {
          dsel = NB - 1 - (BPL * lane + i);
          cum_sel = above;
          cnt_sel = c[i];
        }
        above += c[i];
      }
    }
    const uint64_t who = __ballot(dsel >= 0);
    const int src = (int)__ffsll((unsigned long long)who) - 1;
    const uint32_t d = (uint32_t)__shfl(dsel, src, 64);
    const uint32_t cum = __shfl(cum_sel, src, 64), cnt = __shfl(cnt_sel, src, 64);
    remaining -= cum;
    prefix |= d << shift;
    mask |= dmask << shift;
    hi = shift - 1;
    if (cnt == remaining) all_eq = true;
  };
  if (hi >= 0) radix_pass(std::integral_constant<int, 32>{});
  while (!all_eq && hi >= 0) radix_pass(std::integral_constant<int, 4>{});
  // ordered output: groups of 64 consecutive entries
  uint32_t out_base = 0u, eq_taken = 0u;
  auto emit = [&](int g, uint32_t key) {
    const int j = 64 * g + lane;
    const uint32_t x = key & mask;
    const bool gt = j < nv && x > prefix;
    const bool eq = j < nv && x == prefix;
    const uint64_t eqm = __ballot(eq);
    const uint32_t eq_rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(eqm >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
    const bool sel = gt || (eq && (all_eq || eq_taken + eq_rank < remaining));
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const uint32_t pos = out_base + __builtin_amdgcn_mbcnt_hi(
                                          (uint32_t)(sm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
      orow[pos] = j;
      if (sorow) sorow[pos] = srow[j];
    }
    out_base += (uint32_t)__popcll(sm);
    eq_taken += (uint32_t)__popcll(eqm);
  };
  // when the threshold bin holds exactly the keys still needed (all_eq),
  // every key at or above the threshold is taken: no ranking of equal keys
  auto emit_all = [&](int g, uint32_t key) {
    const int j = 64 * g + lane;
    const bool sel = j < nv && (key & mask) >= prefix;
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const uint32_t pos = out_base + __builtin_amdgcn_mbcnt_hi(
                                          (uint32_t)(sm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
      orow[pos] = j;
      if (sorow) sorow[pos] = srow[j];
    }
    out_base += (uint32_t)__popcll(sm);
  };
  if (all_eq) {
    if constexpr (REG) {
#pragma unroll
      for (int u = 0; u < KPL; ++u)
        if (u < ng) emit_all(u, kr[u]);
    } else {
      for (int g = 0; g < ng; ++g) emit_all(g, keys[64 * g + lane]);
    }
  } else if constexpr (REG) {
#pragma unroll
    for (int u = 0; u < KPL; ++u)
      if (u < ng) emit(u, kr[u]);
  } else {
    for (int g = 0; g < ng; ++g) emit(g, keys[64 * g + lane]);
  }
}

// ---------------------------------------------------------------- long rows
// Grid (n_chunks, rows), 256 threads; wave w owns the 512 consecutive entries
// [j0 + 512 w, + 512) of the chunk.  Each workgroup finds the row's threshold
// bin from the histogram, writes the chunk's words of the row bitmap of
// entries above that bin (certainly selected; 64-entry ballots, one word pair
// per group) and packs the entries inside the bin (candidates: index and low
// key bits) at the start of the chunk's own segment, with their count in
// chunk_cnt.  No counter is shared between workgroups.  Rows that keep every
// visible entry, or none, are left to finalize.
__global__ void __launch_bounds__(256) collect_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ ghist,
    const int64_t* __restrict__ q_pos, const int32_t* __restrict__ n_cmp, int T, int Nc_cap,
    int m, int topk, int n_chunks, int bm_words, uint32_t* __restrict__ def_bm,
    uint32_t* __restrict__ chunk_cnt, uint32_t* __restrict__ cand_idx,
    uint32_t* __restrict__ cand_key) {
  __shared__ uint32_t sh[32];
  const int chunk = blockIdx.x, row = blockIdx.y, b = row / T, t = row % T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = n_visible(q_pos[b] + t, n_cmp[b], m, Nc_cap);
  const int nsel = min(topk, nv);
  const int j0 = chunk * kChunk, j1 = min(nv, j0 + kChunk);
  if (nsel == 0 || nsel == nv || j0 >= j1) return;
  const uint32_t bin = threshold_bin(ghist + (size_t)row * kHistBins, (uint32_t)nsel, sh);
  const float* srow = scores + (size_t)row * Nc_cap;
  uint32_t* bm = def_bm + (size_t)row * bm_words;
  const int wb = j0 + wave * 512;
  constexpr int kGroups = kChunk / 256;
  uint32_t key[kGroups];
  uint32_t n_wave = 0;
  // every score load is issued before the first is used (clamped addresses)
  float sv[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) sv[g] = srow[min(wb + g * 64 + lane, j1 - 1)];
  for (int g = 0; g < kGroups; ++g) {
    const int j = wb + g * 64 + lane;
    const bool valid = j < j1;
    key[g] = valid ? score_key(sv[g]) : 0u;
    const uint32_t kb = key[g] >> kHistShift;
    const uint64_t dm = __ballot(valid && kb > bin);
    const uint64_t cm = __ballot(valid && kb == bin);
    if (lane == 0 && wb + g * 64 < j1) *(uint64_t*)(bm + (wb + g * 64) / 32) = dm;
    n_wave += (uint32_t)__popcll(cm);
  }
  if (lane == 0) sh[24 + wave] = n_wave;
  __syncthreads();
  uint32_t pos = 0;
  for (int w = 0; w < wave; ++w) pos += sh[24 + w];
  if (tid == 0) chunk_cnt[(size_t)row * n_chunks + chunk] = sh[24] + sh[25] + sh[26] + sh[27];
  uint32_t* ci = cand_idx + (size_t)row * Nc_cap + j0;
  uint32_t* ck = cand_key + (size_t)row * Nc_cap + j0;
  for (int g = 0; g < kGroups; ++g) {
    const int j = wb + g * 64 + lane;
    const bool c = j < j1 && (key[g] >> kHistShift) == bin;
    const uint64_t cm = __ballot(c);
    if (c) {
      const uint32_t p = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
      ci[p] = (uint32_t)j;
      ck[p] = key[g] & ((1u << kHistShift) - 1u);
    }
    pos += (uint32_t)__popcll(cm);
  }
}

// MSB-first radix select with 11-bit digits over 22-bit keys (two passes) of
// the `need` largest of n keys, 1 <= need < n; same result convention as
// radix_select.  hist: 2048 words of LDS; sh: >= 32 words; blockDim.x = 1024.
template <class Get>
__device__ RadixResult radix_select22(Get get, int n, uint32_t need, uint32_t* hist,
                                      uint32_t* sh) {
  RadixResult r{0u, 0u, need, false};
  const int tid = threadIdx.x;
  for (int shift = 11; shift >= 0; shift -= 11) {
    for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
      const uint32_t x = get(i);
      if ((x & r.mask) == r.prefix) atomicAdd(&hist[(x >> shift) & 2047u], 1u);
    }
    __syncthreads();
    // thread i owns bins 2047 - 2i (upper) and 2046 - 2i (lower)
    const uint32_t c_hi = hist[2047 - 2 * tid], c_lo = hist[2046 - 2 * tid];
    uint32_t tot;
    const uint32_t above = block_excl_scan(c_hi + c_lo, sh + 8, tot);
    if (above < r.remaining && above + c_hi >= r.remaining) {
      sh[0] = 2047u - 2 * tid;
      sh[1] = above;
      sh[2] = c_hi;
    } else if (above + c_hi < r.remaining && above + c_hi + c_lo >= r.remaining) {
      sh[0] = 2046u - 2 * tid;
      sh[1] = above + c_hi;
      sh[2] = c_lo;
    }
    __syncthreads();
    const uint32_t d = sh[0], cum = sh[1], cnt = sh[2];
    __syncthreads();
    r.remaining -= cum;
    r.prefix |= d << shift;
    r.mask |= 2047u << shift;
    if (cnt == r.remaining) {
      r.all_eq = true;
      break;
    }
  }
  return r;
}

constexpr int FIN_THREADS = 1024;
constexpr int kBitmapLds = 16384;  // 2^19 entries

// Marks in bm the `need` best of n_cand candidates under (key desc, index asc):
// a radix select on the low key bits, then, among candidates whose key
// equals the k-th, one on (Nc_cap - index).  FIN_THREADS threads; hist: 2048
// words of LDS.  Ends with a barrier.
template <class KeyAt, class IdxAt>
__device__ void select_candidates(KeyAt key_at, IdxAt idx_at, uint32_t n_cand, uint32_t need,
                                  int Nc_cap, uint32_t* bm, uint32_t* hist, uint32_t* sh) {
  RadixResult rk{0u, 0u, need, true};
  RadixResult ri{0u, 0u, 0u, true};
  bool tie_break = false;
  if (need < n_cand) {
    rk = radix_select22([&](int i) { return key_at(i); }, (int)n_cand, need, hist, sh);
    if (!rk.all_eq) {
      // rk.remaining of the candidates whose key equals rk.prefix, lowest
      // indices first: the largest values of Nc_cap - index (>= 1, so the
      // other candidates' 0 never ties with them)
      tie_break = true;
      ri = radix_select22(
          [&](int i) { return key_at(i) == rk.prefix ? (uint32_t)Nc_cap - idx_at(i) : 0u; },
          (int)n_cand, rk.remaining, hist, sh);
    }
  }
  for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) {
    bool sel = true;
    if (need < n_cand) {
      const uint32_t x = key_at(i) & rk.mask;
      if (x != rk.prefix) sel = x > rk.prefix;
      else if (tie_break) sel = (((uint32_t)Nc_cap - idx_at(i)) & ri.mask) >= ri.prefix;
    }
    if (sel) {
      const uint32_t j = idx_at(i);
      atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
}

// Ascending output of the entries marked in a row bitmap of nwords words:
// thread t owns words [t per, (t + 1) per); a popcount scan places them.
template <class Word>
__device__ void write_selection(Word word, int nwords, const float* srow, int32_t* orow,
                                float* sorow, uint32_t* sh) {
  const int per = (nwords + (int)blockDim.x - 1) / (int)blockDim.x;
  const int w0 = min(nwords, (int)threadIdx.x * per), w1 = min(nwords, w0 + per);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(word(w));
  uint32_t tot;
  uint32_t pos = block_excl_scan(cnt, sh, tot);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = word(w);
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      const int j = w * 32 + bit;
      orow[pos] = j;
      if (sorow) sorow[pos] = srow[j];
      ++pos;
    }
  }
}

// Padding, and the rows that need no selection (none or every visible entry
// kept).  Returns true when the row is finished.
__device__ bool trivial_row(int nsel, int nv, int topk, const float* srow, int32_t* orow,
                            float* sorow) {
  for (int k = nsel + threadIdx.x; k < topk; k += blockDim.x) {
    orow[k] = -1;
    if (sorow) sorow[k] = __uint_as_float(0x7fc00000u);
  }
  if (nsel == 0) return true;
  if (nsel == nv) {
    for (int j = threadIdx.x; j < nv; j += blockDim.x) {
      orow[j] = j;
      if (sorow) sorow[j] = srow[j];
    }
    return true;
  }
  return false;
}

// One workgroup (1024 threads) per long row after collect.  The selected set
// is the entries marked in the collect bitmap plus the best candidates
// (select_candidates).  Candidates are gathered from the chunk segments into
// LDS (or, beyond kFinalCandLds, a flat workspace list); chosen ones are added
// to the bitmap (in LDS up to kBitmapLds words, else in place in the
// workspace), which then gives the ascending output.
template <bool BM_LDS>
__global__ void __launch_bounds__(FIN_THREADS) finalize_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int T, int Nc_cap, int m, int topk, int n_chunks,
    int bm_words, uint32_t* __restrict__ def_bm, const uint32_t* __restrict__ chunk_cnt,
    const uint32_t* __restrict__ cand_idx, const uint32_t* __restrict__ cand_key,
    uint32_t* __restrict__ cand_flat, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  __shared__ uint32_t ckey[kFinalCandLds];
  __shared__ uint32_t cidx[kFinalCandLds];
  __shared__ uint32_t lbm[BM_LDS ? kBitmapLds : 1];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t coff[FIN_THREADS], ccnt[FIN_THREADS];
  __shared__ uint32_t sh[32];
  const int row = blockIdx.x, b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const int nv = n_visible(q_pos[b] + t, n_cmp[b], m, Nc_cap);
  const int nsel = min(topk, nv);
  const float* srow = scores + (size_t)row * Nc_cap;
  int32_t* orow = idx_out + (size_t)row * topk;
  float* sorow = score_out ? score_out + (size_t)row * topk : nullptr;
  if (trivial_row(nsel, nv, topk, srow, orow, sorow)) return;
  uint32_t* gbm = def_bm + (size_t)row * bm_words;
  uint32_t* bm = BM_LDS ? lbm : gbm;
  const int nwords = (nv + 31) / 32;
  const int nch = (nv + kChunk - 1) / kChunk;  // chunks collect wrote (<= FIN_THREADS)
  uint32_t n_bits = 0;
  // eight words per thread in flight (clamped addresses)
  for (int w0 = 0; w0 < nwords; w0 += 8 * FIN_THREADS) {
    uint32_t xw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) xw[u] = gbm[min(w0 + u * FIN_THREADS + tid, nwords - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int w = w0 + u * FIN_THREADS + tid;
      if (w < nwords) {
        if (BM_LDS) lbm[w] = xw[u];
        n_bits += __popc(xw[u]);
      }
    }
  }
  const uint32_t cc = tid < nch ? chunk_cnt[(size_t)row * n_chunks + tid] : 0u;
  uint32_t n_def, n_cand;
  block_excl_scan(n_bits, sh, n_def);
  const uint32_t off = block_excl_scan(cc, sh, n_cand);
  coff[tid] = off;
  ccnt[tid] = cc;
  __syncthreads();
  const uint32_t need = (uint32_t)nsel - n_def;  // <= n_cand
  const bool in_lds = n_cand <= (uint32_t)kFinalCandLds;
  uint32_t* fkey = cand_flat + (size_t)row * Nc_cap * 2;
  uint32_t* fidx = fkey + Nc_cap;
  if (need > 0) {
    // gather the chunk segments: candidate i (of the flat list) lies in the
    // last chunk whose offset is <= i; four candidates per thread in flight
    const uint32_t* gci = cand_idx + (size_t)row * Nc_cap;
    const uint32_t* gck = cand_key + (size_t)row * Nc_cap;
    for (uint32_t i0 = 0; i0 < n_cand; i0 += 4 * FIN_THREADS) {
      uint32_t kv[4], jv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = min(i0 + u * FIN_THREADS + tid, n_cand - 1);
        int lo = 0, hi = nch - 1;  // coff[lo] <= i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (coff[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        const size_t at = (size_t)lo * kChunk + (i - coff[lo]);
        kv[u] = gck[at];
        jv[u] = gci[at];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = i0 + u * FIN_THREADS + tid;
        if (i < n_cand) {
          if (in_lds) {
            ckey[i] = kv[u];
            cidx[i] = jv[u];
          } else {
            fkey[i] = kv[u];
            fidx[i] = jv[u];
          }
        }
      }
    }
    __syncthreads();
    select_candidates([&](uint32_t i) -> uint32_t { return in_lds ? ckey[i] : fkey[i]; },
                      [&](uint32_t i) -> uint32_t { return in_lds ? cidx[i] : fidx[i]; },
                      n_cand, need, Nc_cap, bm, hist, sh);
  }
  __syncthreads();
  write_selection(
      [&](int w) -> uint32_t {
        return BM_LDS ? lbm[w]
                      : __hip_atomic_load(gbm + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      },
      nwords, srow, orow, sorow, sh);
}

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------- long rows: segments
// The long rows that the histogram path cannot take (bf16 prefill rows,
// whose score workgroups span 16 query rows, and packed sequences) are
// selected in segments: a workgroup of NT
// threads keeps the exact best min(topk, n) of up to 32 NT items.  Level 0
// takes segments of 8192 entries (256 threads, so that a row spreads over
// many compute units); merge levels select again among the candidates of
// several segments, P (a power of two >= topk) being the slot stride of a
// segment's candidates, until one group per row remains (the best topk of a
// row lie among the best topk of its segments); a merge workgroup has 256,
// 512 or 1024 threads, as its candidates need.  Thread t owns the 32 consecutive items [32 t, 32 t + 32):
// they are loaded coalesced into LDS and read back per thread, so that index
// order is thread order, then bit order.
// The k-th key is found by narrowing a key range [lo, lo + span]: each pass
// histograms (key - lo) >> shift over 2048 bins, shift chosen so that the
// range fits, for the items still in range (the first pass from registers,
// later ones through a per-thread bit mask), and keeps the bin holding the
// k-th key.  A final packed scan of the per-thread counts above and inside
// the range places the selection in ascending index order; keys inside the
// range (all equal once it is one key wide) are taken lowest index first.
// Every workgroup writes all it produces and nothing accumulates across
// workgroups, so no workspace starts at zero.
constexpr int LS_KPT = 32, LS_SEG = 256 * LS_KPT;  // level 0: 8192 entries
constexpr int LS_BINS = 2048;
constexpr int LS_GROUP_MAX = 64;  // input segments per merge workgroup

// visible entries of a query row
__device__ __forceinline__ int row_visible(int row, const int64_t* q_pos, const int32_t* n_cmp,
                                           int T, int Nc_cap, int m, Varlen vl) {
  if (vl.cu_q) {
    const int b = varlen_seq(vl, row);
    return n_visible(row - vl.cu_q[b], vl.cu_k[b + 1] - vl.cu_k[b], m, Nc_cap);
  }
  const int b = row / T;
  return n_visible(q_pos[b] + row % T, n_cmp[b], m, Nc_cap);
}

// LDS position of item q: the 16-byte chunk c of thread t's 32 items sits at
// chunk c ^ ((t >> 1) & 7), so that both the coalesced stores (64 consecutive
// items) and the per-thread 16-byte reads (16 threads) hit distinct banks
__device__ __forceinline__ int ls_phys(int q) {
  return (q & ~31) | ((((q >> 2) & 7) ^ ((q >> 6) & 7)) << 2) | (q & 3);
}

// inclusive prefix sum over the wave's lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// FROM_SCORES: level 0, grid (rows, segments); the items are the segment's
// visible entries.  Otherwise a merge level, grid (rows, ceil(n_in /
// group)); the items are the slots s P + i (i below the count of input
// segment s) of the workgroup's `group` input segments, in index order.  The
// last level (one workgroup per row) writes idx_out and score_out, -1 / NaN
// padded; the others write the candidates (key, entry) and their count.
template <int NT, bool FROM_SCORES>
__global__ void __launch_bounds__(NT) select_seg_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int T, int Nc_cap, int m, int topk, int p_log2, int n_in,
    int group, const uint32_t* __restrict__ in_key, const int32_t* __restrict__ in_idx,
    const int32_t* __restrict__ in_cnt, uint32_t* __restrict__ out_key,
    int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, Varlen vl) {
  constexpr int NW = NT / 64, ITEMS = NT * LS_KPT, BPT = LS_BINS / NT;  // bins per thread
  __shared__ __attribute__((aligned(16))) uint32_t keys_s[ITEMS];
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][LS_BINS];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[2][NW];
  __shared__ uint32_t res[4];
  __shared__ int32_t scnt[LS_GROUP_MAX];
  const int row = blockIdx.x, grp = blockIdx.y, n_out = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* srow = scores + (size_t)row * Nc_cap;
  const int P = 1 << p_log2;
  // level 0: entries seg0 + q, q < n_items; merge: slots q of the
  // candidates starting at in_base
  int n_items = 0, seg0 = 0;
  const size_t in_base = ((size_t)row * n_in + (size_t)grp * group) << p_log2;
  if constexpr (FROM_SCORES) {
    const int nv = row_visible(row, q_pos, n_cmp, T, Nc_cap, m, vl);
    seg0 = grp * ITEMS;
    n_items = min(max(nv - seg0, 0), ITEMS);
  } else {
    if (tid < group) {
      const int sg = grp * group + tid;
      scnt[tid] = sg < n_in ? in_cnt[(size_t)row * n_in + sg] : 0;
    }
    __syncthreads();
    for (int sg = 0; sg < group; ++sg) n_items += scnt[sg];
  }
  const int nsel = min(topk, n_items);
  const bool last = n_out == 1;
  int32_t* orow = idx_out + (size_t)row * topk;
  float* sorow = score_out ? score_out + (size_t)row * topk : nullptr;
  const size_t out_base = ((size_t)row * n_out + grp) << p_log2;
  if (last) {
    for (int k = nsel + tid; k < topk; k += NT) {
      orow[k] = -1;
      if (sorow) sorow[k] = __uint_as_float(0x7fc00000u);
    }
  } else if (tid == 0) {
    out_cnt[(size_t)row * n_out + grp] = nsel;
  }
  if (nsel == 0) return;  // uniform

  // whether item q exists
  auto item_ok = [&](int q) -> bool {
    if constexpr (FROM_SCORES) return q < n_items;
    const int sg = q >> p_log2;
    return sg < group && (q & (P - 1)) < scnt[min(sg, group - 1)];
  };
  // coalesced loads (all issued before the first is used; clamped
  // addresses) into LDS; both histogram buffers cleared meanwhile
  {
    uint32_t x[LS_KPT];
#pragma unroll
    for (int r = 0; r < LS_KPT; ++r) {
      const int q = r * NT + tid;
      if constexpr (FROM_SCORES) x[r] = score_key(srow[seg0 + min(q, n_items - 1)]);
      else x[r] = in_key[in_base + (item_ok(q) ? q : 0)];
    }
#pragma unroll
    for (int i = 0; i < BPT; i += 2) *(u32x2*)&hist[0][BPT * tid + i] = u32x2{0u, 0u};
#pragma unroll
    for (int r = 0; r < LS_KPT; ++r) keys_s[ls_phys(r * NT + tid)] = x[r];
  }
  __syncthreads();
  // this thread's items; invalid ones count as absent everywhere below
  uint32_t kr[LS_KPT];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4 v = *(const u32x4*)&keys_s[ls_phys(32 * tid + 4 * c)];
#pragma unroll
    for (int e = 0; e < 4; ++e) kr[4 * c + e] = v[e];
  }
  uint32_t vb;  // bit u: item 32 tid + u exists
  if constexpr (FROM_SCORES) {
    const int nmine = min(max(n_items - 32 * tid, 0), 32);
    vb = nmine >= 32 ? 0xffffffffu : ((1u << nmine) - 1u);
  } else {
    vb = 0u;
#pragma unroll
    for (int u = 0; u < LS_KPT; ++u) vb |= item_ok(32 * tid + u) ? 1u << u : 0u;
  }

  // the selected set: keys above lo + span, plus the `remaining` lowest-index
  // keys in [lo, lo + span] (all of them with all_in)
  uint32_t lo = 0u, span = 0xffffffffu, remaining = (uint32_t)nsel;
  bool all_in = nsel == n_items;  // every item: the full range holds them all
  if (!all_in) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int u = 0; u < LS_KPT; ++u) {
      const bool ok = (vb >> u) & 1u;
      kmin = min(kmin, ok ? kr[u] : 0xffffffffu);
      kmax = max(kmax, ok ? kr[u] : 0u);
    }
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    }
    if (lane == 0) {
      wsum[0][wave] = kmin;
      wsum[1][wave] = kmax;
    }
    __syncthreads();
    kmin = wsum[0][0];
    kmax = wsum[1][0];
    for (int w = 1; w < NW; ++w) {
      kmin = min(kmin, wsum[0][w]);
      kmax = max(kmax, wsum[1][w]);
    }
    lo = kmin;
    span = kmax - kmin;
    uint32_t mb = vb;  // items still in [lo, lo + span]
    for (int pass = 0; !all_in && span != 0u; ++pass) {
      uint32_t* h = hist[pass & 1];
      const int shift = max(0, (32 - __clz((int)span)) - 11);
      // (wsum and the other buffer: their last readers passed the barrier
      // that ended the previous pass)
      __syncthreads();
      if (pass == 0) {
#pragma unroll
        for (int u = 0; u < LS_KPT; ++u)
          if ((vb >> u) & 1u) atomicAdd(&h[(kr[u] - lo) >> shift], 1u);
      } else {
        for (uint32_t bits = mb; bits; bits &= bits - 1u) {
          const int u = __builtin_ctz(bits);
          atomicAdd(&h[(keys_s[ls_phys(32 * tid + u)] - lo) >> shift], 1u);
        }
      }
      __syncthreads();
      // thread t owns the BPT bins below 2048 - BPT t (top bins first);
      // clear the other buffer for the next pass
      uint32_t cb[BPT], csum = 0u;
#pragma unroll
      for (int i = 0; i < BPT; i += 2) {
        const u32x2 v = *(const u32x2*)&h[LS_BINS - BPT * (tid + 1) + i];
        cb[i] = v[0];
        cb[i + 1] = v[1];
        csum += v[0] + v[1];
        *(u32x2*)&hist[(pass + 1) & 1][BPT * tid + i] = u32x2{0u, 0u};
      }
      const uint32_t incl = wave_incl_scan(csum);
      if (lane == 63) wsum[0][wave] = incl;
      __syncthreads();
      uint32_t above_w = 0u;
      for (int w = 0; w < wave; ++w) above_w += wsum[0][w];
      const uint32_t above = above_w + incl - csum;
      if (above < remaining && above + csum >= remaining) {
        // cb[BPT - 1] is this thread's top bin
        uint32_t acc = above;
        for (int i = BPT - 1; i >= 0; --i) {
          if (acc + cb[i] >= remaining) {
            res[0] = (uint32_t)(LS_BINS - BPT * (tid + 1) + i);
            res[1] = acc;
            res[2] = cb[i];
            break;
          }
          acc += cb[i];
        }
      }
      __syncthreads();
      const uint32_t d = res[0], cum = res[1], cnt = res[2];
      remaining -= cum;
      const uint32_t d_lo = d << shift;
      lo += d_lo;
      span = min(span - d_lo, (1u << shift) - 1u);
      if (cnt == remaining) all_in = true;
      // keep the items of the bin
      if (pass == 0) {
        uint32_t nm = 0u;
#pragma unroll
        for (int u = 0; u < LS_KPT; ++u)
          nm |= (((vb >> u) & 1u) && ((kr[u] - (lo - d_lo)) >> shift) == d) ? 1u << u : 0u;
        mb = nm;
      } else {
        for (uint32_t bits = mb; bits; bits &= bits - 1u) {
          const int u = __builtin_ctz(bits);
          if (keys_s[ls_phys(32 * tid + u)] - lo > span) mb &= ~(1u << u);
        }
      }
    }
  }

  // this thread's keys above and inside the range; one packed scan gives
  // the counts before it (ties are taken in index order, so the taken ones
  // before a thread number min(remaining, ties before it))
  uint32_t gtb = 0u, inb = 0u;
  const uint32_t hi_key = lo + span;
#pragma unroll
  for (int u = 0; u < LS_KPT; ++u) {
    const bool ok = (vb >> u) & 1u;
    gtb |= (ok && kr[u] > hi_key) ? 1u << u : 0u;
    inb |= (ok && kr[u] >= lo && kr[u] <= hi_key) ? 1u << u : 0u;
  }
  const uint32_t packed = ((uint32_t)__popc(gtb) << 16) | (uint32_t)__popc(inb);
  const uint32_t incl = wave_incl_scan(packed);
  __syncthreads();  // the last pass's readers of wsum are done
  if (lane == 63) wsum[1][wave] = incl;
  __syncthreads();
  uint32_t before = incl - packed;
  for (int w = 0; w < wave; ++w) before += wsum[1][w];
  const uint32_t gt_before = before >> 16, in_before = before & 0xffffu;
  // one branch-free form for both cases: with all_in every key in range is
  // taken (an unbounded limit), else the first `remaining` of them
  const uint32_t lim = all_in ? 0xffffffffu : remaining;
  // (the headroom as max - in_before: a guarded lim - in_before has let the
  // optimizer assume lim >= in_before and drop the min below)
  uint32_t take = min((uint32_t)__popc(inb), max(lim, in_before) - in_before);
  uint32_t selb = gtb;
  for (uint32_t bits = inb; take; --take) {
    const uint32_t low = bits & (0u - bits);
    selb |= low;
    bits ^= low;
  }
  uint32_t at = gt_before + min(in_before, lim);
  for (uint32_t bits = selb; bits; bits &= bits - 1u, ++at) {
    // (the selection holds exactly nsel items; the bound is a guard)
    if (at >= (uint32_t)nsel) break;
    const int q = 32 * tid + __builtin_ctz(bits);
    const int j = FROM_SCORES ? seg0 + q : in_idx[in_base + q];
    if (last) {
      orow[at] = j;
      if (sorow && (uint32_t)j < (uint32_t)Nc_cap) sorow[at] = srow[j];
    } else {
      out_key[out_base + at] = keys_s[ls_phys(q)];
      out_idx[out_base + at] = j;
    }
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct IdxLayout {
  bool long_rows, bm_lds;
  int n_chunks, bm_words;
  size_t scores, hist, chunk_cnt, def_bm, cand_idx, cand_key, cand_flat, total;
  // segment path: segments of LS_SEG entries, candidate slot stride
  // 2^p_log2, two candidate buffers (keys, entries, counts)
  int n_seg, p_log2;
  size_t seg_cand[2];
};

// The two long-row paths use the space after the scores in turn: its size
// is the larger of theirs.
static IdxLayout idx_layout(int B, int T, int Nc_cap, int topk) {
  IdxLayout L{};
  const size_t rows = (size_t)B * T;
  L.long_rows = Nc_cap > kShortMax;
  L.bm_lds = Nc_cap <= kBitmapLds * 32;
  L.n_chunks = (Nc_cap + kChunk - 1) / kChunk;
  L.bm_words = 2 * ((Nc_cap + 63) / 64);  // even: collect stores word pairs
  L.n_seg = (Nc_cap + LS_SEG - 1) / LS_SEG;
  while ((1 << L.p_log2) < topk) ++L.p_log2;
  size_t off = 0;
  L.scores = off;
  off += align256(rows * (size_t)Nc_cap * 4);
  if (L.long_rows) {
    const size_t base = off;
    L.hist = off;  // the only part that must start at zero
    off += align256(rows * kHistBins * 4);
    L.chunk_cnt = off;
    off += align256(rows * (size_t)L.n_chunks * 4);
    L.def_bm = off;
    off += align256(rows * (size_t)L.bm_words * 4);
    L.cand_idx = off;
    off += align256(rows * (size_t)Nc_cap * 4);
    L.cand_key = off;
    off += align256(rows * (size_t)Nc_cap * 4);
    L.cand_flat = off;
    off += align256(rows * (size_t)Nc_cap * 8);
    size_t off2 = base;
    const size_t slots = rows * (size_t)L.n_seg << L.p_log2;
    for (int k = 0; k < 2; ++k) {
      L.seg_cand[k] = off2;
      off2 += align256(slots * 8 + rows * (size_t)L.n_seg * 4);
    }
    off = std::max(off, off2);
  }
  L.total = off;
  return L;
}

size_t indexer_ws_bytes(int B, int T, int H_I, int d_I, int Nc_cap, int topk, csa_dtype_t dt) {
  (void)H_I;
  (void)d_I;
  (void)dt;
  return idx_layout(B, T, Nc_cap, topk).total;
}

hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t st) {
  // packed sequences: one row per query token of every sequence
  const int rows = a.vl.cu_q ? a.total_rows : a.B * a.T;
  const IdxLayout L = idx_layout(1, rows, a.Nc_cap, a.topk);
  char* ws = (char*)a.ws;
  float* scores = (float*)(ws + L.scores);
  // long rows: the histogram path when each score workgroup owns one query
  // row of one sequence, else the segment path
  const bool seg_path = L.long_rows && (a.vl.cu_q || (a.dt == CSA_DT_BF16 && a.T != 1));
  const bool hist_path = L.long_rows && !seg_path;
  uint32_t* hist = hist_path ? (uint32_t*)(ws + L.hist) : nullptr;
  if (hist_path) {
    size_t n = (size_t)rows * kHistBins;
    zero_u32_kernel<<<(unsigned)std::min<size_t>((n + 255) / 256, 1024), 256, 0, st>>>(hist, n);
  }
  if (a.Nc_cap == 0) {
    // no entry exists: every output row is padding
  } else if (a.dt == CSA_DT_F32) {
    dim3 g((a.Nc_cap + 255) / 256, rows);
    if (hist_path)
      score_f32_kernel<true><<<g, 256, 0, st>>>((const float*)a.q_idx, a.w_idx,
                                                (const float*)a.k_idx, a.q_pos, a.n_cmp, a.T,
                                                a.H_I, a.d_I, a.Nc_cap, a.m, scores, hist, a.vl);
    else
      score_f32_kernel<false><<<g, 256, 0, st>>>((const float*)a.q_idx, a.w_idx,
                                                 (const float*)a.k_idx, a.q_pos, a.n_cmp, a.T,
                                                 a.H_I, a.d_I, a.Nc_cap, a.m, scores, hist, a.vl);
  } else if (a.dt == CSA_DT_BF16) {
    // long rows need one histogram per row: one row per workgroup then;
    // short rows split their entries in chunks of 512 so that the causal
    // growth of the visible range spreads over more, smaller workgroups
    const int key_chunk = hist_path ? kChunk : std::min(a.Nc_cap, 512);
    dim3 g((a.T + SB_ROWS - 1) / SB_ROWS, (a.Nc_cap + key_chunk - 1) / key_chunk, a.B);
#define CSA_LAUNCH_SB(HS)                                                                     \
  if (a.pages.block_table)                                                                    \
    score_bf16_kernel<HS, true><<<g, 256, 0, st>>>(                                           \
        (const uint16_t*)a.q_idx, a.w_idx, (const uint16_t*)a.k_idx, a.q_pos, a.n_cmp, a.T,   \
        a.Nc_cap, a.m, key_chunk, scores, hist, a.pages, a.vl);                                \
  else                                                                                        \
    score_bf16_kernel<HS, false><<<g, 256, 0, st>>>(                                          \
        (const uint16_t*)a.q_idx, a.w_idx, (const uint16_t*)a.k_idx, a.q_pos, a.n_cmp, a.T,   \
        a.Nc_cap, a.m, key_chunk, scores, hist, a.pages, a.vl)
    if (hist_path) {
      CSA_LAUNCH_SB(true);  // (T == 1: the workgroup's rows share the histogram)
    } else {
      CSA_LAUNCH_SB(false);
    }
#undef CSA_LAUNCH_SB
  } else {
    dim3 g((a.Nc_cap + kChunk - 1) / kChunk, rows);
#define CSA_LAUNCH_SF(HS, QK)                                                                 \
  if (a.pages.block_table)                                                                    \
    score_fp8_kernel<HS, QK, true><<<g, 256, 0, st>>>(                                        \
        (const uint8_t*)a.q_idx, a.q_scale, a.w_idx, (const uint8_t*)a.k_idx, a.k_scale,      \
        a.q_pos, a.n_cmp, a.T, a.Nc_cap, a.m, scores, hist, a.pages);                         \
  else                                                                                        \
    score_fp8_kernel<HS, QK, false><<<g, 256, 0, st>>>(                                       \
        (const uint8_t*)a.q_idx, a.q_scale, a.w_idx, (const uint8_t*)a.k_idx, a.k_scale,      \
        a.q_pos, a.n_cmp, a.T, a.Nc_cap, a.m, scores, hist, a.pages)
    if (a.dt == CSA_DT_MXFP4) {
      if (hist_path) {
        CSA_LAUNCH_SF(true, CSA_DT_MXFP4);
      } else {
        CSA_LAUNCH_SF(false, CSA_DT_MXFP4);
      }
    } else {
      if (hist_path) {
        CSA_LAUNCH_SF(true, CSA_DT_FP8E4M3);
      } else {
        CSA_LAUNCH_SF(false, CSA_DT_FP8E4M3);
      }
    }
#undef CSA_LAUNCH_SF
  }
  if (!L.long_rows) {
    const unsigned g = (unsigned)((rows + 3) / 4);
    if (a.Nc_cap <= 2048)
      select_short_kernel<2048><<<g, 256, 0, st>>>(scores, a.q_pos, a.n_cmp, rows, a.T, a.Nc_cap,
                                                   a.m, a.topk, a.idx_out, a.score_out, a.vl);
    else
      select_short_kernel<kShortMax><<<g, 256, 0, st>>>(scores, a.q_pos, a.n_cmp, rows, a.T,
                                                        a.Nc_cap, a.m, a.topk, a.idx_out,
                                                        a.score_out, a.vl);
  } else if (seg_path) {
    // level 0 over segments of LS_SEG entries, then merge levels until one
    // workgroup per row remains
    const size_t slots = (size_t)rows * L.n_seg << L.p_log2;
    uint32_t* ck[2];
    int32_t *ci[2], *cc[2];
    for (int k = 0; k < 2; ++k) {
      ck[k] = (uint32_t*)(ws + L.seg_cand[k]);
      ci[k] = (int32_t*)(ck[k] + slots);
      cc[k] = ci[k] + slots;
    }
    select_seg_kernel<256, true><<<dim3(rows, L.n_seg), 256, 0, st>>>(
        scores, a.q_pos, a.n_cmp, a.T, a.Nc_cap, a.m, a.topk, L.p_log2, 1, 1, nullptr, nullptr,
        nullptr, ck[0], ci[0], cc[0], a.idx_out, a.score_out, a.vl);
    // each merge level: one workgroup per row when the candidates fit 32768
    // slots (with the thread count they need), else groups of at least four
    // segments
    int n_in = L.n_seg, cur = 0;
    while (n_in > 1) {
      const long slots_in = (long)n_in << L.p_log2;
      const int nt = slots_in <= 8192    ? 256
                     : slots_in <= 16384 ? 512
                     : slots_in <= 32768 ? 1024
                                         : std::max(256, (4 << L.p_log2) / LS_KPT);
      const int group = std::min(LS_GROUP_MAX, (nt * LS_KPT) >> L.p_log2);
      const int n_out = (n_in + group - 1) / group;
#define CSA_LAUNCH_MERGE(NT_)                                                                 \
  select_seg_kernel<NT_, false><<<dim3(rows, n_out), NT_, 0, st>>>(                          \
      scores, a.q_pos, a.n_cmp, a.T, a.Nc_cap, a.m, a.topk, L.p_log2, n_in, group, ck[cur],  \
      ci[cur], cc[cur], ck[cur ^ 1], ci[cur ^ 1], cc[cur ^ 1], a.idx_out, a.score_out, a.vl)
      if (nt == 256) CSA_LAUNCH_MERGE(256);
      else if (nt == 512) CSA_LAUNCH_MERGE(512);
      else CSA_LAUNCH_MERGE(1024);
#undef CSA_LAUNCH_MERGE
      n_in = n_out;
      cur ^= 1;
    }
  } else {
    uint32_t* cnt = (uint32_t*)(ws + L.chunk_cnt);
    uint32_t* bm = (uint32_t*)(ws + L.def_bm);
    uint32_t* ci = (uint32_t*)(ws + L.cand_idx);
    uint32_t* ck = (uint32_t*)(ws + L.cand_key);
    uint32_t* cf = (uint32_t*)(ws + L.cand_flat);
    collect_kernel<<<dim3(L.n_chunks, rows), 256, 0, st>>>(scores, hist, a.q_pos, a.n_cmp, a.T,
                                                           a.Nc_cap, a.m, a.topk, L.n_chunks,
                                                           L.bm_words, bm, cnt, ci, ck);
    if (L.bm_lds)
      finalize_kernel<true><<<rows, FIN_THREADS, 0, st>>>(scores, a.q_pos, a.n_cmp, a.T, a.Nc_cap,
                                                          a.m, a.topk, L.n_chunks, L.bm_words, bm,
                                                          cnt, ci, ck, cf, a.idx_out, a.score_out);
    else
      finalize_kernel<false><<<rows, FIN_THREADS, 0, st>>>(scores, a.q_pos, a.n_cmp, a.T,
                                                           a.Nc_cap, a.m, a.topk, L.n_chunks,
                                                           L.bm_words, bm, cnt, ci, ck, cf,
                                                           a.idx_out, a.score_out);
  }
  return hipGetLastError();
}

}  // namespace csa_host
