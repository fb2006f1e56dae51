// Sparse / dense MQA attention over compressed entries plus the raw sliding
// window, for gfx950.
//
// DS-V4 analysis section 1.2 (attend to the k selected compressed entries and
// the sliding-window KV), section 1.4 (HCA: every compressed entry), Notion
// copy section 1.1 (softmax(q K^T / sqrt(d)) V) and the MQA remark there (one
// KV head shared by every query head).
//
// Key list of a query row (b, t) at position pos: first the compressed part
// (CSA: the topk slots of idx; HCA: entries 0 .. n_vis - 1), then the raw
// tokens max(0, pos - W + 1) .. pos.  Invalid slots are masked.  One softmax
// runs over the whole list.
//
// Two bf16 kernels share the tile arithmetic (S^T = K Q^T and O^T += V^T P^T
// on MFMA with online softmax, V^T from the LDS transpose read):
//  * prefill (many rows): one row per wave, all heads per wave, key ranges
//    common to neighbouring rows shared through LDS;
//  * decode (few rows): the waves of a workgroup split the heads of one row,
//    split-K across workgroups, partials merged by log-sum-exp in a combine
//    kernel.
// fp32 runs a plain per-(row, head) wave kernel.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace csa {


struct KeyList {
  int n_c;       // compressed positions (topk slots or n_vis)
  int64_t lo;    // first window token
  int n_w;       // window tokens
};

__device__ __forceinline__ KeyList key_list(bool dense, int topk, int window, int64_t pos,
                                            int32_t ncmp, int m, int Nc_cap) {
  KeyList L;
  L.n_c = dense ? n_visible(pos, ncmp, m, Nc_cap) : topk;
  if (window > 0 && pos >= 0) {
    L.lo = pos - window + 1;
    if (L.lo < 0) L.lo = 0;
    L.n_w = (int)(pos - L.lo + 1);
  } else {
    L.lo = 0;
    L.n_w = 0;
  }
  return L;
}

// Source row of list position p (nullptr if the slot is empty).  With a
// block table (cmp_pt for the dense form's entries, raw_pt for the window),
// the row is found in the pool, and a row of an absent page is empty.
template <typename Tp>
__device__ __forceinline__ const Tp* key_row(int p, const KeyList& L, bool dense,
                                             const int32_t* idx_row, const Tp* kv_cmp_b,
                                             int Nc_cap, const Tp* kv_raw_b, int R_cap,
                                             int64_t raw_base, int row_elems, int b,
                                             const PageTable& cmp_pt, const PageTable& raw_pt) {
  if (p < L.n_c) {
    int64_t j = dense ? p : idx_row[p];
    if (j < 0 || j >= Nc_cap) return nullptr;
    if (dense && cmp_pt.block_table) j = paged_row(cmp_pt, b, (int)j);
    if (j < 0) return nullptr;
    return kv_cmp_b + (size_t)j * row_elems;
  }
  int64_t r = L.lo + (p - L.n_c) - raw_base;
  if (r < 0 || r >= R_cap) return nullptr;
  if (raw_pt.block_table) r = paged_row(raw_pt, b, (int)r);
  if (r < 0) return nullptr;
  return kv_raw_b + (size_t)r * row_elems;
}

typedef __attribute__((ext_vector_type(4))) short s16x4;

// LDS transpose read: lane i of each 16-lane group receives element i % 4 of
// the 8-byte chunks whose addresses lanes i/4 + 4 v (v = 0..3) supplied.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// Final normalisation of one (row, head) softmax from its running maximum m
// (log2 units of the scaled logits) and sum l, with the head's sink logit
// (natural-log units, one more term with no value) when sink is given and
// the head's entry is finite: inv multiplies the numerator accumulated
// relative to m; lse is the natural-log sum.
__device__ __forceinline__ void finish_softmax(float m, float l, const float* sink, int h,
                                               float& inv, float& lse_out) {
  const float z = sink ? sink[h] * kLog2e : -INFINITY;
  if (z > -INFINITY) {
    const float mn = fmaxf(m, z);
    const float c = m == -INFINITY ? 0.0f : exp2f(m - mn);
    const float lt = l * c + exp2f(z - mn);
    inv = c / lt;
    lse_out = (mn + __log2f(lt)) * kLn2;
  } else {
    inv = l > 0.0f ? 1.0f / l : 0.0f;
    lse_out = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- bf16 prefill
// Many query rows: a workgroup owns PF_ROWS consecutive rows of one sequence;
// each row has H/32 waves, one per 32-head slice (8 waves for H = 64, two per
// SIMD, so one wave's softmax overlaps another's MFMAs).
//  * phase A - key ranges shared by the rows (HCA: the compressed entries;
//    always: the union of the rows' windows) go through LDS once per
//    workgroup (double-buffered, one barrier per tile); each wave masks keys
//    outside its own row's visibility;
//  * phase B - CSA only: each row's selected compressed rows are gathered into
//    that row's own pair of LDS tiles by the row's waves (the index row is
//    staged first).
// Tiles move from global memory straight into LDS (global_load_lds_dwordx4:
// lane l of one instruction writes the 16 bytes at instruction base + 16 l),
// two 512-byte [K | V] rows per instruction, with no register staging and no
// LDS store instructions; one barrier per tile publishes a tile and frees the
// other buffer.  Rows are 512 bytes apart in a tile and the 16-byte chunk c
// of row r sits at slot c ^ pf_swz(r): 16 consecutive rows read at one chunk
// by the K fragment loads, and 4 rows read by the V transpose loads, fall in
// distinct bank groups.  The loader places a chunk by choosing, per lane, the
// global chunk that belongs in that lane's slot.
// Per wave and 32-key tile: S^T (32 keys x 32 heads) = K Q^T in 8 MFMA
// 32x32x16 and O^T (128 dims x 32 heads) += V^T P^T in 8 more; the S^T
// accumulator is the P^T operand once the second product's k order is
// permuted to match, and V^T fragments come from the LDS transpose read.
// Every tile load is issued unconditionally (empty slots read a valid dummy
// row and are masked).  The running maximum is only raised when a tile
// exceeds it by more than 2^8 (the final normalisation makes the result
// independent of the maximum used).
constexpr int PF_KT = 32;
constexpr int PF_ROWB = 512;                // bytes of one [K | V] row
constexpr int PF_TILEB = PF_KT * PF_ROWB;   // 16 KB per tile
constexpr int PF_IDX_MAX = 1024;            // index slots per row staged in LDS
constexpr float PF_RESCALE = 8.0f;          // log2 headroom before the maximum is raised

// chunk slot permutation of tile row r (an involution on the 16 chunks of
// either half of the row)
__device__ __forceinline__ int pf_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// H = 32 NH; PF_ROWS query rows per workgroup; SPARSE: CSA (top-k entries +
// window) rather than HCA (every visible entry + window).  Two waves per
// SIMD: the register budget is held to 256 so that a second workgroup hides
// the first one's load and barrier latency.
// PG: paged window rows (raw_pt) and, for HCA, paged compressed entries
// (cmp_pt): a shared-segment row is found through its sequence's block
// table, and rows of absent pages are masked.
template <int NH, int PF_ROWS, bool SPARSE, bool PG>
__global__ void __launch_bounds__(64 * PF_ROWS * NH, 2) attn_pf_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv_cmp,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw,
    const int64_t* __restrict__ q_pos, const int32_t* __restrict__ n_cmp,
    const int64_t* __restrict__ raw_base, int T, int topk, int window, int m, int Nc_cap,
    int R_cap, float scale_log2, const float* __restrict__ sink, uint16_t* __restrict__ out,
    float* __restrict__ lse, int64_t cmp_rows_b, Varlen vl, PageTable cmp_pt, PageTable raw_pt) {
  constexpr int H = 32 * NH, D = 128, NT = 64 * PF_ROWS * NH, NW = NT / 64;
  constexpr bool dense = !SPARSE;
  // phase A: tiles tile0[0] and tile1[0] (shared); phase B: row r's tiles
  // tile0[r] and tile1[r].  The two buffers are distinct variables so that the
  // compiler can tell reads of one from the loads in flight into the other
  // (otherwise it waits for every load before any read of the tile memory).
  constexpr int NROWBUF = SPARSE ? PF_ROWS : 1;
  static_assert(16 % NW == 0 && 16 % NH == 0, "a tile is 16 two-row load instructions");
  __shared__ __attribute__((aligned(16))) uint8_t tile0[NROWBUF][PF_TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[NROWBUF][PF_TILEB];
  __shared__ __attribute__((aligned(16))) int idx_all[SPARSE ? PF_ROWS : 1][SPARSE ? PF_IDX_MAX : 1];
  // paged shared segments: whether each row of the two tile buffers exists
  __shared__ int rowok[PG ? 2 : 1][PG ? PF_KT : 1];
  // the wave index is a scalar so that every per-wave decision below is a
  // uniform branch
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_w = wave / NH, hh = wave % NH;     // query row and 32-head slice
  const int h2 = lane >> 5, l32 = lane & 31;

  const int tiles_per_b = (T + PF_ROWS - 1) / PF_ROWS;
  const int b = blockIdx.x / tiles_per_b;
  const int t0 = (blockIdx.x % tiles_per_b) * PF_ROWS;
  // the sequence's rows, compressed entries and raw rows (packed sequences:
  // offsets into the packed tensors, the raw rows being the sequence's own
  // tokens from position 0; T is then the longest sequence)
  size_t qrow0 = (size_t)b * T;
  // (a paged segment addresses its shared pool: no per-sequence offset; the
  // host passes cmp_rows_b = 0 for a paged compressed cache)
  const uint16_t* kvc_b = kv_cmp + (size_t)b * cmp_rows_b * 2 * D;
  const uint16_t* kvr_b = kv_raw + (PG && raw_pt.block_table ? 0 : (size_t)b * R_cap * 2 * D);
  if (vl.cu_q) {
    qrow0 = (size_t)vl.cu_q[b];
    T = vl.cu_q[b + 1] - vl.cu_q[b];
    R_cap = T;
    kvc_b = kv_cmp + (size_t)vl.cu_k[b] * 2 * D;
    kvr_b = kv_raw + qrow0 * 2 * D;
    Nc_cap = vl.cu_k[b + 1] - vl.cu_k[b];
    if (t0 >= T) return;  // uniform, before any barrier
  }
  const int t = t0 + row_w;
  const bool active = t < T;
  const int t_last = min(T - 1, t0 + PF_ROWS - 1);
  const int64_t qp = vl.cu_q ? 0 : q_pos[b];
  const int64_t pos = qp + t, pos_first = qp + t0, pos_last = qp + t_last;
  const int32_t ncb = vl.cu_q ? Nc_cap : (n_cmp ? n_cmp[b] : 0);
  const int64_t rbase = vl.cu_q ? 0 : raw_base[b];
  const size_t rowi = qrow0 + (active ? t : t_last);

  // this row's visibility
  const int nv_me = dense ? n_visible(pos, ncb, m, Nc_cap) : 0;
  const int64_t w_lo = window > 0 ? (pos - window + 1 < 0 ? 0 : pos - window + 1) : 1;
  const int64_t w_hi = window > 0 ? pos : 0;   // window empty when w_lo > w_hi

  // Q^T operand: head 32 hh + l32, dims 16 s + 8 h2 .. + 8
  bf16x8 qf[8];
  {
    const uint16_t* qr = q + (rowi * H + 32 * hh + l32) * D + 8 * h2;
    for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(qr + 16 * s);
  }
  f32x16 o[4];
  for (int dt = 0; dt < 4; ++dt)
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float mrun = -INFINITY, lrun = 0.0f;

  // byte offsets of this lane's fragments inside a tile: K fragment s is key
  // row l32, chunk 2 s + h2 (dims 16 s + 8 h2 ..); the transpose reads of V
  // take key row 4 (g / 2) + j / 4 (+ 8 for the second read, + 16 per k
  // step), dims 32 dt + 16 (g & 1) + 4 (j & 3), for lane j of 16-lane group g
  const int gg = lane >> 4, jj = lane & 15;
  uint32_t kofs[8], vofs[4][2];
  {
    const int fk = pf_swz(l32);
#pragma unroll
    for (int s = 0; s < 8; ++s) kofs[s] = (uint32_t)(l32 * PF_ROWB + 16 * ((2 * s + h2) ^ fk));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * (gg >> 1) + (jj >> 2) + 8 * e;
      const int fr = pf_swz(r);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int c = 16 + 4 * dt + 2 * (gg & 1) + ((jj & 3) >> 1);
        vofs[dt][e] = (uint32_t)(r * PF_ROWB + 16 * (c ^ fr) + 8 * (jj & 1));
      }
    }
  }
  // phase base: the fragment offsets then point into buffer 0 of the phase
  auto rebase = [&](uint32_t base) {
#pragma unroll
    for (int s = 0; s < 8; ++s) kofs[s] += base;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      vofs[dt][0] += base;
      vofs[dt][1] += base;
    }
  };

  // One tile in the phase's buffer BUF; vmask bit k: key k attended.
  auto compute = [&](auto buf_tag, uint32_t vmask) {
    const uint8_t* const tb = decltype(buf_tag)::value ? &tile1[0][0] : &tile0[0][0];
    f32x16 sacc;
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
    // all eight K fragments are read before the products start, so that one
    // LDS latency is exposed per tile instead of one per pair
    bf16x8 kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = *(const bf16x8*)(tb + kofs[s]);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // keys of register r: 8 (r/4) + 4 h2 + r%4; partial tiles mask, full
    // tiles skip the per-key work; the scale (> 0) is applied inside the FMA
    if (vmask != 0xffffffffu) {
      // one per-lane shift, then constant bit positions
      const uint32_t mv = vmask >> (4 * h2);
      for (int r = 0; r < 16; ++r)
        if (!((mv >> (8 * (r >> 2) + (r & 3))) & 1u)) sacc[r] = -INFINITY;
    }
    float x = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
    for (int r = 3; r < 15; r += 2) x = fmaxf(fmaxf(x, sacc[r]), sacc[r + 1]);
    x = fmaxf(x, sacc[15]);
    x = max_xor32(x) * scale_log2;
    const bool up = x > mrun + PF_RESCALE;
    if (__ballot(up)) {
      const float corr = up ? __builtin_amdgcn_exp2f(mrun - x) : 1.0f;
      if (up) mrun = x;
      lrun *= corr;
      for (int dt = 0; dt < 4; ++dt)
        for (int r = 0; r < 16; ++r) o[dt][r] *= corr;
    }
    const float nmuse = mrun == -INFINITY ? 0.0f : -mrun;
    float ps = 0.0f;
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], scale_log2, nmuse));
      ps += pv;
      sacc[r] = pv;
    }
    ps = sum_xor32(ps);
    lrun += ps;
    bf16x8 pf[2];
    for (int ks = 0; ks < 2; ++ks)
      for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)sacc[8 * ks + e];
    for (int ks = 0; ks < 2; ++ks)
      for (int dt = 0; dt < 4; ++dt) {
        const uint32_t ko = (uint32_t)ks * 16 * PF_ROWB;
        const u32x2 v1 = __builtin_bit_cast(u32x2, lds_read_tr16((const uint16_t*)(tb + vofs[dt][0] + ko)));
        const u32x2 v2 = __builtin_bit_cast(u32x2, lds_read_tr16((const uint16_t*)(tb + vofs[dt][1] + ko)));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{v1[0], v1[1], v2[0], v2[1]});
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[dt], 0, 0, 0);
      }
  };
  // the loads of a tile (global_load_lds) complete before the barrier that
  // publishes it
  auto wait_loads = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // one two-row load instruction: tile rows 2 i, 2 i + 1 (lane halves) into
  // the LDS tile at `dst`; the lane's global row byte offset is `roff`
  auto dma = [&](uint8_t* dst, int i, const char* base, uint32_t roff) {
    const int r = 2 * i + h2;
    const uint32_t c = (uint32_t)(l32 ^ pf_swz(r));  // the chunk that belongs in this slot
    __builtin_amdgcn_global_load_lds((const void*)(base + roff + 16u * c),
                                     (__attribute__((address_space(3))) void*)(dst + 1024 * i),
                                     16, 0, 0);
  };

  // ---------------- phase A: shared contiguous segments
  // segment 0 (HCA): entries [0, nv_max); segment 1: window tokens
  // [win_first, pos_last]
  const int nv_max = dense ? n_visible(pos_last, ncb, m, Nc_cap) : 0;
  int64_t win_first = pos_first - window + 1;
  if (win_first < 0) win_first = 0;
  // (no window tile without a raw cache: none of its tokens could be present)
  const int n_win = window > 0 && R_cap > 0 ? (int)(pos_last - win_first + 1) : 0;
  const int tiles0 = (nv_max + PF_KT - 1) / PF_KT;
  const int tiles1 = (n_win + PF_KT - 1) / PF_KT;
  const int ntA = tiles0 + tiles1;
  // cache row of window key 0, clamped into the int range (rows outside
  // [0, R_cap) are skipped either way)
  const int64_t rw0_64 = win_first - rbase;
  const int rw0 = (int)(rw0_64 < -(1 << 30) ? -(1 << 30) : (rw0_64 > (1 << 30) ? (1 << 30) : rw0_64));
  // Key kk of a segment is cache row row0 + kk; it is loaded when kk < kk_lim
  // and the row is below row_lim, else row 0 of the same cache stands in (a
  // segment has tiles only when its cache has rows).  Byte offsets fit in 32
  // bits: caches hold at most 2^23 rows of 512 bytes.  Paged: the row's pool
  // row, pool row 0 standing in for an absent page.  Wave w issues the
  // instructions w, w + NW, ... of the tile.
  // the lane's byte offset inside a tile's rows for each of the wave's load
  // instructions (instruction i: rows 2 i, 2 i + 1; the lane's chunk)
  uint32_t doff[16 / NW];
#pragma unroll
  for (int k = 0; k < 16 / NW; ++k) {
    const int r = 2 * (wave + NW * k) + h2;
    doff[k] = (uint32_t)(r * PF_ROWB + 16 * (l32 ^ pf_swz(r)));
  }
  auto issueA = [&](int ti, auto buf_tag) {
    constexpr int buf = decltype(buf_tag)::value;
    uint8_t* const dst = buf ? &tile1[0][0] : &tile0[0][0];
    const bool seg0 = ti < tiles0;  // uniform
    const char* base = (const char*)(seg0 ? kvc_b : kvr_b);
    const int kk0 = (seg0 ? ti : ti - tiles0) * PF_KT;
    const int kk_lim = seg0 ? nv_max : n_win;
    const int row0 = seg0 ? kk0 : rw0 + kk0;
    const uint32_t row_lim = (uint32_t)(seg0 ? Nc_cap : R_cap);
    if (!PG && kk0 + PF_KT <= kk_lim && row0 >= 0 && (uint32_t)row0 + PF_KT <= row_lim) {
      // (uniform) every row of the tile exists: one scalar base per tile
      const char* tb = base + (size_t)(uint32_t)row0 * PF_ROWB;
#pragma unroll
      for (int k = 0; k < 16 / NW; ++k) {
        const int i = wave + NW * k;
        __builtin_amdgcn_global_load_lds((const void*)(tb + doff[k]),
                                         (__attribute__((address_space(3))) void*)(dst + 1024 * i),
                                         16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < 16 / NW; ++k) {
      const int i = wave + NW * k;
      const int rr = 2 * i + h2;
      const int row = row0 + rr;
      bool ok = (kk0 + rr < kk_lim) & ((uint32_t)row < row_lim);
      int prow = row;
      if constexpr (PG) {
        const PageTable& spt = seg0 ? cmp_pt : raw_pt;
        if (spt.block_table) {  // uniform: this segment's cache is paged
          const int64_t pr = ok ? paged_row(spt, b, row) : -1;
          ok = pr >= 0;
          prow = (int)pr;
        }
        if (l32 == 0) rowok[buf][rr] = ok;
      }
      dma(dst, i, base, (uint32_t)(ok ? prow : 0) * (uint32_t)PF_ROWB);
    }
  };
  // this wave's mask over tile ti's 32 keys (key = lane & 31)
  auto maskA = [&](int ti, int buf) -> uint32_t {
    bool ok;
    if (ti < tiles0) {
      if (!PG && (ti + 1) * PF_KT <= nv_me) return 0xffffffffu;  // (uniform)
      ok = ti * PF_KT + l32 < nv_me;
    } else {
      const int64_t tok0 = win_first + (int64_t)(ti - tiles0) * PF_KT;
      if (!PG && tok0 >= w_lo && tok0 + PF_KT - 1 <= w_hi && tok0 - rbase >= 0 &&
          tok0 - rbase + PF_KT <= R_cap)
        return 0xffffffffu;  // (uniform) every key of the tile is in the row's window
      const int64_t tok = win_first + (int64_t)(ti - tiles0) * PF_KT + l32;
      const int64_t r = tok - rbase;
      ok = tok >= w_lo && tok <= w_hi && r >= 0 && r < R_cap;
    }
    if constexpr (PG) ok = ok && rowok[buf][l32];
    return (uint32_t)__ballot(ok);
  };
  // step of tile ti in buffer BUF: publish it, start tile ti + 1 in the
  // other buffer (free: every wave finished tile ti - 1 before the barrier)
  auto stepA = [&](auto buf_tag, int ti) {
    constexpr int BUF = decltype(buf_tag)::value;
    wait_loads();
    __syncthreads();
    if (ti + 1 < ntA) issueA(ti + 1, std::integral_constant<int, BUF ^ 1>{});
    const uint32_t vmask = maskA(ti, BUF);
    if (active && vmask) compute(buf_tag, vmask);
  };
  if (ntA > 0) {
    issueA(0, std::integral_constant<int, 0>{});
    for (int ti = 0; ti < ntA; ti += 2) {
      stepA(std::integral_constant<int, 0>{}, ti);
      if (ti + 1 < ntA) stepA(std::integral_constant<int, 1>{}, ti + 1);
    }
  }

  // ---------------- phase B: each row's selected compressed entries
  // The index rows are staged in LDS, PF_IDX_MAX slots at a time, as entry
  // numbers or -1 (padding, out of range, past the list, a row past T), so
  // that a tile's loads need one LDS read per instruction and never wait on a
  // global index load.  Row r's tiles are tile0[r] and tile1[r].
  if (SPARSE && topk > 0 && Nc_cap > 0) {
    const int32_t* idx_rows = idx + (qrow0 + t0) * topk;
    const int nrows = t_last - t0 + 1;
    const int* idx_s = idx_all[row_w];
    rebase((uint32_t)row_w * PF_TILEB);
    for (int c0 = 0; c0 < topk; c0 += PF_IDX_MAX) {
      const int cn = min(PF_IDX_MAX, topk - c0);
      const int cw = (cn + PF_KT - 1) / PF_KT * PF_KT;  // whole tiles
      // every thread takes part: the barrier below orders these stores
      // after every read of the previous chunk's slots and tiles (loads
      // batched four per thread, from clamped addresses)
      __syncthreads();
      const int n_st = PF_ROWS * cw;
      for (int i0 = 0; i0 < n_st; i0 += 4 * NT) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * NT + tid;
          const int r = i / cw, pp = i - r * cw;
          v[u] = idx_rows[(size_t)min(r, nrows - 1) * topk + c0 + min(pp, cn - 1)];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * NT + tid;
          const int r = i / cw, pp = i - r * cw;
          const bool ok = r < nrows && pp < cn && (uint32_t)v[u] < (uint32_t)Nc_cap;
          if (i < n_st) idx_all[r][pp] = ok ? v[u] : -1;
        }
      }
      __syncthreads();
      // the row's NH waves issue the 16 instructions of its tile: wave hh
      // takes hh, hh + NH, ...
      auto issueB = [&](int ti, auto buf_tag) {
        uint8_t* const dst = decltype(buf_tag)::value ? &tile1[row_w][0] : &tile0[row_w][0];
#pragma unroll
        for (int k = 0; k < 16 / NH; ++k) {
          const int i = hh + NH * k;
          const int j = idx_s[ti * PF_KT + 2 * i + h2];
          dma(dst, i, (const char*)kvc_b,
              (uint32_t)max(j, 0) * (uint32_t)PF_ROWB);
        }
      };
      const int ntB = cw / PF_KT;
      auto stepB = [&](auto buf_tag, int ti) {
        constexpr int BUF = decltype(buf_tag)::value;
        wait_loads();
        __syncthreads();
        if (ti + 1 < ntB) issueB(ti + 1, std::integral_constant<int, BUF ^ 1>{});
        const uint32_t vmask = (uint32_t)__ballot(idx_s[ti * PF_KT + l32] >= 0);
        if (vmask) compute(buf_tag, vmask);
      };
      issueB(0, std::integral_constant<int, 0>{});
      for (int ti = 0; ti < ntB; ti += 2) {
        stepB(std::integral_constant<int, 0>{}, ti);
        if (ti + 1 < ntB) stepB(std::integral_constant<int, 1>{}, ti + 1);
      }
    }
  }

  // ---------------- output: lane holds head 32 hh + l32, dims
  // 32 dt + 8 (r/4) + 4 h2 + r%4
  if (!active) return;
  const int h = 32 * hh + l32;
  float inv, lse_v;
  finish_softmax(mrun, lrun, sink, h, inv, lse_v);
  uint16_t* orow = out + (rowi * H + h) * D;
  for (int dt = 0; dt < 4; ++dt)
    for (int rq = 0; rq < 4; ++rq) {
      const int d = 32 * dt + 8 * rq + 4 * h2;
      uint32_t lo = (uint32_t)f32_to_bf16(o[dt][4 * rq] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * rq + 1] * inv) << 16);
      uint32_t hi = (uint32_t)f32_to_bf16(o[dt][4 * rq + 2] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * rq + 3] * inv) << 16);
      *(u32x2*)(orow + d) = u32x2{lo, hi};
    }
  if (lse && h2 == 0) lse[rowi * H + h] = lse_v;
}

// ---------------------------------------------------------------- bf16 decode
// Few query rows, long key lists (decode): a work item is (row, split) and its
// waves split the heads - wave w owns heads 16 w .. 16 w + 15 - so a 64-key
// tile of [K | V] rows is loaded once per workgroup and read by every wave.
// Per wave and tile:
//     S^T (16 keys x 16 heads) = K Q^T        4 blocks x 4 MFMA 16x16x32
//     O^T (16 dims x 16 heads) += V^T P^T     8 dim tiles x 2 MFMA
// The S^T accumulator of lane l holds head l%16 and keys 4 (l/16) + i of each
// 16-key block, which is the P^T operand once the k order of the second
// product pairs keys {32 ks + 4 g + i} and {32 ks + 16 + 4 g + i}; V^T
// fragments of 4 consecutive keys per lane come from the LDS transpose read
// (lane i of a 16-lane group gets element i % 4 of the 8-byte chunks whose
// addresses lanes i/4 + 4 v supplied).  The rows of the next two tiles are
// loaded into registers while the current one is computed.
constexpr int DC_KT = 64;                // keys per tile
// K and V halves in separate LDS arrays: K rows of 68 dwords (16 rows of
// 16-byte reads hit 16 distinct 4-bank groups), V rows of 72 dwords (the
// transpose reads of a 32-lane half cover 8 rows x 8 dwords)
constexpr int DC_KS = 128 + 8, DC_VS = 128 + 16;
constexpr int DC_IDX_MAX = 4096;         // index slots staged in LDS per work item
constexpr float DC_RESCALE = 8.0f;       // log2 headroom before the maximum is raised

template <int WAVES>  // H = 16 WAVES
__global__ void __launch_bounds__(64 * WAVES) attn_dec_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv_cmp,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw,
    const int64_t* __restrict__ q_pos, const int32_t* __restrict__ n_cmp,
    const int64_t* __restrict__ raw_base, int T, int topk, int window, int m, int Nc_cap,
    int R_cap, bool dense, float scale_log2, const float* __restrict__ sink, int n_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int64_t cmp_rows_b, PageTable pt, int nc_logical, Varlen vl,
    PageTable raw_pt, int phase, int n_split_c) {
  constexpr int H = 16 * WAVES, D = 128, NT = 64 * WAVES;
  constexpr int CH = DC_KT * 32 / NT;       // 16-byte chunks per thread per tile
  constexpr uint32_t kRowBytes = 2 * D * 2;  // one [K | V] row
  __shared__ __attribute__((aligned(16))) uint16_t tile[DC_KT * (DC_KS + DC_VS)];
  uint16_t* const vtile = tile + DC_KT * DC_KS;
  __shared__ __attribute__((aligned(16))) int vmask[DC_KT];
  __shared__ __attribute__((aligned(16))) int partial[4];
  __shared__ int idx_s[DC_IDX_MAX];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, hl = lane & 15;
  // phase 0: the n_split splits of each row share its tile list evenly.
  // Phases 1 and 2 (the two halves of a split call): splits [0, n_split_c)
  // take the selected entries' tiles, splits [n_split_c, n_split) the
  // window's; phase 1 launches only the window splits, phase 2 only the
  // others.  item is the partial slot (row, split).
  const int n_launch = phase == 0 ? n_split : (phase == 1 ? n_split - n_split_c : n_split_c);
  const int rowi = blockIdx.x / n_launch;
  const int split = (phase == 1 ? n_split_c : 0) + blockIdx.x % n_launch;
  const int item = rowi * n_split + split;
  const int b = vl.cu_q ? varlen_seq(vl, rowi) : rowi / T;
  const int t = vl.cu_q ? rowi - vl.cu_q[b] : rowi % T;
  // packed sequences: the sequence's entries and its own tokens as the raw
  // rows, positions from 0
  // (pt with the dense form and raw_pt: rows found in the shared pools on
  // load; pt with the sparse form: the staged indices are pool rows)
  const bool cmp_paged = dense && pt.block_table;
  const uint16_t* kvc_b = kv_cmp + (cmp_paged ? 0 : (size_t)b * cmp_rows_b * 2 * D);
  const uint16_t* kvr_b = kv_raw + (raw_pt.block_table ? 0 : (size_t)b * R_cap * 2 * D);
  if (vl.cu_q) {
    kvc_b = kv_cmp + (size_t)vl.cu_k[b] * 2 * D;
    kvr_b = kv_raw + (size_t)vl.cu_q[b] * 2 * D;
    Nc_cap = vl.cu_k[b + 1] - vl.cu_k[b];
    R_cap = vl.cu_q[b + 1] - vl.cu_q[b];
  }
  const int64_t pos = vl.cu_q ? t : q_pos[b] + t;
  // n_cmp exists only for the dense (HCA) form: csa_sparse_attn passes none
  const int32_t ncmp_b = vl.cu_q ? Nc_cap : (dense ? n_cmp[b] : 0);
  const KeyList L = key_list(dense, topk, window, pos, ncmp_b, m, Nc_cap);
  // Tile-aligned list: compressed slots [0, n_c) padded to a whole tile, then
  // the window, so that every tile reads from one of the two caches.  Splits
  // take whole tiles.
  const int nc_pad = (L.n_c + DC_KT - 1) / DC_KT * DC_KT;
  const int n_tiles_row = (nc_pad + L.n_w + DC_KT - 1) / DC_KT;
  int ta, tb;
  if (phase == 0) {
    const int tiles_per = (n_tiles_row + n_split - 1) / n_split;
    ta = min(n_tiles_row, split * tiles_per);
    tb = min(n_tiles_row, ta + tiles_per);
  } else {
    // the selected part's tiles [0, nc_pad / DC_KT) over n_split_c splits,
    // the window's [nc_pad / DC_KT, n_tiles_row) over the rest
    const int c_tiles = nc_pad / DC_KT;
    const bool wpart = split >= n_split_c;
    const int t0 = wpart ? c_tiles : 0, nt = wpart ? n_tiles_row - c_tiles : c_tiles;
    const int ns = wpart ? n_split - n_split_c : n_split_c, s = wpart ? split - n_split_c : split;
    const int per = (nt + ns - 1) / ns;
    ta = t0 + min(nt, s * per);
    tb = t0 + min(nt, s * per + per);
  }
  const int ntiles = tb - ta;
  const int kb = ta * DC_KT;
  const int32_t* idx_row = dense ? nullptr : idx + (size_t)rowi * topk;
  const uint16_t* dummy = q + (size_t)rowi * H * D;  // a valid row for empty slots
  const char* cbase = Nc_cap > 0 ? (const char*)kvc_b : (const char*)dummy;
  const char* wbase = R_cap > 0 ? (const char*)kvr_b : (const char*)dummy;
  const int n_c = L.n_c, n_w = L.n_w;
  const int64_t w_row0 = L.lo - (vl.cu_q ? 0 : raw_base[b]);  // cache row of window slot 0
  // index slots of this item's compressed positions, staged once (loads
  // batched four per thread before their LDS stores); the host splits the
  // list so that an item holds at most DC_IDX_MAX of them
  const int c_lo = min(kb, L.n_c), c_hi = min(tb * DC_KT, L.n_c);
  if (!dense) {
    for (int i0 = 0; i0 < c_hi - c_lo; i0 += 4 * NT) {
      int v[4];
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + tid;
        v[u] = i < c_hi - c_lo ? idx_row[c_lo + i] : 0;
      }
      if (pt.block_table && !dense) {  // paged: logical entries to pool rows
        for (int u = 0; u < 4; ++u)
          v[u] = (v[u] >= 0 && v[u] < nc_logical) ? (int)paged_row(pt, b, v[u]) : -1;
      }
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + tid;
        if (i < c_hi - c_lo) idx_s[i] = v[u];
      }
    }
  }
  __syncthreads();

  // Q^T operand: lane holds head 16 wave + hl, dims 32 s + 8 g .. + 8
  bf16x8 qf[4];
  {
    const uint16_t* qr = q + ((size_t)rowi * H + 16 * wave + hl) * D;
    for (int s = 0; s < 4; ++s) qf[s] = *(const bf16x8*)(qr + 32 * s + 8 * g);
  }
  f32x4 o[8];
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float mrun = -INFINITY, lrun = 0.0f;

  const int col = tid & 31;
  // Tile rows in registers: byte offsets from the tile's cache base (empty
  // slots: offset 0 of a valid base, masked), loads issued unconditionally
  // so that the waits count them exactly.  Tiles past the end read the
  // dummy row.
  u32x4 pfa[CH], pfb[CH];
  bool pva[CH], pvb[CH];
  auto issue = [&](int ti, u32x4(&pf)[CH], bool(&pv)[CH]) __attribute__((always_inline)) {
    const int p0 = kb + ti * DC_KT;
    const bool ct = p0 < nc_pad && ti < ntiles;  // uniform
    // base by masks rather than a select: a select between captured
    // variables would be folded into one between their addresses, which
    // keeps the whole capture block in scratch memory
    const uint64_t mc = 0 - (uint64_t)ct, md = 0 - (uint64_t)(ti >= ntiles);
    const uint64_t bsel = ((uint64_t)cbase & mc) | ((uint64_t)wbase & ~mc);
    const char* base = (const char*)(((uint64_t)dummy & md) | (bsel & ~md));
    uint32_t off[CH];
    if (ct) {
      #pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int p = p0 + i * (NT / 32) + (tid >> 5);
        int j = dense ? p : idx_s[min(max(0, p - c_lo), DC_IDX_MAX - 1)];
        bool ok = (p < n_c) & (j >= 0) & (j < Nc_cap);
        if (cmp_paged && ok) {
          j = (int)paged_row(pt, b, j);
          ok = j >= 0;
        }
        pv[i] = ok;
        off[i] = ok ? (uint32_t)j * kRowBytes : 0u;
      }
    } else {
      #pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int w = p0 - nc_pad + i * (NT / 32) + (tid >> 5);
        int64_t r = w_row0 + w;
        bool ok = (ti < ntiles) & (w < n_w) & (r >= 0) & (r < R_cap);
        if (raw_pt.block_table && ok) {
          r = paged_row(raw_pt, b, (int)r);
          ok = r >= 0;
        }
        pv[i] = ok;
        off[i] = ok ? (uint32_t)r * kRowBytes : 0u;
      }
    }
    #pragma unroll
    for (int i = 0; i < CH; ++i)
      pf[i] = __builtin_nontemporal_load((const u32x4*)(base + off[i] + 16 * col));
  };
  // step(ti, regs, refill): tile ti moves from regs to LDS and is computed;
  // with refill the registers then request tile ti + 2, unconditionally.
  auto step = [&](int ti, u32x4(&pf)[CH], bool(&pv)[CH], auto refill)
                  __attribute__((always_inline)) {
    __syncthreads();  // every wave is done reading the previous tile
    bool mine = true;
    #pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int rr = i * (NT / 32) + (tid >> 5);
      const int off = col < 16 ? rr * DC_KS + 8 * col : DC_KT * DC_KS + rr * DC_VS + 8 * (col - 16);
      *(u32x4*)(tile + off) = pf[i];
      if (col == 0) vmask[rr] = pv[i];
      mine = mine && pv[i];
    }
    const bool wave_partial = __ballot(!mine) != 0;
    if (lane == 0) partial[wave] = wave_partial;
    __syncthreads();
    if constexpr (decltype(refill)::value) issue(ti + 2, pf, pv);
    // ---- S^T = K Q^T for 4 blocks of 16 keys; the fragments of a k step are
    // read together, the next step's while the current one multiplies
    // k step s of all four blocks back to back: consecutive MFMAs are
    // independent (a dependent 16x16x32 waits out the full result latency)
    f32x4 sacc[4];
    bf16x8 kf[2][4];
    auto read_k = [&](int s, bf16x8(&f)[4]) {
      for (int kb4 = 0; kb4 < 4; ++kb4)
        f[kb4] = *(const bf16x8*)(tile + (16 * kb4 + hl) * DC_KS + 8 * g + 32 * s);
    };
    for (int kb4 = 0; kb4 < 4; ++kb4) sacc[kb4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    read_k(0, kf[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) read_k(s + 1, kf[(s + 1) & 1]);
      for (int kb4 = 0; kb4 < 4; ++kb4)
        sacc[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s & 1][kb4], qf[s], sacc[kb4], 0,
                                                           0, 0);
    }
    // ---- online softmax over the 64 keys; lane: head hl, keys 16 kb4 + 4 g + i.
    // Only tiles with empty slots pay for the mask.  The running maximum is
    // raised only when a score exceeds it by more than DC_RESCALE (log2
    // units), so most tiles skip the rescale of the accumulators.
    const int4 pw = *(const int4*)partial;
    if (pw[0] | pw[1] | (WAVES > 2 ? pw[2] | pw[3] : 0)) {
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const int4 vm = *(const int4*)(vmask + 16 * kb4 + 4 * g);
        for (int i = 0; i < 4; ++i)
          if (!vm[i]) sacc[kb4][i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
    for (int kb4 = 0; kb4 < 4; ++kb4)
      mx = fmaxf(fmaxf(mx, fmaxf(sacc[kb4][0], sacc[kb4][1])), fmaxf(sacc[kb4][2], sacc[kb4][3]));
    mx = max_xor32(max_xor16(mx)) * scale_log2;
    const bool up = mx > mrun + DC_RESCALE;
    if (__ballot(up)) {
      const float corr = up ? __builtin_amdgcn_exp2f(mrun - mx) : 1.0f;
      if (up) mrun = mx;
      lrun *= corr;
      for (int dt = 0; dt < 8; ++dt) o[dt] *= corr;
    }
    const float nmuse = mrun == -INFINITY ? 0.0f : -mrun;
    float ps = 0.0f;
    for (int kb4 = 0; kb4 < 4; ++kb4)
      for (int i = 0; i < 4; ++i) {
        const float pv2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb4][i], scale_log2, nmuse));
        sacc[kb4][i] = pv2;
        ps += pv2;
      }
    ps = sum_xor32(sum_xor16(ps));
    lrun += ps;
    // ---- O^T += V^T P^T (k slot 8 g + i: key 32 ks + 4 g + i, then 32 ks + 16 + 4 g + i)
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pfr;
      for (int i = 0; i < 4; ++i) {
        pfr[i] = (__bf16)sacc[2 * ks][i];
        pfr[4 + i] = (__bf16)sacc[2 * ks + 1][i];
      }
      // transpose-read addresses: lane j of the group supplies row k0 + j/4,
      // dims D0 + 4 (j % 4)
      const uint16_t* base1 = vtile + (32 * ks + 4 * g + (hl >> 2)) * DC_VS + 4 * (hl & 3);
      const uint16_t* base2 = base1 + 16 * DC_VS;
      // all 16 transpose reads first, then the 8 products (whole-register
      // moves only: the four 16-bit values of a transpose read are not
      // extracted one by one)
      u32x2 v1[8], v2[8];
      for (int dt = 0; dt < 8; ++dt) {
        v1[dt] = __builtin_bit_cast(u32x2, lds_read_tr16(base1 + 16 * dt));
        v2[dt] = __builtin_bit_cast(u32x2, lds_read_tr16(base2 + 16 * dt));
      }
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 vf =
            __builtin_bit_cast(bf16x8, u32x4{v1[dt][0], v1[dt][1], v2[dt][0], v2[dt][1]});
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfr, o[dt], 0, 0, 0);
      }
    }
  };
  issue(0, pfa, pva);
  issue(1, pfb, pvb);
  int ti = 0;
  for (; ti + 1 < ntiles; ti += 2) {
    step(ti, pfa, pva, std::true_type{});
    step(ti + 1, pfb, pvb, std::true_type{});
  }
  if (ti < ntiles) step(ti, pfa, pva, std::false_type{});
  // ---- results: lane holds head 16 wave + hl, dims 16 dt + 4 g + i
  const int h = 16 * wave + hl;
  if (n_split == 1) {
    float inv, lse_v;
    finish_softmax(mrun, lrun, sink, h, inv, lse_v);
    uint16_t* orow = out + ((size_t)rowi * H + h) * D;
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + 4 * g;
      uint32_t lo = (uint32_t)f32_to_bf16(o[dt][0] * inv) | ((uint32_t)f32_to_bf16(o[dt][1] * inv) << 16);
      uint32_t hi = (uint32_t)f32_to_bf16(o[dt][2] * inv) | ((uint32_t)f32_to_bf16(o[dt][3] * inv) << 16);
      *(u32x2*)(orow + d) = u32x2{lo, hi};
    }
    if (lse && g == 0) lse[(size_t)rowi * H + h] = lse_v;
  } else {
    float* po = part_o + ((size_t)item * H + h) * D;
    for (int dt = 0; dt < 8; ++dt) *(f32x4*)(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0) {
      part_ml[((size_t)item * H + h) * 2 + 0] = mrun;
      part_ml[((size_t)item * H + h) * 2 + 1] = lrun;
    }
  }
}

// ---------------------------------------------------------------- combine
// Grid (rows, H / 2), 256 threads: thread (h, d) merges output element d of
// head h over the splits, O = sum_s exp2(m_s - M) O_s / sum_s exp2(m_s - M) l_s
// with M = max_s m_s.  Lane s of each wave computes the weight of split s
// (n_split <= 64); the partial loads are issued eight splits at a time.
// D = 128.
constexpr int CB_MAX_SPLIT = 64;

template <int OUT_DT>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_split, int H,
                                                      const float* __restrict__ sink,
                                                      void* __restrict__ out,
                                                      float* __restrict__ lse) {
  constexpr int D = 128;
  const int rowi = blockIdx.x;
  const int h = blockIdx.y * 2 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);
  const int d = threadIdx.x & (D - 1), lane = threadIdx.x & 63;
  const float* ml = part_ml + ((size_t)rowi * n_split * H + h) * 2;  // split s at + 2 H s
  const float* po = part_o + ((size_t)rowi * n_split * H + h) * D + d;  // split s at + H D s
  // lane s holds split s: weights exp2(m_s - M) and the merged sum
  const float ms = lane < n_split ? ml[(size_t)2 * H * lane] : -INFINITY;
  const float ls = lane < n_split ? ml[(size_t)2 * H * lane + 1] : 0.0f;
  const float M = wave_max(ms);
  const float Mu = M == -INFINITY ? 0.0f : M;
  const float c = lane < n_split ? exp2f(ms - Mu) : 0.0f;
  const float Ls = wave_sum(ls * c);
  float O = 0.0f;
  for (int s0 = 0; s0 < n_split; s0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = s0 + k < n_split ? po[(size_t)H * D * (s0 + k)] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) O = fmaf(v[k], __shfl(c, s0 + k, 64), O);
  }
  float inv, lse_v;
  finish_softmax(M, Ls, sink, h, inv, lse_v);
  const float v = O * inv;
  if (OUT_DT == CSA_DT_BF16)
    ((uint16_t*)out)[((size_t)rowi * H + h) * D + d] = f32_to_bf16(v);
  else
    ((float*)out)[((size_t)rowi * H + h) * D + d] = v;
  if (lse && d == 0) lse[(size_t)rowi * H + h] = lse_v;
}

// ---------------------------------------------------------------- fp32
// One wave per (row, head); lane owns dims lane and lane + 64.
__global__ void __launch_bounds__(64) attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv_cmp, const int32_t* __restrict__ idx,
    const float* __restrict__ kv_raw, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, const int64_t* __restrict__ raw_base, int T, int H, int D,
    int topk, int window, int m, int Nc_cap, int R_cap, bool dense, float scale_log2,
    const float* __restrict__ sink, float* __restrict__ out, float* __restrict__ lse,
    int64_t cmp_rows_b, Varlen vl, PageTable cmp_pt, PageTable raw_pt) {
  const int lane = threadIdx.x;
  const int rowi = blockIdx.x / H, h = blockIdx.x % H;
  const int b = vl.cu_q ? varlen_seq(vl, rowi) : rowi / T;
  const int t = vl.cu_q ? rowi - vl.cu_q[b] : rowi % T;
  const float* kvc_b = kv_cmp + (cmp_pt.block_table ? 0 : (size_t)b * cmp_rows_b * 2 * D);
  const float* kvr_b = kv_raw + (raw_pt.block_table ? 0 : (size_t)b * R_cap * 2 * D);
  if (vl.cu_q) {  // packed sequences (positions from 0, own tokens as raw rows)
    kvc_b = kv_cmp + (size_t)vl.cu_k[b] * 2 * D;
    kvr_b = kv_raw + (size_t)vl.cu_q[b] * 2 * D;
    Nc_cap = vl.cu_k[b + 1] - vl.cu_k[b];
    R_cap = vl.cu_q[b + 1] - vl.cu_q[b];
  }
  const int64_t pos = vl.cu_q ? t : q_pos[b] + t;
  // n_cmp exists only for the dense (HCA) form: csa_sparse_attn passes none
  const int32_t ncmp_b = vl.cu_q ? Nc_cap : (dense ? n_cmp[b] : 0);
  const KeyList L = key_list(dense, topk, window, pos, ncmp_b, m, Nc_cap);
  const int nk = L.n_c + L.n_w;
  const int32_t* idx_row = dense ? nullptr : idx + (size_t)rowi * topk;
  const int64_t rbase = vl.cu_q ? 0 : raw_base[b];
  const float* qr = q + ((size_t)rowi * H + h) * D;
  const float q0 = lane < D ? qr[lane] : 0.0f;
  const float q1 = lane + 64 < D ? qr[lane + 64] : 0.0f;
  float mrun = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int p = 0; p < nk; ++p) {
    const float* src = key_row(p, L, dense, idx_row, kvc_b, Nc_cap, kvr_b, R_cap, rbase, 2 * D,
                               b, cmp_pt, raw_pt);
    if (!src) continue;
    float part = (lane < D ? q0 * src[lane] : 0.0f) + (lane + 64 < D ? q1 * src[lane + 64] : 0.0f);
    const float s = wave_sum(part) * scale_log2;
    const float mnew = fmaxf(mrun, s);
    const float corr = exp2f(mrun - mnew);
    const float pv = exp2f(s - mnew);
    l = l * corr + pv;
    o0 = o0 * corr + pv * (lane < D ? src[D + lane] : 0.0f);
    o1 = o1 * corr + pv * (lane + 64 < D ? src[D + lane + 64] : 0.0f);
    mrun = mnew;
  }
  float inv, lse_v;
  finish_softmax(mrun, l, sink, h, inv, lse_v);
  float* orow = out + ((size_t)rowi * H + h) * D;
  if (lane < D) orow[lane] = o0 * inv;
  if (lane + 64 < D) orow[lane + 64] = o1 * inv;
  if (lse && lane == 0) lse[(size_t)rowi * H + h] = lse_v;
}

// Selected logical entries of a paged compressed cache to pool rows (-1
// stays -1, as does an index outside [0, Nc_cap)); rows of topk slots.
__global__ void page_index_kernel(const int32_t* __restrict__ idx, size_t n, int T, int topk,
                                  int Nc_cap, PageTable pt, int32_t* __restrict__ phys) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int j = idx[i];
    const int b = (int)(i / topk) / T;
    phys[i] = (j >= 0 && j < Nc_cap) ? (int32_t)paged_row(pt, b, j) : -1;
  }
}

}  // namespace csa

// Scratch of csa_sparse_attn_noalloc (for callers that cannot allocate):
// the split-key partials of the decode kernel live here instead of in a
// caller workspace.  Each GPU the library runs on holds one copy for the
// life of the process; every call on that GPU shares it.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace csa_host {
using namespace csa;

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the host-side name is only a stand-in
// for the symbol, never a device address).
hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// Rows at or above this count use the one-row-per-wave kernel; fewer rows
// (decode) use the head-split kernel with split-K.
constexpr int AT_DECODE_ROWS = 1024;
constexpr int DC_MIN_SPLIT_KEYS = 128;

static bool use_decode_kernel(int rows, int H) {
  return rows < AT_DECODE_ROWS && (H == 32 || H == 64);
}

// Splits of the decode kernel: about one workgroup per CU of the 256 (more,
// shorter work items measured slower: each carries fixed index, query and
// partial-output costs, and the combine reads more partials), each with >= 128
// keys, and for index lists enough that no split holds more than DC_IDX_MAX
// index slots (its staging buffer).  0: unsupported.
static int attn_splits(int rows, int keys_per_row, bool sparse, int H) {
  if (use_decode_kernel(rows, H)) {
    int s = (256 + rows - 1) / rows;
    int smax = (keys_per_row + DC_MIN_SPLIT_KEYS - 1) / DC_MIN_SPLIT_KEYS;
    if (smax > CB_MAX_SPLIT) smax = CB_MAX_SPLIT;
    s = s < smax ? s : smax;
    if (sparse) {
      // the kernel's tile-aligned list has at most this many tiles; a split
      // takes ceil(tiles / s) of them
      const int tiles = (keys_per_row + 2 * DC_KT - 1) / DC_KT;
      const int smin = (tiles + DC_IDX_MAX / DC_KT - 1) / (DC_IDX_MAX / DC_KT);
      if (s < smin) s = smin;
      if (s > CB_MAX_SPLIT) return 0;
    }
    return s < 1 ? 1 : s;
  }
  return 1;  // the prefill kernel has enough rows to fill the chip
}

// Splits of a call taken in two halves (decode rows, sparse form): the
// window's tiles over about 128 workgroups, so that they fit beside the
// indexer that runs at the same time, and the selected entries' tiles over
// about one workgroup per CU, each split holding at most DC_IDX_MAX slots.
// Both counts are fixed by (rows, topk, window) alone.  {0, 0}: unsupported.
struct HalfSplits {
  int s_c, s_w;
};
static HalfSplits half_splits(int rows, int H, int topk, int window) {
  if (!use_decode_kernel(rows, H) || rows < 1) return {0, 0};
  const int c_tiles = (topk + DC_KT - 1) / DC_KT, w_tiles = (window + DC_KT - 1) / DC_KT;
  int s_w = std::min(std::max(w_tiles, 1), std::max(1, (128 + rows - 1) / rows));
  int s_c = std::min(std::max(c_tiles, 1), std::max(1, (256 + rows - 1) / rows));
  s_c = std::max(s_c, (c_tiles + DC_IDX_MAX / DC_KT - 1) / (DC_IDX_MAX / DC_KT));
  if (s_c + s_w > CB_MAX_SPLIT) return {0, 0};
  return {s_c, s_w};
}

bool attn_half_supported(int B, int T, int H, int topk, int window) {
  return half_splits(B * T, H, topk, window).s_c > 0;
}

size_t attn_half_ws_bytes(int B, int T, int H, int D, int topk, int window) {
  const HalfSplits hs = half_splits(B * T, H, topk, window);
  return (size_t)B * T * (hs.s_c + hs.s_w) * H * (D + 2) * sizeof(float);
}

bool attn_supported(int B, int T, int H, int keys_per_row, bool sparse) {
  return attn_splits(B * T, keys_per_row, sparse, H) > 0;
}

size_t attn_ws_bytes(int B, int T, int H, int D, int keys_per_row, bool sparse) {
  const int rows = B * T;
  const int s = attn_splits(rows, keys_per_row, sparse, H);
  if (s <= 1) return 0;
  return (size_t)rows * s * H * (D + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a_in, hipStream_t st) {
  AttnArgs a = a_in;
  // packed sequences: one row per query token of every sequence (a.T is the
  // longest sequence)
  const int rows = a.vl.cu_q ? a.total_rows : a.B * a.T;
  const float scale_log2 = a.scale * kLog2e;
  int64_t cmp_rows_b = a.Nc_cap;  // rows of one sequence's compressed cache
  const int nc_logical = a.Nc_cap;
  PageTable dec_pages{nullptr, 0, 0, 0}, cmp_pt{nullptr, 0, 0, 0};
  const PageTable raw_pt = a.raw_pages;
  if (a.pages.block_table && a.dense) {
    // paged entries of the dense form: every kernel finds each visible entry
    // through the table when it loads it
    cmp_pt = a.pages;
    cmp_rows_b = 0;
  } else if (a.pages.block_table && a.dt != CSA_DT_F32 && use_decode_kernel(rows, a.H)) {
    // paged decode rows: the kernel maps each staged index to its pool row
    dec_pages = a.pages;
    a.Nc_cap = a.pages.n_pages << a.pages.page_log2;
    cmp_rows_b = 0;
  } else if (a.pages.block_table) {
    // paged (sparse only): the selected entries become pool rows in the
    // workspace (after the split partials); the kernels then address the
    // pool as one cache shared by every sequence
    int32_t* phys = (int32_t*)((char*)a.ws + attn_ws_bytes(a.B, a.T, a.H, a.D, a.topk + a.window,
                                                           true));
    const size_t n = (size_t)rows * a.topk;
    page_index_kernel<<<(unsigned)std::max<size_t>(1, std::min<size_t>((n + 255) / 256, 4096)),
                        256, 0, st>>>(a.idx, n, a.T, a.topk, a.Nc_cap, a.pages, phys);
    a.idx = phys;
    a.Nc_cap = a.pages.n_pages << a.pages.page_log2;
    cmp_rows_b = 0;
  }
  if (a.dt == CSA_DT_F32) {
    attn_f32_kernel<<<rows * a.H, 64, 0, st>>>(
        (const float*)a.q, (const float*)a.kv_cmp, a.idx, (const float*)a.kv_raw, a.q_pos,
        a.n_cmp, a.raw_base, a.T, a.H, a.D, a.topk, a.window, a.m, a.Nc_cap, a.R_cap, a.dense,
        scale_log2, a.sink, (float*)a.out, a.lse, cmp_rows_b, a.vl, cmp_pt, raw_pt);
    return hipGetLastError();
  }
  const int keys = (a.dense ? a.Nc_cap : a.topk) + a.window;
  int n_split = attn_splits(rows, keys, !a.dense, a.H), n_split_c = 0;
  unsigned grid = (unsigned)(rows * n_split);
  if (a.phase != 0) {
    // one half of a split call: its own split layout (see half_splits)
    const HalfSplits hs = half_splits(rows, a.H, a.topk, a.window);
    n_split = hs.s_c + hs.s_w;
    n_split_c = hs.s_c;
    grid = (unsigned)(rows * (a.phase == 1 ? hs.s_w : hs.s_c));
  }
  if (n_split == 0) return hipErrorNotSupported;
  float* part_o = (float*)a.ws;
  float* part_ml = part_o ? part_o + (size_t)rows * n_split * a.H * a.D : nullptr;
  if (use_decode_kernel(rows, a.H)) {
    if (a.H == 64)
      attn_dec_kernel<4><<<grid, 256, 0, st>>>(
          (const uint16_t*)a.q, (const uint16_t*)a.kv_cmp, a.idx, (const uint16_t*)a.kv_raw,
          a.q_pos, a.n_cmp, a.raw_base, a.T, a.topk, a.window, a.m, a.Nc_cap, a.R_cap, a.dense,
          scale_log2, a.sink, n_split, (uint16_t*)a.out, a.lse, part_o, part_ml, cmp_rows_b,
          a.dense ? cmp_pt : dec_pages, nc_logical, a.vl, raw_pt, a.phase, n_split_c);
    else
      attn_dec_kernel<2><<<grid, 128, 0, st>>>(
          (const uint16_t*)a.q, (const uint16_t*)a.kv_cmp, a.idx, (const uint16_t*)a.kv_raw,
          a.q_pos, a.n_cmp, a.raw_base, a.T, a.topk, a.window, a.m, a.Nc_cap, a.R_cap, a.dense,
          scale_log2, a.sink, n_split, (uint16_t*)a.out, a.lse, part_o, part_ml, cmp_rows_b,
          a.dense ? cmp_pt : dec_pages, nc_logical, a.vl, raw_pt, a.phase, n_split_c);
  } else {
    // HCA rows share the whole compressed range: 4 rows per workgroup; CSA
    // rows share only the window: 2 rows, so that two independent
    // workgroups fill each CU.
#define CSA_LAUNCH_PF(NH, ROWS, SP, PG)                                                           \
  attn_pf_kernel<NH, ROWS, SP, PG><<<(unsigned)(a.B * ((a.T + ROWS - 1) / ROWS)), 64 * ROWS * NH, \
                                     0, st>>>(                                                     \
      (const uint16_t*)a.q, (const uint16_t*)a.kv_cmp, a.idx, (const uint16_t*)a.kv_raw, a.q_pos,  \
      a.n_cmp, a.raw_base, a.T, a.topk, a.window, a.m, a.Nc_cap, a.R_cap, scale_log2, a.sink,      \
      (uint16_t*)a.out, a.lse, cmp_rows_b, a.vl, cmp_pt, raw_pt)
    // paged window rows or paged dense entries: the variant that looks rows
    // up in the block tables
    const bool pg = cmp_pt.block_table || raw_pt.block_table;
    if (a.H == 64) {
      if (a.dense) {
        if (pg) CSA_LAUNCH_PF(2, 4, false, true);
        else CSA_LAUNCH_PF(2, 4, false, false);
      } else {
        if (pg) CSA_LAUNCH_PF(2, 2, true, true);
        else CSA_LAUNCH_PF(2, 2, true, false);
      }
    } else {
      if (a.dense) {
        if (pg) CSA_LAUNCH_PF(1, 4, false, true);
        else CSA_LAUNCH_PF(1, 4, false, false);
      } else {
        if (pg) CSA_LAUNCH_PF(1, 2, true, true);
        else CSA_LAUNCH_PF(1, 2, true, false);
      }
    }
#undef CSA_LAUNCH_PF
  }
  // the window half leaves its partials for the selected half's combine
  if (n_split > 1 && a.phase != 1)
    combine_kernel<CSA_DT_BF16><<<dim3(rows, a.H / 2), 256, 0, st>>>(part_o, part_ml, n_split,
                                                                      a.H, a.sink, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace csa_host
