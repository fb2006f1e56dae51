// Indexer KL loss and its gradients for gfx950 (bf16 queries and keys,
// H_I = 16, d_I = 64).
//
// The migration page (sections 1 and 3.2) names an indexer loss for training
// and a fused sparse "lightning indexer grad + KL loss" operator; section 4.3
// gives a loss coefficient and a sparse-loss switch.  The loss's formula is
// not on the pages; the reading used here (sparse form): per query token,
// over its selected entries S, the target p is the main attention's
// probability mass per entry summed over heads and normalised over S, the
// indexer's distribution is the softmax over S of its scores
// I_k = sum_h w_h ReLU(q_h . k_j), and the loss is KL(p || softmax(I)).
// With g the row's gradient scale, dI_k = g (softmax(I)_k - p_k) and
//   dw[h] = sum_k dI_k ReLU(v_hk),  dq[h] = sum_k dI_k w_h [v_hk > 0] k_j,
//   dk[j] += sum_h dI_k w_h [v_hk > 0] q_h.
//
// Two kernels.  A row kernel (one workgroup per query token) computes the
// selected entries' scores on the 16x16x32 MFMA (heads x entries, the keys
// gathered straight from global memory), the loss, dI, dw and dq (dq^T =
// K_sel^T C^T on the MFMA, the selected key rows staged in LDS 256 at a time).
// A key-major kernel sums dk over the rows that select each entry (a
// workgroup owns 128 entries, pairs of query rows are 32 MFMA rows of
// heads), so no per-(row, entry) atomics are needed.
//
// The dense form (the switch off) is the same loss over every visible entry
// of a row, with the dense attention's per-entry mass as the target: a row
// kernel that streams the entries in two passes (statistics, then gradients)
// and the same key-major kernel with visibility in place of the bitmap.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace csa {

constexpr int KL_HI = 16, KL_DI = 64;
constexpr int KL_TOPK_MAX = 1024;
constexpr int KL_CH = 256;                        // slots per dq chunk
constexpr int KL_RC = 64;                         // query rows per dk workgroup

typedef __attribute__((ext_vector_type(4))) short kl_s16x4;
__device__ __forceinline__ kl_s16x4 kl_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) kl_s16x4*)p);
}
__device__ __forceinline__ void kl_dma(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void kl_wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// block reductions over 256 threads (sh: >= 8 floats; ends with a barrier)
__device__ __forceinline__ float kl_block_max(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return v;
}
__device__ __forceinline__ float kl_block_sum(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return v;
}

// ---------------------------------------------------------------- row kernel
// Slot tile u (16 slots) belongs to wave u % 4; lane l holds slot 16 u + l % 16
// and, after the MFMA, v of heads 4 (l / 16) .. + 3 for it.
// TW: 16-slot tiles per wave (topk <= 64 TW); fewer tiles keep fewer
// registers, so that three workgroups share a CU at topk 512
template <int TW>
__global__ void __launch_bounds__(256) idx_kl_row_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ idx,
    const float* __restrict__ mass, const float* __restrict__ gscale, int T, int Nc_cap, int topk,
    float* __restrict__ loss, float* __restrict__ dq_idx, float* __restrict__ dw_idx,
    float* __restrict__ dIw) {
  // key rows of a chunk: 16-byte chunk c of row r at slot c ^ (r & 7), so the
  // row-per-lane staging stores and the transposing reads spread over the banks
  __shared__ __attribute__((aligned(16))) uint8_t ks[KL_CH * 128];
  // C^T of a chunk (bf16), rows padded by 16 bytes: the 16 head rows read at
  // one slot fall in distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t cs[KL_HI][KL_CH + 8];
  // the row's index slots (entry, or -1 for padding and entries past the
  // cache) and attention mass, staged once with coalesced loads
  __shared__ int32_t idx_l[KL_TOPK_MAX];
  __shared__ float mass_l[KL_TOPK_MAX];
  __shared__ float sh[8];
  __shared__ float dws[4][KL_HI];
  const int row = blockIdx.x, b = row / T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int ntile = (topk + 15) / 16;
  const uint16_t* kb = k_idx + (size_t)b * Nc_cap * KL_DI;
  // A operands: head l16, dims 32 s + 8 g4 .. + 8
  bf16x8 qa[2];
  {
    const uint16_t* qr = q_idx + ((size_t)row * KL_HI + l16) * KL_DI + 8 * g4;
    qa[0] = *(const bf16x8*)qr;
    qa[1] = *(const bf16x8*)(qr + 32);
  }
  float wq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wq[i] = w_idx[(size_t)row * KL_HI + 4 * g4 + i];
  {
    const int32_t* ir = idx + (size_t)row * topk;
    const float* mr = mass + (size_t)row * topk;
    for (int k = tid; k < topk; k += 256) {
      const int32_t j = ir[k];
      idx_l[k] = j >= 0 && j < Nc_cap ? j : -1;
      mass_l[k] = mr[k];
    }
  }
  __syncthreads();

  // scores of this wave's tiles, four tiles' key rows in flight at a time
  // (empty slots read row 0 and are ignored)
  float v[TW][4];
  float sc[TW];
  int jv[TW];
  float imax = -INFINITY, msum = 0.0f;
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    jv[i] = -1;
    sc[i] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[i][e] = 0.0f;
  }
#pragma unroll
  for (int i0 = 0; i0 < TW; i0 += 4) {
    if (wave + 4 * i0 >= ntile) break;  // uniform: no tile of this wave left
    bf16x8 k0[4], k1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = wave + 4 * (i0 + q);
      const int k = 16 * u + l16;
      const int j = u < ntile && k < topk ? idx_l[k] : -1;
      jv[i0 + q] = j;
      const uint16_t* kr = kb + (size_t)(j >= 0 ? j : 0) * KL_DI + 8 * g4;
      k0[q] = *(const bf16x8*)kr;
      k1[q] = *(const bf16x8*)(kr + 32);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q;
      const int u = wave + 4 * i;
      if (u < ntile) {  // uniform
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], k0[q], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], k1[q], acc, 0, 0, 0);
        float p = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[i][e] = acc[e];
          p = fmaf(wq[e], fmaxf(acc[e], 0.0f), p);
        }
        p += lane_xor16(p);
        p += lane_xor32(p);
        if (jv[i] >= 0) {
          sc[i] = p;
          imax = fmaxf(imax, p);
          if (g4 == 0) msum += mass_l[16 * u + l16];
        }
      }
    }
  }
  imax = kl_block_max(imax, sh);
  msum = kl_block_sum(msum, sh);
  float zs = 0.0f;
  if (imax > -INFINITY) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
      if (jv[i] >= 0 && g4 == 0) zs += __expf(sc[i] - imax);
  }
  zs = kl_block_sum(zs, sh);
  const bool live = imax > -INFINITY && msum > 0.0f;  // uniform
  const float lz = live ? imax + __logf(zs) : 0.0f;
  const float g = gscale ? gscale[row] : 1.0f;
  // dI, the loss and dw
  float dI[TW];
  float kl = 0.0f, dwp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int u = wave + 4 * i;
    const int k = 16 * u + l16;
    dI[i] = 0.0f;
    if (live && jv[i] >= 0) {
      const float p = mass_l[k] / msum;
      const float lq = sc[i] - lz;
      if (g4 == 0 && p > 0.0f) kl += p * (__logf(p) - lq);
      dI[i] = g * (__expf(lq) - p);
#pragma unroll
      for (int e = 0; e < 4; ++e) dwp[e] = fmaf(dI[i], fmaxf(v[i][e], 0.0f), dwp[e]);
    }
    if (u < ntile && g4 == 0 && k < topk) dIw[(size_t)row * topk + k] = dI[i];
  }
  kl = kl_block_sum(kl, sh);
  if (tid == 0) loss[row] = live ? kl : 0.0f;
  // dw: sum over the 16 slot lanes of each head group, then over the waves
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = dwp[e];
    for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
    dwp[e] = x;
  }
  if (l16 == 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) dws[wave][4 * g4 + e] = dwp[e];
  __syncthreads();
  if (tid < KL_HI) dw_idx[(size_t)row * KL_HI + tid] = dws[0][tid] + dws[1][tid] + dws[2][tid] + dws[3][tid];

  // dq^T (64 dims x 16 heads) = K_sel^T C^T over chunks of 256 slots; wave w
  // owns dims 16 w .. 16 w + 15.  A: the transposing reads of the chunk's
  // key rows (lane l16: dim 16 w + l16; slots 8 g4 + 32 step ..); B: C^T
  // (lane l16: head, the same slots).
  f32x4 dqa = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < ntile * 16; c0 += KL_CH) {
    // stage the chunk's key rows (row r of the chunk at 128 r) and C^T
    for (int r = tid; r < KL_CH; r += 256) {
      const int k = c0 + r;
      const int j = k < topk ? idx_l[k] : -1;
      const u32x4* src = (const u32x4*)(kb + (size_t)(j >= 0 ? j : 0) * KL_DI);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        ((u32x4*)(ks + 128 * r))[c ^ (r & 7)] = j >= 0 ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
    // slots past the last tile: zero (their key rows are zero too)
    if (c0 + tid >= ntile * 16)
#pragma unroll
      for (int h = 0; h < KL_HI; ++h) cs[h][tid] = 0;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int u = wave + 4 * i;
      const int k = 16 * u + l16;
      if (k >= c0 && k < c0 + KL_CH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = v[i][e] > 0.0f ? dI[i] * wq[e] : 0.0f;
          cs[4 * g4 + e][k - c0] = f32_to_bf16(c);
        }
      }
    }
    __syncthreads();
    const int nst = (min(KL_CH, ntile * 16 - c0) + 31) / 32;  // 32-slot steps in the chunk
    for (int st = 0; st < nst; ++st) {
      // lane jj of 16-lane group gg reads slot rows 32 st + 8 gg + 4 e + jj / 4,
      // dims 16 w + 4 (jj & 3) .. + 4; after the transpose lane l holds dim
      // 16 w + l16 of slots 32 st + 8 g4 + 4 e .. + 4
      bf16x8 ka;
      {
        const int jj = lane & 15, gg = lane >> 4;
        u32x2 t[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 32 * st + 8 * gg + 4 * e + (jj >> 2);
          const int d0 = 16 * wave + 4 * (jj & 3);  // first dim: chunk d0 / 8, byte 2 (d0 % 8)
          t[e] = __builtin_bit_cast(
              u32x2, kl_read_tr16(ks + 128 * r + 16 * ((d0 >> 3) ^ (r & 7)) + 2 * (d0 & 7)));
        }
        ka = __builtin_bit_cast(bf16x8, u32x4{t[0][0], t[0][1], t[1][0], t[1][1]});
      }
      const bf16x8 cb = *(const bf16x8*)&cs[l16][32 * st + 8 * g4];
      dqa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, cb, dqa, 0, 0, 0);
    }
    __syncthreads();
  }
  // dqa[e]: dim 16 w + 4 g4 + e, head l16
  float* o = dq_idx + ((size_t)row * KL_HI + l16) * KL_DI + 16 * wave + 4 * g4;
  *(f32x4*)o = dqa;
}

// ---------------------------------------------------------------- dense row kernel
// The dense form (the sparse-loss switch off): the selected set of row t is
// every visible entry j < n_vis(t), the target the dense attention's mass per
// entry ([B, T, Nc_cap]).  A wave's 16-entry tiles are w, w + 4, ... of a
// chunk (lane l: entry 16 u + l % 16, heads 4 (l / 16) .. + 3 after the
// MFMA).  Pass 1 streams 256-entry chunks straight into registers, the next
// chunk's keys and mass in flight while the current one is reduced, for the
// softmax statistics (a running max and sum per lane) and the mass sum.
// Pass 2 stages 128-entry chunks of key rows in LDS by direct loads, one
// chunk ahead in the other of two buffers, recomputes the scores from them,
// forms dI, the loss and dw, and adds the chunk's dq^T = K^T C^T from the
// same rows.  Entries past n_vis read row n_vis - 1 (a row of the cache that
// is set) and are masked.  Workgroups take the rows from the last (the
// longest) down.
constexpr int KL_DC = 128;  // entries per pass-2 chunk

__global__ void __launch_bounds__(256) idx_kl_dense_row_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const float* __restrict__ mass,
    const float* __restrict__ gscale, const int64_t* __restrict__ q_pos,
    const int32_t* __restrict__ n_cmp, int T, int Nc_cap, int m, float* __restrict__ loss,
    float* __restrict__ dq_idx, float* __restrict__ dw_idx, float* __restrict__ dIw) {
  // key rows of a chunk: 16-byte chunk c of row r at slot c ^ (r & 7)
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[KL_DC * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[KL_DC * 128];
  __shared__ __attribute__((aligned(16))) uint16_t cs[KL_HI][KL_DC + 8];
  __shared__ float sh[8];
  __shared__ float dws[4][KL_HI];
  const int row = gridDim.x - 1 - blockIdx.x, b = row / T, t = row - b * T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int nv = n_visible(q_pos[b] + t, n_cmp[b], m, Nc_cap);
  const uint16_t* kb = k_idx + (size_t)b * Nc_cap * KL_DI;
  const float* mr = mass + (size_t)row * Nc_cap;
  float* dIr = dIw + (size_t)row * Nc_cap;
  bf16x8 qa[2];
  {
    const uint16_t* qr = q_idx + ((size_t)row * KL_HI + l16) * KL_DI + 8 * g4;
    qa[0] = *(const bf16x8*)qr;
    qa[1] = *(const bf16x8*)(qr + 32);
  }
  float wq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wq[i] = w_idx[(size_t)row * KL_HI + 4 * g4 + i];
  // the row's score of this lane's entry (all four 16-lane groups end with it)
  auto score = [&](const bf16x8& x0, const bf16x8& x1, f32x4& acc) -> float {
    acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], x0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], x1, acc, 0, 0, 0);
    float p = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) p = fmaf(wq[e], fmaxf(acc[e], 0.0f), p);
    p += lane_xor16(p);
    p += lane_xor32(p);
    return p;
  };

  // pass 1: max and sum of exp of the scores, and the mass sum
  float mx = -INFINITY, zs = 0.0f, msum = 0.0f;
  auto load1 = [&](int c0, bf16x8 (&x0)[4], bf16x8 (&x1)[4], float (&mm)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kc = min(c0 + 16 * (wave + 4 * q) + l16, nv - 1);
      const uint16_t* kr = kb + (size_t)kc * KL_DI + 8 * g4;
      x0[q] = *(const bf16x8*)kr;
      x1[q] = *(const bf16x8*)(kr + 32);
      mm[q] = mr[kc];
    }
  };
  auto stats = [&](int c0, const bf16x8 (&x0)[4], const bf16x8 (&x1)[4], const float (&mm)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0t = c0 + 16 * (wave + 4 * q);
      if (k0t < nv) {  // uniform
        f32x4 acc;
        const float p = score(x0[q], x1[q], acc);
        if (k0t + l16 < nv && g4 == 0) {
          if (p > mx) {
            zs = zs * __expf(mx - p) + 1.0f;
            mx = p;
          } else {
            zs += __expf(p - mx);
          }
          msum += mm[q];
        }
      }
    }
  };
  // (the next chunk's loads are issued unconditionally, clamped into the
  // row: the same count in flight on every path, so each wait leaves them
  // in flight)
  if (nv > 0) {
    bf16x8 a0[4], a1[4], b0[4], b1[4];
    float ma[4], mb[4];
    load1(0, a0, a1, ma);
    for (int c0 = 0; c0 < nv; c0 += 2 * KL_CH) {
      load1(c0 + KL_CH, b0, b1, mb);
      stats(c0, a0, a1, ma);
      if (c0 + KL_CH >= nv) break;
      load1(c0 + 2 * KL_CH, a0, a1, ma);
      stats(c0 + KL_CH, b0, b1, mb);
    }
  }
  const float imax = kl_block_max(mx, sh);
  zs = kl_block_sum(mx > -INFINITY ? zs * __expf(mx - imax) : 0.0f, sh);
  msum = kl_block_sum(msum, sh);
  const bool live = nv > 0 && msum > 0.0f;  // uniform
  if (!live) {  // loss 0, no gradient
    for (int k = tid; k < nv; k += 256) dIr[k] = 0.0f;
    if (tid == 0) loss[row] = 0.0f;
    if (tid < KL_HI) dw_idx[(size_t)row * KL_HI + tid] = 0.0f;
    float* o = dq_idx + (size_t)row * KL_HI * KL_DI;
    for (int k = tid; k < KL_HI * KL_DI; k += 256) o[k] = 0.0f;
    return;
  }
  const float lz = imax + __logf(zs);
  const float g = gscale ? gscale[row] : 1.0f;
  const float rms = 1.0f / msum;

  // pass 2
  float kl = 0.0f, dwp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 dqa = {0.0f, 0.0f, 0.0f, 0.0f};
  // load instruction i (wave, wave + 4, ...): chunk rows 8 i .. 8 i + 7, lane
  // l writing slot l % 8 of row 8 i + l / 8; and the mass of this lane's
  // entries
  auto stage2 = [&](int c0, uint8_t* dst, float (&mm)[2]) {
#pragma unroll
    for (int u = 0; u < KL_DC / 32; ++u) {
      const int i = wave + 4 * u;
      const int r = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      kl_dma(kb + (size_t)min(c0 + r, nv - 1) * KL_DI + 8 * c, dst + 1024 * i);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) mm[q] = mr[min(c0 + 16 * (wave + 4 * q) + l16, nv - 1)];
  };
  auto grad = [&](int c0, const uint8_t* kbuf, const float (&mm)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rl = 16 * (wave + 4 * q) + l16;  // entry c0 + rl
      if (c0 + 16 * (wave + 4 * q) < nv) {       // uniform
        const bf16x8 x0 = *(const bf16x8*)(kbuf + 128 * rl + 16 * (g4 ^ (rl & 7)));
        const bf16x8 x1 = *(const bf16x8*)(kbuf + 128 * rl + 16 * ((4 + g4) ^ (rl & 7)));
        f32x4 acc;
        const float p = score(x0, x1, acc);
        const int k = c0 + rl;
        float dI = 0.0f;
        if (k < nv) {
          const float pt = mm[q] * rms;
          const float lq = p - lz;
          dI = g * (__expf(lq) - pt);
          if (g4 == 0) {
            if (pt > 0.0f) kl += pt * (__logf(pt) - lq);
            dIr[k] = dI;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dwp[e] = fmaf(dI, fmaxf(acc[e], 0.0f), dwp[e]);
          cs[4 * g4 + e][rl] = f32_to_bf16(acc[e] > 0.0f ? dI * wq[e] : 0.0f);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[4 * g4 + e][rl] = 0;
      }
    }
    lds_barrier();  // cs is complete (the other buffer's loads stay in flight)
    // dq^T (64 dims x 16 heads) += K^T C^T over the chunk's 32-entry steps;
    // wave w owns dims 16 w .. 16 w + 15 (lane layout as in the sparse form)
    const int nst = (min(KL_DC, nv - c0) + 31) / 32;
    for (int st = 0; st < nst; ++st) {
      bf16x8 ka;
      {
        const int jj = lane & 15, gg = lane >> 4;
        u32x2 tr[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 32 * st + 8 * gg + 4 * e + (jj >> 2);
          const int d0 = 16 * wave + 4 * (jj & 3);
          tr[e] = __builtin_bit_cast(
              u32x2, kl_read_tr16(kbuf + 128 * r + 16 * ((d0 >> 3) ^ (r & 7)) + 2 * (d0 & 7)));
        }
        ka = __builtin_bit_cast(bf16x8, u32x4{tr[0][0], tr[0][1], tr[1][0], tr[1][1]});
      }
      const bf16x8 cb = *(const bf16x8*)&cs[l16][32 * st + 8 * g4];
      dqa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, cb, dqa, 0, 0, 0);
    }
  };
  // the barrier at the top of each half: the staged chunk is in, and every
  // wave is done with the other buffer and with cs.  The next chunk is staged
  // unconditionally (clamped into the row; one spare chunk at the end), so
  // the loads in flight are the same on every path and nothing inside a
  // chunk waits for them.
  {
    float ma[2], mb[2];
    stage2(0, ks0, ma);
    for (int c0 = 0; c0 < nv; c0 += 2 * KL_DC) {
      kl_wait_loads();
      __syncthreads();
      stage2(c0 + KL_DC, ks1, mb);
      grad(c0, ks0, ma);
      if (c0 + KL_DC >= nv) break;
      kl_wait_loads();
      __syncthreads();
      stage2(c0 + 2 * KL_DC, ks0, ma);
      grad(c0 + KL_DC, ks1, mb);
    }
    kl_wait_loads();  // the spare chunk is in before the buffers go
  }
  kl = kl_block_sum(kl, sh);
  if (tid == 0) loss[row] = kl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = dwp[e];
    for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
    dwp[e] = x;
  }
  if (l16 == 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) dws[wave][4 * g4 + e] = dwp[e];
  __syncthreads();
  if (tid < KL_HI)
    dw_idx[(size_t)row * KL_HI + tid] = dws[0][tid] + dws[1][tid] + dws[2][tid] + dws[3][tid];
  float* o = dq_idx + ((size_t)row * KL_HI + l16) * KL_DI + 16 * wave + 4 * g4;
  *(f32x4*)o = dqa;
}

// ---------------------------------------------------------------- dk kernel
// Workgroup (kt, chunk, b): entries [128 kt, + 128) (wave w: 32 from 128 kt +
// 32 w), up to 64 query rows from the chunk, taken two at a time: the pair's
// 2 x 16 heads are the 32 MFMA rows.  Per wave and pair:
//   V = Q2 K^T (4 MFMAs), C = dI w [V > 0], dk^T += Q2^T C (4 MFMAs).
// Sparse form: a row takes part when it selects an entry of the tile (its
// bitmap), dI of the slot from the rank; dense form (DENSE): when it sees
// one (n_vis > 128 kt), dI at [row, entry].
template <bool DENSE>
__global__ void __launch_bounds__(256) idx_kl_dk_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const uint32_t* __restrict__ bm,
    const uint32_t* __restrict__ rank, const float* __restrict__ dIw, int nw, int T, int Nc_cap,
    int topk, const int64_t* __restrict__ q_pos, const int32_t* __restrict__ n_cmp, int m,
    float* __restrict__ dk_idx) {
  constexpr int PB = 32 * 128;  // bytes of a pair's 32 head rows
  constexpr int SB = 2 * 32 * 65 * 4;   // >= PB + 128; the epilogue's rows
  __shared__ __attribute__((aligned(1024))) uint8_t st0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[SB];
  __shared__ int32_t rows_s[KL_RC + 1];
  // the active rows' bitmap words over the tile's 128 entries and their ranks
  // (dense form: n_vis in word 0; row n_rows: the odd row's absent partner,
  // all zero)
  __shared__ uint32_t rows_w[KL_RC + 1][4], rows_r[KL_RC + 1][4];
  __shared__ uint32_t shc[16];
  const int kt = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int j0 = 128 * kt;
  const int jw = j0 + 32 * wave + l32;
  const int c0 = chunk * KL_RC;
  if (c0 >= T) return;  // uniform
  const int nc = min(KL_RC, T - c0);
  {
    bool act = false;
    uint32_t wv[4] = {0u, 0u, 0u, 0u}, rv[4] = {0u, 0u, 0u, 0u};
    if (tid < nc) {
      if (DENSE) {
        const int nvr = n_visible(q_pos[b] + c0 + tid, n_cmp[b], m, Nc_cap);
        wv[0] = (uint32_t)nvr;
        act = nvr > j0;
      } else {
        const size_t wi = ((size_t)b * T + c0 + tid) * nw + (j0 >> 5);
        uint32_t any = 0;
        for (int k = 0; k < 4; ++k)
          if ((j0 >> 5) + k < nw) {
            wv[k] = bm[wi + k];
            rv[k] = rank[wi + k];
            any |= wv[k];
          }
        act = any != 0;
      }
    }
    uint32_t tot;
    const uint32_t at = block_excl_scan(act ? 1u : 0u, shc, tot);
    if (act) {
      rows_s[at] = c0 + tid;
      for (int k = 0; k < 4; ++k) {
        rows_w[at][k] = wv[k];
        rows_r[at][k] = rv[k];
      }
    }
    shc[8] = tot;
  }
  __syncthreads();
  const int n_rows = (int)shc[8];
  if (n_rows == 0) return;  // uniform
  if (tid == 0) {
    rows_s[n_rows] = -1;  // the odd row's partner: none
    for (int k = 0; k < 4; ++k) rows_w[n_rows][k] = rows_r[n_rows][k] = 0u;
  }
  __syncthreads();

  const bool key_in = jw < Nc_cap;
  bf16x8 kf[4];
  {
    const uint16_t* kr = k_idx + ((size_t)b * Nc_cap + (key_in ? jw : 0)) * KL_DI + 8 * h2;
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[s] = *(const bf16x8*)(kr + 16 * s);
  }
  // LDS rows: head row m (0..31) at 128 m, 16-byte chunk c at slot c ^ ((m >> 1) & 7)
  uint32_t aofs[4], tofs[2][2];
  {
#pragma unroll
    for (int s = 0; s < 4; ++s) aofs[s] = (uint32_t)(128 * l32 + 16 * ((2 * s + h2) ^ ((l32 >> 1) & 7)));
    const int gg = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * (gg >> 1) + (jj >> 2) + 8 * e;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int d = 32 * dt + 16 * (gg & 1) + 4 * (jj & 3);
        tofs[dt][e] = (uint32_t)(128 * r + 16 * (((d >> 3)) ^ ((r >> 1) & 7)) + 2 * (d & 7));
      }
    }
  }
  // stage pair (t0, t1): head rows of t0 then t1 (t1 < 0: zeros), then w
  auto stage = [&](int t0, int t1, uint8_t* dst) {
    const int i = wave;  // load instruction i: head rows 8 i .. 8 i + 7
    const int m = 8 * i + (lane >> 3), c = lane & 7;
    const int t = m < 16 ? t0 : t1;
    const int hd = m & 15;
    const int lc = c ^ ((m >> 1) & 7);
    const size_t src_row = ((size_t)b * T + (t >= 0 ? t : t0)) * KL_HI + hd;
    kl_dma(q_idx + src_row * KL_DI + 8 * lc, dst + 1024 * i);
    if (wave == 0 && lane < 8) {
      const int tt = lane < 4 ? t0 : (t1 >= 0 ? t1 : t0);
      kl_dma(w_idx + ((size_t)b * T + tt) * KL_HI + 4 * (lane & 3), dst + PB);
    }
  };
  f32x16 dk[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[dt][r] = 0.0f;
  bool touched = false;

  // dI of this lane's entry for active row ri (0: not selected); the word
  // and rank come from LDS, so one global load remains
  auto fetch_di = [&](int ri) -> float {
    const int t = rows_s[ri];
    float v = 0.0f;
    if (DENSE) {
      if (t >= 0 && key_in && jw < (int)rows_w[ri][0]) v = dIw[((size_t)b * T + t) * Nc_cap + jw];
      return v;
    }
    const uint32_t word = rows_w[ri][wave];  // zero past the bitmap's words
    if (t >= 0 && key_in && ((word >> l32) & 1u)) {
      const uint32_t slot = rows_r[ri][wave] + __popc(word & ((1u << l32) - 1u));
      if (slot < (uint32_t)topk) v = dIw[((size_t)b * T + t) * topk + slot];
    }
    return v;
  };
  auto compute = [&](const uint8_t* sb, const float (&di)[2]) {
    if (!__ballot(di[0] != 0.0f || di[1] != 0.0f)) return;
    touched = true;
    f32x16 va;
#pragma unroll
    for (int r = 0; r < 16; ++r) va[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      va = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(sb + aofs[s]), kf[s], va, 0, 0, 0);
    // register r: head row 8 (r / 4) + 4 h2 + r % 4 (row r >= 8 of the pair's second token)
    const float* ws = (const float*)(sb + PB);
    bf16x8 cb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * h2 + (r & 3);
      const float c = va[r] > 0.0f ? di[r >> 3] * ws[m] : 0.0f;
      cb[r >> 3][r & 7] = (__bf16)c;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const uint32_t ho = (uint32_t)(16 * ks) * 128;
        const u32x2 a1 = __builtin_bit_cast(u32x2, kl_read_tr16(sb + ho + tofs[dt][0]));
        const u32x2 a2 = __builtin_bit_cast(u32x2, kl_read_tr16(sb + ho + tofs[dt][1]));
        const bf16x8 qt = __builtin_bit_cast(bf16x8, u32x4{a1[0], a1[1], a2[0], a2[1]});
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, cb[ks], dk[dt], 0, 0, 0);
      }
  };

  // pair pi = active rows 2 pi, 2 pi + 1; its dI values are fetched while the
  // previous pair computes
  const int npairs = (n_rows + 1) / 2;
  stage(rows_s[0], rows_s[1], st0);
  float di_cur[2] = {fetch_di(0), fetch_di(1)};
  for (int pi = 0; pi < npairs; pi += 2) {
    kl_wait_loads();
    __syncthreads();
    float di_nxt[2] = {0.0f, 0.0f};
    if (pi + 1 < npairs) {
      stage(rows_s[2 * pi + 2], rows_s[2 * pi + 3], st1);
      di_nxt[0] = fetch_di(2 * pi + 2);
      di_nxt[1] = fetch_di(2 * pi + 3);
    }
    compute(st0, di_cur);
    if (pi + 1 >= npairs) break;
    kl_wait_loads();
    __syncthreads();
    di_cur[0] = di_cur[1] = 0.0f;
    if (pi + 2 < npairs) {
      stage(rows_s[2 * pi + 4], rows_s[2 * pi + 5], st0);
      di_cur[0] = fetch_di(2 * pi + 4);
      di_cur[1] = fetch_di(2 * pi + 5);
    }
    compute(st1, di_nxt);
  }
  // dk^T (entry jw on columns, dims 32 dt + 8 (r / 4) + 4 h2 + r % 4)
  // through LDS into entry rows (stride 65 floats), then atomics of 64
  // consecutive floats (one entry row) per instruction
  __syncthreads();  // every wave is done with the staging buffers
  float* red = (float*)(wave < 2 ? st0 : st1) + (wave & 1) * 32 * 65;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[l32 * 65 + 32 * dt + 8 * (r >> 2) + 4 * h2 + (r & 3)] = dk[dt][r];
  __syncthreads();
  const int nkeys = min(32, Nc_cap - (j0 + 32 * wave));  // uniform
  if (touched) {
    float* gk0 = dk_idx + ((size_t)b * Nc_cap + j0 + 32 * wave) * KL_DI;
    for (int k = 0; k < nkeys; ++k) atomicAdd(gk0 + (size_t)k * KL_DI + lane, red[k * 65 + lane]);
  }
}

}  // namespace csa

// ---------------------------------------------------------------- host side
namespace csa_host {
using namespace csa;

static size_t kl_al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t indexer_kl_ws_bytes(int B, int T, int Nc_cap, int topk) {
  const size_t rows = (size_t)B * T, nw = ((size_t)Nc_cap + 31) / 32;
  return kl_al256(rows * topk * sizeof(float)) + 2 * kl_al256(rows * nw * sizeof(uint32_t));
}

hipError_t launch_indexer_kl_bwd(const IndexerKlArgs& a, hipStream_t s) {
  const int rows = a.B * a.T;
  const int nw = (a.Nc_cap + 31) / 32;
  char* ws = (char*)a.ws;
  float* dIw = (float*)ws;
  ws += kl_al256((size_t)rows * a.topk * sizeof(float));
  uint32_t* bm = (uint32_t*)ws;
  uint32_t* rank = (uint32_t*)(ws + kl_al256((size_t)rows * nw * sizeof(uint32_t)));
  const size_t nk = (size_t)a.B * a.Nc_cap * KL_DI;
  hipError_t e = launch_zero_f32(a.dk_idx, nk, s);
  if (e != hipSuccess) return e;
  if (a.topk > 0 && a.Nc_cap > 0) {
    e = launch_sel_bitmap(a.idx, rows, a.topk, a.Nc_cap, bm, rank, s);
    if (e != hipSuccess) return e;
  }
#define CSA_KL_ROW(TW_)                                                                      \
  idx_kl_row_kernel<TW_><<<rows, 256, 0, s>>>((const uint16_t*)a.q_idx, a.w_idx,           \
                                              (const uint16_t*)a.k_idx, a.idx, a.mass,     \
                                              a.grad_scale, a.T, a.Nc_cap, a.topk, a.loss, \
                                              a.dq_idx, a.dw_idx, dIw)
  if (a.topk <= 512) CSA_KL_ROW(8);
  else CSA_KL_ROW(KL_TOPK_MAX / 64);
#undef CSA_KL_ROW
  if (a.topk > 0 && a.Nc_cap > 0)
    idx_kl_dk_kernel<false><<<dim3((a.Nc_cap + 127) / 128, (a.T + KL_RC - 1) / KL_RC, a.B), 256,
                              0, s>>>((const uint16_t*)a.q_idx, a.w_idx, (const uint16_t*)a.k_idx,
                                      bm, rank, dIw, nw, a.T, a.Nc_cap, a.topk, nullptr, nullptr,
                                      1, a.dk_idx);
  return hipGetLastError();
}

size_t indexer_kl_dense_ws_bytes(int B, int T, int Nc_cap) {
  return kl_al256((size_t)B * T * Nc_cap * sizeof(float));
}

hipError_t launch_indexer_kl_dense_bwd(const IndexerKlArgs& a, hipStream_t s) {
  const int rows = a.B * a.T;
  float* dIw = (float*)a.ws;
  hipError_t e = launch_zero_f32(a.dk_idx, (size_t)a.B * a.Nc_cap * KL_DI, s);
  if (e != hipSuccess) return e;
  idx_kl_dense_row_kernel<<<rows, 256, 0, s>>>(
      (const uint16_t*)a.q_idx, a.w_idx, (const uint16_t*)a.k_idx, a.mass, a.grad_scale, a.q_pos,
      a.n_cmp, a.T, a.Nc_cap, a.m, a.loss, a.dq_idx, a.dw_idx, dIw);
  if (a.Nc_cap > 0)
    idx_kl_dk_kernel<true><<<dim3((a.Nc_cap + 127) / 128, (a.T + KL_RC - 1) / KL_RC, a.B), 256,
                             0, s>>>((const uint16_t*)a.q_idx, a.w_idx, (const uint16_t*)a.k_idx,
                                     nullptr, nullptr, dIw, 0, a.T, a.Nc_cap, 0, a.q_pos, a.n_cmp,
                                     a.m, a.dk_idx);
  return hipGetLastError();
}

}  // namespace csa_host
