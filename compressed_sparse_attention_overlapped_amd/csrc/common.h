// Internal helpers shared by the gfx950 kernels of libcsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// ---- scalar format conversions -------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// OCP e4m3 code -> fp32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  uint32_t s = (uint32_t)(c & 0x80) << 24;
  uint32_t e = (c >> 3) & 15, m = c & 7;
  float v;
  if (e == 0)
    v = (float)m * 0.001953125f;  // m * 2^-9
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(v) | s);
}

// fp32 pair -> two e4m3 codes (round to nearest even).  The hardware
// conversion turns magnitudes >= 464 into NaN, so values are clamped to the
// largest finite code first (saturating conversion).
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Order-preserving map of an fp32 score to an unsigned key (larger score ->
// larger key).  -0 is folded onto +0 so equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Typed loads of one element as fp32.
template <int DT> __device__ __forceinline__ float ld_elem(const void* p, size_t i);
template <> __device__ __forceinline__ float ld_elem<CSA_DT_F32>(const void* p, size_t i) {
  return ((const float*)p)[i];
}
template <> __device__ __forceinline__ float ld_elem<CSA_DT_BF16>(const void* p, size_t i) {
  return bf16_to_f32(((const uint16_t*)p)[i]);
}
template <> __device__ __forceinline__ float ld_elem<CSA_DT_FP8E4M3>(const void* p, size_t i) {
  return e4m3_to_f32(((const uint8_t*)p)[i]);
}

// Visible compressed entries of a query at absolute position t.
__device__ __forceinline__ int n_visible(int64_t t, int32_t n_cmp, int m, int cap) {
  int64_t n = t < 0 ? 0 : (t + 1) / m;
  if (n > n_cmp) n = n_cmp;
  if (n > cap) n = cap;
  return n < 0 ? 0 : (int)n;
}

// ---- wave helpers ---------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Value of lane l ^ 32 (resp. l ^ 16) through the gfx950 permlane swaps, a
// VALU path instead of the LDS crossbar of a shuffle.  permlane32_swap(x, x)
// gives (x[l], x[l - 32]) for l >= 32 and (x[l], x[l + 32]) as its second
// word for l < 32 - in lane order: word 0 = l < 32 ? x[l] : x[l - 32],
// word 1 = l < 32 ? x[l + 32] : x[l]; the 16-lane swap does the same between
// the even and odd rows of 16 lanes.
__device__ __forceinline__ float lane_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
// max / sum of a value and its partner: both words of the swap, no select
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- paged compressed caches ---------------------------------------------
// Logical entry j of sequence b lives in pool row
//   (block_table[b * max_pages + j / 2^page_log2] * 2^page_log2) + j % 2^page_log2;
// a null block_table means the unpaged layout [B, Nc_cap, row].  Page ids are
// clamped into [0, n_pages) so that a stale table entry cannot leave the pool.
struct PageTable {
  const int32_t* block_table;
  int page_log2, max_pages, n_pages;
};
__device__ __forceinline__ int64_t paged_row(const PageTable& pt, int b, int j) {
  int pg = pt.block_table[(size_t)b * pt.max_pages + (j >> pt.page_log2)];
  pg = min(max(pg, 0), pt.n_pages - 1);
  return ((int64_t)pg << pt.page_log2) | (int64_t)(j & ((1 << pt.page_log2) - 1));
}

}  // namespace csa

// ---- host-side launch entry points (defined in the kernel sources) --------

namespace csa_host {

struct CompressArgs {
  int B, L, d_model, E, m, overlap, rotate, Nc_cap;
  const int64_t* pos0;
  const void* x;
  const void* w_kv;
  const void* w_gate;
  csa_dtype_t in_dt, out_dt;
  const float* ape;
  const float* state_in;
  float* state_out;
  void* out;
  void* out_scale;
  void* ws;
  csa::PageTable pages;  // block_table null: unpaged out
};
size_t compress_ws_bytes(int B, int L, int d_model, int E, int m, int overlap, csa_dtype_t in_dt);
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

struct IndexerArgs {
  int B, T, H_I, d_I, Nc_cap, m, topk;
  const int64_t* q_pos;
  const int32_t* n_cmp;
  const void* q_idx;
  const void* q_scale;  // fp32 (e4m3) or E8M0 bytes (mxfp4)
  const float* w_idx;
  const void* k_idx;
  const void* k_scale;
  csa_dtype_t dt;
  int32_t* idx_out;
  float* score_out;
  void* ws;
  csa::PageTable pages;  // block_table null: unpaged k_idx / k_scale
};
size_t indexer_ws_bytes(int B, int T, int H_I, int d_I, int Nc_cap, int topk, csa_dtype_t dt);
hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t s);

struct AttnArgs {
  int B, T, H, D, topk, window, m, Nc_cap, R_cap;
  bool dense;  // HCA: every visible entry instead of an index list
  float scale;
  const float* sink;  // [H] per-head sink logits or null
  const int64_t* q_pos;
  const int32_t* n_cmp;
  const void* q;
  const void* kv_cmp;
  const int32_t* idx;
  const void* kv_raw;
  const int64_t* raw_base;
  csa_dtype_t dt;
  void* out;
  float* lse;
  void* ws;
  csa::PageTable pages;  // block_table null: unpaged kv_cmp (sparse only)
};
size_t attn_ws_bytes(int B, int T, int H, int D, int keys_per_row, bool sparse);
bool attn_supported(int B, int T, int H, int keys_per_row, bool sparse);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);

}  // namespace csa_host
