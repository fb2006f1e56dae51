// C ABI of libcsa: argument validation, workspace sizing and dispatch to the
// gfx950 kernels.  Every check runs on the host before any launch; nothing is
// allocated and nothing synchronises.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <algorithm>
#include <climits>
#include "common.h"

namespace {

thread_local char g_err[512];

csa_status_t fail(csa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

csa_status_t ok() {
  g_err[0] = 0;
  return CSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

csa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace {
// Validates an optional page table; null means the unpaged layout.
csa_status_t check_pages(const char* fn, const csa_page_table_t* pg, int Nc_cap,
                         csa::PageTable& out) {
  out = csa::PageTable{nullptr, 0, 0, 0};
  if (!pg) return CSA_OK;
  if (!pg->block_table) return fail(CSA_E_ARG, "%s: pages->block_table is required", fn);
  const int ps = pg->page_size;
  if (ps < 16 || ps > (1 << 20) || (ps & (ps - 1)))
    return fail(CSA_E_ARG, "%s: page_size must be a power of two in [16, 2^20] (got %d)", fn, ps);
  if (pg->max_pages < 1 || pg->n_pages < 1)
    return fail(CSA_E_ARG, "%s: max_pages and n_pages must be >= 1", fn);
  if ((int64_t)pg->max_pages * ps < (int64_t)Nc_cap)
    return fail(CSA_E_ARG, "%s: Nc_cap %d exceeds max_pages * page_size", fn, Nc_cap);
  if ((int64_t)pg->n_pages * ps > (int64_t)1 << 30)
    return fail(CSA_E_UNSUPPORTED, "%s: pools hold at most 2^30 rows", fn);
  int lg = 0;
  while ((1 << lg) < ps) ++lg;
  out = csa::PageTable{pg->block_table, lg, pg->max_pages, pg->n_pages};
  return CSA_OK;
}
}  // namespace

extern "C" {

const char* csa_status_string(csa_status_t s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_E_ARG: return "invalid argument";
    case CSA_E_UNSUPPORTED: return "unsupported shape or dtype";
    case CSA_E_WORKSPACE: return "workspace too small";
    case CSA_E_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* csa_last_error(void) { return g_err; }

size_t csa_compress_workspace_size(int B, int L, int d_model, int E, int m, int overlap,
                                   csa_dtype_t in_dt) {
  if (B <= 0 || L <= 0 || d_model <= 0 || E <= 0) return 0;
  return csa_host::compress_ws_bytes(B, L, d_model, E, m, overlap, in_dt);
}

static csa_status_t compress_impl(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                          const int64_t* pos0, const void* x, const void* w_kv,
                          const void* w_gate, csa_dtype_t in_dt, const float* ape,
                          const float* state_in, float* state_out, void* out, void* out_scale,
                          csa_dtype_t out_dt, int Nc_cap, void* workspace, size_t ws_bytes,
                          hipStream_t stream, const csa_page_table_t* pages) {
  if (B <= 0 || L <= 0 || d_model <= 0 || E <= 0 || Nc_cap < 0)
    return fail(CSA_E_ARG, "csa_compress: B, L, d_model, E must be > 0 and Nc_cap >= 0");
  if (m < 1) return fail(CSA_E_ARG, "csa_compress: m must be >= 1 (got %d)", m);
  if (overlap != 0 && overlap != 1) return fail(CSA_E_ARG, "csa_compress: overlap must be 0 or 1");
  if (rotate != 0 && rotate != 1) return fail(CSA_E_ARG, "csa_compress: rotate must be 0 or 1");
  if (rotate && (E & (E - 1)))
    return fail(CSA_E_ARG, "csa_compress: rotate needs E a power of two (got %d)", E);
  if (!pos0 || !x || !w_kv || !w_gate || !out)
    return fail(CSA_E_ARG, "csa_compress: pos0, x, w_kv, w_gate and out are required");
  if (state_in && state_in == state_out)
    return fail(CSA_E_ARG, "csa_compress: state_out must not alias state_in");
  if (in_dt != CSA_DT_F32 && in_dt != CSA_DT_BF16)
    return fail(CSA_E_UNSUPPORTED, "csa_compress: in_dt must be F32 or BF16");
  if (out_dt != CSA_DT_F32 && out_dt != CSA_DT_BF16 && out_dt != CSA_DT_FP8E4M3 &&
      out_dt != CSA_DT_MXFP4)
    return fail(CSA_E_ARG, "csa_compress: bad out_dt %d", (int)out_dt);
  if ((out_dt == CSA_DT_FP8E4M3 || out_dt == CSA_DT_MXFP4) && !out_scale)
    return fail(CSA_E_ARG, "csa_compress: fp8 and mxfp4 outputs need out_scale");
  if (out_dt == CSA_DT_MXFP4 && E % 32 != 0)
    return fail(CSA_E_UNSUPPORTED, "csa_compress: mxfp4 output needs E %% 32 == 0 (got %d)", E);
  if (E > 1024) return fail(CSA_E_UNSUPPORTED, "csa_compress: E > 1024");
  if (in_dt == CSA_DT_BF16 && (d_model % 64 != 0 || !aligned16(x) || !aligned16(w_kv) ||
                               !aligned16(w_gate)))
    return fail(CSA_E_UNSUPPORTED,
                "csa_compress: bf16 needs d_model %% 64 == 0 and 16-byte aligned x and weights");
  const size_t need = csa_host::compress_ws_bytes(B, L, d_model, E, m, overlap, in_dt);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "csa_compress: workspace %zu < %zu bytes", ws_bytes, need);
  csa::PageTable pt;
  const csa_status_t pst = check_pages("csa_compress", pages, Nc_cap, pt);
  if (pst != CSA_OK) return pst;
  csa_host::CompressArgs a{B, L, d_model, E, m, overlap, rotate, Nc_cap, pos0, x, w_kv, w_gate,
                           in_dt, out_dt, ape, state_in, state_out, out, out_scale, workspace};
  a.pages = pt;
  return hip_status(csa_host::launch_compress(a, stream), "csa_compress launch");
}

csa_status_t csa_compress(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                          const int64_t* pos0, const void* x, const void* w_kv,
                          const void* w_gate, csa_dtype_t in_dt, const float* ape,
                          const float* state_in, float* state_out, void* out, void* out_scale,
                          csa_dtype_t out_dt, int Nc_cap, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  return compress_impl(B, L, d_model, E, m, overlap, rotate, pos0, x, w_kv, w_gate, in_dt, ape,
                       state_in, state_out, out, out_scale, out_dt, Nc_cap, workspace, ws_bytes,
                       stream, nullptr);
}

csa_status_t csa_compress_paged(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                                const int64_t* pos0, const void* x, const void* w_kv,
                                const void* w_gate, csa_dtype_t in_dt, const float* ape,
                                const float* state_in, float* state_out, void* out,
                                void* out_scale, csa_dtype_t out_dt, int Nc_cap,
                                const csa_page_table_t* pages, void* workspace, size_t ws_bytes,
                                hipStream_t stream) {
  if (!pages) return fail(CSA_E_ARG, "csa_compress_paged: pages is required");
  return compress_impl(B, L, d_model, E, m, overlap, rotate, pos0, x, w_kv, w_gate, in_dt, ape,
                       state_in, state_out, out, out_scale, out_dt, Nc_cap, workspace, ws_bytes,
                       stream, pages);
}

size_t csa_indexer_topk_workspace_size(int B, int T, int H_I, int d_I, int Nc_cap, int topk,
                                       csa_dtype_t qk_dt) {
  if (B <= 0 || T <= 0 || Nc_cap <= 0) return 0;
  return csa_host::indexer_ws_bytes(B, T, H_I, d_I, Nc_cap, topk, qk_dt);
}

static csa_status_t indexer_impl(int B, int T, int H_I, int d_I, int Nc_cap, int m, int topk,
                                 const int64_t* q_pos, const int32_t* n_cmp, const void* q_idx,
                                 const void* q_scale, const float* w_idx, const void* k_idx,
                                 const void* k_scale, csa_dtype_t qk_dt, int32_t* idx_out,
                                 float* score_out, void* workspace, size_t ws_bytes,
                                 hipStream_t stream, const csa_page_table_t* pages) {
  if (B <= 0 || T <= 0 || H_I <= 0 || d_I <= 0 || Nc_cap < 0 || topk < 0)
    return fail(CSA_E_ARG, "csa_indexer_topk: B, T, H_I, d_I must be > 0; Nc_cap, topk >= 0");
  if (m < 1) return fail(CSA_E_ARG, "csa_indexer_topk: m must be >= 1");
  if (topk == 0) return ok();  // nothing to select, nothing to write
  if (!q_pos || !n_cmp || !q_idx || !w_idx || !idx_out || (Nc_cap > 0 && !k_idx))
    return fail(CSA_E_ARG, "csa_indexer_topk: missing required pointer");
  if ((qk_dt == CSA_DT_FP8E4M3 || qk_dt == CSA_DT_MXFP4) &&
      (!q_scale || (Nc_cap > 0 && !k_scale)))
    return fail(CSA_E_ARG, "csa_indexer_topk: fp8 and mxfp4 need q_scale and k_scale");
  if (topk > 8192) return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk: topk > 8192");
  if (Nc_cap > 1024 * 2048) return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk: Nc_cap > 2^21");
  if (qk_dt == CSA_DT_F32) {
    if (!((H_I == 4 && d_I == 32) || (H_I == 16 && d_I == 64)))
      return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk: f32 needs (H_I, d_I) in {(4,32),(16,64)}");
  } else if (qk_dt == CSA_DT_BF16 || qk_dt == CSA_DT_FP8E4M3 || qk_dt == CSA_DT_MXFP4) {
    if (H_I != 16 || d_I != 64)
      return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk: bf16/fp8/mxfp4 need H_I = 16, d_I = 64");
    if (!aligned16(q_idx) || (Nc_cap > 0 && !aligned16(k_idx)))
      return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk: q_idx and k_idx must be 16-byte aligned");
    if (qk_dt == CSA_DT_BF16 && Nc_cap > 8192 && T != 1)
      return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk: bf16 rows longer than 8192 need T == 1");
  } else {
    return fail(CSA_E_ARG, "csa_indexer_topk: bad qk_dt %d", (int)qk_dt);
  }
  const size_t need = csa_host::indexer_ws_bytes(B, T, H_I, d_I, Nc_cap, topk, qk_dt);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "csa_indexer_topk: workspace %zu < %zu bytes", ws_bytes, need);
  csa::PageTable pt;
  const csa_status_t pst = check_pages("csa_indexer_topk", pages, Nc_cap, pt);
  if (pst != CSA_OK) return pst;
  if (pages && qk_dt == CSA_DT_F32)
    return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk_paged: paged keys need BF16, FP8E4M3 or MXFP4");
  csa_host::IndexerArgs a{B, T, H_I, d_I, Nc_cap, m, topk, q_pos, n_cmp, q_idx, q_scale, w_idx,
                          k_idx, k_scale, qk_dt, idx_out, score_out, workspace};
  a.pages = pt;
  return hip_status(csa_host::launch_indexer_topk(a, stream), "csa_indexer_topk launch");
}

csa_status_t csa_indexer_topk(int B, int T, int H_I, int d_I, int Nc_cap, int m, int topk,
                              const int64_t* q_pos, const int32_t* n_cmp, const void* q_idx,
                              const void* q_scale, const float* w_idx, const void* k_idx,
                              const void* k_scale, csa_dtype_t qk_dt, int32_t* idx_out,
                              float* score_out, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  return indexer_impl(B, T, H_I, d_I, Nc_cap, m, topk, q_pos, n_cmp, q_idx, q_scale, w_idx, k_idx,
                      k_scale, qk_dt, idx_out, score_out, workspace, ws_bytes, stream, nullptr);
}

csa_status_t csa_indexer_topk_paged(int B, int T, int H_I, int d_I, int Nc_cap, int m, int topk,
                                    const int64_t* q_pos, const int32_t* n_cmp,
                                    const void* q_idx, const void* q_scale, const float* w_idx,
                                    const void* k_idx, const void* k_scale, csa_dtype_t qk_dt,
                                    const csa_page_table_t* pages, int32_t* idx_out,
                                    float* score_out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!pages) return fail(CSA_E_ARG, "csa_indexer_topk_paged: pages is required");
  return indexer_impl(B, T, H_I, d_I, Nc_cap, m, topk, q_pos, n_cmp, q_idx, q_scale, w_idx, k_idx,
                      k_scale, qk_dt, idx_out, score_out, workspace, ws_bytes, stream, pages);
}

static csa_status_t check_attn(const char* fn, int B, int T, int H, int D, int window,
                               const int64_t* q_pos, const void* q, const void* kv_cmp, int Nc_cap,
                               const void* kv_raw, int R_cap, const int64_t* raw_base,
                               csa_dtype_t dt, void* out) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || window < 0 || Nc_cap < 0 || R_cap < 0)
    return fail(CSA_E_ARG, "%s: B, T, H, D must be > 0; window, Nc_cap, R_cap >= 0", fn);
  if (!q_pos || !q || !out || !raw_base || (Nc_cap > 0 && !kv_cmp) || (R_cap > 0 && !kv_raw))
    return fail(CSA_E_ARG, "%s: missing required pointer", fn);
  if (dt == CSA_DT_F32) {
    if (D != 64 && D != 128) return fail(CSA_E_UNSUPPORTED, "%s: f32 needs D in {64, 128}", fn);
  } else if (dt == CSA_DT_BF16) {
    if (D != 128 || (H != 32 && H != 64))
      return fail(CSA_E_UNSUPPORTED, "%s: bf16 needs D = 128 and H in {32, 64}", fn);
    if (!aligned16(q) || (kv_cmp && !aligned16(kv_cmp)) || (kv_raw && !aligned16(kv_raw)) ||
        !aligned16(out))
      return fail(CSA_E_UNSUPPORTED, "%s: bf16 tensors must be 16-byte aligned", fn);
    if (Nc_cap > (1 << 23) || R_cap > (1 << 23))
      return fail(CSA_E_UNSUPPORTED, "%s: bf16 caches hold at most 2^23 rows", fn);
  } else {
    return fail(CSA_E_UNSUPPORTED, "%s: dt must be F32 or BF16", fn);
  }
  return CSA_OK;
}

size_t csa_sparse_attn_workspace_size(int B, int T, int H, int D, int topk, int window) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0) return 0;
  return csa_host::attn_ws_bytes(B, T, H, D, topk + window, true);
}

size_t csa_sparse_attn_paged_workspace_size(int B, int T, int H, int D, int topk, int window) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || topk < 0) return 0;
  return csa_host::attn_ws_bytes(B, T, H, D, topk + window, true) +
         (size_t)B * T * topk * sizeof(int32_t);
}

static csa_status_t sparse_attn_impl(int B, int T, int H, int D, int topk, int window,
                                     float scale, const float* sink, const int64_t* q_pos,
                                     const void* q, const void* kv_cmp, int Nc_cap,
                                     const int32_t* idx, const void* kv_raw, int R_cap,
                                     const int64_t* raw_base, csa_dtype_t dt, void* out,
                                     float* lse, void* workspace, size_t ws_bytes,
                                     hipStream_t stream, const csa_page_table_t* pages) {
  csa::PageTable pt;
  csa_status_t st = check_pages("csa_sparse_attn", pages, Nc_cap, pt);
  if (st != CSA_OK) return st;
  // a paged kv_cmp is the pool: its row count is what the kernels bound
  const int cmp_rows =
      pages ? (int)std::min<int64_t>((int64_t)pages->n_pages * pages->page_size, INT32_MAX)
            : Nc_cap;
  st = check_attn("csa_sparse_attn", B, T, H, D, window, q_pos, q, kv_cmp, cmp_rows, kv_raw,
                  R_cap, raw_base, dt, out);
  if (st != CSA_OK) return st;
  if (topk < 0) return fail(CSA_E_ARG, "csa_sparse_attn: topk must be >= 0");
  if (topk > 0 && !idx) return fail(CSA_E_ARG, "csa_sparse_attn: idx is required when topk > 0");
  if (dt == CSA_DT_BF16 && !csa_host::attn_supported(B, T, H, topk + window, true))
    return fail(CSA_E_UNSUPPORTED, "csa_sparse_attn: topk + window too large for %d rows", B * T);
  const size_t need =
      pages ? csa_sparse_attn_paged_workspace_size(B, T, H, D, topk, window)
            : (dt == CSA_DT_F32 ? 0 : csa_host::attn_ws_bytes(B, T, H, D, topk + window, true));
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "csa_sparse_attn: workspace %zu < %zu bytes", ws_bytes, need);
  csa_host::AttnArgs a{B, T, H, D, topk, window, 1, Nc_cap, R_cap, false, scale, sink, q_pos,
                       nullptr, q, kv_cmp, idx, kv_raw, raw_base, dt, out, lse, workspace};
  a.pages = pt;
  return hip_status(csa_host::launch_attn(a, stream), "csa_sparse_attn launch");
}

csa_status_t csa_sparse_attn(int B, int T, int H, int D, int topk, int window, float scale,
                             const float* sink, const int64_t* q_pos, const void* q,
                             const void* kv_cmp, int Nc_cap,
                             const int32_t* idx, const void* kv_raw, int R_cap,
                             const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  return sparse_attn_impl(B, T, H, D, topk, window, scale, sink, q_pos, q, kv_cmp, Nc_cap, idx,
                          kv_raw, R_cap, raw_base, dt, out, lse, workspace, ws_bytes, stream,
                          nullptr);
}

csa_status_t csa_sparse_attn_paged(int B, int T, int H, int D, int topk, int window, float scale,
                                   const float* sink, const int64_t* q_pos, const void* q,
                                   const void* kv_cmp, int Nc_cap, const csa_page_table_t* pages,
                                   const int32_t* idx, const void* kv_raw, int R_cap,
                                   const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!pages) return fail(CSA_E_ARG, "csa_sparse_attn_paged: pages is required");
  return sparse_attn_impl(B, T, H, D, topk, window, scale, sink, q_pos, q, kv_cmp, Nc_cap, idx,
                          kv_raw, R_cap, raw_base, dt, out, lse, workspace, ws_bytes, stream,
                          pages);
}

size_t hca_dense_attn_workspace_size(int B, int T, int H, int D, int Nc_cap, int window) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0) return 0;
  return csa_host::attn_ws_bytes(B, T, H, D, Nc_cap + window, false);
}

csa_status_t hca_dense_attn(int B, int T, int H, int D, int m, int window, float scale,
                            const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                            const void* q,
                            const void* kv_cmp, int Nc_cap, const void* kv_raw, int R_cap,
                            const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
  csa_status_t st = check_attn("hca_dense_attn", B, T, H, D, window, q_pos, q, kv_cmp, Nc_cap,
                               kv_raw, R_cap, raw_base, dt, out);
  if (st != CSA_OK) return st;
  if (m < 1) return fail(CSA_E_ARG, "hca_dense_attn: m must be >= 1");
  if (!n_cmp) return fail(CSA_E_ARG, "hca_dense_attn: n_cmp is required");
  const size_t need =
      dt == CSA_DT_F32 ? 0 : csa_host::attn_ws_bytes(B, T, H, D, Nc_cap + window, false);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "hca_dense_attn: workspace %zu < %zu bytes", ws_bytes, need);
  csa_host::AttnArgs a{B, T, H, D, 0, window, m, Nc_cap, R_cap, true, scale, sink, q_pos,
                       n_cmp, q, kv_cmp, nullptr, kv_raw, raw_base, dt, out, lse, workspace};
  return hip_status(csa_host::launch_attn(a, stream), "hca_dense_attn launch");
}

}  // extern "C"
