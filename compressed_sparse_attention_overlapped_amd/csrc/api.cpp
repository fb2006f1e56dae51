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
                          hipStream_t stream, const csa_page_table_t* pages,
                          const csa_compress_opts_t* opts) {
  csa_host::EntryOpts eo{nullptr, 0.0f, 0, 0, 0, 10000.0f};
  if (opts) {
    const int R = opts->rope_dim;
    if (R < 0 || (R & 1) || opts->rope_offset < 0 || (int64_t)opts->rope_offset + R > E)
      return fail(CSA_E_ARG,
                  "csa_compress: rope_dim must be even and [rope_offset, rope_offset + rope_dim) "
                  "inside [0, E)");
    if (R > 0 && !(opts->rope_base > 0.0f))
      return fail(CSA_E_ARG, "csa_compress: rope_base must be > 0");
    if (opts->rope_interleaved != 0 && opts->rope_interleaved != 1)
      return fail(CSA_E_ARG, "csa_compress: rope_interleaved must be 0 or 1");
    if (opts->norm_weight && !(opts->norm_eps >= 0.0f))
      return fail(CSA_E_ARG, "csa_compress: norm_eps must be >= 0");
    eo = csa_host::EntryOpts{opts->norm_weight, opts->norm_eps, R, opts->rope_offset,
                             opts->rope_interleaved, opts->rope_base};
  }
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
  a.opt = eo;
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
                       stream, nullptr, nullptr);
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
                       stream, pages, nullptr);
}

csa_status_t csa_compress_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                             const int64_t* pos0, const void* x, const void* w_kv,
                             const void* w_gate, csa_dtype_t in_dt, const float* ape,
                             const float* state_in, float* state_out, void* out,
                             void* out_scale, csa_dtype_t out_dt, int Nc_cap,
                             const csa_page_table_t* pages, const csa_compress_opts_t* opts,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  return compress_impl(B, L, d_model, E, m, overlap, rotate, pos0, x, w_kv, w_gate, in_dt, ape,
                       state_in, state_out, out, out_scale, out_dt, Nc_cap, workspace, ws_bytes,
                       stream, pages, opts);
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
                                     hipStream_t stream, const csa_page_table_t* pages,
                                     const csa_page_table_t* raw_pages) {
  csa::PageTable pt, rpt;
  csa_status_t st = check_pages("csa_sparse_attn", pages, Nc_cap, pt);
  if (st != CSA_OK) return st;
  st = check_pages("csa_sparse_attn (window)", raw_pages, R_cap, rpt);
  if (st != CSA_OK) return st;
  // a paged cache is its pool: its row count is what the kernels bound
  const int cmp_rows =
      pages ? (int)std::min<int64_t>((int64_t)pages->n_pages * pages->page_size, INT32_MAX)
            : Nc_cap;
  const int raw_rows =
      raw_pages
          ? (int)std::min<int64_t>((int64_t)raw_pages->n_pages * raw_pages->page_size, INT32_MAX)
          : R_cap;
  st = check_attn("csa_sparse_attn", B, T, H, D, window, q_pos, q, kv_cmp, cmp_rows, kv_raw,
                  raw_rows, raw_base, dt, out);
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
  a.raw_pages = rpt;
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
                          nullptr, nullptr);
}

csa_status_t csa_sparse_attn_paged(int B, int T, int H, int D, int topk, int window, float scale,
                                   const float* sink, const int64_t* q_pos, const void* q,
                                   const void* kv_cmp, int Nc_cap, const csa_page_table_t* pages,
                                   const int32_t* idx, const void* kv_raw, int R_cap,
                                   const int64_t* raw_base, const csa_page_table_t* raw_pages,
                                   csa_dtype_t dt, void* out, float* lse, void* workspace,
                                   size_t ws_bytes, hipStream_t stream) {
  if (!pages && !raw_pages)
    return fail(CSA_E_ARG, "csa_sparse_attn_paged: pages or raw_pages is required");
  return sparse_attn_impl(B, T, H, D, topk, window, scale, sink, q_pos, q, kv_cmp, Nc_cap, idx,
                          kv_raw, R_cap, raw_base, dt, out, lse, workspace, ws_bytes, stream,
                          pages, raw_pages);
}

csa_status_t csa_sparse_attn_noalloc(int B, int T, int H, int D, int topk, int window,
                                     float scale, const float* sink, const int64_t* q_pos,
                                     const void* q, const void* kv_cmp, int Nc_cap,
                                     const int32_t* idx, const void* kv_raw, int R_cap,
                                     const int64_t* raw_base, csa_dtype_t dt, void* out,
                                     float* lse, hipStream_t stream) {
  csa_status_t st = check_attn("csa_sparse_attn_noalloc", B, T, H, D, window, q_pos, q, kv_cmp,
                               Nc_cap, kv_raw, R_cap, raw_base, dt, out);
  if (st != CSA_OK) return st;
  if (topk < 0) return fail(CSA_E_ARG, "csa_sparse_attn_noalloc: topk must be >= 0");
  if (dt == CSA_DT_BF16 && !csa_host::attn_supported(B, T, H, topk + window, true))
    return fail(CSA_E_UNSUPPORTED, "csa_sparse_attn_noalloc: topk + window too large for %d rows",
                B * T);
  const size_t need =
      dt == CSA_DT_F32 ? 0 : csa_host::attn_ws_bytes(B, T, H, D, topk + window, true);
  const size_t cap = csa_host::noalloc_scratch_bytes();
  if (need > cap)
    return fail(CSA_E_UNSUPPORTED,
                "csa_sparse_attn_noalloc: this call needs %zu bytes of scratch; the static "
                "scratch holds %zu (use csa_sparse_attn with a workspace)", need, cap);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = csa_host::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "csa_sparse_attn_noalloc: scratch address");
  }
  return sparse_attn_impl(B, T, H, D, topk, window, scale, sink, q_pos, q, kv_cmp, Nc_cap, idx,
                          kv_raw, R_cap, raw_base, dt, out, lse, ws, need > 0 ? cap : 0, stream,
                          nullptr, nullptr);
}

size_t csa_sparse_attn_split_workspace_size(int B, int T, int H, int D, int topk, int window) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || topk < 0 || window < 0) return 0;
  if (!csa_host::attn_half_supported(B, T, H, topk, window)) return 0;
  return csa_host::attn_half_ws_bytes(B, T, H, D, topk, window);
}

// One half of csa_sparse_attn taken in two calls (phase 1: the window,
// phase 2: the selected entries and the merge).
static csa_status_t sparse_attn_half(const char* fn, int phase, int B, int T, int H, int D,
                                     int topk, int window, float scale, const float* sink,
                                     const int64_t* q_pos, const void* q, const void* kv_cmp,
                                     int Nc_cap, const int32_t* idx, const void* kv_raw,
                                     int R_cap, const int64_t* raw_base, csa_dtype_t dt,
                                     void* out, float* lse, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  // the window half writes no output: q stands in for out in the checks
  csa_status_t st = check_attn(fn, B, T, H, D, window, q_pos, q, phase == 2 ? kv_cmp : nullptr,
                               phase == 2 ? Nc_cap : 0, kv_raw, R_cap, raw_base, dt,
                               phase == 2 ? out : const_cast<void*>(q));
  if (st != CSA_OK) return st;
  if (topk < 0) return fail(CSA_E_ARG, "%s: topk must be >= 0", fn);
  if (phase == 2 && topk > 0 && !idx) return fail(CSA_E_ARG, "%s: idx is required when topk > 0", fn);
  if (dt != CSA_DT_BF16 || !csa_host::attn_half_supported(B, T, H, topk, window))
    return fail(CSA_E_UNSUPPORTED,
                "%s: needs bf16 with fewer than 1024 query rows and at most 64 splits "
                "(%d rows, topk %d, window %d)", fn, B * T, topk, window);
  const size_t need = csa_host::attn_half_ws_bytes(B, T, H, D, topk, window);
  if (ws_bytes < need || !workspace)
    return fail(CSA_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  csa_host::AttnArgs a{B, T, H, D, topk, window, 1, phase == 2 ? Nc_cap : 0, R_cap, false,
                       scale, sink, q_pos, nullptr, q, phase == 2 ? kv_cmp : nullptr,
                       phase == 2 ? idx : nullptr, kv_raw, raw_base, dt,
                       phase == 2 ? out : nullptr, phase == 2 ? lse : nullptr, workspace};
  a.phase = phase;
  return hip_status(csa_host::launch_attn(a, stream), fn);
}

csa_status_t csa_sparse_attn_window_half(int B, int T, int H, int D, int topk, int window,
                                         float scale, const int64_t* q_pos, const void* q,
                                         const void* kv_raw, int R_cap, const int64_t* raw_base,
                                         csa_dtype_t dt, void* workspace, size_t ws_bytes,
                                         hipStream_t stream) {
  return sparse_attn_half("csa_sparse_attn_window_half", 1, B, T, H, D, topk, window, scale,
                          nullptr, q_pos, q, nullptr, 0, nullptr, kv_raw, R_cap, raw_base, dt,
                          nullptr, nullptr, workspace, ws_bytes, stream);
}

csa_status_t csa_sparse_attn_selected_half(int B, int T, int H, int D, int topk, int window,
                                           float scale, const float* sink, const int64_t* q_pos,
                                           const void* q, const void* kv_cmp, int Nc_cap,
                                           const int32_t* idx, const void* kv_raw, int R_cap,
                                           const int64_t* raw_base, csa_dtype_t dt, void* out,
                                           float* lse, void* workspace, size_t ws_bytes,
                                           hipStream_t stream) {
  return sparse_attn_half("csa_sparse_attn_selected_half", 2, B, T, H, D, topk, window, scale,
                          sink, q_pos, q, kv_cmp, Nc_cap, idx, kv_raw, R_cap, raw_base, dt, out,
                          lse, workspace, ws_bytes, stream);
}

size_t hca_dense_attn_workspace_size(int B, int T, int H, int D, int Nc_cap, int window) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0) return 0;
  return csa_host::attn_ws_bytes(B, T, H, D, Nc_cap + window, false);
}

static csa_status_t hca_impl(int B, int T, int H, int D, int m, int window, float scale,
                             const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                             const void* q, const void* kv_cmp, int Nc_cap, const void* kv_raw,
                             int R_cap, const int64_t* raw_base, csa_dtype_t dt, void* out,
                             float* lse, void* workspace, size_t ws_bytes, hipStream_t stream,
                             const csa_page_table_t* pages, const csa_page_table_t* raw_pages) {
  csa::PageTable pt, rpt;
  csa_status_t st = check_pages("hca_dense_attn", pages, Nc_cap, pt);
  if (st != CSA_OK) return st;
  st = check_pages("hca_dense_attn (window)", raw_pages, R_cap, rpt);
  if (st != CSA_OK) return st;
  const int cmp_rows =
      pages ? (int)std::min<int64_t>((int64_t)pages->n_pages * pages->page_size, INT32_MAX)
            : Nc_cap;
  const int raw_rows =
      raw_pages
          ? (int)std::min<int64_t>((int64_t)raw_pages->n_pages * raw_pages->page_size, INT32_MAX)
          : R_cap;
  st = check_attn("hca_dense_attn", B, T, H, D, window, q_pos, q, kv_cmp, cmp_rows, kv_raw,
                  raw_rows, raw_base, dt, out);
  if (st != CSA_OK) return st;
  if (m < 1) return fail(CSA_E_ARG, "hca_dense_attn: m must be >= 1");
  if (!n_cmp) return fail(CSA_E_ARG, "hca_dense_attn: n_cmp is required");
  const size_t need =
      dt == CSA_DT_F32 ? 0 : csa_host::attn_ws_bytes(B, T, H, D, Nc_cap + window, false);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "hca_dense_attn: workspace %zu < %zu bytes", ws_bytes, need);
  csa_host::AttnArgs a{B, T, H, D, 0, window, m, Nc_cap, R_cap, true, scale, sink, q_pos,
                       n_cmp, q, kv_cmp, nullptr, kv_raw, raw_base, dt, out, lse, workspace};
  a.pages = pt;
  a.raw_pages = rpt;
  return hip_status(csa_host::launch_attn(a, stream), "hca_dense_attn launch");
}

csa_status_t hca_dense_attn(int B, int T, int H, int D, int m, int window, float scale,
                            const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                            const void* q,
                            const void* kv_cmp, int Nc_cap, const void* kv_raw, int R_cap,
                            const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
  return hca_impl(B, T, H, D, m, window, scale, sink, q_pos, n_cmp, q, kv_cmp, Nc_cap, kv_raw,
                  R_cap, raw_base, dt, out, lse, workspace, ws_bytes, stream, nullptr, nullptr);
}

csa_status_t hca_dense_attn_paged(int B, int T, int H, int D, int m, int window, float scale,
                                  const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                                  const void* q, const void* kv_cmp, int Nc_cap,
                                  const csa_page_table_t* pages, const void* kv_raw, int R_cap,
                                  const int64_t* raw_base, const csa_page_table_t* raw_pages,
                                  csa_dtype_t dt, void* out, float* lse, void* workspace,
                                  size_t ws_bytes, hipStream_t stream) {
  if (!pages && !raw_pages)
    return fail(CSA_E_ARG, "hca_dense_attn_paged: pages or raw_pages is required");
  return hca_impl(B, T, H, D, m, window, scale, sink, q_pos, n_cmp, q, kv_cmp, Nc_cap, kv_raw,
                  R_cap, raw_base, dt, out, lse, workspace, ws_bytes, stream, pages, raw_pages);
}

/* ---- packed variable-length sequences --------------------------------- */

csa_status_t csa_build_cmp_cu_seqlens(int n, const int32_t* cu_seqlens, int m,
                                      int32_t* cmp_cu_seqlens, hipStream_t stream) {
  if (n < 1 || m < 1 || !cu_seqlens || !cmp_cu_seqlens)
    return fail(CSA_E_ARG, "csa_build_cmp_cu_seqlens: n, m >= 1 and both arrays are required");
  return hip_status(csa_host::launch_cmp_cu(n, cu_seqlens, m, cmp_cu_seqlens, stream),
                    "csa_build_cmp_cu_seqlens launch");
}

static csa_status_t check_varlen(const char* fn, int n, int total, int max_len,
                                 const int32_t* cu, const int32_t* cmp_cu) {
  if (n < 1 || total < 1 || max_len < 1)
    return fail(CSA_E_ARG, "%s: n, total and max_len must be >= 1", fn);
  if (!cu || !cmp_cu) return fail(CSA_E_ARG, "%s: cu_seqlens and cmp_cu_seqlens are required", fn);
  return CSA_OK;
}

size_t csa_compress_varlen_workspace_size(int total, int d_model, int E, int m, int overlap,
                                          csa_dtype_t in_dt) {
  if (total <= 0 || d_model <= 0 || E <= 0) return 0;
  return csa_host::compress_ws_bytes(1, total, d_model, E, m, overlap, in_dt);
}

csa_status_t csa_compress_varlen(int n, int total, int max_len, int d_model, int E, int m,
                                 int overlap, int rotate, const int32_t* cu_seqlens,
                                 const int32_t* cmp_cu_seqlens, const void* x, const void* w_kv,
                                 const void* w_gate, csa_dtype_t in_dt, const float* ape,
                                 float* state_out, void* out, void* out_scale, csa_dtype_t out_dt,
                                 const csa_compress_opts_t* opts, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  csa_status_t st = check_varlen("csa_compress_varlen", n, total, max_len, cu_seqlens,
                                 cmp_cu_seqlens);
  if (st != CSA_OK) return st;
  static const int64_t zero = 0;  // a stand-in pos0 (packed sequences start at 0)
  const size_t need = csa_host::compress_ws_bytes(1, total, d_model, E, m, overlap, in_dt);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "csa_compress_varlen: workspace %zu < %zu bytes", ws_bytes, need);
  if (m < 1) return fail(CSA_E_ARG, "csa_compress_varlen: m must be >= 1");
  if (overlap != 0 && overlap != 1)
    return fail(CSA_E_ARG, "csa_compress_varlen: overlap must be 0 or 1");
  if (rotate != 0 && rotate != 1) return fail(CSA_E_ARG, "csa_compress_varlen: rotate must be 0 or 1");
  if (rotate && (E & (E - 1)))
    return fail(CSA_E_ARG, "csa_compress_varlen: rotate needs E a power of two (got %d)", E);
  if (!x || !w_kv || !w_gate || !out)
    return fail(CSA_E_ARG, "csa_compress_varlen: x, w_kv, w_gate and out are required");
  if (in_dt != CSA_DT_F32 && in_dt != CSA_DT_BF16)
    return fail(CSA_E_UNSUPPORTED, "csa_compress_varlen: in_dt must be F32 or BF16");
  if (out_dt != CSA_DT_F32 && out_dt != CSA_DT_BF16 && out_dt != CSA_DT_FP8E4M3 &&
      out_dt != CSA_DT_MXFP4)
    return fail(CSA_E_ARG, "csa_compress_varlen: bad out_dt %d", (int)out_dt);
  if ((out_dt == CSA_DT_FP8E4M3 || out_dt == CSA_DT_MXFP4) && !out_scale)
    return fail(CSA_E_ARG, "csa_compress_varlen: fp8 and mxfp4 outputs need out_scale");
  if (out_dt == CSA_DT_MXFP4 && E % 32 != 0)
    return fail(CSA_E_UNSUPPORTED, "csa_compress_varlen: mxfp4 output needs E %% 32 == 0");
  if (E > 1024) return fail(CSA_E_UNSUPPORTED, "csa_compress_varlen: E > 1024");
  if (in_dt == CSA_DT_BF16 && (d_model % 64 != 0 || !aligned16(x) || !aligned16(w_kv) ||
                               !aligned16(w_gate)))
    return fail(CSA_E_UNSUPPORTED,
                "csa_compress_varlen: bf16 needs d_model %% 64 == 0 and 16-byte aligned x and "
                "weights");
  csa_host::EntryOpts eo{nullptr, 0.0f, 0, 0, 0, 10000.0f};
  if (opts) {
    const int R = opts->rope_dim;
    if (R < 0 || (R & 1) || opts->rope_offset < 0 || (int64_t)opts->rope_offset + R > E ||
        (R > 0 && !(opts->rope_base > 0.0f)) ||
        (opts->rope_interleaved != 0 && opts->rope_interleaved != 1) ||
        (opts->norm_weight && !(opts->norm_eps >= 0.0f)))
      return fail(CSA_E_ARG, "csa_compress_varlen: bad rope / norm options");
    eo = csa_host::EntryOpts{opts->norm_weight, opts->norm_eps, R, opts->rope_offset,
                             opts->rope_interleaved, opts->rope_base};
  }
  csa_host::CompressArgs a{n, max_len, d_model, E, m, overlap, rotate, 0, &zero, x, w_kv,
                           w_gate, in_dt, out_dt, ape, nullptr, state_out, out, out_scale,
                           workspace};
  a.opt = eo;
  a.vl = csa::Varlen{cu_seqlens, cmp_cu_seqlens, n};
  a.total_rows = total;
  return hip_status(csa_host::launch_compress(a, stream), "csa_compress_varlen launch");
}

size_t csa_indexer_topk_varlen_workspace_size(int total, int max_cmp, int topk,
                                              csa_dtype_t qk_dt) {
  if (total <= 0 || max_cmp <= 0) return 0;
  return csa_host::indexer_ws_bytes(1, total, 16, 64, max_cmp, topk, qk_dt);
}

csa_status_t csa_indexer_topk_varlen(int n, int total, int max_len, int H_I, int d_I,
                                     int max_cmp, int m, int topk, const int32_t* cu_seqlens,
                                     const int32_t* cmp_cu_seqlens, const void* q_idx,
                                     const float* w_idx, const void* k_idx, csa_dtype_t qk_dt,
                                     int32_t* idx_out, float* score_out, void* workspace,
                                     size_t ws_bytes, hipStream_t stream) {
  csa_status_t st = check_varlen("csa_indexer_topk_varlen", n, total, max_len, cu_seqlens,
                                 cmp_cu_seqlens);
  if (st != CSA_OK) return st;
  if (H_I <= 0 || d_I <= 0 || max_cmp < 0 || topk < 0 || m < 1)
    return fail(CSA_E_ARG, "csa_indexer_topk_varlen: H_I, d_I, m >= 1; max_cmp, topk >= 0");
  if (topk == 0) return ok();
  if (!q_idx || !w_idx || !idx_out || (max_cmp > 0 && !k_idx))
    return fail(CSA_E_ARG, "csa_indexer_topk_varlen: missing required pointer");
  if (topk > 8192) return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk_varlen: topk > 8192");
  if (max_cmp > 1024 * 2048)
    return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk_varlen: max_cmp > 2^21");
  if (qk_dt == CSA_DT_F32) {
    if (!((H_I == 4 && d_I == 32) || (H_I == 16 && d_I == 64)))
      return fail(CSA_E_UNSUPPORTED,
                  "csa_indexer_topk_varlen: f32 needs (H_I, d_I) in {(4,32),(16,64)}");
  } else if (qk_dt == CSA_DT_BF16) {
    if (H_I != 16 || d_I != 64)
      return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk_varlen: bf16 needs H_I = 16, d_I = 64");
    if (!aligned16(q_idx) || (max_cmp > 0 && !aligned16(k_idx)))
      return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk_varlen: q_idx, k_idx 16-byte aligned");
  } else {
    return fail(CSA_E_UNSUPPORTED, "csa_indexer_topk_varlen: qk_dt must be F32 or BF16");
  }
  const size_t need = csa_host::indexer_ws_bytes(1, total, H_I, d_I, max_cmp, topk, qk_dt);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "csa_indexer_topk_varlen: workspace %zu < %zu bytes", ws_bytes,
                need);
  // (max_cmp 0: no sequence has an entry and every row is padding; the
  // kernels run with a one-entry cap and read no key)
  csa_host::IndexerArgs a{n, max_len, H_I, d_I, max_cmp > 0 ? max_cmp : 1, m, topk, nullptr,
                          nullptr, q_idx, nullptr, w_idx, k_idx, nullptr, qk_dt, idx_out,
                          score_out, workspace};
  a.vl = csa::Varlen{cu_seqlens, cmp_cu_seqlens, n};
  a.total_rows = total;
  return hip_status(csa_host::launch_indexer_topk(a, stream), "csa_indexer_topk_varlen launch");
}

size_t csa_sparse_attn_varlen_workspace_size(int total, int H, int D, int topk, int window) {
  if (total <= 0 || H <= 0 || D <= 0) return 0;
  return csa_host::attn_ws_bytes(1, total, H, D, topk + window, true);
}

csa_status_t csa_sparse_attn_varlen(int n, int total, int max_len, int H, int D, int topk,
                                    int window, float scale, const float* sink,
                                    const int32_t* cu_seqlens, const int32_t* cmp_cu_seqlens,
                                    const void* q, const void* kv_cmp, int max_cmp,
                                    const int32_t* idx, const void* kv_raw, csa_dtype_t dt,
                                    void* out, float* lse, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  csa_status_t st = check_varlen("csa_sparse_attn_varlen", n, total, max_len, cu_seqlens,
                                 cmp_cu_seqlens);
  if (st != CSA_OK) return st;
  static const int64_t zero = 0;
  st = check_attn("csa_sparse_attn_varlen", 1, total, H, D, window, &zero, q, kv_cmp, max_cmp,
                  kv_raw, max_len, &zero, dt, out);
  if (st != CSA_OK) return st;
  if (topk < 0) return fail(CSA_E_ARG, "csa_sparse_attn_varlen: topk must be >= 0");
  if (topk > 0 && !idx) return fail(CSA_E_ARG, "csa_sparse_attn_varlen: idx is required");
  if (!kv_raw) return fail(CSA_E_ARG, "csa_sparse_attn_varlen: kv_raw is required");
  if (dt == CSA_DT_BF16 && !csa_host::attn_supported(1, total, H, topk + window, true))
    return fail(CSA_E_UNSUPPORTED, "csa_sparse_attn_varlen: topk + window too large");
  const size_t need =
      dt == CSA_DT_F32 ? 0 : csa_host::attn_ws_bytes(1, total, H, D, topk + window, true);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "csa_sparse_attn_varlen: workspace %zu < %zu bytes", ws_bytes,
                need);
  csa_host::AttnArgs a{n, max_len, H, D, topk, window, 1, max_cmp, max_len, false, scale, sink,
                       nullptr, nullptr, q, kv_cmp, idx, kv_raw, nullptr, dt, out, lse, workspace};
  a.vl = csa::Varlen{cu_seqlens, cmp_cu_seqlens, n};
  a.total_rows = total;
  return hip_status(csa_host::launch_attn(a, stream), "csa_sparse_attn_varlen launch");
}

}  // extern "C"

// ---------------------------------------------------------------- backward

size_t csa_sparse_attn_bwd_workspace_size(int B, int T, int H, int Nc_cap, int R_cap,
                                          int window) {
  if (B <= 0 || T <= 0 || H <= 0 || Nc_cap < 0 || R_cap < 0 || window < 0) return 0;
  return csa_host::attn_bwd_ws_bytes(B, T, H, Nc_cap, R_cap, window, true);
}

size_t hca_dense_attn_bwd_workspace_size(int B, int T, int H, int Nc_cap, int R_cap, int window) {
  if (B <= 0 || T <= 0 || H <= 0 || Nc_cap < 0 || R_cap < 0 || window < 0) return 0;
  return csa_host::attn_bwd_ws_bytes(B, T, H, Nc_cap, R_cap, window, false);
}

static csa_status_t attn_bwd_impl(const char* fn, csa_host::AttnBwdArgs& a, int D,
                                  csa_dtype_t dt, size_t ws_bytes, hipStream_t stream) {
  if (a.B <= 0 || a.T <= 0 || a.H <= 0 || D <= 0 || a.window < 0 || a.Nc_cap < 0 ||
      a.R_cap < 0 || a.topk < 0)
    return fail(CSA_E_ARG, "%s: B, T, H, D must be > 0; window, Nc_cap, R_cap, topk >= 0", fn);
  if (!a.q_pos || !a.q || !a.raw_base || !a.lse || !a.dout || !a.dq)
    return fail(CSA_E_ARG, "%s: q_pos, q, raw_base, lse, dout and dq are required", fn);
  if ((a.Nc_cap > 0 && (!a.kv_cmp || !a.dkv_cmp)) || (a.R_cap > 0 && (!a.kv_raw || !a.dkv_raw)))
    return fail(CSA_E_ARG, "%s: a cache with rows needs its tensor and its gradient", fn);
  if (a.dsink && !a.sink) return fail(CSA_E_ARG, "%s: dsink needs sink", fn);
  if (dt != CSA_DT_BF16) return fail(CSA_E_UNSUPPORTED, "%s: dt must be BF16", fn);
  if (D != 128 || (a.H != 32 && a.H != 64))
    return fail(CSA_E_UNSUPPORTED, "%s: needs D = 128 and H in {32, 64}", fn);
  const void* al[] = {a.q, a.dout, a.kv_cmp, a.kv_raw, a.dq};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(CSA_E_UNSUPPORTED, "%s: tensors must be 16-byte aligned", fn);
  if (a.Nc_cap > (1 << 23) || a.R_cap > (1 << 23))
    return fail(CSA_E_UNSUPPORTED, "%s: caches hold at most 2^23 rows", fn);
  if ((a.T + 63) / 64 > 65535 || a.B > 65535)
    return fail(CSA_E_UNSUPPORTED, "%s: T <= 65535 * 64 and B <= 65535", fn);
  const size_t need =
      csa_host::attn_bwd_ws_bytes(a.B, a.T, a.H, a.Nc_cap, a.R_cap, a.window, !a.dense);
  if (ws_bytes < need || !a.ws)
    return fail(CSA_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return hip_status(csa_host::launch_attn_bwd(a, stream), fn);
}

csa_status_t csa_sparse_attn_bwd(int B, int T, int H, int D, int topk, int window, float scale,
                                 const float* sink, const int64_t* q_pos, const void* q,
                                 const void* kv_cmp, int Nc_cap, const int32_t* idx,
                                 const void* kv_raw, int R_cap, const int64_t* raw_base,
                                 csa_dtype_t dt, const float* lse, const void* dout, float* dq,
                                 float* dkv_cmp, float* dkv_raw, float* dsink, float* attn_mass,
                                 void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (topk > 4096) return fail(CSA_E_UNSUPPORTED, "csa_sparse_attn_bwd: topk > 4096");
  if (Nc_cap > 65536) return fail(CSA_E_UNSUPPORTED, "csa_sparse_attn_bwd: Nc_cap > 65536");
  if (topk > 0 && !idx) return fail(CSA_E_ARG, "csa_sparse_attn_bwd: idx is required when topk > 0");
  csa_host::AttnBwdArgs a{B,      T,      H,       topk,    window,  1,       Nc_cap,
                          R_cap,  false,  scale,   sink,    q_pos,   nullptr, q,
                          kv_cmp, idx,    kv_raw,  raw_base, lse,    dout,    dq,
                          dkv_cmp, dkv_raw, dsink, attn_mass, workspace};
  return attn_bwd_impl("csa_sparse_attn_bwd", a, D, dt, ws_bytes, stream);
}

csa_status_t hca_dense_attn_bwd(int B, int T, int H, int D, int m, int window, float scale,
                                const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                                const void* q, const void* kv_cmp, int Nc_cap, const void* kv_raw,
                                int R_cap, const int64_t* raw_base, csa_dtype_t dt,
                                const float* lse, const void* dout, float* dq, float* dkv_cmp,
                                float* dkv_raw, float* dsink, float* attn_mass, void* workspace,
                                size_t ws_bytes, hipStream_t stream) {
  if (m < 1) return fail(CSA_E_ARG, "hca_dense_attn_bwd: m must be >= 1");
  if (!n_cmp) return fail(CSA_E_ARG, "hca_dense_attn_bwd: n_cmp is required");
  csa_host::AttnBwdArgs a{B,      T,       H,       0,       window,  m,       Nc_cap,
                          R_cap,  true,    scale,   sink,    q_pos,   n_cmp,   q,
                          kv_cmp, nullptr, kv_raw,  raw_base, lse,    dout,    dq,
                          dkv_cmp, dkv_raw, dsink,  attn_mass, workspace};
  return attn_bwd_impl("hca_dense_attn_bwd", a, D, dt, ws_bytes, stream);
}

size_t csa_indexer_kl_bwd_workspace_size(int B, int T, int Nc_cap, int topk) {
  if (B <= 0 || T <= 0 || Nc_cap < 0 || topk < 0) return 0;
  return csa_host::indexer_kl_ws_bytes(B, T, Nc_cap, topk);
}

csa_status_t csa_indexer_kl_bwd(int B, int T, int H_I, int d_I, int Nc_cap, int topk,
                                const void* q_idx, const float* w_idx, const void* k_idx,
                                csa_dtype_t qk_dt, const int32_t* idx, const float* attn_mass,
                                const float* grad_scale, float* loss, float* dq_idx,
                                float* dw_idx, float* dk_idx, void* workspace, size_t ws_bytes,
                                hipStream_t stream) {
  const char* fn = "csa_indexer_kl_bwd";
  if (B <= 0 || T <= 0 || H_I <= 0 || d_I <= 0 || Nc_cap < 0 || topk < 0)
    return fail(CSA_E_ARG, "%s: B, T, H_I, d_I must be > 0; Nc_cap, topk >= 0", fn);
  if (!q_idx || !w_idx || !loss || !dq_idx || !dw_idx || (topk > 0 && (!idx || !attn_mass)) ||
      (Nc_cap > 0 && (!k_idx || !dk_idx)))
    return fail(CSA_E_ARG, "%s: missing required pointer", fn);
  if (qk_dt != CSA_DT_BF16) return fail(CSA_E_UNSUPPORTED, "%s: qk_dt must be BF16", fn);
  if (H_I != 16 || d_I != 64) return fail(CSA_E_UNSUPPORTED, "%s: needs H_I = 16, d_I = 64", fn);
  if (topk > 1024) return fail(CSA_E_UNSUPPORTED, "%s: topk > 1024", fn);
  if (Nc_cap > 65536) return fail(CSA_E_UNSUPPORTED, "%s: Nc_cap > 65536", fn);
  if ((T + 63) / 64 > 65535 || B > 65535)
    return fail(CSA_E_UNSUPPORTED, "%s: T <= 65535 * 64 and B <= 65535", fn);
  if (!aligned16(q_idx) || (k_idx && !aligned16(k_idx)) || !aligned16(w_idx) ||
      !aligned16(dq_idx))
    return fail(CSA_E_UNSUPPORTED, "%s: q_idx, k_idx, w_idx and dq_idx must be 16-byte aligned", fn);
  const size_t need = csa_host::indexer_kl_ws_bytes(B, T, Nc_cap, topk);
  if (ws_bytes < need || !workspace)
    return fail(CSA_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  csa_host::IndexerKlArgs a{B,          T,    Nc_cap, topk,   q_idx,  w_idx, k_idx, idx,
                            attn_mass,  grad_scale, loss, dq_idx, dw_idx, dk_idx, workspace};
  return hip_status(csa_host::launch_indexer_kl_bwd(a, stream), fn);
}

size_t csa_indexer_kl_dense_bwd_workspace_size(int B, int T, int Nc_cap) {
  if (B <= 0 || T <= 0 || Nc_cap < 0) return 0;
  return csa_host::indexer_kl_dense_ws_bytes(B, T, Nc_cap);
}

csa_status_t csa_indexer_kl_dense_bwd(int B, int T, int H_I, int d_I, int Nc_cap, int m,
                                      const int64_t* q_pos, const int32_t* n_cmp,
                                      const void* q_idx, const float* w_idx, const void* k_idx,
                                      csa_dtype_t qk_dt, const float* attn_mass,
                                      const float* grad_scale, float* loss, float* dq_idx,
                                      float* dw_idx, float* dk_idx, void* workspace,
                                      size_t ws_bytes, hipStream_t stream) {
  const char* fn = "csa_indexer_kl_dense_bwd";
  if (B <= 0 || T <= 0 || H_I <= 0 || d_I <= 0 || Nc_cap < 0 || m < 1)
    return fail(CSA_E_ARG, "%s: B, T, H_I, d_I, m must be > 0; Nc_cap >= 0", fn);
  if (!q_pos || !n_cmp || !q_idx || !w_idx || !loss || !dq_idx || !dw_idx ||
      (Nc_cap > 0 && (!k_idx || !dk_idx || !attn_mass)))
    return fail(CSA_E_ARG, "%s: missing required pointer", fn);
  if (qk_dt != CSA_DT_BF16) return fail(CSA_E_UNSUPPORTED, "%s: qk_dt must be BF16", fn);
  if (H_I != 16 || d_I != 64) return fail(CSA_E_UNSUPPORTED, "%s: needs H_I = 16, d_I = 64", fn);
  if (Nc_cap > 65536) return fail(CSA_E_UNSUPPORTED, "%s: Nc_cap > 65536", fn);
  if ((T + 63) / 64 > 65535 || B > 65535)
    return fail(CSA_E_UNSUPPORTED, "%s: T <= 65535 * 64 and B <= 65535", fn);
  if (!aligned16(q_idx) || (k_idx && !aligned16(k_idx)) || !aligned16(w_idx) ||
      !aligned16(dq_idx))
    return fail(CSA_E_UNSUPPORTED, "%s: q_idx, k_idx, w_idx and dq_idx must be 16-byte aligned", fn);
  const size_t need = csa_host::indexer_kl_dense_ws_bytes(B, T, Nc_cap);
  if (ws_bytes < need || (need && !workspace))
    return fail(CSA_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  csa_host::IndexerKlArgs a{B,         T,          0,    0,      q_idx,  w_idx, k_idx, nullptr,
                            attn_mass, grad_scale, loss, dq_idx, dw_idx, dk_idx, workspace};
  a.Nc_cap = Nc_cap;
  a.m = m;
  a.q_pos = q_pos;
  a.n_cmp = n_cmp;
  return hip_status(csa_host::launch_indexer_kl_dense_bwd(a, stream), fn);
}

size_t csa_compress_bwd_workspace_size(int B, int L, int d_model, int E, int m, int Nc_cap) {
  if (B <= 0 || L <= 0 || d_model <= 0 || E <= 0 || m < 1 || Nc_cap < 0) return 0;
  return csa_host::compress_bwd_ws_bytes(B, L, d_model, E, m, Nc_cap);
}

csa_status_t csa_compress_bwd(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                              const void* x, const void* w_kv, const void* w_gate,
                              csa_dtype_t in_dt, const float* ape, int Nc_cap, const float* d_out,
                              float* dx, float* dw_kv, float* dw_gate, float* dape,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  return csa_compress_bwd_ex(B, L, d_model, E, m, overlap, rotate, x, w_kv, w_gate, in_dt, ape,
                             Nc_cap, d_out, nullptr, dx, dw_kv, dw_gate, dape, nullptr, workspace,
                             ws_bytes, stream);
}

csa_status_t csa_compress_bwd_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                                 const void* x, const void* w_kv, const void* w_gate,
                                 csa_dtype_t in_dt, const float* ape, int Nc_cap,
                                 const float* d_out, const csa_compress_opts_t* opts, float* dx,
                                 float* dw_kv, float* dw_gate, float* dape, float* d_norm_weight,
                                 void* workspace, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "csa_compress_bwd";
  csa_host::EntryOpts eo{nullptr, 0.0f, 0, 0, 0, 10000.0f};
  if (opts) {
    const int R = opts->rope_dim;
    if (R < 0 || (R & 1) || opts->rope_offset < 0 || (int64_t)opts->rope_offset + R > E ||
        (R > 0 && !(opts->rope_base > 0.0f)) ||
        (opts->rope_interleaved != 0 && opts->rope_interleaved != 1) ||
        (opts->norm_weight && !(opts->norm_eps >= 0.0f)))
      return fail(CSA_E_ARG,
                  "%s: rope_dim must be even with [rope_offset, rope_offset + rope_dim) inside "
                  "[0, E), rope_base > 0, rope_interleaved 0 or 1, norm_eps >= 0", fn);
    if (opts->norm_weight && !d_norm_weight)
      return fail(CSA_E_ARG, "%s: a norm weight needs d_norm_weight", fn);
    eo = csa_host::EntryOpts{opts->norm_weight, opts->norm_eps, R, opts->rope_offset,
                             opts->rope_interleaved, opts->rope_base};
  }
  if (B <= 0 || L <= 0 || d_model <= 0 || E <= 0 || Nc_cap < 0)
    return fail(CSA_E_ARG, "%s: B, L, d_model, E must be > 0 and Nc_cap >= 0", fn);
  if (m < 1) return fail(CSA_E_ARG, "%s: m must be >= 1", fn);
  if (overlap != 0 && overlap != 1) return fail(CSA_E_ARG, "%s: overlap must be 0 or 1", fn);
  if (rotate != 0 && rotate != 1) return fail(CSA_E_ARG, "%s: rotate must be 0 or 1", fn);
  if (rotate && (E & (E - 1))) return fail(CSA_E_ARG, "%s: rotate needs E a power of two", fn);
  if (!x || !w_kv || !w_gate || !dx || !dw_kv || !dw_gate || (Nc_cap > 0 && !d_out) ||
      (dape && !ape))
    return fail(CSA_E_ARG, "%s: missing required pointer (dape needs ape)", fn);
  if (in_dt != CSA_DT_BF16) return fail(CSA_E_UNSUPPORTED, "%s: in_dt must be BF16", fn);
  if (E > 1024 || d_model % 64 != 0)
    return fail(CSA_E_UNSUPPORTED, "%s: needs E <= 1024 and d_model a multiple of 64", fn);
  if ((1 + overlap) * m > 1024) return fail(CSA_E_UNSUPPORTED, "%s: (1 + overlap) m > 1024", fn);
  if ((int64_t)B * L > INT32_MAX / 2 || (L + 127) / 128 > 65535 || B > 65535)
    return fail(CSA_E_UNSUPPORTED, "%s: B * L too large", fn);
  if (!aligned16(x) || !aligned16(w_kv) || !aligned16(w_gate))
    return fail(CSA_E_UNSUPPORTED, "%s: x and the weights must be 16-byte aligned", fn);
  const size_t need = csa_host::compress_bwd_ws_bytes(B, L, d_model, E, m, Nc_cap);
  if (ws_bytes < need || !workspace)
    return fail(CSA_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  csa_host::CompressBwdArgs a{B,     L,     d_model, E,       m,       overlap, rotate, Nc_cap,
                              x,     w_kv,  w_gate,  ape,     d_out,   dx,      dw_kv,  dw_gate,
                              dape,  workspace, eo, d_norm_weight};
  return hip_status(csa_host::launch_compress_bwd(a, stream), fn);
}
