/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed sparse attention library.
 *
 * The library implements the data-parallel hot path of DeepSeek-V4-style
 * hybrid attention as described by the DS-V4 analysis pages (sections 1.2 to
 * 1.5: compression, Lightning Indexer top-k, sparse attention plus a sliding
 * window; HCA: heavy compression with dense attention) and the hyper-parallel
 * migration notes (section 3.2: the gated overlapping compressor; section 4.2:
 * the attention entry point and its layouts).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers into caller-owned memory; the
 *    library allocates nothing and keeps no state besides a thread-local
 *    error string.  Layouts are dense, row-major, batch-first ([B, S, ...];
 *    the pages' seq-first layout is the same for B = 1).
 *  - Per-sequence metadata (pos0, q_pos, n_cmp, raw_base) is device-resident
 *    so calls can be captured in a HIP graph; no call synchronises the host,
 *    and none issues hipMemset.
 *  - Calls are asynchronous on `stream`.  The status covers argument checks
 *    and the launch itself (hipGetLastError); faults inside kernels surface
 *    at the caller's next synchronisation.
 *  - Positions are absolute token indices.  A query at position t sees the
 *    compressed entry i iff that entry's last token m (i + 1) - 1 is at or
 *    before t, and the raw token j iff max(0, t - W + 1) <= j <= t (article
 *    section 5.2 window rule).  Entries >= n_cmp[b] do not exist.
 *  - Unsupported shape/dtype combinations return CSA_E_UNSUPPORTED; the
 *    library has exactly one implementation per supported case and no
 *    fallback.
 *  - fp8 means OCP FP8 E4M3 ("e4m3fn", largest finite value 448) codes with a
 *    positive fp32 scale per row: value = code * scale.
 *  - mxfp4 means OCP MXFP4: E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
 *    6; sign in bit 3) packed two per byte, element 2i of a row in the low
 *    nibble, with one E8M0 scale byte per 32 consecutive values of a row:
 *    value = e2m1(code) * 2^(scale - 127).  A row of n values takes n / 2
 *    code bytes and n / 32 scale bytes.  (The CSA/HCA article, section 3.2,
 *    notes that the indexer computes in FP4 and names no format; MXFP4 is
 *    the reading taken.)
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CSA_DT_F32 = 0, CSA_DT_BF16 = 1, CSA_DT_FP8E4M3 = 2, CSA_DT_MXFP4 = 3 } csa_dtype_t;

typedef enum {
  CSA_OK = 0,
  CSA_E_ARG = 1,          /* invalid argument (sizes, null pointers)          */
  CSA_E_UNSUPPORTED = 2,  /* valid but not implemented (shape / dtype combo)  */
  CSA_E_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_size */
  CSA_E_HIP = 4           /* a HIP launch error                                */
} csa_status_t;

/*
 * Gated overlapping compressor (migration notes section 3.2: linear_wkv and
 * linear_wgate projections, a softmax over an overlapping window with an
 * absolute position bias `ape`; ratio 4 overlaps, ratio 128 does not; DS-V4
 * analysis section 1.3: each entry looks at 2m adjacent positions and decode
 * keeps a tail state).
 *
 * For token j:  P_j = W_kv x_j,  G_j = W_gate x_j   (width E each).
 * Entry i pools the window of tokens [m (i - o), m (i + 1)) restricted to
 * j >= 0 (o = overlap):
 *     a_{j,e} = softmax_j (G_{j,e} + ape[j - m (i - o), e]),
 *     C_{i,e} = sum_j a_{j,e} P_{j,e}.
 * The call consumes tokens [pos0[b], pos0[b] + L) of every sequence and writes
 * every entry i < Nc_cap whose last token m (i + 1) - 1 lies in that range.
 * Window tokens before pos0[b] come from state_in.
 *
 *  B, L         sequences, new tokens per sequence (L >= 1)
 *  d_model, E   input width, output width per entry (main compressor:
 *               E = 2 D = [K | V]; indexer compressor: E = d_I)
 *  m, overlap   ratio (>= 1) and overlap flag (0 or 1)
 *  rotate       0, or 1: each entry is multiplied by H_E / sqrt(E) before the
 *               storage rounding, H_E the Walsh-Hadamard matrix in Sylvester
 *               order (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]); E must be
 *               a power of two (the migration notes name a Hadamard step in the
 *               compressor and the indexer, section 3.2; the rotation is
 *               orthogonal, so indexer scores of rotated queries and keys are
 *               unchanged while e4m3 rounding sees flatter rows)
 *  pos0         int64 [B]: absolute position of x[b, 0]
 *  x            [B, L, d_model] in in_dt
 *  w_kv, w_gate [E, d_model] each, in in_dt (output-major, like a Linear weight)
 *  in_dt        CSA_DT_F32 or CSA_DT_BF16
 *  ape          fp32 [(1 + overlap) m, E] or NULL (= zero); row s biases window
 *               slot s, slot 0 being the oldest token of the window
 *  state_in     fp32 [B, (1 + overlap) m - 1, 2, E] or NULL: P (index 0) and G
 *               (index 1) of the tokens at positions pos0 - ns .. pos0 - 1,
 *               ns = (1 + overlap) m - 1, in position order.  A token that does
 *               not exist carries G = -inf (and P = 0).  NULL or a position < 0
 *               means "absent".
 *  state_out    same layout for positions pos0 + L - ns .. pos0 + L - 1, or
 *               NULL.  Must not alias state_in (ping-pong two buffers).
 *  out          [B, Nc_cap, E] in out_dt (F32, BF16 or FP8E4M3; MXFP4: bytes
 *               [B, Nc_cap, E / 2]); rows of entries not completed by this
 *               call are left untouched
 *  out_scale    FP8E4M3: fp32 [B, Nc_cap], the row scale amax|C_i| / 448 (1
 *               for an all-zero row), the codes e4m3(C / scale) rounded to
 *               nearest even and saturated at 448.  MXFP4: E8M0 bytes
 *               [B, Nc_cap, E / 32]; per block of 32 values X =
 *               floor(log2 amax) - 2 clamped to [-127, 127] (0 for an
 *               all-zero block), the codes e2m1(C / 2^X) rounded to nearest
 *               even and saturated at 6 (E % 32 == 0).  NULL otherwise.
 *  workspace    device scratch of at least csa_compress_workspace_size() bytes
 *               (NULL allowed when that size is 0)
 * Supported: in_dt F32 with any d_model; in_dt BF16 with d_model % 64 == 0.
 */
csa_status_t csa_compress(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                          const int64_t* pos0, const void* x, const void* w_kv,
                          const void* w_gate, csa_dtype_t in_dt, const float* ape,
                          const float* state_in, float* state_out, void* out,
                          void* out_scale, csa_dtype_t out_dt, int Nc_cap,
                          void* workspace, size_t ws_bytes, hipStream_t stream);
size_t csa_compress_workspace_size(int B, int L, int d_model, int E, int m, int overlap,
                                   csa_dtype_t in_dt);

/*
 * Lightning Indexer score and per-query top-k (DS-V4 analysis section 1.2;
 * article section 3.2: score each query against every compressed entry, keep
 * the top k).  Score, with sq = q_scale and sk = k_scale (1 unless fp8):
 *     s(t, j) = sum_h w[t, h] * ReLU(sq[t, h] * sk[j] * sum_e q[t, h, e] k[j, e])
 * over the visible entries j < n_vis(t) = min(n_cmp[b], floor((t + 1) / m),
 * Nc_cap), t = q_pos[b] + row.  The selection keeps the min(topk, n_vis)
 * largest scores, ties broken toward the lower index, and writes them in
 * ascending index order padded with -1.
 *
 *  q_idx     [B, T, H_I, d_I] in qk_dt;  q_scale fp32 [B, T, H_I] iff fp8
 *  w_idx     fp32 [B, T, H_I]
 *  k_idx     [B, Nc_cap, d_I] in qk_dt;  k_scale fp32 [B, Nc_cap] iff fp8
 *            (mxfp4: q_idx bytes [B, T, H_I, d_I / 2] with q_scale E8M0 bytes
 *            [B, T, H_I, d_I / 32], k_idx bytes [B, Nc_cap, d_I / 2] with
 *            k_scale E8M0 bytes [B, Nc_cap, d_I / 32]; the score uses the
 *            decoded values, each with its block scale, and sq = sk = 1)
 *  idx_out   int32 [B, T, topk]
 *  score_out fp32 [B, T, topk] or NULL: the score of each selected index
 *            (NaN in padded slots)
 *  workspace at least csa_indexer_topk_workspace_size() bytes
 * Supported: (H_I, d_I) in {(4, 32), (16, 64)} for F32; (16, 64) for BF16,
 * FP8E4M3 and MXFP4; topk <= 8192.  fp8 scales must be positive.
 */
csa_status_t csa_indexer_topk(int B, int T, int H_I, int d_I, int Nc_cap, int m, int topk,
                              const int64_t* q_pos, const int32_t* n_cmp, const void* q_idx,
                              const void* q_scale, const float* w_idx, const void* k_idx,
                              const void* k_scale, csa_dtype_t qk_dt, int32_t* idx_out,
                              float* score_out, void* workspace, size_t ws_bytes,
                              hipStream_t stream);
size_t csa_indexer_topk_workspace_size(int B, int T, int H_I, int d_I, int Nc_cap, int topk,
                                       csa_dtype_t qk_dt);

/*
 * Sparse MQA attention over the selected compressed entries plus the sliding
 * window of raw KV (DS-V4 analysis section 1.2: attend to the k compressed
 * entries and the window; Notion copy section 1: MQA, scale 1/sqrt(head_dim)).
 * For query row t (position q_pos[b] + t) and head h, one softmax runs over
 * J = {kv_cmp[b, idx[b, t, k]] : 0 <= idx < Nc_cap} followed by the raw rows
 * r = j - raw_base[b] in [0, R_cap) of tokens j in [max(0, t - W + 1), t]:
 *     l_j = scale * q[b, t, h] . K_j,  out = sum_j softmax(l)_j V_j,
 *     lse = ln sum_j exp(l_j).
 * A KV row is [K | V] of width 2 D; every head shares it.  Slots with idx < 0
 * or idx >= Nc_cap are skipped; an empty J gives out = 0 and lse = -inf.
 * Attention sink (the migration page, section 3.2, lists attn_sink among the
 * attention's state): when sink is given, head h's softmax has one more term
 * with logit sink[h] (natural-log units of l) and no value:
 *     out = sum_j e^{l_j} V_j / (e^{sink[h]} + sum_j e^{l_j}),
 *     lse = ln(e^{sink[h]} + sum_j e^{l_j});
 * a sink of -inf is none, and an empty J then gives out = 0, lse = sink[h].
 *
 *  sink     fp32 [H] (device) or NULL
 *  q        [B, T, H, D] in dt;  out [B, T, H, D] in dt;  lse fp32 [B, T, H] or NULL
 *  kv_cmp   [B, Nc_cap, 2 D] in dt;  idx int32 [B, T, topk] (topk may be 0)
 *  kv_raw   [B, R_cap, 2 D] in dt;   raw_base int64 [B]
 * Supported: dt F32 with D in {64, 128}; dt BF16 with D = 128, H in {32, 64}
 * and Nc_cap, R_cap <= 2^23; with BF16 and fewer than 1024 query rows (the
 * split-key decode kernel), topk + window <= 64 * 4032.
 */
csa_status_t csa_sparse_attn(int B, int T, int H, int D, int topk, int window, float scale,
                             const float* sink, const int64_t* q_pos, const void* q,
                             const void* kv_cmp,
                             int Nc_cap, const int32_t* idx, const void* kv_raw, int R_cap,
                             const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                             void* workspace, size_t ws_bytes, hipStream_t stream);
size_t csa_sparse_attn_workspace_size(int B, int T, int H, int D, int topk, int window);

/*
 * HCA: heavily compressed attention (DS-V4 analysis sections 1.4-1.5: ratio
 * m' >> m, dense attention over every compressed entry, plus the window).
 * As csa_sparse_attn (sink included) with the compressed part of J being
 * every visible entry j < n_vis(t) = min(n_cmp[b], floor((t + 1) / m), Nc_cap).
 */
csa_status_t hca_dense_attn(int B, int T, int H, int D, int m, int window, float scale,
                            const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                            const void* q,
                            const void* kv_cmp, int Nc_cap, const void* kv_raw, int R_cap,
                            const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                            void* workspace, size_t ws_bytes, hipStream_t stream);
size_t hca_dense_attn_workspace_size(int B, int T, int H, int D, int Nc_cap, int window);

/* Static text of a status code. */
/*
 * Paged compressed caches (serving-shaped storage: the million-token CSA/HCA
 * article, section 8.3, lists paged-attention style cache management for
 * the compressed caches among the serving adaptations; the CSA migration
 * analysis, section 5, lists packed variable-length batches).
 * Instead of one [B, Nc_cap, row] tensor, the compressed entries of every
 * sequence live in a shared pool of n_pages pages of page_size rows each;
 * logical entry j of sequence b is pool row
 *     block_table[b * max_pages + j / page_size] * page_size + j % page_size.
 *  block_table  device int32 [B, max_pages], read-only; entries past a
 *               sequence's last used page are not read.  A page id outside
 *               [0, n_pages) is clamped into it (no fault; the caller's
 *               table is wrong then)
 *  page_size    rows per page, a power of two in [16, 2^20]
 *  max_pages    row stride of block_table; Nc_cap <= max_pages * page_size
 *  n_pages      pages in the pool (pool rows = n_pages * page_size)
 * The struct is read on the host during the call; the caller owns it and the
 * table.  Errors: CSA_E_ARG for a missing table or a bad size.
 */
typedef struct {
  const int32_t* block_table;
  int page_size;
  int max_pages;
  int n_pages;
} csa_page_table_t;

/*
 * csa_compress with a paged output: out (and out_scale) are pools of
 * n_pages * page_size rows in the layouts above ([rows, E] in out_dt,
 * [rows] fp32 scales for FP8E4M3, [rows, E / 32] E8M0 bytes for MXFP4);
 * entry i of sequence b goes to its pool row.  Everything else is as in
 * csa_compress (the same workspace size).
 */
csa_status_t csa_compress_paged(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                                const int64_t* pos0, const void* x, const void* w_kv,
                                const void* w_gate, csa_dtype_t in_dt, const float* ape,
                                const float* state_in, float* state_out, void* out,
                                void* out_scale, csa_dtype_t out_dt, int Nc_cap,
                                const csa_page_table_t* pages, void* workspace, size_t ws_bytes,
                                hipStream_t stream);

/*
 * csa_indexer_topk over paged keys: k_idx and k_scale are pools (BF16:
 * [rows, d_I]; FP8E4M3: [rows, d_I] codes and [rows] fp32 scales; MXFP4:
 * [rows, d_I / 2] bytes and [rows, d_I / 32] E8M0 scales).  Indices in
 * idx_out stay logical (0 .. Nc_cap - 1).  qk_dt BF16, FP8E4M3 or MXFP4
 * (F32: CSA_E_UNSUPPORTED); the workspace is
 * csa_indexer_topk_workspace_size().
 */
csa_status_t csa_indexer_topk_paged(int B, int T, int H_I, int d_I, int Nc_cap, int m, int topk,
                                    const int64_t* q_pos, const int32_t* n_cmp,
                                    const void* q_idx, const void* q_scale, const float* w_idx,
                                    const void* k_idx, const void* k_scale, csa_dtype_t qk_dt,
                                    const csa_page_table_t* pages, int32_t* idx_out,
                                    float* score_out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * csa_sparse_attn over a paged kv_cmp pool ([rows, 2 D]); idx holds logical
 * indices as csa_indexer_topk writes them.  The workspace is
 * csa_sparse_attn_paged_workspace_size() bytes (it also holds the selected
 * entries' pool rows).  BF16 pools hold at most 2^23 rows.
 */
csa_status_t csa_sparse_attn_paged(int B, int T, int H, int D, int topk, int window, float scale,
                                   const float* sink, const int64_t* q_pos, const void* q,
                                   const void* kv_cmp, int Nc_cap, const csa_page_table_t* pages,
                                   const int32_t* idx, const void* kv_raw, int R_cap,
                                   const int64_t* raw_base, csa_dtype_t dt, void* out, float* lse,
                                   void* workspace, size_t ws_bytes, hipStream_t stream);
size_t csa_sparse_attn_paged_workspace_size(int B, int T, int H, int D, int topk, int window);

const char* csa_status_string(csa_status_t status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* csa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
