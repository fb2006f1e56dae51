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
 * Post-processing of every emitted compressor entry (migration notes section
 * 3.2: the compressor carries a norm submodule and applies the rotary
 * position embedding to the key positions, ApplyRotaryPosEmb with
 * for_k_pos_emb; section 4.3: layernorm_epsilon 1e-6, rotary_interleaved
 * False).  Applied to the pooled entry C_i, in this order, before the
 * Hadamard rotation and the storage rounding:
 *  norm_weight      device fp32 [E], or NULL for no norm: RMS norm over the
 *                   entry, C_e <- C_e / sqrt(mean_e C_e^2 + norm_eps) * w_e
 *  norm_eps         >= 0
 *  rope_dim         0 (none) or an even count of channels starting at
 *                   rope_offset (rope_offset + rope_dim <= E) that rotate by
 *                   the angles p * rope_base^(-2k / rope_dim), k <
 *                   rope_dim / 2, at the entry's position p = m i (the first
 *                   token of its own block; angles in double precision)
 *  rope_interleaved 0: channel k of the slice pairs with k + rope_dim / 2
 *                   ("rotate half"); 1: channel 2k pairs with 2k + 1.  A pair
 *                   (a, b) becomes (a cos - b sin, b cos + a sin)
 *  rope_base        > 0 when rope_dim > 0 (10000 is the usual value)
 * For the main compressor (E = 2 D = [K | V]) the key's rotary channels are
 * a slice of the first D channels; queries get the same rotation at their
 * token positions from the caller.
 */
typedef struct {
  const float* norm_weight;
  float norm_eps;
  int rope_dim;
  int rope_offset;
  float rope_base;
  int rope_interleaved;
} csa_compress_opts_t;

/*
 * csa_compress with the entry post-processing above (opts, or NULL for
 * none) and an optional paged output (pages, or NULL for the [B, Nc_cap,
 * ...] layout; see csa_page_table_t below).  Everything else, the workspace
 * included, is as in csa_compress.  Errors: CSA_E_ARG for a rotary slice
 * outside the entry, an odd rope_dim, rope_base <= 0 or norm_eps < 0.
 */
typedef struct csa_page_table_s csa_page_table_t;
csa_status_t csa_compress_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                             const int64_t* pos0, const void* x, const void* w_kv,
                             const void* w_gate, csa_dtype_t in_dt, const float* ape,
                             const float* state_in, float* state_out, void* out,
                             void* out_scale, csa_dtype_t out_dt, int Nc_cap,
                             const csa_page_table_t* pages, const csa_compress_opts_t* opts,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

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
 * FP8E4M3 and MXFP4; topk <= 8192; Nc_cap <= 2^21.  fp8 scales must be
 * positive.  The workspace holds scores and selection candidates only; its
 * contents on entry do not matter.
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
 * csa_sparse_attn in two halves, so that the sliding-window half of a decode
 * step can run while the indexer is still choosing the entries.  The
 * attention of a query is one softmax over the selected compressed entries
 * and the raw window tokens (DS-V4 analysis section 1.2); the window half
 * does not depend on the top-k indices, and
 * the softmax over the union of two key sets is the log-sum-exp merge of the
 * softmaxes over each (the partials and merge of the split-key decode form).
 *
 * csa_sparse_attn_window_half attends each row to its window tokens only and
 * leaves fp32 partial results (unnormalised output, running maximum and sum
 * per head) in the workspace.  csa_sparse_attn_selected_half then attends the
 * rows to their selected entries, merges both halves (and the sink) and writes
 * out and lse exactly as csa_sparse_attn defines them (equal up to fp32
 * summation order).  Both calls take the same B, T, H, D, topk, window, scale,
 * q_pos, q, kv_raw, R_cap, raw_base, dt and workspace; the caller orders the
 * selected half after the window half (same stream, or an event between the
 * two streams); nothing else may use the workspace in between.  The window
 * half reads no index, compressed row, sink or output.
 * Supported: dt BF16, D = 128, H in {32, 64}, fewer than 1024 query rows
 * (decode), unpaged caches and the [B, T] layout; CSA_E_UNSUPPORTED otherwise.
 * Workspace: csa_sparse_attn_split_workspace_size() bytes (0: unsupported).
 */
size_t csa_sparse_attn_split_workspace_size(int B, int T, int H, int D, int topk, int window);
csa_status_t csa_sparse_attn_window_half(int B, int T, int H, int D, int topk, int window,
                                         float scale, const int64_t* q_pos, const void* q,
                                         const void* kv_raw, int R_cap, const int64_t* raw_base,
                                         csa_dtype_t dt, void* workspace, size_t ws_bytes,
                                         hipStream_t stream);
csa_status_t csa_sparse_attn_selected_half(int B, int T, int H, int D, int topk, int window,
                                           float scale, const float* sink, const int64_t* q_pos,
                                           const void* q, const void* kv_cmp, int Nc_cap,
                                           const int32_t* idx, const void* kv_raw, int R_cap,
                                           const int64_t* raw_base, csa_dtype_t dt, void* out,
                                           float* lse, void* workspace, size_t ws_bytes,
                                           hipStream_t stream);

/*
 * csa_sparse_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  Arguments, results and errors are those of
 * csa_sparse_attn; the split-key partials of few-row calls go to a static
 * device buffer of 16 MiB that the library holds on each GPU it runs on
 * until the process ends, instead of a caller workspace.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * its first call on a device looks up the buffer's device address once.
 * A call whose partials would exceed 16 MiB returns CSA_E_UNSUPPORTED (the
 * message gives the size); csa_sparse_attn_workspace_size() tells the size
 * a call needs.  Every call on one GPU shares the buffer, and it keeps the
 * last call's contents: calls that overlap on one GPU (concurrent streams,
 * host threads) race and must be serialised by the caller.
 */
csa_status_t csa_sparse_attn_noalloc(int B, int T, int H, int D, int topk, int window,
                                     float scale, const float* sink, const int64_t* q_pos,
                                     const void* q, const void* kv_cmp, int Nc_cap,
                                     const int32_t* idx, const void* kv_raw, int R_cap,
                                     const int64_t* raw_base, csa_dtype_t dt, void* out,
                                     float* lse, hipStream_t stream);

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

/*
 * Paged compressed caches (serving-shaped storage: the million-token CSA/HCA
 * article, section 8.3, lists paged-attention style cache management for
 * the compressed caches among the serving adaptations; the CSA migration
 * analysis, section 5, lists packed variable-length batches).
 * Instead of one [B, Nc_cap, row] tensor, the compressed entries of every
 * sequence live in a shared pool of n_pages pages of page_size rows each;
 * logical entry j of sequence b is pool row
 *     block_table[b * max_pages + j / page_size] * page_size + j % page_size.
 *  block_table  device int32 [B, max_pages], read-only.  Table entries of
 *               the pages that cover logical entries 0 .. Nc_cap - 1 may be
 *               read whatever n_cmp[b] is; only those of pages holding
 *               existing entries (j < n_cmp[b]) affect results.  A page id
 *               outside [0, n_pages) marks its entries absent: the
 *               compressor does not store them, the indexer gives them the
 *               score -inf (they are selected only when fewer than topk
 *               other visible entries exist), and sparse attention skips
 *               them as it skips a -1 slot.  No pool row is read or written
 *               for an absent page.
 *  page_size    rows per page, a power of two in [16, 2^20]
 *  max_pages    row stride of block_table; Nc_cap <= max_pages * page_size
 *  n_pages      pages in the pool (pool rows = n_pages * page_size)
 * The struct is read on the host during the call; the caller owns it and the
 * table.  Errors: CSA_E_ARG for a missing table or a bad size.
 */
struct csa_page_table_s {
  const int32_t* block_table;
  int page_size;
  int max_pages;
  int n_pages;
};

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
 * csa_sparse_attn over a paged kv_cmp pool ([rows, 2 D]; pages), a paged raw
 * window cache (raw_pages: raw row r of sequence b, the token raw_base[b] +
 * r, is pool row block_table[b, r / page_size] * page_size + r % page_size
 * of a kv_raw pool [rows, 2 D]; R_cap logical rows per sequence), or both;
 * either may be NULL, not both.  idx holds logical indices as
 * csa_indexer_topk writes them.  Rows of absent pages are skipped.  The
 * workspace is csa_sparse_attn_paged_workspace_size() bytes with pages (it
 * also holds the selected entries' pool rows), csa_sparse_attn_workspace_size()
 * without.  BF16 pools hold at most 2^23 rows.
 */
csa_status_t csa_sparse_attn_paged(int B, int T, int H, int D, int topk, int window, float scale,
                                   const float* sink, const int64_t* q_pos, const void* q,
                                   const void* kv_cmp, int Nc_cap, const csa_page_table_t* pages,
                                   const int32_t* idx, const void* kv_raw, int R_cap,
                                   const int64_t* raw_base, const csa_page_table_t* raw_pages,
                                   csa_dtype_t dt, void* out, float* lse, void* workspace,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * hca_dense_attn over a paged compressed cache (pages: entry j of sequence b
 * at its pool row of kv_cmp [rows, 2 D]), a paged raw window cache
 * (raw_pages, as for csa_sparse_attn_paged), or both; either may be NULL,
 * not both.  Entries and window rows of absent pages are skipped.  Everything
 * else, the workspace included, is as in hca_dense_attn.
 */
csa_status_t hca_dense_attn_paged(int B, int T, int H, int D, int m, int window, float scale,
                                  const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                                  const void* q, const void* kv_cmp, int Nc_cap,
                                  const csa_page_table_t* pages, const void* kv_raw, int R_cap,
                                  const int64_t* raw_base, const csa_page_table_t* raw_pages,
                                  csa_dtype_t dt, void* out, float* lse, void* workspace,
                                  size_t ws_bytes, hipStream_t stream);
size_t csa_sparse_attn_paged_workspace_size(int B, int T, int H, int D, int topk, int window);

/*
 * Packed variable-length prefill (the CSA migration analysis, section 4.2:
 * the attention entry point takes actual_seq_len; its phase 3 builds
 * cmp_cu_seqlens for packed sequences).  n sequences of lengths
 * len_b = cu_seqlens[b + 1] - cu_seqlens[b] are packed along the token
 * axis (total = cu_seqlens[n] tokens), every one starting at position 0:
 * token j of sequence b is row cu_seqlens[b] + j of every per-token tensor,
 * and its compressed entry i is row cmp_cu_seqlens[b] + i of every per-entry
 * tensor.  A sequence never sees another sequence's tokens or entries.  The
 * raw window rows of a sequence are its own packed tokens (kv_raw row
 * cu_seqlens[b] + j is token j).  Offsets are device int32 arrays of n + 1
 * elements; max_len (host) is at least every len_b, and max_cmp the largest
 * entry count floor(len_b / m).
 */

/* cmp_cu_seqlens[0] = 0, cmp_cu_seqlens[b + 1] = cmp_cu_seqlens[b] +
 * floor(len_b / m): the entry offsets of the packed sequences (device). */
csa_status_t csa_build_cmp_cu_seqlens(int n, const int32_t* cu_seqlens, int m,
                                      int32_t* cmp_cu_seqlens, hipStream_t stream);

/* csa_compress over packed sequences, each from position 0 (no carried state
 * in): x [total, d_model]; out [cmp_cu_seqlens[n], E] (and out_scale) in the
 * layouts of csa_compress; state_out [n, (1 + overlap) m - 1, 2, E] or NULL
 * receives each sequence's tail for a later decode step.  opts as for
 * csa_compress_ex.  Workspace: csa_compress_varlen_workspace_size(). */
csa_status_t csa_compress_varlen(int n, int total, int max_len, int d_model, int E, int m,
                                 int overlap, int rotate, const int32_t* cu_seqlens,
                                 const int32_t* cmp_cu_seqlens, const void* x, const void* w_kv,
                                 const void* w_gate, csa_dtype_t in_dt, const float* ape,
                                 float* state_out, void* out, void* out_scale, csa_dtype_t out_dt,
                                 const csa_compress_opts_t* opts, void* workspace,
                                 size_t ws_bytes, hipStream_t stream);
size_t csa_compress_varlen_workspace_size(int total, int d_model, int E, int m, int overlap,
                                          csa_dtype_t in_dt);

/* csa_indexer_topk over packed sequences: q_idx [total, H_I, d_I], w_idx
 * [total, H_I], k_idx [cmp_cu_seqlens[n], d_I]; idx_out [total, topk] holds
 * indices local to the row's sequence (entry i of sequence b is i).
 * Supported: F32 and BF16 as for csa_indexer_topk, max_cmp <= 2^21.
 * Workspace: csa_indexer_topk_varlen_workspace_size(). */
csa_status_t csa_indexer_topk_varlen(int n, int total, int max_len, int H_I, int d_I,
                                     int max_cmp, int m, int topk, const int32_t* cu_seqlens,
                                     const int32_t* cmp_cu_seqlens, const void* q_idx,
                                     const float* w_idx, const void* k_idx, csa_dtype_t qk_dt,
                                     int32_t* idx_out, float* score_out, void* workspace,
                                     size_t ws_bytes, hipStream_t stream);
size_t csa_indexer_topk_varlen_workspace_size(int total, int max_cmp, int topk,
                                              csa_dtype_t qk_dt);

/* csa_sparse_attn over packed sequences: q and out [total, H, D], kv_cmp
 * [cmp_cu_seqlens[n], 2 D], idx [total, topk] local to each sequence (as
 * csa_indexer_topk_varlen writes it; slots outside [0, floor(len_b / m))
 * are skipped), kv_raw [total, 2 D] the packed tokens' own KV rows.  Other
 * arguments and the supported set as for csa_sparse_attn.  Workspace:
 * csa_sparse_attn_varlen_workspace_size(). */
csa_status_t csa_sparse_attn_varlen(int n, int total, int max_len, int H, int D, int topk,
                                    int window, float scale, const float* sink,
                                    const int32_t* cu_seqlens, const int32_t* cmp_cu_seqlens,
                                    const void* q, const void* kv_cmp, int max_cmp,
                                    const int32_t* idx, const void* kv_raw, csa_dtype_t dt,
                                    void* out, float* lse, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);
size_t csa_sparse_attn_varlen_workspace_size(int total, int H, int D, int topk, int window);

/*
 * ---- training: backward passes ----------------------------------------------
 * The migration page (sections 1 and 3.2) places the training path of
 * CompressedSparseAttention in scope: its backward, the indexer loss and a
 * fused "sparse lightning indexer grad + KL loss" operator.  The gradients
 * below are those of the forward definitions above (chain rule); the call
 * recomputes the attention probabilities from the forward's lse, and delta
 * as sum_j P_j dP_j (equal to dout . out, without the rounding of a stored
 * output).
 *
 * Gradients of csa_sparse_attn for an upstream gradient dout of out.  Per
 * query token and head, over the forward's key set J:
 *     P_j = exp(l_j - lse),  dP_j = dout . V_j,  delta = sum_j P_j dP_j,
 *     dS_j = P_j (dP_j - delta),
 *     dq = scale sum_j dS_j K_j,  dK_j += scale dS_j q,  dV_j += P_j dout,
 *     dsink[h] = -sum over tokens of exp(sink[h] - lse) delta.
 *  q, dout  bf16 [B, T, H, D];  lse fp32 [B, T, H] (the forward's)
 *  kv_cmp, idx, kv_raw, raw_base, q_pos, sink, scale, window: as in the forward
 *  dq        fp32 [B, T, H, D] (written)
 *  dkv_cmp   fp32 [B, Nc_cap, 2 D] = [dK | dV] per compressed row (written in
 *            full; rows no token attends get 0); dkv_raw fp32 [B, R_cap, 2 D]
 *  dsink     fp32 [H] or NULL (needs sink)
 *  attn_mass fp32 [B, T, topk] or NULL: per slot, the attention probability
 *            of its entry summed over heads (0 in skipped slots), the target
 *            of csa_indexer_kl_bwd
 * Each row of idx must name an entry at most once (csa_indexer_topk's rows
 * do; the forward attends a repeated entry twice, this call once), and
 * attn_mass assumes the valid indices of a row ascend before its -1 pads, as
 * csa_indexer_topk writes them.  Supported: dt BF16, D = 128, H in {32, 64},
 * topk <= 4096, Nc_cap <= 65536, R_cap <= 2^23, 16-byte aligned tensors.
 * Workspace: csa_sparse_attn_bwd_workspace_size() bytes (contents on entry do
 * not matter; about 10 KB per window row plus 16 MB per 128 compressed rows
 * of row-chunk partials, 2^26 bytes at most for the compressed part at
 * B = 1).  The per-key sums over query rows are reduced in a fixed order:
 * repeated calls give the same bits.  The sink gradient alone is summed with
 * a few fp32 atomics per head.
 */
csa_status_t csa_sparse_attn_bwd(int B, int T, int H, int D, int topk, int window, float scale,
                                 const float* sink, const int64_t* q_pos, const void* q,
                                 const void* kv_cmp, int Nc_cap, const int32_t* idx,
                                 const void* kv_raw, int R_cap, const int64_t* raw_base,
                                 csa_dtype_t dt, const float* lse, const void* dout, float* dq,
                                 float* dkv_cmp, float* dkv_raw, float* dsink, float* attn_mass,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);
size_t csa_sparse_attn_bwd_workspace_size(int B, int T, int H, int Nc_cap, int R_cap,
                                          int window);

/*
 * Gradients of hca_dense_attn (the compressed part of J is every visible
 * entry j < n_vis(t)); arguments, outputs and limits as in
 * csa_sparse_attn_bwd without idx (Nc_cap <= 2^23), except:
 *  attn_mass fp32 [B, T, Nc_cap] or NULL: per compressed entry, the attention
 *            probability summed over heads (0 for entries the row does not
 *            see), the target of csa_indexer_kl_dense_bwd
 * Workspace: hca_dense_attn_bwd_workspace_size() bytes.
 */
csa_status_t hca_dense_attn_bwd(int B, int T, int H, int D, int m, int window, float scale,
                                const float* sink, const int64_t* q_pos, const int32_t* n_cmp,
                                const void* q, const void* kv_cmp, int Nc_cap, const void* kv_raw,
                                int R_cap, const int64_t* raw_base, csa_dtype_t dt,
                                const float* lse, const void* dout, float* dq, float* dkv_cmp,
                                float* dkv_raw, float* dsink, float* attn_mass, void* workspace,
                                size_t ws_bytes, hipStream_t stream);
size_t hca_dense_attn_bwd_workspace_size(int B, int T, int H, int Nc_cap, int R_cap, int window);

/*
 * Indexer KL loss and its gradients, the training signal of the Lightning
 * Indexer (migration page, sections 1 and 3.2: the indexer loss and the fused
 * sparse "lightning indexer grad + KL loss" operator; section 4.3: the loss
 * coefficient and the sparse-loss switch).  The pages do not print the loss;
 * the reading implemented (sparse form): for query row t with selected slots
 * S (0 <= idx < Nc_cap), the target is the main attention's mass per entry,
 * p_k = attn_mass[k] / sum_S attn_mass, the indexer's distribution is the
 * softmax over S of its scores I_k = sum_h w[h] ReLU(q[h] . k_idx[idx_k]),
 * and
 *     loss[t] = KL(p || softmax(I)) = sum_S p_k (ln p_k - ln softmax(I)_k).
 * The target carries no gradient.  With g = grad_scale[t] (1 if NULL; the
 * caller's loss coefficient and averaging), dI_k = g (softmax(I)_k - p_k) and
 *     dw_idx[t, h] = sum_k dI_k ReLU(v_hk),
 *     dq_idx[t, h] = sum_k dI_k w[h] [v_hk > 0] k_idx[idx_k],
 *     dk_idx[j]   += sum over rows and heads of dI_k w[h] [v_hk > 0] q[h],
 * v_hk = q[h] . k_idx[idx_k].  A row with no selected entry or zero total
 * mass has loss 0 and no gradient.
 *  q_idx  bf16 [B, T, 16, 64];  w_idx fp32 [B, T, 16];  k_idx bf16 [B, Nc_cap, 64]
 *  idx    int32 [B, T, topk] (each row's valid indices distinct and ascending
 *         before its -1 pads, as csa_indexer_topk writes them)
 *  attn_mass fp32 [B, T, topk] (csa_sparse_attn_bwd's);  grad_scale fp32 [B, T] or NULL
 *  loss fp32 [B, T]; dq_idx fp32 [B, T, 16, 64]; dw_idx fp32 [B, T, 16];
 *  dk_idx fp32 [B, Nc_cap, 64] (written in full)
 * Supported: qk_dt BF16, H_I = 16, d_I = 64, topk <= 1024, Nc_cap <= 65536.
 * Workspace: csa_indexer_kl_bwd_workspace_size() bytes (contents on entry do
 * not matter).  dk_idx sums rows with fp32 atomics (run-to-run last bits).
 */
csa_status_t csa_indexer_kl_bwd(int B, int T, int H_I, int d_I, int Nc_cap, int topk,
                                const void* q_idx, const float* w_idx, const void* k_idx,
                                csa_dtype_t qk_dt, const int32_t* idx, const float* attn_mass,
                                const float* grad_scale, float* loss, float* dq_idx,
                                float* dw_idx, float* dk_idx, void* workspace, size_t ws_bytes,
                                hipStream_t stream);
size_t csa_indexer_kl_bwd_workspace_size(int B, int T, int Nc_cap, int topk);

/*
 * The dense form of the indexer KL loss (migration page, section 4.3: the
 * sparse-loss switch off): the loss and gradients of csa_indexer_kl_bwd with
 * the selected set of row t being every visible entry j < n_vis(t) =
 * min((q_pos + t + 1) / m, n_cmp, Nc_cap), and the target the dense
 * attention's mass per entry.  Reading: the dense form is the sparse form
 * over that set (the pages give no separate formula).
 *  q_pos int64 [B];  n_cmp int32 [B];  m: the compression ratio of the cache
 *  q_idx, w_idx, k_idx, grad_scale, loss, dq_idx, dw_idx, dk_idx: as in
 *  csa_indexer_kl_bwd
 *  attn_mass fp32 [B, T, Nc_cap] (hca_dense_attn_bwd's; entries past n_vis
 *  are not read)
 * Supported: qk_dt BF16, H_I = 16, d_I = 64, Nc_cap <= 65536.  Workspace:
 * csa_indexer_kl_dense_bwd_workspace_size() bytes (B T Nc_cap floats of dI;
 * contents on entry do not matter).  dk_idx sums rows with fp32 atomics.
 */
csa_status_t csa_indexer_kl_dense_bwd(int B, int T, int H_I, int d_I, int Nc_cap, int m,
                                      const int64_t* q_pos, const int32_t* n_cmp,
                                      const void* q_idx, const float* w_idx, const void* k_idx,
                                      csa_dtype_t qk_dt, const float* attn_mass,
                                      const float* grad_scale, float* loss, float* dq_idx,
                                      float* dw_idx, float* dk_idx, void* workspace,
                                      size_t ws_bytes, hipStream_t stream);
size_t csa_indexer_kl_dense_bwd_workspace_size(int B, int T, int Nc_cap);

/*
 * Gradients of a one-shot compressor call (csa_compress from position 0 with
 * no carried state, bf16 tokens and weights, entries post-processed by
 * nothing or by the Hadamard rotation; csa_compress_bwd_ex below adds the
 * RMS norm and the rotary embedding) for an upstream gradient d_out
 * [B, Nc_cap, E] (fp32) of the entries it writes, rows i < min(L / m, Nc_cap)
 * (other rows are ignored).  By the chain rule through the compressor's
 * definition (migration page, section 3.2), for entry i and window token j
 * (slot s = j - m (i - overlap)), per channel, with g the entry's gradient
 * (H d_out / sqrt(E) under the rotation, H being symmetric):
 *     a_j = softmax_j(G_j + ape[s]),  C_i = sum_j a_j P_j,
 *     dP_j += a_j g,  dG_j += a_j (P_j - C_i) g,  dape[s] += a_j (P_j - C_i) g,
 *     dx = dP W_kv + dG W_gate,  dw_kv = sum_j dP_j x_j^T,  dw_gate = sum_j dG_j x_j^T.
 *  x bf16 [B, L, d_model];  w_kv, w_gate bf16 [E, d_model];  ape fp32 [(1+o) m, E] or NULL
 *  dx fp32 [B, L, d_model];  dw_kv, dw_gate fp32 [E, d_model];  dape fp32 [(1+o) m, E]
 *  or NULL (needs ape); every output is written in full.
 * dP and dG enter the weight and input products as bf16 (fp32 accumulation);
 * those products run on rocBLAS.  Supported: in_dt BF16, E <= 1024, d_model a
 * multiple of 64, (1 + overlap) m <= 1024.  Workspace:
 * csa_compress_bwd_workspace_size() bytes (contents on entry do not matter;
 * it holds P | G, dP | dG, the two weights stacked and their gradients
 * stacked).  When w_gate starts right where w_kv ends (one [2E, d_model]
 * buffer), the weights are read in place, and likewise dw_gate right after
 * dw_kv receives the weight gradients directly: no stacking copies.
 */
csa_status_t csa_compress_bwd(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                              const void* x, const void* w_kv, const void* w_gate,
                              csa_dtype_t in_dt, const float* ape, int Nc_cap, const float* d_out,
                              float* dx, float* dw_kv, float* dw_gate, float* dape,
                              void* workspace, size_t ws_bytes, hipStream_t stream);
size_t csa_compress_bwd_workspace_size(int B, int L, int d_model, int E, int m, int Nc_cap);

/*
 * csa_compress_bwd for a compressor whose entries were post-processed by
 * csa_compress_ex with opts (RMS norm, rotary embedding; NULL: none, which
 * is csa_compress_bwd).  The entry's gradient goes back through the
 * post-processing in reverse order (migration page, section 3.2: the
 * compressor's norm and its rotary embedding of the key positions; chain
 * rule through the definitions at csa_compress_opts_t): the Hadamard
 * rotation, the rotary embedding (the pair rotation at position -m i), and
 * the RMS norm y = C r w with r = (mean_e C_e^2 + norm_eps)^(-1/2):
 *     dC = r u - C r^3 (sum_e u_e C_e) / E,   u = g w,
 *     d_norm_weight[e] = sum over entries of g_e C_e r
 * (g the gradient reaching the norm's output).  d_norm_weight fp32 [E] is
 * required when opts has a norm weight (written in full; a fixed-order sum,
 * so repeated calls agree bit for bit) and ignored otherwise.  Errors: as
 * csa_compress_bwd, and CSA_E_ARG for opts that csa_compress_ex rejects or a
 * norm weight without d_norm_weight.  The workspace is
 * csa_compress_bwd_workspace_size() bytes, as for csa_compress_bwd.
 */
csa_status_t csa_compress_bwd_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                                 const void* x, const void* w_kv, const void* w_gate,
                                 csa_dtype_t in_dt, const float* ape, int Nc_cap,
                                 const float* d_out, const csa_compress_opts_t* opts, float* dx,
                                 float* dw_kv, float* dw_gate, float* dape, float* d_norm_weight,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);

/* Static text of a status code. */
const char* csa_status_string(csa_status_t status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* csa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
