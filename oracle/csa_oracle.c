/*
 * csa_oracle.c -- plain, slow CPU oracle for the compressed sparse attention
 * (CSA) / heavily compressed attention (HCA) path.
 *
 * TEST INFRASTRUCTURE ONLY.  It is loaded by tests/, by the smoke check and by
 * the CPU-baseline leg of the benchmark; the GPU library never links, includes
 * or calls it, and it shares no source with the GPU library.
 *
 * Everything is computed in IEEE double with plain loops, in the order the
 * method states its steps.  The only parallelism is an OpenMP loop over
 * independent rows (a batch element, a query token or a compressed entry).
 * Inputs are read in their stored formats (fp32, bf16 bits, OCP e4m3 codes)
 * and decoded by this file's own routines.
 *
 * Sources (web pages on DeepSeek-V4 hybrid attention):
 *  - "DeepSeek V4 CSA + CP migration to HP" (gitcode hyper-parallel issue 4),
 *    section 3.2: the compressor is linear_wkv + linear_wgate with a softmax
 *    over an overlapping window and an absolute position embedding `ape`;
 *    ratio 4 overlaps, ratio 128 does not.
 *  - "DS-V4 analysis" (edward-lyz), sections 1.2-1.5: m tokens -> one entry,
 *    each entry looks at 2m adjacent positions; indexer scores -> top-k ->
 *    attend to the k entries plus a sliding window of raw KV; HCA is dense
 *    over all compressed entries.
 *  - notion copy of the same, section 1.1: attention with 1/sqrt(head_dim)
 *    scale; MQA (one shared KV head).
 *  - chenxutan article, section 3.2 (mean-pool special case, entry count
 *    seq_len // m, simplified indexer einsum + topk) and section 5.2 (window
 *    rule: token i sees [max(0, i - W + 1), i]).
 *
 * Parity status per function (see the tests under tests/):
 *  - number formats: orc_bf16_decode is pinned to torch's bfloat16 on all
 *    65536 bit patterns, orc_e4m3_decode on all 256 codes, the encoders to
 *    torch's round-to-nearest-even casts (midpoints included), and
 *    orc_quant_rows_e4m3 (row scale amax / 448 in fp32, codes of the fp32
 *    quotient) to torch's float8_e4m3fn cast of the same quotient, zero rows
 *    and midpoint rows included.  Every stage fed bf16 patterns equals the
 *    same stage fed their torch-decoded values.
 *  - orc_compress: the uniform-gate / no-overlap case is pinned to the
 *    mean-pool closed form; the non-uniform overlapping gate form is the
 *    plainest reading of section 3.2 of the migration page and is otherwise
 *    "parity unpinned" by the pages.  The optional Hadamard rotation of an
 *    entry (the migration page names a Hadamard step in the compressor and
 *    the indexer, section 3.2; read as the Sylvester-ordered Walsh-Hadamard
 *    matrix scaled by 1/sqrt(E)) is pinned to a library Hadamard matrix.
 *  - orc_indexer_topk: the score formula (sum over heads of w * ReLU(q.k)) is
 *    the published Lightning Indexer form; the pages print only its one-head
 *    special case, so the multi-head form is "parity unpinned"; the top-k
 *    order is pinned against a library sort.  The optional MXFP4
 *    inputs (the CSA/HCA article, section 3.2, notes that the indexer
 *    computes in FP4 and nothing more; read as OCP MXFP4: E2M1 values with an
 *    E8M0 scale per 32) are pinned to the standard's E2M1 table, to nearest-value
 *    rounding by brute force, to a library E8M0 decode, and to the fp32
 *    path on the decoded values.
 *  - orc_sparse_attn / orc_hca_dense_attn: pinned to a library scaled
 *    dot-product attention with an explicit mask.  The optional per-head
 *    attention sink (the migration page lists `attn_sink` among the state of
 *    CompressedSparseAttention; read as one more softmax term with logit
 *    sink[h] and no value) is pinned to the same attention with one extra
 *    key whose logit equals the sink and whose value is zero.
 *  - orc_attn_bwd (both attention forms, sink and per-slot attention mass):
 *    pinned to torch autograd through the library attention with an explicit
 *    mask, to central differences of orc_sparse_attn, and to the identities
 *    sum dV = sum dO, sum dK = 0, sum q.dq = sum K.dK.
 *  - orc_indexer_kl_bwd: the loss form is a reading (the pages name the
 *    loss, not its formula; see the function); given that reading it is
 *    pinned to torch autograd through torch's kl_div and log_softmax (sparse
 *    and dense forms), and to its closed forms (zero at the indexer's own
 *    distribution, linearity in the gradient scale); the HCA form's
 *    per-entry mass to the library softmax summed over heads.
 *  - orc_compress_bwd / orc_compress_bwd_ex: pinned to central differences
 *    of orc_compress_ex (with and without the norm, the rotary embedding and
 *    the Hadamard step, the norm weight's gradient included) and to the
 *    mean-pool closed form.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_E4M3 = 2, ODT_MXFP4 = 3 };

/* ---- number formats ---------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32 value. */
double orc_bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite magnitude 1.75 * 2^8 = 448;
 * exponent field 0 encodes subnormals m/8 * 2^-6. */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, mant = c & 7;
  double v;
  if (e == 15 && mant == 7) return NAN;
  if (e == 0)
    v = ldexp((double)mant / 8.0, -6);
  else
    v = ldexp(1.0 + (double)mant / 8.0, e - 7);
  return s ? -v : v;
}

/* Round half to even of a non-negative double to an integer value. */
static double rne(double r) {
  double f = floor(r);
  double d = r - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* Encode a double as e4m3 with round-to-nearest-even; magnitudes beyond the
 * largest finite value saturate to +-448 (the saturating conversion). */
uint8_t orc_e4m3_encode(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v), q, r;
  int ex, e;
  if (isnan(v)) return 0x7f;
  if (a == 0) return sign;
  frexp(a, &ex);
  e = ex - 1;            /* a lies in [2^e, 2^(e+1)) */
  if (e < -6) e = -6;    /* subnormals share the binade-(-6) spacing 2^-9 */
  q = ldexp(1.0, e - 3); /* spacing of the 3-bit mantissa in this binade */
  r = rne(a / q) * q;    /* a / q is exact: q is a power of two */
  if (r > 448.0) return sign | 0x7e;
  if (r == 0) return sign;
  frexp(r, &ex);
  e = ex - 1;
  if (e < -6) return sign | (uint8_t)(r / ldexp(1.0, -9));
  return sign | (uint8_t)(((e + 7) << 3) | (int)((r / ldexp(1.0, e) - 1.0) * 8.0));
}

/* bf16 round-to-nearest-even of a double (rounded to binary32 first). */
uint16_t orc_bf16_encode(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP MX FP4 element (E2M1): 1 sign, 2 exponent (bias 1), 1 mantissa bit, no
 * infinities or NaN.  Exponent field e > 0: (1 + m / 2) 2^(e - 1); e = 0: the
 * subnormal m / 2.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_e2m1_decode(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, mant = c & 1;
  double v = e == 0 ? 0.5 * mant : ldexp(1.0 + 0.5 * mant, e - 1);
  return s ? -v : v;
}

/* Encode a double as E2M1 with round-to-nearest-even; magnitudes beyond 6
 * saturate to +-6.  The 4-bit code is returned in the low nibble. */
uint8_t orc_e2m1_encode(double v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double a = fabs(v), q, r;
  int ex, e;
  if (isnan(v) || a == 0) return sign;
  frexp(a, &ex);
  e = ex - 1;           /* a lies in [2^e, 2^(e+1)) */
  if (e < 0) e = 0;     /* below 1 the subnormal spacing 0.5 continues */
  q = ldexp(1.0, e - 1); /* spacing of the 1-bit mantissa in this binade */
  r = rne(a / q) * q;
  if (r > 6.0) r = 6.0;
  if (r == 0) return sign;
  if (r == 0.5) return sign | 1;
  frexp(r, &ex);
  e = ex - 1;
  return sign | (uint8_t)(((e + 1) << 1) | (int)((r / ldexp(1.0, e) - 1.0) * 2.0));
}

/* MX block scale (OCP Microscaling formats v1.0, the conversion section):
 * shared exponent X = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent),
 * clamped to the E8M0 range [-127, 127]; X = 0 for an all-zero block.  The
 * E8M0 code is X + 127 and the scale 2^X. */
static int mx_exponent(double amax) {
  int ex, x;
  if (!(amax > 0)) return 0;
  frexp(amax, &ex);
  x = (ex - 1) - 2;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

/* MXFP4 quantisation of rows of `cols` values (cols a multiple of 32): per
 * 32-value block the shared exponent above, then code = E2M1(v / 2^X).  Codes
 * pack two per byte, element 2i in the low nibble; scales are E8M0 codes,
 * cols / 32 per row. */
void orc_quant_rows_mxfp4(int rows, int cols, const double* in, uint8_t* codes,
                          uint8_t* scales) {
  for (int r = 0; r < rows; ++r)
    for (int blk = 0; blk < cols / 32; ++blk) {
      const double* v = in + (size_t)r * cols + 32 * blk;
      double amax = 0;
      int x;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[i]));
      x = mx_exponent(amax);
      scales[(size_t)r * (cols / 32) + blk] = (uint8_t)(x + 127);
      for (int i = 0; i < 32; i += 2) {
        uint8_t lo = orc_e2m1_encode(ldexp(v[i], -x));
        uint8_t hi = orc_e2m1_encode(ldexp(v[i + 1], -x));
        codes[(size_t)r * (cols / 2) + 16 * blk + i / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
}

/* Value of element i of an MXFP4 row store (codes as above, scales E8M0). */
static double ld_mxfp4(const uint8_t* codes, const uint8_t* scales, size_t i) {
  uint8_t byte = codes[i / 2];
  uint8_t c = (i & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  return ldexp(orc_e2m1_decode(c), (int)scales[i / 32] - 127);
}

static double ld(const void* p, size_t i, int dt) {
  switch (dt) {
    case ODT_F32: return (double)((const float*)p)[i];
    case ODT_BF16: return orc_bf16_decode(((const uint16_t*)p)[i]);
    default: return orc_e4m3_decode(((const uint8_t*)p)[i]);
  }
}

/* Per-row e4m3 quantisation as the compressor's fp8 store defines it: the
 * stored row scale is the fp32 value s = amax / 448 (s = 1 for an all-zero
 * row), and each code is the e4m3 rounding (nearest even, saturating at 448)
 * of the IEEE fp32 quotient v / s.  The quotient is formed in fp32 because
 * that is the precision the scale is stored and applied in; rounding it to
 * e4m3 afterwards is the reading taken of "divide by the row scale, then
 * round". */
void orc_quant_rows_e4m3(int rows, int cols, const double* in, uint8_t* codes,
                         double* scales) {
  for (int r = 0; r < rows; ++r) {
    double amax = 0;
    float s;
    for (int c = 0; c < cols; ++c) amax = fmax(amax, fabs(in[(size_t)r * cols + c]));
    s = amax > 0 ? (float)(amax / 448.0) : 1.0f;
    scales[r] = (double)s;
    for (int c = 0; c < cols; ++c) {
      volatile float q = (float)in[(size_t)r * cols + c] / s; /* one fp32 divide */
      codes[(size_t)r * cols + c] = orc_e4m3_encode((double)q);
    }
  }
}

/* ---- compressor ---------------------------------------------------------
 * Token j (absolute position) has a projected value P_j = W_kv x_j and gate
 * logits G_j = W_gate x_j, both of width E (weights stored [E, d_model]).  Compressed entry i pools the
 * window of tokens [m (i - o), m (i + 1)) (o = 1: the previous block and its
 * own block, 2m tokens; o = 0: its own m tokens), restricted to j >= 0:
 *     a_{j,e} = softmax over the window of (G_{j,e} + ape[j - m (i - o), e])
 *     C_{i,e} = sum_j a_{j,e} P_{j,e}.
 * Entry i exists once its last token m (i + 1) - 1 has been seen.  A call
 * processes tokens [pos0, pos0 + L) of each sequence; the previous
 * (1 + o) m - 1 tokens come from state_in (P then G per token, in position
 * order; absent tokens carry P = 0, G = -inf, which gives them zero weight).
 * state_out receives the same record for the last (1 + o) m - 1 tokens.
 * Output rows are written (double, before any storage rounding) for every
 * entry completed in the call with i < Nc_cap; written[b, i] flags them.
 * With rotate, each written row C_i is replaced by H C_i / sqrt(E), H the
 * Walsh-Hadamard matrix of order E (a power of two) in Sylvester order,
 * H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]. */
static void hadamard_rows(double* v, int E) {
  for (int len = 1; len < E; len <<= 1)
    for (int blk = 0; blk < E; blk += 2 * len)
      for (int j = blk; j < blk + len; ++j) {
        const double a = v[j], c = v[j + len];
        v[j] = a + c;
        v[j + len] = a - c;
      }
  for (int e = 0; e < E; ++e) v[e] /= sqrt((double)E);
}

/* Entry post-processing, applied in this order to each emitted entry C_i
 * (migration page, section 3.2: the compressor carries a norm submodule,
 * ApplyRotaryPosEmb for the key positions, and a Hadamard step; section 4.3
 * gives layernorm_epsilon and rotary_interleaved = False as its config):
 *  - RMS norm (norm_w != NULL): C_e <- C_e / sqrt(mean_e C_e^2 + eps) * w_e
 *    over the entry's E channels;
 *  - rotary position embedding (rope_dim > 0): the channels
 *    [rope_off, rope_off + rope_dim) rotate by the angles p * base^(-2k/rope_dim),
 *    k < rope_dim / 2, at the entry's position p = m i (the first token of its
 *    own block).  Non-interleaved: channel k pairs with k + rope_dim / 2;
 *    interleaved: 2k with 2k + 1.  A pair (a, b) becomes
 *    (a cos - b sin, b cos + a sin);
 *  - the Hadamard rotation (rotate).
 * The three readings (RMS norm over the whole entry, the block's first token
 * as the position, this order) are the plainest ones the pages leave open. */
typedef struct {
  const double* norm_w;
  double norm_eps;
  int rope_dim, rope_off, rope_interleaved;
  double rope_base;
} orc_compress_opts;

static void rms_norm_row(double* v, int E, const double* w, double eps) {
  double ss = 0;
  for (int e = 0; e < E; ++e) ss += v[e] * v[e];
  const double r = 1.0 / sqrt(ss / E + eps);
  for (int e = 0; e < E; ++e) v[e] = v[e] * r * w[e];
}

static void rope_row(double* v, int R, int interleaved, double base, int64_t pos) {
  for (int k = 0; k < R / 2; ++k) {
    const double ang = (double)pos * pow(base, -2.0 * k / R);
    const double c = cos(ang), s = sin(ang);
    const int i0 = interleaved ? 2 * k : k, i1 = interleaved ? 2 * k + 1 : k + R / 2;
    const double a = v[i0], b = v[i1];
    v[i0] = a * c - b * s;
    v[i1] = b * c + a * s;
  }
}

int orc_compress_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                    const int64_t* pos0, const void* x, const void* w_kv,
                    const void* w_gate, int in_dt, const double* ape,
                    const double* state_in, double* state_out, int Nc_cap,
                    double* out, uint8_t* written, const orc_compress_opts* opts);

int orc_compress(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                 const int64_t* pos0, const void* x, const void* w_kv,
                 const void* w_gate, int in_dt, const double* ape,
                 const double* state_in, double* state_out, int Nc_cap,
                 double* out, uint8_t* written) {
  return orc_compress_ex(B, L, d_model, E, m, overlap, rotate, pos0, x, w_kv, w_gate, in_dt,
                         ape, state_in, state_out, Nc_cap, out, written, NULL);
}

int orc_compress_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                    const int64_t* pos0, const void* x, const void* w_kv,
                    const void* w_gate, int in_dt, const double* ape,
                    const double* state_in, double* state_out, int Nc_cap,
                    double* out, uint8_t* written, const orc_compress_opts* opts) {
  const int Sw = (1 + overlap) * m, ns = Sw - 1;
  if (B < 0 || L < 0 || m < 1 || E < 1 || d_model < 1) return 1;
  if (rotate && (E & (E - 1))) return 1;
  if (opts && opts->rope_dim &&
      (opts->rope_dim < 0 || opts->rope_dim % 2 || opts->rope_off < 0 ||
       opts->rope_off + opts->rope_dim > E))
    return 1;
  for (int b = 0; b < B; ++b) {
    const int64_t p0 = pos0[b];
    const int64_t base = p0 - ns; /* position of token-table row 0 */
    const int ntok = ns + L;
    double* P = (double*)calloc((size_t)ntok * E, sizeof(double));
    double* G = (double*)malloc((size_t)ntok * E * sizeof(double));
    for (size_t k = 0; k < (size_t)ntok * E; ++k) G[k] = -INFINITY;
    /* carried tokens */
    for (int s = 0; s < ns; ++s) {
      int64_t pos = base + s;
      if (pos < 0 || !state_in) continue;
      for (int e = 0; e < E; ++e) {
        P[(size_t)s * E + e] = state_in[(((size_t)b * ns + s) * 2 + 0) * E + e];
        G[(size_t)s * E + e] = state_in[(((size_t)b * ns + s) * 2 + 1) * E + e];
      }
    }
    /* projections of the new tokens */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < L; ++t) {
      for (int e = 0; e < E; ++e) {
        double pk = 0, gk = 0;
        for (int k = 0; k < d_model; ++k) {
          double xv = ld(x, ((size_t)b * L + t) * d_model + k, in_dt);
          pk += xv * ld(w_kv, (size_t)e * d_model + k, in_dt);
          gk += xv * ld(w_gate, (size_t)e * d_model + k, in_dt);
        }
        P[(size_t)(ns + t) * E + e] = pk;
        G[(size_t)(ns + t) * E + e] = gk;
      }
    }
    /* entries completed by this chunk */
    {
      int64_t i_lo = (p0 + 1 + m - 1) / m - 1; /* smallest i with m(i+1)-1 >= p0 */
      int64_t i_hi = (p0 + L) / m - 1;         /* largest i with m(i+1)-1 < p0+L */
      if (i_lo < 0) i_lo = 0;
#pragma omp parallel for schedule(static)
      for (int64_t i = i_lo; i <= i_hi; ++i) {
        int64_t first = (int64_t)m * (i - overlap);
        int64_t last = (int64_t)m * (i + 1) - 1;
        if (i >= Nc_cap) continue;
        for (int e = 0; e < E; ++e) {
          double mx = -INFINITY, den = 0, num = 0;
          for (int64_t j = first; j <= last; ++j) {
            double z;
            if (j < 0) continue;
            z = G[(size_t)(j - base) * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
            if (z > mx) mx = z;
          }
          for (int64_t j = first; j <= last; ++j) {
            double z, w;
            if (j < 0) continue;
            z = G[(size_t)(j - base) * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
            if (z == -INFINITY) continue;
            w = exp(z - mx);
            den += w;
            num += w * P[(size_t)(j - base) * E + e];
          }
          out[((size_t)b * Nc_cap + i) * E + e] = num / den;
        }
        if (opts && opts->norm_w)
          rms_norm_row(out + ((size_t)b * Nc_cap + i) * E, E, opts->norm_w, opts->norm_eps);
        if (opts && opts->rope_dim)
          rope_row(out + ((size_t)b * Nc_cap + i) * E + opts->rope_off, opts->rope_dim,
                   opts->rope_interleaved, opts->rope_base, (int64_t)m * i);
        if (rotate) hadamard_rows(out + ((size_t)b * Nc_cap + i) * E, E);
        if (written) written[(size_t)b * Nc_cap + i] = 1;
      }
    }
    /* carried state for the next call */
    if (state_out) {
      for (int s = 0; s < ns; ++s) {
        int64_t pos = p0 + L - ns + s;
        int64_t row = pos - base;
        for (int e = 0; e < E; ++e) {
          double pv = 0, gv = -INFINITY;
          if (pos >= 0) {
            pv = P[(size_t)row * E + e];
            gv = G[(size_t)row * E + e];
          }
          state_out[(((size_t)b * ns + s) * 2 + 0) * E + e] = pv;
          state_out[(((size_t)b * ns + s) * 2 + 1) * E + e] = gv;
        }
      }
    }
    free(P);
    free(G);
  }
  return 0;
}

/* ---- visibility -----------------------------------------------------------
 * A query at absolute position t sees compressed entry i iff the entry's last
 * token m (i + 1) - 1 is at or before t; at most n_cmp entries exist. */
static int64_t n_visible(int64_t t, int64_t n_cmp, int m, int64_t cap) {
  int64_t n = (t + 1) / m;
  if (t < 0) n = 0;
  if (n > n_cmp) n = n_cmp;
  if (n > cap) n = cap;
  if (n < 0) n = 0;
  return n;
}

/* ---- Lightning Indexer score + top-k --------------------------------------
 * score(t, j) = sum_h w[t,h] * ReLU(sq[t,h] * sk[j] * sum_e q[t,h,e] k[j,e])
 * over the visible entries j < n_vis(t) (sq = sk = 1 unless e4m3; MXFP4
 * values carry their block scales: q and k are the decoded values).
 * Selection: the first min(topk, n_vis) entries under the order
 * (score descending, index ascending), written in ascending index order and
 * padded with -1.  sel_score receives the selected scores aligned with
 * idx_out (NaN in padded slots); kth receives the score of the last selected
 * entry in selection order (NaN if none); all_scores (optional) every score,
 * NaN for invisible entries. */
typedef struct {
  double s;
  int32_t j;
} scored;

static int by_score_desc_index_asc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int by_int_asc(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int orc_indexer_topk(int B, int T, int H_I, int d_I, int Nc_cap, int m, int topk,
                     const int64_t* q_pos, const int32_t* n_cmp, const void* q_idx,
                     const void* q_scale, const float* w_idx, const void* k_idx,
                     const void* k_scale, int qk_dt, int32_t* idx_out,
                     double* sel_score, double* kth, double* all_scores) {
  if (B < 0 || T < 0 || H_I < 1 || d_I < 1 || m < 1 || topk < 0) return 1;
  if (qk_dt == ODT_MXFP4 && d_I % 32 != 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
    int b = (int)(bt / T), t = (int)(bt % T);
    int64_t pos = q_pos[b] + t;
    int64_t nv = n_visible(pos, n_cmp[b], m, Nc_cap);
    int nsel = (int)(nv < topk ? nv : topk);
    scored* row = (scored*)malloc(sizeof(scored) * (nv > 0 ? nv : 1));
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (nsel > 0 ? nsel : 1));
    for (int64_t j = 0; j < nv; ++j) {
      const size_t krow = (size_t)b * Nc_cap + j;
      double sk = (qk_dt == ODT_E4M3) ? (double)((const float*)k_scale)[krow] : 1.0;
      double s = 0;
      for (int h = 0; h < H_I; ++h) {
        size_t qrow = (((size_t)b * T + t) * H_I + h);
        double sq = (qk_dt == ODT_E4M3) ? (double)((const float*)q_scale)[qrow] : 1.0;
        double dot = 0, v;
        if (qk_dt == ODT_MXFP4) {
          /* per-block scales are part of each value */
          const uint8_t* qc = (const uint8_t*)q_idx + qrow * (d_I / 2);
          const uint8_t* qs = (const uint8_t*)q_scale + qrow * (d_I / 32);
          const uint8_t* kc = (const uint8_t*)k_idx + krow * (d_I / 2);
          const uint8_t* ks = (const uint8_t*)k_scale + krow * (d_I / 32);
          for (int e = 0; e < d_I; ++e) dot += ld_mxfp4(qc, qs, e) * ld_mxfp4(kc, ks, e);
        } else {
          for (int e = 0; e < d_I; ++e)
            dot += ld(q_idx, qrow * d_I + e, qk_dt) * ld(k_idx, krow * d_I + e, qk_dt);
        }
        v = sq * sk * dot;
        s += (double)w_idx[qrow] * (v > 0 ? v : 0.0);
      }
      row[j].s = s;
      row[j].j = (int32_t)j;
      if (all_scores) all_scores[((size_t)b * T + t) * Nc_cap + j] = s;
    }
    if (all_scores)
      for (int64_t j = nv; j < Nc_cap; ++j) all_scores[((size_t)b * T + t) * Nc_cap + j] = NAN;
    qsort(row, (size_t)nv, sizeof(scored), by_score_desc_index_asc);
    for (int k = 0; k < nsel; ++k) sel[k] = row[k].j;
    if (kth) kth[(size_t)b * T + t] = nsel > 0 ? row[nsel - 1].s : NAN;
    qsort(sel, (size_t)nsel, sizeof(int32_t), by_int_asc);
    for (int k = 0; k < topk; ++k) {
      size_t o = ((size_t)b * T + t) * topk + k;
      idx_out[o] = k < nsel ? sel[k] : -1;
      if (sel_score) {
        double sv = NAN;
        if (k < nsel) {
          /* recover the score of sel[k] from the sorted row */
          for (int q = 0; q < nsel; ++q)
            if (row[q].j == sel[k]) { sv = row[q].s; break; }
        }
        sel_score[o] = sv;
      }
    }
    free(row);
    free(sel);
  }
  return 0;
}

/* ---- attention ------------------------------------------------------------
 * MQA: all H query heads share one KV head; a KV row is [K | V] of width 2D.
 * For query token t (absolute position pos) and head h, the attended key set
 * J is the union of the compressed rows named by idx (entries outside
 * [0, Nc_cap) are skipped) and the raw tokens j in [max(0, pos - W + 1), pos]
 * whose row r = j - raw_base lies in [0, R_cap).  One softmax runs over J:
 *     l_j = scale * q . K_j,  out = sum_j softmax(l)_j V_j,
 *     lse = log sum_j exp(l_j)   (natural log).
 * With a sink z (finite), the softmax runs over the logits l_j and z, the
 * sink carrying no value:  out = sum_j e^{l_j} V_j / (e^z + sum_j e^{l_j}),
 * lse = log(e^z + sum_j e^{l_j}).  sink = -inf is no sink.
 * An empty J gives out = 0 and lse = -inf (= z with a sink). */
static void attend_row(int D, double scale, const void* q, size_t qoff, int dt,
                       const void* const* rows_src, const size_t* rows_off, int n,
                       double sink, double* o, double* lse) {
  double mx = sink, den = 0;
  double* l = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
  for (int d = 0; d < D; ++d) o[d] = 0;
  for (int r = 0; r < n; ++r) {
    double dot = 0;
    for (int d = 0; d < D; ++d) dot += ld(q, qoff + d, dt) * ld(rows_src[r], rows_off[r] + d, dt);
    l[r] = scale * dot;
    if (l[r] > mx) mx = l[r];
  }
  for (int r = 0; r < n; ++r) {
    double p = exp(l[r] - mx);
    den += p;
    for (int d = 0; d < D; ++d) o[d] += p * ld(rows_src[r], rows_off[r] + D + d, dt);
  }
  if (sink > -INFINITY) den += exp(sink - mx);
  if (den > 0) {
    for (int d = 0; d < D; ++d) o[d] /= den;
    *lse = mx + log(den);
  } else {
    *lse = -INFINITY;
  }
  free(l);
}

/* sink: [H] logits or NULL (no sink), for both attention forms. */
int orc_sparse_attn(int B, int T, int H, int D, int topk, int window, double scale,
                    const double* sink, const int64_t* q_pos, const void* q, const void* kv_cmp,
                    int Nc_cap, const int32_t* idx, const void* kv_raw, int R_cap,
                    const int64_t* raw_base, int dt, double* out, double* lse) {
  if (B < 0 || T < 0 || H < 1 || D < 1 || topk < 0 || window < 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
    int b = (int)(bt / T), t = (int)(bt % T);
    int64_t pos = q_pos[b] + t;
    int cap = topk + window;
    const void** src = (const void**)malloc(sizeof(void*) * (cap > 0 ? cap : 1));
    size_t* off = (size_t*)malloc(sizeof(size_t) * (cap > 0 ? cap : 1));
    int n = 0;
    for (int k = 0; k < topk; ++k) {
      int32_t j = idx[((size_t)b * T + t) * topk + k];
      if (j < 0 || j >= Nc_cap) continue;
      src[n] = kv_cmp;
      off[n++] = ((size_t)b * Nc_cap + j) * 2 * D;
    }
    if (window > 0) {
      int64_t lo = pos - window + 1;
      if (lo < 0) lo = 0;
      for (int64_t j = lo; j <= pos; ++j) {
        int64_t r = j - raw_base[b];
        if (r < 0 || r >= R_cap) continue;
        src[n] = kv_raw;
        off[n++] = ((size_t)b * R_cap + (size_t)r) * 2 * D;
      }
    }
    for (int h = 0; h < H; ++h) {
      size_t row = ((size_t)b * T + t) * H + h;
      double l;
      attend_row(D, scale, q, row * D, dt, src, off, n, sink ? sink[h] : -INFINITY, out + row * D,
                 &l);
      if (lse) lse[row] = l;
    }
    free(src);
    free(off);
  }
  return 0;
}

/* HCA: the compressed part of the key set is every visible entry
 * [0, n_vis(pos)), n_vis as for the indexer; the window part is as above. */
int orc_hca_dense_attn(int B, int T, int H, int D, int m, int window, double scale,
                       const double* sink, const int64_t* q_pos, const int32_t* n_cmp, const void* q,
                       const void* kv_cmp, int Nc_cap, const void* kv_raw, int R_cap,
                       const int64_t* raw_base, int dt, double* out, double* lse) {
  if (B < 0 || T < 0 || H < 1 || D < 1 || m < 1 || window < 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
    int b = (int)(bt / T), t = (int)(bt % T);
    int64_t pos = q_pos[b] + t;
    int64_t nv = n_visible(pos, n_cmp[b], m, Nc_cap);
    int64_t cap = nv + window;
    const void** src = (const void**)malloc(sizeof(void*) * (cap > 0 ? cap : 1));
    size_t* off = (size_t*)malloc(sizeof(size_t) * (cap > 0 ? cap : 1));
    int n = 0;
    for (int64_t j = 0; j < nv; ++j) {
      src[n] = kv_cmp;
      off[n++] = ((size_t)b * Nc_cap + j) * 2 * D;
    }
    if (window > 0) {
      int64_t lo = pos - window + 1;
      if (lo < 0) lo = 0;
      for (int64_t j = lo; j <= pos; ++j) {
        int64_t r = j - raw_base[b];
        if (r < 0 || r >= R_cap) continue;
        src[n] = kv_raw;
        off[n++] = ((size_t)b * R_cap + (size_t)r) * 2 * D;
      }
    }
    for (int h = 0; h < H; ++h) {
      size_t row = ((size_t)b * T + t) * H + h;
      double l;
      attend_row(D, scale, q, row * D, dt, src, off, n, sink ? sink[h] : -INFINITY, out + row * D,
                 &l);
      if (lse) lse[row] = l;
    }
    free(src);
    free(off);
  }
  return 0;
}

/* ---- attention backward ---------------------------------------------------
 * Gradients of the attention above (either form) for an upstream gradient dO
 * of out, by the chain rule through its definition.  Per query token and head,
 * over the same key set J and softmax:
 *     P_j = e^{l_j - lse},  P_z = e^{z - lse} (the sink, no value),
 *     dP_j = dO . V_j,      delta = sum_j P_j dP_j = dO . out,
 *     dl_j = P_j (dP_j - delta),  dz = -P_z delta,
 *     dq += scale sum_j dl_j K_j,  dK_j += scale dl_j q,  dV_j += P_j dO.
 * dK_j and dV_j sum over every (token, head) whose key set holds row j (the
 * compressed entry or the raw row), so they land in dkv_cmp [B, Nc_cap, 2D] /
 * dkv_raw [B, R_cap, 2D] as [dK | dV]; dsink [H] sums dz over all tokens.
 * idx == NULL selects the HCA form (every visible entry, m and n_cmp as for
 * the indexer), otherwise the CSA form over idx.  attn_mass (optional)
 * receives sum_h P_j, the attention's probability mass on an entry over all
 * heads: per selected slot in the CSA form ([B, T, topk], 0 in skipped
 * slots), per entry in the HCA form ([B, T, Nc_cap], 0 past the visible
 * entries) - the dense indexer loss's target.
 * The caller zeroes nothing: every output is written in full. */
int orc_attn_bwd(int B, int T, int H, int D, int topk, int window, double scale,
                 const double* sink, const int64_t* q_pos, const void* q, const void* kv_cmp,
                 int Nc_cap, const int32_t* idx, int m, const int32_t* n_cmp,
                 const void* kv_raw, int R_cap, const int64_t* raw_base, int dt,
                 const double* dout, double* dq, double* dkv_cmp, double* dkv_raw,
                 double* dsink, double* attn_mass) {
  if (B < 0 || T < 0 || H < 1 || D < 1 || topk < 0 || window < 0) return 1;
  if (!idx && (m < 1 || !n_cmp)) return 1;
  memset(dkv_cmp, 0, sizeof(double) * (size_t)B * Nc_cap * 2 * D);
  memset(dkv_raw, 0, sizeof(double) * (size_t)B * R_cap * 2 * D);
  if (dsink) memset(dsink, 0, sizeof(double) * H);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
    const int b = (int)(bt / T), t = (int)(bt % T);
    const int64_t pos = q_pos[b] + t;
    const int64_t nv = idx ? 0 : n_visible(pos, n_cmp[b], m, Nc_cap);
    const int64_t cap = (idx ? topk : nv) + window;
    /* key list: source flag (0 compressed, 1 raw), row, and the slot of a
     * selected entry (-1 otherwise) */
    int* src = (int*)malloc(sizeof(int) * (cap > 0 ? cap : 1));
    int64_t* row = (int64_t*)malloc(sizeof(int64_t) * (cap > 0 ? cap : 1));
    int* slot = (int*)malloc(sizeof(int) * (cap > 0 ? cap : 1));
    double* l = (double*)malloc(sizeof(double) * (cap > 0 ? cap : 1));
    double* P = (double*)malloc(sizeof(double) * (cap > 0 ? cap : 1));
    double* o = (double*)malloc(sizeof(double) * D);
    int n = 0;
    if (idx) {
      for (int k = 0; k < topk; ++k) {
        const int32_t j = idx[((size_t)b * T + t) * topk + k];
        if (attn_mass) attn_mass[((size_t)b * T + t) * topk + k] = 0;
        if (j < 0 || j >= Nc_cap) continue;
        src[n] = 0, row[n] = j, slot[n++] = k;
      }
    } else {
      if (attn_mass)
        for (int64_t j = 0; j < Nc_cap; ++j) attn_mass[((size_t)b * T + t) * Nc_cap + j] = 0;
      for (int64_t j = 0; j < nv; ++j) src[n] = 0, row[n] = j, slot[n++] = (int)j;
    }
    if (window > 0) {
      int64_t lo = pos - window + 1;
      if (lo < 0) lo = 0;
      for (int64_t j = lo; j <= pos; ++j) {
        const int64_t r = j - raw_base[b];
        if (r < 0 || r >= R_cap) continue;
        src[n] = 1, row[n] = r, slot[n++] = -1;
      }
    }
    for (int h = 0; h < H; ++h) {
      const size_t qr = ((size_t)b * T + t) * H + h;
      const double z = sink ? sink[h] : -INFINITY;
      const double* dO = dout + qr * D;
      /* forward quantities */
      double mx = z, den = 0;
      for (int r = 0; r < n; ++r) {
        const void* kv = src[r] ? kv_raw : kv_cmp;
        const size_t ko = ((size_t)b * (src[r] ? R_cap : Nc_cap) + row[r]) * 2 * D;
        double dot = 0;
        for (int d = 0; d < D; ++d) dot += ld(q, qr * D + d, dt) * ld(kv, ko + d, dt);
        l[r] = scale * dot;
        if (l[r] > mx) mx = l[r];
      }
      for (int r = 0; r < n; ++r) den += exp(l[r] - mx);
      if (z > -INFINITY) den += exp(z - mx);
      for (int d = 0; d < D; ++d) dq[qr * D + d] = 0;
      if (den == 0) continue; /* empty key set: out = 0, no gradient */
      const double lse = mx + log(den);
      for (int d = 0; d < D; ++d) o[d] = 0;
      for (int r = 0; r < n; ++r) {
        const void* kv = src[r] ? kv_raw : kv_cmp;
        const size_t ko = ((size_t)b * (src[r] ? R_cap : Nc_cap) + row[r]) * 2 * D;
        P[r] = exp(l[r] - lse);
        for (int d = 0; d < D; ++d) o[d] += P[r] * ld(kv, ko + D + d, dt);
      }
      double delta = 0;
      for (int d = 0; d < D; ++d) delta += dO[d] * o[d];
      if (dsink && z > -INFINITY) {
        const double dz = -exp(z - lse) * delta;
#pragma omp atomic
        dsink[h] += dz;
      }
      /* backward through the softmax and both products */
      for (int r = 0; r < n; ++r) {
        const void* kv = src[r] ? kv_raw : kv_cmp;
        double* g = (src[r] ? dkv_raw : dkv_cmp) +
                    ((size_t)b * (src[r] ? R_cap : Nc_cap) + row[r]) * 2 * D;
        const size_t ko = ((size_t)b * (src[r] ? R_cap : Nc_cap) + row[r]) * 2 * D;
        double dP = 0;
        for (int d = 0; d < D; ++d) dP += dO[d] * ld(kv, ko + D + d, dt);
        const double dl = P[r] * (dP - delta);
        for (int d = 0; d < D; ++d) {
          const double gk = scale * dl * ld(q, qr * D + d, dt);
          const double gv = P[r] * dO[d];
          dq[qr * D + d] += scale * dl * ld(kv, ko + d, dt);
#pragma omp atomic
          g[d] += gk;
#pragma omp atomic
          g[D + d] += gv;
        }
        if (attn_mass && slot[r] >= 0)
          attn_mass[((size_t)b * T + t) * (idx ? topk : Nc_cap) + slot[r]] += P[r];
      }
    }
    free(src);
    free(row);
    free(slot);
    free(l);
    free(P);
    free(o);
  }
  return 0;
}

/* ---- indexer KL loss and its gradient --------------------------------------
 * The migration page (sections 1 and 3.2) names an indexer loss for training,
 * a fused sparse "lightning indexer grad + KL loss" operator, a loss
 * coefficient and a sparse-loss switch (config, section 4.3), but not the
 * formula.  Reading (sparse form): per query token, over its selected entries
 * S (the slots of idx with 0 <= idx < Nc_cap), the target is the main
 * attention's probability mass on each entry summed over heads (attn_mass,
 * from orc_attn_bwd), normalised over S:  p_k = mass_k / sum_S mass; the
 * indexer's distribution is the softmax over S of its scores I_k (as in
 * orc_indexer_topk):  q_k = e^{I_k} / sum_S e^{I}.  The row's loss is
 * KL(p || q) = sum_S p_k (log p_k - log q_k), with 0 log 0 = 0.  The target
 * carries no gradient; with g = grad_scale[row] (the caller's loss
 * coefficient and averaging), dI_k = g (q_k - p_k), and through the score
 * (v_hk = q_h . k_j, I_k = sum_h w_h ReLU(v_hk), ReLU'(0) = 0):
 *     dw[t,h] = sum_k dI_k ReLU(v_hk),
 *     dq[t,h] = sum_k dI_k w_h [v_hk > 0] k_j,
 *     dk[j]  += sum_h dI_k w_h [v_hk > 0] q_h     (j = idx_k).
 * Inputs fp32 or bf16 (the training formats).  A row with no selected entry
 * or zero total mass has loss 0 and no gradient.  The dense form (the
 * config's sparse-loss switch off) is this function over every visible entry:
 * slots 0 .. n_vis - 1 in order, with the HCA form's per-entry mass of
 * orc_attn_bwd as the target (oracle.py builds that index list). */
int orc_indexer_kl_bwd(int B, int T, int H_I, int d_I, int Nc_cap, int topk, const void* q_idx,
                       const float* w_idx, const void* k_idx, int qk_dt, const int32_t* idx,
                       const double* mass, const double* grad_scale, double* loss,
                       double* dq_idx, double* dw_idx, double* dk_idx) {
  if (B < 0 || T < 0 || H_I < 1 || d_I < 1 || topk < 0) return 1;
  if (qk_dt != ODT_F32 && qk_dt != ODT_BF16) return 1;
  memset(dk_idx, 0, sizeof(double) * (size_t)B * Nc_cap * d_I);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
    const int b = (int)(bt / T);
    double* I = (double*)malloc(sizeof(double) * (topk > 0 ? topk : 1));
    double* dI = (double*)malloc(sizeof(double) * (topk > 0 ? topk : 1));
    const int32_t* irow = idx + (size_t)bt * topk;
    const double* mrow = mass + (size_t)bt * topk;
    double msum = 0, imax = -INFINITY;
    int any = 0;
    for (int h = 0; h < H_I; ++h) {
      dw_idx[(size_t)bt * H_I + h] = 0;
      for (int e = 0; e < d_I; ++e) dq_idx[((size_t)bt * H_I + h) * d_I + e] = 0;
    }
    loss[bt] = 0;
    for (int k = 0; k < topk; ++k) {
      const int32_t j = irow[k];
      dI[k] = 0;
      if (j < 0 || j >= Nc_cap) continue;
      double s = 0;
      for (int h = 0; h < H_I; ++h) {
        const size_t qr = (size_t)bt * H_I + h;
        double v = 0;
        for (int e = 0; e < d_I; ++e)
          v += ld(q_idx, qr * d_I + e, qk_dt) * ld(k_idx, ((size_t)b * Nc_cap + j) * d_I + e, qk_dt);
        s += (double)w_idx[qr] * (v > 0 ? v : 0.0);
      }
      I[k] = s;
      if (s > imax) imax = s;
      msum += mrow[k];
      any = 1;
    }
    if (!any || !(msum > 0)) {
      free(I);
      free(dI);
      continue;
    }
    double zsum = 0;
    for (int k = 0; k < topk; ++k)
      if (irow[k] >= 0 && irow[k] < Nc_cap) zsum += exp(I[k] - imax);
    const double logz = imax + log(zsum);
    const double g = grad_scale ? grad_scale[bt] : 1.0;
    double kl = 0;
    for (int k = 0; k < topk; ++k) {
      const int32_t j = irow[k];
      if (j < 0 || j >= Nc_cap) continue;
      const double p = mrow[k] / msum, lq = I[k] - logz;
      if (p > 0) kl += p * (log(p) - lq);
      dI[k] = g * (exp(lq) - p);
    }
    loss[bt] = kl;
    for (int k = 0; k < topk; ++k) {
      const int32_t j = irow[k];
      if (j < 0 || j >= Nc_cap) continue;
      const size_t kr = ((size_t)b * Nc_cap + j) * d_I;
      for (int h = 0; h < H_I; ++h) {
        const size_t qr = (size_t)bt * H_I + h;
        double v = 0;
        for (int e = 0; e < d_I; ++e) v += ld(q_idx, qr * d_I + e, qk_dt) * ld(k_idx, kr + e, qk_dt);
        if (v > 0) {
          const double c = dI[k] * (double)w_idx[qr];
          dw_idx[qr] += dI[k] * v;
          for (int e = 0; e < d_I; ++e) {
            dq_idx[qr * d_I + e] += c * ld(k_idx, kr + e, qk_dt);
            const double gk = c * ld(q_idx, qr * d_I + e, qk_dt);
#pragma omp atomic
            dk_idx[kr + e] += gk;
          }
        }
      }
    }
    free(I);
    free(dI);
  }
  return 0;
}

/* ---- compressor backward ----------------------------------------------------
 * Gradients of a one-shot compressor call over tokens [0, L) (pos0 = 0, no
 * carried state; entries post-processed as orc_compress_ex does with opts,
 * or not at all with opts NULL) for an upstream gradient dC [B, Nc_cap, E]
 * of the entries it writes (rows i < min(L / m, Nc_cap); other rows are
 * ignored).  The entry's gradient goes back through the post-processing in
 * reverse order (the chain rule through the definitions above):
 *  - the Hadamard rotation: g <- H g / sqrt(E) (H symmetric and orthogonal);
 *  - the rotary embedding: the pair rotation's transpose, i.e. the same
 *    rotation at position -m i;
 *  - the RMS norm y = C r w, r = (mean C^2 + eps)^(-1/2): with u = g w,
 *    g_C = r u - C r^3 (sum_e u_e C_e) / E, and dnorm_w += g C r.
 * Through the pool, for every entry i and token j of its window (slot
 * s = j - m (i - o)), with dC_i now that gradient of the pooled entry:
 *     dP_j += a_{i,j} dC_i,   dG_j += a_{i,j} (P_j - C_i) dC_i,
 *     dape[s] += a_{i,j} (P_j - C_i) dC_i            (all per channel),
 * and through the projections P = W_kv x, G = W_gate x:
 *     dx_j = W_kv^T dP_j + W_gate^T dG_j,
 *     dW_kv = sum_j dP_j x_j^T,  dW_gate = sum_j dG_j x_j^T  (over b and j).
 * dape may be NULL (no ape); dnorm_w [E] is written when opts has a norm. */
int orc_compress_bwd_ex(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                        const void* x, const void* w_kv, const void* w_gate, int in_dt,
                        const double* ape, int Nc_cap, const double* dC,
                        const orc_compress_opts* opts, double* dx, double* dw_kv,
                        double* dw_gate, double* dape, double* dnorm_w) {
  const int Sw = (1 + overlap) * m;
  if (B < 0 || L < 0 || m < 1 || E < 1 || d_model < 1) return 1;
  if (rotate && (E & (E - 1))) return 1;
  if (opts && opts->rope_dim &&
      (opts->rope_dim < 0 || opts->rope_dim % 2 || opts->rope_off < 0 ||
       opts->rope_off + opts->rope_dim > E))
    return 1;
  const double* nw = opts ? opts->norm_w : NULL;
  if (nw && !dnorm_w) return 1;
  memset(dw_kv, 0, sizeof(double) * (size_t)E * d_model);
  memset(dw_gate, 0, sizeof(double) * (size_t)E * d_model);
  if (dape) memset(dape, 0, sizeof(double) * (size_t)Sw * E);
  if (nw) memset(dnorm_w, 0, sizeof(double) * (size_t)E);
  const int64_t n_ent = (int64_t)L / m < Nc_cap ? (int64_t)L / m : Nc_cap;
  for (int b = 0; b < B; ++b) {
    double* P = (double*)malloc(sizeof(double) * ((size_t)L * E + 1));
    double* G = (double*)malloc(sizeof(double) * ((size_t)L * E + 1));
    double* dP = (double*)calloc((size_t)L * E + 1, sizeof(double));
    double* dG = (double*)calloc((size_t)L * E + 1, sizeof(double));
#pragma omp parallel for schedule(static)
    for (int t = 0; t < L; ++t)
      for (int e = 0; e < E; ++e) {
        double pk = 0, gk = 0;
        for (int k = 0; k < d_model; ++k) {
          const double xv = ld(x, ((size_t)b * L + t) * d_model + k, in_dt);
          pk += xv * ld(w_kv, (size_t)e * d_model + k, in_dt);
          gk += xv * ld(w_gate, (size_t)e * d_model + k, in_dt);
        }
        P[(size_t)t * E + e] = pk;
        G[(size_t)t * E + e] = gk;
      }
    /* through the pool: entries are independent; the token rows they share
     * are summed with atomics */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_ent; ++i) {
      double* g = (double*)malloc(sizeof(double) * E);
      double* Cv = (double*)malloc(sizeof(double) * E);
      for (int e = 0; e < E; ++e) g[e] = dC[((size_t)b * Nc_cap + i) * E + e];
      if (rotate) hadamard_rows(g, E);
      const int64_t first = (int64_t)m * (i - overlap), last = (int64_t)m * (i + 1) - 1;
      if (opts && opts->rope_dim)
        rope_row(g + opts->rope_off, opts->rope_dim, opts->rope_interleaved, opts->rope_base,
                 -((int64_t)m * i));
      if (nw) {
        /* the pooled entry, then the norm's backward */
        for (int e = 0; e < E; ++e) {
          double mx = -INFINITY, den = 0, C = 0;
          for (int64_t j = first; j <= last; ++j) {
            if (j < 0) continue;
            const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
            if (z > mx) mx = z;
          }
          for (int64_t j = first; j <= last; ++j) {
            if (j < 0) continue;
            const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
            den += exp(z - mx);
          }
          for (int64_t j = first; j <= last; ++j) {
            if (j < 0) continue;
            const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
            C += exp(z - mx) / den * P[(size_t)j * E + e];
          }
          Cv[e] = C;
        }
        double ss = 0, dot = 0;
        for (int e = 0; e < E; ++e) {
          ss += Cv[e] * Cv[e];
          dot += g[e] * nw[e] * Cv[e];
        }
        const double r = 1.0 / sqrt(ss / E + opts->norm_eps);
        for (int e = 0; e < E; ++e) {
#pragma omp atomic
          dnorm_w[e] += g[e] * Cv[e] * r;
          g[e] = r * g[e] * nw[e] - Cv[e] * r * r * r * dot / E;
        }
      }
      for (int e = 0; e < E; ++e) {
        double mx = -INFINITY, den = 0, C = 0;
        for (int64_t j = first; j <= last; ++j) {
          if (j < 0) continue;
          const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
          if (z > mx) mx = z;
        }
        for (int64_t j = first; j <= last; ++j) {
          if (j < 0) continue;
          const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
          den += exp(z - mx);
        }
        for (int64_t j = first; j <= last; ++j) {
          if (j < 0) continue;
          const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
          C += exp(z - mx) / den * P[(size_t)j * E + e];
        }
        for (int64_t j = first; j <= last; ++j) {
          if (j < 0) continue;
          const double z = G[(size_t)j * E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0);
          const double a = exp(z - mx) / den;
          const double gp = a * g[e], gg = a * (P[(size_t)j * E + e] - C) * g[e];
#pragma omp atomic
          dP[(size_t)j * E + e] += gp;
#pragma omp atomic
          dG[(size_t)j * E + e] += gg;
          if (dape) {
#pragma omp atomic
            dape[(size_t)(j - first) * E + e] += gg;
          }
        }
      }
      free(g);
      free(Cv);
    }
    /* through the projections */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < L; ++t)
      for (int k = 0; k < d_model; ++k) {
        double s = 0;
        for (int e = 0; e < E; ++e)
          s += dP[(size_t)t * E + e] * ld(w_kv, (size_t)e * d_model + k, in_dt) +
               dG[(size_t)t * E + e] * ld(w_gate, (size_t)e * d_model + k, in_dt);
        dx[((size_t)b * L + t) * d_model + k] = s;
      }
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e)
      for (int k = 0; k < d_model; ++k) {
        double sk = 0, sg = 0;
        for (int t = 0; t < L; ++t) {
          const double xv = ld(x, ((size_t)b * L + t) * d_model + k, in_dt);
          sk += dP[(size_t)t * E + e] * xv;
          sg += dG[(size_t)t * E + e] * xv;
        }
        dw_kv[(size_t)e * d_model + k] += sk;
        dw_gate[(size_t)e * d_model + k] += sg;
      }
    free(P);
    free(G);
    free(dP);
    free(dG);
  }
  return 0;
}

int orc_compress_bwd(int B, int L, int d_model, int E, int m, int overlap, int rotate,
                     const void* x, const void* w_kv, const void* w_gate, int in_dt,
                     const double* ape, int Nc_cap, const double* dC, double* dx,
                     double* dw_kv, double* dw_gate, double* dape) {
  return orc_compress_bwd_ex(B, L, d_model, E, m, overlap, rotate, x, w_kv, w_gate, in_dt, ape,
                             Nc_cap, dC, NULL, dx, dw_kv, dw_gate, dape, NULL);
}

/* Number of threads an OpenMP parallel region will use (for reporting). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
