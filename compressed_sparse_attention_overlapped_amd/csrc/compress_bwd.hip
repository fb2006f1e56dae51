// Compressor backward for gfx950: gradients of a one-shot compressor call
// over tokens [0, L) of each sequence (bf16 tokens and weights, no carried
// state; entries optionally Hadamard-rotated) for an upstream gradient dC of
// its entries (migration page, section 3.2: the compressor is two linear maps
// and a softmax-gated pool over overlapping windows; its training path is
// listed in sections 1 and 3.2).
//
// For entry i over its window tokens j (slot s = j - m (i - o)), per channel:
//   a_j = softmax_j(G_j + ape_s),  C_i = sum_j a_j P_j,
//   dP_j += a_j dC_i,  dG_j += a_j (P_j - C_i) dC_i,  dape_s += the same;
// and through P = x W_kv^T, G = x W_gate^T:
//   dx = dP W_kv + dG W_gate,  dW_kv = dP^T x,  dW_gate = dG^T x.
//
// Launches: the forward projection (recomputes P | G in fp32); an entry
// kernel (each entry's softmax statistics lse and C per channel, and the
// entry's gradient back through the post-processing the forward applied, in
// reverse order: the Hadamard rotation (H dC / sqrt(E), H symmetric), the
// rotary embedding (its transpose: the pair rotation at -m i) and the RMS
// norm y = C r w, r = (mean C^2 + eps)^(-1/2), whose gradient is
// r u - C r^3 (sum u C) / E with u = g w, and whose weight gradient sums
// g C r over the entries - per-entry rows, then a fixed-order column sum); a token
// kernel (owner computes: token j takes its share of the one or two entries
// whose windows hold it, so no two threads write one element, and dape is
// summed per workgroup in LDS, then one atomic per slot and channel); and two
// plain GEMMs (rocBLAS, bf16 operands, fp32 accumulation and output) over the
// [dP | dG] rows: dx against the two weights stacked as one [2E, d_model]
// matrix (one pass over the fp32 dx instead of a write and an accumulate),
// and both weight gradients as one [2E, d_model] product, split afterwards.
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"

namespace csa {

constexpr int CB_TT = 128;  // tokens per workgroup of the token kernel

// Sum over the block (any blockDim.x <= 1024; red: 1024 floats); every
// thread gets the total.  Ends with a barrier.
__device__ float cb_block_sum(float v, float* red) {
  const int tid = threadIdx.x, n = blockDim.x;
  red[tid] = v;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o && tid + o < n) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float t = red[0];
  __syncthreads();
  return t;
}

// Per (b, entry i < n_ent, channel e): lse and C of the window softmax, and
// the entry's gradient back through the Hadamard rotation, the rotary
// embedding and the RMS norm (each when the forward applied it).  One
// workgroup per entry row, E threads (E <= 1024).  dnw_part [B n_ent, E]:
// the entry's terms of the norm weight's gradient (when opt.norm_w).
__global__ void __launch_bounds__(1024) cmp_bwd_entry_kernel(
    const float* __restrict__ pg, const float* __restrict__ ape, const float* __restrict__ dC,
    int L, int E, int m, int overlap, int Nc_cap, int n_ent, int rotate, float rs,
    csa_host::EntryOpts opt, float* __restrict__ stats, float* __restrict__ gent,
    float* __restrict__ dnw_part) {
  __shared__ float hv[1024];
  __shared__ float red[1024];
  const int i = blockIdx.x, b = blockIdx.y, e = threadIdx.x;
  const int N = 2 * E;
  const size_t prow = (size_t)b * L;
  // the pooled entry's statistics for this channel
  const int first = m * (i - overlap), last = m * (i + 1) - 1;
  float mx = -INFINITY;
  for (int j = max(first, 0); j <= last; ++j)
    mx = fmaxf(mx, pg[(prow + j) * N + E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0f));
  float den = 0.0f, num = 0.0f;
  for (int j = max(first, 0); j <= last; ++j) {
    const float w = __expf(pg[(prow + j) * N + E + e] + (ape ? ape[(size_t)(j - first) * E + e] : 0.0f) - mx);
    den += w;
    num = fmaf(w, pg[(prow + j) * N + e], num);
  }
  const float C = num / den;
  float g = dC[((size_t)b * Nc_cap + i) * E + e];
  if (rotate) {
    // fast Walsh-Hadamard transform of the row (Sylvester order), / sqrt(E)
    hv[e] = g;
    __syncthreads();
    for (int len = 1; len < E; len <<= 1) {
      const int blk = e / (2 * len), off = e % (2 * len);
      float val;
      if (off < len) val = hv[blk * 2 * len + off] + hv[blk * 2 * len + off + len];
      else val = hv[blk * 2 * len + off - len] - hv[blk * 2 * len + off];
      __syncthreads();
      hv[e] = val;
      __syncthreads();
    }
    g = hv[e] * rs;
  }
  if (opt.rope_dim) {
    // the forward turned pair (a, b) into (a cos - b sin, b cos + a sin); its
    // transpose takes (g_a, g_b) to (g_a cos + g_b sin, g_b cos - g_a sin)
    __syncthreads();  // (hv's last reads above)
    hv[e] = g;
    __syncthreads();
    const int R = opt.rope_dim, half = R / 2, c = e - opt.rope_off;
    if (c >= 0 && c < R) {
      const int k = opt.rope_interleaved ? c >> 1 : (c < half ? c : c - half);
      const bool lo = opt.rope_interleaved ? (c & 1) == 0 : c < half;
      const int partner = opt.rope_interleaved ? (lo ? e + 1 : e - 1) : (lo ? e + half : e - half);
      const double ang = (double)m * (double)i * pow((double)opt.rope_base, -2.0 * k / R);
      const float cs = (float)cos(ang), sn = (float)sin(ang);
      g = fmaf(g, cs, (lo ? hv[partner] : -hv[partner]) * sn);
    }
  }
  if (opt.norm_w) {
    const float w = opt.norm_w[e];
    const float ss = cb_block_sum(C * C, red);
    const float dot = cb_block_sum(g * w * C, red);
    const float r = 1.0f / sqrtf(ss / (float)E + opt.norm_eps);
    dnw_part[((size_t)b * n_ent + i) * E + e] = g * C * r;
    g = r * g * w - C * (r * r * r) * dot / (float)E;
  }
  const size_t o = ((size_t)b * n_ent + i) * E + e;
  stats[2 * o] = mx + __logf(den);
  stats[2 * o + 1] = C;
  gent[o] = g;
}

// dnw[e] = sum over rows of part[row][e], rows in a fixed order per thread
// then a fixed tree: workgroup of 256 threads per 64 channels
__global__ void __launch_bounds__(256) cmp_bwd_colsum_kernel(const float* __restrict__ part,
                                                             int rows, int E,
                                                             float* __restrict__ out) {
  __shared__ float sh[4][64];
  const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + c;
  float acc = 0.0f;
  if (e < E)
    for (int r = rg; r < rows; r += 4) acc += part[(size_t)r * E + e];
  sh[rg][c] = acc;
  __syncthreads();
  if (rg == 0 && e < E) out[e] = (sh[0][c] + sh[1][c]) + (sh[2][c] + sh[3][c]);
}

// Token j (workgroup: CB_TT tokens x 64 channels; thread: a channel and
// every fourth token): dP_j, dG_j as bf16 [M, 2 E] rows, and dape.
__global__ void __launch_bounds__(256) cmp_bwd_token_kernel(
    const float* __restrict__ pg, const float* __restrict__ ape, const float* __restrict__ stats,
    const float* __restrict__ gent, int L, int E, int m, int overlap, int n_ent,
    uint16_t* __restrict__ dpg, float* __restrict__ dape) {
  extern __shared__ float dsh[];  // [(1 + o) m][64]
  const int Sw = (1 + overlap) * m;
  const int c = threadIdx.x & 63, tq = threadIdx.x >> 6;
  const int e = blockIdx.y * 64 + c, b = blockIdx.z;
  const int j0 = blockIdx.x * CB_TT;
  const int N = 2 * E;
  const bool ch = e < E;
  for (int k = threadIdx.x; k < Sw * 64; k += 256) dsh[k] = 0.0f;
  __syncthreads();
  for (int j = j0 + tq; j < min(j0 + CB_TT, L) && ch; j += 4) {
    const size_t r = (size_t)b * L + j;
    const float P = pg[r * N + e], G = pg[r * N + E + e];
    float dP = 0.0f, dG = 0.0f;
    const int q = j / m;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      if (w == 1 && !overlap) break;
      const int i = q + w;  // own block's entry, then the next one (its previous block)
      if (i >= n_ent) continue;
      const int s = j - m * (i - overlap);
      const size_t o = ((size_t)b * n_ent + i) * E + e;
      const float a = __expf(G + (ape ? ape[(size_t)s * E + e] : 0.0f) - stats[2 * o]);
      const float g = gent[o];
      const float gg = a * (P - stats[2 * o + 1]) * g;
      dP = fmaf(a, g, dP);
      dG += gg;
      if (dape) atomicAdd(&dsh[s * 64 + c], gg);
    }
    dpg[r * N + e] = f32_to_bf16(dP);
    dpg[r * N + E + e] = f32_to_bf16(dG);
  }
  __syncthreads();
  if (dape)
    for (int k = threadIdx.x; k < Sw * 64; k += 256) {
      const int ee = blockIdx.y * 64 + (k & 63);
      if (ee < E && dsh[k] != 0.0f) atomicAdd(&dape[(size_t)(k >> 6) * E + ee], dsh[k]);
    }
}

// out[i] = sum over s < S of part[s n + i] (the token-split weight gradient)
__global__ void __launch_bounds__(256) cmp_bwd_sum_kernel(const float* __restrict__ part, int S,
                                                          size_t n, float* __restrict__ out) {
  const size_t n4 = n / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    f32x4 acc = *(const f32x4*)(part + 4 * i);
    for (int k = 1; k < S; ++k) {
      const f32x4 v = *(const f32x4*)(part + (size_t)k * n + 4 * i);
      acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
    }
    *(f32x4*)(out + 4 * i) = acc;
  }
  for (size_t i = 4 * n4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    float acc = part[i];
    for (int k = 1; k < S; ++k) acc += part[(size_t)k * n + i];
    out[i] = acc;
  }
}

}  // namespace csa

// ---------------------------------------------------------------- host side
namespace csa_host {
using namespace csa;

static size_t cb_al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Token splits of the weight-gradient product: a [d_model, 2E] output too
// small to fill the chip on its own (below about 256 tiles of 64 x 128) is
// computed as S partial products over token ranges, then summed.
static int dw_splits(size_t M, int d_model, int E) {
  if ((size_t)d_model * 2 * E >= (size_t)256 * 64 * 128) return 1;
  return (M % 4 == 0 && M >= 4096) ? 4 : 1;
}

// workspace: P | G fp32 [M, 2E], dP | dG bf16 [M, 2E], the entries' stats,
// gradients and norm-weight terms, the stacked weights bf16 [2E, d_model],
// the stacked weight gradients fp32 [2E, d_model] and, with token splits,
// their partials
size_t compress_bwd_ws_bytes(int B, int L, int d_model, int E, int m, int Nc_cap) {
  const size_t M = (size_t)B * L;
  const size_t n_ent = std::min<size_t>((size_t)L / m, (size_t)Nc_cap);
  const size_t WK = (size_t)2 * E * d_model;
  const int S = dw_splits(M, d_model, E);
  return cb_al256(M * 2 * E * sizeof(float)) + cb_al256(M * 2 * E * sizeof(uint16_t)) +
         cb_al256((size_t)B * n_ent * E * 2 * sizeof(float)) +
         2 * cb_al256((size_t)B * n_ent * E * sizeof(float)) + cb_al256(WK * sizeof(uint16_t)) +
         cb_al256(WK * sizeof(float)) + (S > 1 ? cb_al256(S * WK * sizeof(float)) : 0);
}

// one rocBLAS handle per device, created on first use
static rocblas_handle blas_handle(hipError_t& err) {
  static std::mutex mu;
  static rocblas_handle h[64] = {};
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess || dev < 0 || dev >= 64) {
    if (err == hipSuccess) err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!h[dev] && rocblas_create_handle(&h[dev]) != rocblas_status_success) {
    err = hipErrorUnknown;
    return nullptr;
  }
  return h[dev];
}

// C (col-major rows x cols) = op(A) op(B) + beta C, bf16 operands, fp32 C
static bool gemm_bf16_f32(rocblas_handle hb, rocblas_operation ta, rocblas_operation tb, int rows,
                          int cols, int k, const void* A, int lda, const void* B, int ldb,
                          float beta, float* C, int ldc) {
  const float alpha = 1.0f;
  return rocblas_gemm_ex(hb, ta, tb, rows, cols, k, &alpha, A, rocblas_datatype_bf16_r, lda, B,
                         rocblas_datatype_bf16_r, ldb, &beta, C, rocblas_datatype_f32_r, ldc, C,
                         rocblas_datatype_f32_r, ldc, rocblas_datatype_f32_r,
                         rocblas_gemm_algo_standard, 0, 0) == rocblas_status_success;
}

hipError_t launch_compress_bwd(const CompressBwdArgs& a, hipStream_t s) {
  const int M = a.B * a.L, E = a.E, K = a.d_model, N = 2 * E;
  const int n_ent = std::min(a.L / a.m, a.Nc_cap);
  char* ws = (char*)a.ws;
  float* pg = (float*)ws;
  ws += cb_al256((size_t)M * N * sizeof(float));
  uint16_t* dpg = (uint16_t*)ws;
  ws += cb_al256((size_t)M * N * sizeof(uint16_t));
  float* stats = (float*)ws;
  ws += cb_al256((size_t)a.B * std::max(n_ent, 0) * E * 2 * sizeof(float));
  float* gent = (float*)ws;
  ws += cb_al256((size_t)a.B * std::max(n_ent, 0) * E * sizeof(float));
  float* dnw_part = (float*)ws;
  ws += cb_al256((size_t)a.B * std::max(n_ent, 0) * E * sizeof(float));
  uint16_t* wcat = (uint16_t*)ws;
  ws += cb_al256((size_t)2 * E * K * sizeof(uint16_t));
  float* dwcat = (float*)ws;
  ws += cb_al256((size_t)2 * E * K * sizeof(float));
  float* dwpart = (float*)ws;  // S partials [2E, K] when the tokens are split
  const int S = dw_splits((size_t)M, K, E);
  const size_t wb = (size_t)E * K * sizeof(uint16_t), dwb = (size_t)E * K * sizeof(float);
  // weights (and weight gradients) the caller already keeps stacked - w_gate
  // right after w_kv - are used in place
  const bool w_stacked = (const char*)a.w_gate == (const char*)a.w_kv + wb;
  const bool dw_stacked = (char*)a.dw_gate == (char*)a.dw_kv + dwb;
  const uint16_t* wsrc = w_stacked ? (const uint16_t*)a.w_kv : wcat;
  float* dwdst = dw_stacked ? a.dw_kv : dwcat;
  hipError_t e = hipSuccess;
  if (!w_stacked) {
    e = hipMemcpyAsync(wcat, a.w_kv, wb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(wcat + (size_t)E * K, a.w_gate, wb, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  e = launch_proj_pg(a.x, a.w_kv, a.w_gate, M, E, K, pg, s);
  if (e != hipSuccess) return e;
  const int Sw = (1 + a.overlap) * a.m;
  if (a.dape) {
    e = launch_zero_f32(a.dape, (size_t)Sw * E, s);
    if (e != hipSuccess) return e;
  }
  if (n_ent > 0)
    cmp_bwd_entry_kernel<<<dim3(n_ent, a.B), E, 0, s>>>(
        pg, a.ape, a.dC, a.L, E, a.m, a.overlap, a.Nc_cap, n_ent, a.rotate,
        (float)(1.0 / std::sqrt((double)E)), a.opt, stats, gent, dnw_part);
  if (a.opt.norm_w) {
    if (n_ent > 0)
      cmp_bwd_colsum_kernel<<<(E + 63) / 64, 256, 0, s>>>(dnw_part, a.B * n_ent, E, a.dnorm_w);
    else
      e = launch_zero_f32(a.dnorm_w, (size_t)E, s);
    if (e != hipSuccess) return e;
  }
  cmp_bwd_token_kernel<<<dim3((a.L + CB_TT - 1) / CB_TT, (E + 63) / 64, a.B), 256,
                         (size_t)Sw * 64 * sizeof(float), s>>>(
      pg, a.ape, stats, gent, a.L, E, a.m, a.overlap, n_ent, dpg, a.dape);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  rocblas_handle hb = blas_handle(e);
  if (!hb) return e;
  if (rocblas_set_stream(hb, s) != rocblas_status_success) return hipErrorUnknown;
  // row-major views as column-major: dx^T (K x M) = [W_kv; W_gate]^T [dP | dG]^T,
  // [dW_kv; dW_gate]^T (K x 2E) = x^T [dP | dG]  (x: K x M column-major)
  bool ok = gemm_bf16_f32(hb, rocblas_operation_none, rocblas_operation_none, K, M, N, wsrc, K,
                          dpg, N, 0.0f, a.dx, K);
  if (ok && S == 1) {
    ok = gemm_bf16_f32(hb, rocblas_operation_none, rocblas_operation_transpose, K, N, M, a.x, K,
                       dpg, N, 0.0f, dwdst, K);
  } else if (ok) {
    // partial s over tokens [s M / S, (s + 1) M / S), then their sum
    const int Ms = M / S;
    const float alpha = 1.0f, beta = 0.0f;
    ok = rocblas_gemm_strided_batched_ex(
             hb, rocblas_operation_none, rocblas_operation_transpose, K, N, Ms, &alpha, a.x,
             rocblas_datatype_bf16_r, K, (rocblas_stride)Ms * K, dpg, rocblas_datatype_bf16_r, N,
             (rocblas_stride)Ms * N, &beta, dwpart, rocblas_datatype_f32_r, K,
             (rocblas_stride)K * N, dwpart, rocblas_datatype_f32_r, K, (rocblas_stride)K * N, S,
             rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) == rocblas_status_success;
    if (ok) {
      const size_t n = (size_t)K * N;
      cmp_bwd_sum_kernel<<<(unsigned)std::min<size_t>((n / 4 + 255) / 256, 1024), 256, 0, s>>>(
          dwpart, S, n, dwdst);
    }
  }
  if (!ok) return hipErrorUnknown;
  if (!dw_stacked) {
    e = hipMemcpyAsync(a.dw_kv, dwcat, dwb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(a.dw_gate, dwcat + (size_t)E * K, dwb, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace csa_host
