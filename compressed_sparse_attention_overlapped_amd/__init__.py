"""Python binding of libcsa, the gfx950 compressed sparse attention library.

The functions mirror the C ABI in ``include/csa.h`` one to one and only
marshal arguments: they read shapes off torch tensors, pass device pointers
and the current HIP stream, and raise ``CsaError`` on a non-zero status.
Every step of the computation runs in the library's HIP kernels; PyTorch only
owns the device memory (outputs and workspaces are allocated here when the
caller does not pass them).  If ``libcsa.so`` has not been built the first
call raises - there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

__all__ = ["csa_compress", "csa_indexer_topk", "csa_sparse_attn", "hca_dense_attn",
           "csa_sparse_attn_noalloc", "csa_sparse_attn_window_half",
           "csa_sparse_attn_selected_half", "csa_sparse_attn_split_workspace_size", "csa_build_cmp_cu_seqlens", "csa_compress_varlen",
           "csa_indexer_topk_varlen", "csa_sparse_attn_varlen", "csa_sparse_attn_bwd",
           "hca_dense_attn_bwd", "csa_indexer_kl_bwd", "csa_indexer_kl_dense_bwd", "csa_compress_bwd", "csa_compress_bwd_ex",
           "csa_compress_workspace_size", "csa_indexer_topk_workspace_size",
           "csa_sparse_attn_workspace_size", "hca_dense_attn_workspace_size",
           "CsaError", "PageTable", "lib", "LIB_PATH", "DT_F32", "DT_BF16", "DT_FP8", "DT_MXFP4"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
DT_F32, DT_BF16, DT_FP8, DT_MXFP4 = 0, 1, 2, 3
_DT = {torch.float32: DT_F32, torch.bfloat16: DT_BF16, torch.float8_e4m3fn: DT_FP8,
       torch.float4_e2m1fn_x2: DT_MXFP4}

_lib = None


class CsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__("%s failed: status %d (%s)" % (fn, status, detail))
        self.status = status


class _CPageTable(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("page_size", C.c_int), ("max_pages", C.c_int),
                ("n_pages", C.c_int)]


class _COpts(C.Structure):
    _fields_ = [("norm_weight", C.c_void_p), ("norm_eps", C.c_float), ("rope_dim", C.c_int),
                ("rope_offset", C.c_int), ("rope_base", C.c_float), ("rope_interleaved", C.c_int)]


class PageTable:
    """Paged compressed caches (``csa_page_table_t`` in include/csa.h): logical
    entry j of sequence b is pool row ``block_table[b, j // page_size] *
    page_size + j % page_size``.  block_table: device int32 [B, max_pages];
    n_pages: pages in the pool.  The logical capacity Nc_cap defaults to
    max_pages * page_size."""

    def __init__(self, block_table: torch.Tensor, page_size: int, n_pages: int, nc_cap=None):
        if block_table.dtype != torch.int32 or block_table.dim() != 2:
            raise ValueError("block_table must be an int32 tensor [B, max_pages]")
        self.block_table = block_table.contiguous()
        self.page_size = int(page_size)
        self.n_pages = int(n_pages)
        self.max_pages = int(block_table.shape[1])
        self.nc_cap = self.max_pages * self.page_size if nc_cap is None else int(nc_cap)

    def c(self):
        return C.byref(_CPageTable(self.block_table.data_ptr(), self.page_size, self.max_pages,
                                   self.n_pages))

    def check(self, B: int, *pools):
        """Raise ValueError unless the table can serve B sequences on the
        pools' device and every pool holds n_pages * page_size rows (the C
        ABI sees only pointers, so a short table or pool would be read or
        written out of bounds)."""
        bt = self.block_table
        if bt.shape[0] < B:
            raise ValueError("block_table has %d rows for %d sequences" % (bt.shape[0], B))
        for p in pools:
            if p is None:
                continue
            if p.dim() < 1 or p.shape[0] < self.n_pages * self.page_size:
                raise ValueError("a paged pool needs n_pages * page_size = %d rows (got %s)"
                                 % (self.n_pages * self.page_size, tuple(p.shape)))
            if not bt.is_cuda or bt.device != p.device:
                raise ValueError("block_table must live on the caches' device (%s, got %s)"
                                 % (p.device, bt.device))


def lib():
    """Load libcsa.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcsa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        vp, i32, f32, sz = C.c_void_p, C.c_int, C.c_float, C.c_size_t
        L.csa_compress.argtypes = [i32] * 7 + [vp] * 4 + [i32, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
        L.csa_compress_workspace_size.argtypes = [i32] * 7
        L.csa_indexer_topk.argtypes = [i32] * 7 + [vp] * 7 + [i32, vp, vp, vp, sz, vp]
        L.csa_indexer_topk_workspace_size.argtypes = [i32] * 7
        L.csa_sparse_attn.argtypes = [i32] * 6 + [f32, vp, vp, vp, vp, i32, vp, vp, i32, vp, i32, vp, vp, vp, sz, vp]
        L.csa_sparse_attn_workspace_size.argtypes = [i32] * 6
        L.csa_sparse_attn_window_half.argtypes = [i32] * 6 + [f32, vp, vp, vp, i32, vp, i32, vp, sz, vp]
        L.csa_sparse_attn_selected_half.argtypes = L.csa_sparse_attn.argtypes
        L.csa_sparse_attn_split_workspace_size.argtypes = [i32] * 6
        L.csa_sparse_attn_window_half.restype = C.c_int
        L.csa_sparse_attn_selected_half.restype = C.c_int
        L.csa_sparse_attn_split_workspace_size.restype = C.c_size_t
        L.hca_dense_attn.argtypes = [i32] * 6 + [f32, vp, vp, vp, vp, vp, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
        L.hca_dense_attn_workspace_size.argtypes = [i32] * 6
        pt = C.POINTER(_CPageTable)
        L.csa_compress_paged.argtypes = ([i32] * 7 + [vp] * 4 + [i32, vp, vp, vp, vp, vp, i32, i32,
                                         pt, vp, sz, vp])
        L.csa_indexer_topk_paged.argtypes = [i32] * 7 + [vp] * 7 + [i32, pt, vp, vp, vp, sz, vp]
        L.csa_compress_ex.argtypes = ([i32] * 7 + [vp] * 4 + [i32, vp, vp, vp, vp, vp, i32, i32,
                                      pt, C.POINTER(_COpts), vp, sz, vp])
        L.csa_compress_ex.restype = C.c_int
        L.csa_build_cmp_cu_seqlens.argtypes = [i32, vp, i32, vp, vp]
        L.csa_compress_varlen.argtypes = ([i32] * 8 + [vp] * 5 + [i32, vp, vp, vp, vp, i32,
                                          C.POINTER(_COpts), vp, sz, vp])
        L.csa_compress_varlen_workspace_size.argtypes = [i32] * 6
        L.csa_indexer_topk_varlen.argtypes = ([i32] * 8 + [vp] * 5 + [i32, vp, vp, vp, sz, vp])
        L.csa_indexer_topk_varlen_workspace_size.argtypes = [i32] * 4
        L.csa_sparse_attn_varlen.argtypes = ([i32] * 7 + [f32] + [vp] * 5 + [i32, vp, vp, i32,
                                             vp, vp, vp, sz, vp])
        L.csa_sparse_attn_varlen_workspace_size.argtypes = [i32] * 5
        for f in (L.csa_build_cmp_cu_seqlens, L.csa_compress_varlen, L.csa_indexer_topk_varlen,
                  L.csa_sparse_attn_varlen):
            f.restype = C.c_int
        for f in (L.csa_compress_varlen_workspace_size, L.csa_indexer_topk_varlen_workspace_size,
                  L.csa_sparse_attn_varlen_workspace_size):
            f.restype = C.c_size_t
        L.csa_sparse_attn_paged.argtypes = ([i32] * 6 + [f32, vp, vp, vp, vp, i32, pt, vp, vp, i32,
                                            vp, pt, i32, vp, vp, vp, sz, vp])
        L.hca_dense_attn_paged.argtypes = ([i32] * 6 + [f32, vp, vp, vp, vp, vp, i32, pt, vp, i32,
                                           vp, pt, i32, vp, vp, vp, sz, vp])
        L.hca_dense_attn_paged.restype = C.c_int
        L.csa_sparse_attn_noalloc.argtypes = ([i32] * 6 + [f32, vp, vp, vp, vp, i32, vp, vp, i32,
                                              vp, i32, vp, vp, vp])
        L.csa_sparse_attn_noalloc.restype = C.c_int
        L.csa_sparse_attn_paged_workspace_size.argtypes = [i32] * 6
        L.csa_sparse_attn_paged_workspace_size.restype = C.c_size_t
        for f in (L.csa_compress, L.csa_indexer_topk, L.csa_sparse_attn, L.hca_dense_attn,
                  L.csa_compress_paged, L.csa_indexer_topk_paged, L.csa_sparse_attn_paged):
            f.restype = C.c_int
        for f in (L.csa_compress_workspace_size, L.csa_indexer_topk_workspace_size,
                  L.csa_sparse_attn_workspace_size, L.hca_dense_attn_workspace_size):
            f.restype = C.c_size_t
        L.csa_sparse_attn_bwd.argtypes = ([i32] * 6 + [f32, vp, vp, vp, vp, i32, vp, vp, i32, vp,
                                          i32] + [vp] * 8 + [sz, vp])
        L.csa_sparse_attn_bwd.restype = C.c_int
        L.csa_sparse_attn_bwd_workspace_size.argtypes = [i32] * 6
        L.csa_sparse_attn_bwd_workspace_size.restype = C.c_size_t
        L.hca_dense_attn_bwd.argtypes = ([i32] * 6 + [f32, vp, vp, vp, vp, vp, i32, vp, i32, vp,
                                         i32] + [vp] * 8 + [sz, vp])
        L.hca_dense_attn_bwd.restype = C.c_int
        L.hca_dense_attn_bwd_workspace_size.argtypes = [i32] * 6
        L.hca_dense_attn_bwd_workspace_size.restype = C.c_size_t
        L.csa_indexer_kl_bwd.argtypes = [i32] * 6 + [vp, vp, vp, i32] + [vp] * 7 + [vp, sz, vp]
        L.csa_indexer_kl_bwd.restype = C.c_int
        L.csa_indexer_kl_bwd_workspace_size.argtypes = [i32] * 4
        L.csa_indexer_kl_bwd_workspace_size.restype = C.c_size_t
        L.csa_indexer_kl_dense_bwd.argtypes = [i32] * 6 + [vp] * 5 + [i32] + [vp] * 7 + [sz, vp]
        L.csa_indexer_kl_dense_bwd.restype = C.c_int
        L.csa_indexer_kl_dense_bwd_workspace_size.argtypes = [i32] * 3
        L.csa_indexer_kl_dense_bwd_workspace_size.restype = C.c_size_t
        L.csa_compress_bwd.argtypes = [i32] * 7 + [vp, vp, vp, i32, vp, i32] + [vp] * 5 + [vp, sz, vp]
        L.csa_compress_bwd.restype = C.c_int
        L.csa_compress_bwd_workspace_size.argtypes = [i32] * 6
        L.csa_compress_bwd_workspace_size.restype = C.c_size_t
        L.csa_compress_bwd_ex.argtypes = ([i32] * 7 + [vp, vp, vp, i32, vp, i32, vp,
                                                       C.POINTER(_COpts)] + [vp] * 5 + [vp, sz, vp])
        L.csa_compress_bwd_ex.restype = C.c_int
        L.csa_status_string.argtypes = [i32]
        L.csa_status_string.restype = C.c_char_p
        L.csa_last_error.argtypes = []
        L.csa_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        L = lib()
        raise CsaError(fn, rc, "%s: %s" % (L.csa_status_string(rc).decode(),
                                           L.csa_last_error().decode()))


def _dense(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libcsa must be contiguous")


def _workspace(nbytes: int, like: torch.Tensor, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------- sizes

def csa_compress_workspace_size(B, L, d_model, E, m, overlap, in_dtype) -> int:
    return lib().csa_compress_workspace_size(B, L, d_model, E, m, overlap, _DT[in_dtype])


def csa_indexer_topk_workspace_size(B, T, H_I, d_I, Nc_cap, topk, qk_dtype) -> int:
    return lib().csa_indexer_topk_workspace_size(B, T, H_I, d_I, Nc_cap, topk, _DT[qk_dtype])


def csa_sparse_attn_workspace_size(B, T, H, D, topk, window) -> int:
    return lib().csa_sparse_attn_workspace_size(B, T, H, D, topk, window)


def hca_dense_attn_workspace_size(B, T, H, D, Nc_cap, window) -> int:
    return lib().hca_dense_attn_workspace_size(B, T, H, D, Nc_cap, window)


# ---------------------------------------------------------------- calls

def csa_compress(x, w_kv, w_gate, pos0, m, overlap, out, out_scale=None, ape=None,
                 state_in=None, state_out=None, workspace=None, rotate=False, pages=None,
                 norm_weight=None, norm_eps=1e-6, rope_dim=0, rope_offset=0, rope_base=10000.0,
                 rope_interleaved=False):
    """Gated overlapping compressor; see ``csa_compress`` in include/csa.h.

    x [B, L, d_model]; w_kv, w_gate [E, d_model]; pos0 int64 [B];
    out [B, Nc_cap, E] (f32, bf16 or float8_e4m3fn, then out_scale f32 [B, Nc_cap]),
    or float4_e2m1fn_x2 [B, Nc_cap, E / 2] with out_scale E8M0 bytes [B, Nc_cap, E / 32]
    (float8_e8m0fnu or uint8);
    ape f32 [(1+o) m, E]; state_in / state_out f32 [B, (1+o) m - 1, 2, E];
    rotate: entries times the Hadamard matrix / sqrt(E) before storage.
    pages: a PageTable; out (and out_scale) are then pools [n_pages * page_size, ...].
    norm_weight f32 [E] (RMS norm of each entry, eps norm_eps) and rope_dim / rope_offset /
    rope_base / rope_interleaved (rotary embedding of a channel slice at the entry's
    position m * i): csa_compress_opts_t in include/csa.h."""
    _dense(x, w_kv, w_gate, pos0, out, out_scale, ape, state_in, state_out, norm_weight)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    ws, nb = _workspace(csa_compress_workspace_size(B, L, d_model, E, m, overlap, x.dtype), x,
                        workspace)
    if norm_weight is not None or rope_dim:
        if norm_weight is not None and (norm_weight.dtype != torch.float32 or
                                        norm_weight.shape != (E,)):
            raise ValueError("norm_weight must be a float32 tensor of shape [E]")
        if pages is not None:
            pages.check(B, out, out_scale)
        opts = _COpts(None if norm_weight is None else norm_weight.data_ptr(), float(norm_eps),
                      int(rope_dim), int(rope_offset), float(rope_base), int(bool(rope_interleaved)))
        nc_cap = pages.nc_cap if pages is not None else out.shape[1]
        rc = lib().csa_compress_ex(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(pos0),
                                   _p(x), _p(w_kv), _p(w_gate), _DT[x.dtype], _p(ape),
                                   _p(state_in), _p(state_out), _p(out), _p(out_scale),
                                   _DT[out.dtype], nc_cap, pages.c() if pages is not None else None,
                                   C.byref(opts), _p(ws), nb, _stream(x))
    elif pages is not None:
        pages.check(B, out, out_scale)
        rc = lib().csa_compress_paged(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(pos0),
                                      _p(x), _p(w_kv), _p(w_gate), _DT[x.dtype], _p(ape),
                                      _p(state_in), _p(state_out), _p(out), _p(out_scale),
                                      _DT[out.dtype], pages.nc_cap, pages.c(), _p(ws), nb,
                                      _stream(x))
    else:
        rc = lib().csa_compress(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(pos0), _p(x),
                                _p(w_kv), _p(w_gate),
                                _DT[x.dtype], _p(ape), _p(state_in), _p(state_out), _p(out),
                                _p(out_scale), _DT[out.dtype], out.shape[1], _p(ws), nb,
                                _stream(x))
    _check("csa_compress", rc)
    return out


def csa_indexer_topk(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale=None, k_scale=None,
                     idx_out=None, score_out=None, want_scores=False, workspace=None, pages=None):
    """Lightning-indexer scores + top-k; returns (idx int32 [B, T, topk], scores or None).
    fp8: float8_e4m3fn q_idx / k_idx with f32 q_scale [B, T, H_I], k_scale [B, Nc_cap];
    mxfp4: float4_e2m1fn_x2 q_idx [B, T, H_I, d_I / 2], k_idx [B, Nc_cap, d_I / 2] with
    E8M0 byte scales q_scale [B, T, H_I, d_I / 32], k_scale [B, Nc_cap, d_I / 32].
    pages: a PageTable; k_idx and k_scale are then pools (rows first), fp8 or mxfp4."""
    _dense(q_idx, w_idx, k_idx, q_pos, n_cmp, q_scale, k_scale)
    B, T, H_I, d_I = q_idx.shape
    if q_idx.dtype == torch.float4_e2m1fn_x2:
        d_I *= 2                       # two E2M1 codes per element
    Nc_cap = pages.nc_cap if pages is not None else k_idx.shape[1]
    if idx_out is None:
        idx_out = torch.empty(B, T, topk, dtype=torch.int32, device=q_idx.device)
    if want_scores and score_out is None:
        score_out = torch.empty(B, T, topk, dtype=torch.float32, device=q_idx.device)
    ws, nb = _workspace(csa_indexer_topk_workspace_size(B, T, H_I, d_I, Nc_cap, topk, q_idx.dtype),
                        q_idx, workspace)
    if pages is not None:
        pages.check(B, k_idx, k_scale)
        rc = lib().csa_indexer_topk_paged(B, T, H_I, d_I, Nc_cap, m, topk, _p(q_pos), _p(n_cmp),
                                          _p(q_idx), _p(q_scale), _p(w_idx), _p(k_idx),
                                          _p(k_scale), _DT[q_idx.dtype], pages.c(), _p(idx_out),
                                          _p(score_out), _p(ws), nb, _stream(q_idx))
    else:
        rc = lib().csa_indexer_topk(B, T, H_I, d_I, Nc_cap, m, topk, _p(q_pos), _p(n_cmp),
                                    _p(q_idx), _p(q_scale), _p(w_idx), _p(k_idx), _p(k_scale),
                                    _DT[q_idx.dtype], _p(idx_out), _p(score_out), _p(ws), nb,
                                    _stream(q_idx))
    _check("csa_indexer_topk", rc)
    return idx_out, score_out


def _sink(sink, H):
    if sink is None:
        return None
    if sink.dtype != torch.float32 or sink.shape != (H,) or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor of shape [H]")
    return sink


def csa_sparse_attn(q, kv_cmp, idx, kv_raw, window, q_pos, raw_base, scale=None, out=None,
                    lse=None, want_lse=False, workspace=None, sink=None, pages=None,
                    raw_pages=None):
    """CSA attention; returns (out [B, T, H, D], lse f32 [B, T, H] or None).
    sink: f32 [H] per-head sink logits or None.  pages: a PageTable; kv_cmp is then
    the pool [n_pages * page_size, 2 D] and idx holds logical indices.  raw_pages: a
    PageTable for the window cache; kv_raw is then a pool and raw_pages.nc_cap the
    logical rows per sequence."""
    _dense(q, kv_cmp, idx, kv_raw, q_pos, raw_base, sink)
    B, T, H, D = q.shape
    topk = idx.shape[2] if idx is not None else 0
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    if pages is not None or raw_pages is not None:
        if pages is not None:
            pages.check(B, kv_cmp)
            nb_ws = lib().csa_sparse_attn_paged_workspace_size(B, T, H, D, topk, window)
        else:
            nb_ws = csa_sparse_attn_workspace_size(B, T, H, D, topk, window)
        if raw_pages is not None:
            raw_pages.check(B, kv_raw)
        ws, nb = _workspace(nb_ws, q, workspace)
        rc = lib().csa_sparse_attn_paged(
            B, T, H, D, topk, window, scale, _p(_sink(sink, H)), _p(q_pos), _p(q), _p(kv_cmp),
            pages.nc_cap if pages is not None else kv_cmp.shape[1],
            pages.c() if pages is not None else None, _p(idx), _p(kv_raw),
            raw_pages.nc_cap if raw_pages is not None else kv_raw.shape[1], _p(raw_base),
            raw_pages.c() if raw_pages is not None else None, _DT[q.dtype], _p(out), _p(lse),
            _p(ws), nb, _stream(q))
        _check("csa_sparse_attn_paged", rc)
        return out, lse
    ws, nb = _workspace(csa_sparse_attn_workspace_size(B, T, H, D, topk, window), q, workspace)
    rc = lib().csa_sparse_attn(B, T, H, D, topk, window, scale, _p(_sink(sink, H)), _p(q_pos),
                               _p(q), _p(kv_cmp),
                               kv_cmp.shape[1], _p(idx), _p(kv_raw), kv_raw.shape[1],
                               _p(raw_base), _DT[q.dtype], _p(out), _p(lse), _p(ws), nb,
                               _stream(q))
    _check("csa_sparse_attn", rc)
    return out, lse


def csa_sparse_attn_split_workspace_size(B, T, H, D, topk, window) -> int:
    """Bytes of the workspace both halves of a split csa_sparse_attn share (0: unsupported)."""
    return lib().csa_sparse_attn_split_workspace_size(B, T, H, D, topk, window)


def csa_sparse_attn_window_half(q, kv_raw, window, q_pos, raw_base, topk, workspace, scale=None):
    """First half of csa_sparse_attn (decode rows, bf16): attends each row to its window
    tokens only and leaves the partial results in workspace (a uint8 tensor of
    csa_sparse_attn_split_workspace_size bytes) on q's current stream; it reads no
    index, so it may run while the indexer chooses them."""
    _dense(q, kv_raw, q_pos, raw_base)
    B, T, H, D = q.shape
    scale = D ** -0.5 if scale is None else float(scale)
    rc = lib().csa_sparse_attn_window_half(B, T, H, D, topk, window, scale, _p(q_pos), _p(q),
                                           _p(kv_raw), kv_raw.shape[1], _p(raw_base),
                                           _DT[q.dtype], _p(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(q))
    _check("csa_sparse_attn_window_half", rc)


def csa_sparse_attn_selected_half(q, kv_cmp, idx, kv_raw, window, q_pos, raw_base, workspace,
                                  scale=None, out=None, lse=None, want_lse=False, sink=None):
    """Second half of csa_sparse_attn: attends the rows to their selected entries and merges
    them with the window half's partials in workspace (which must have run first, on this
    stream or ordered before it by an event); returns (out, lse) as csa_sparse_attn does."""
    _dense(q, kv_cmp, idx, kv_raw, q_pos, raw_base, sink)
    B, T, H, D = q.shape
    topk = idx.shape[2] if idx is not None else 0
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    rc = lib().csa_sparse_attn_selected_half(
        B, T, H, D, topk, window, scale, _p(_sink(sink, H)), _p(q_pos), _p(q), _p(kv_cmp),
        kv_cmp.shape[1], _p(idx), _p(kv_raw), kv_raw.shape[1], _p(raw_base), _DT[q.dtype],
        _p(out), _p(lse), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(q))
    _check("csa_sparse_attn_selected_half", rc)
    return out, lse


def csa_sparse_attn_noalloc(q, kv_cmp, idx, kv_raw, window, q_pos, raw_base, out, scale=None,
                            lse=None, sink=None):
    """csa_sparse_attn that allocates nothing: out (and lse, if wanted) are
    the caller's; split-key partials use the library's static device scratch
    (see csa_sparse_attn_noalloc in include/csa.h).  Returns (out, lse)."""
    _dense(q, kv_cmp, idx, kv_raw, q_pos, raw_base, sink, out, lse)
    B, T, H, D = q.shape
    topk = idx.shape[2] if idx is not None else 0
    scale = D ** -0.5 if scale is None else float(scale)
    rc = lib().csa_sparse_attn_noalloc(B, T, H, D, topk, window, scale, _p(_sink(sink, H)),
                                       _p(q_pos), _p(q), _p(kv_cmp), kv_cmp.shape[1], _p(idx),
                                       _p(kv_raw), kv_raw.shape[1], _p(raw_base), _DT[q.dtype],
                                       _p(out), _p(lse), _stream(q))
    _check("csa_sparse_attn_noalloc", rc)
    return out, lse


def hca_dense_attn(q, kv_cmp, kv_raw, m, window, q_pos, n_cmp, raw_base, scale=None, out=None,
                   lse=None, want_lse=False, workspace=None, sink=None, pages=None,
                   raw_pages=None):
    """HCA attention; returns (out [B, T, H, D], lse or None).
    sink: f32 [H] per-head sink logits or None.  pages / raw_pages: PageTables of the
    compressed and window caches (each then a pool; nc_cap the logical rows)."""
    _dense(q, kv_cmp, kv_raw, q_pos, n_cmp, raw_base, sink)
    B, T, H, D = q.shape
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    if pages is not None or raw_pages is not None:
        nc = pages.nc_cap if pages is not None else kv_cmp.shape[1]
        rcap = raw_pages.nc_cap if raw_pages is not None else kv_raw.shape[1]
        if pages is not None:
            pages.check(B, kv_cmp)
        if raw_pages is not None:
            raw_pages.check(B, kv_raw)
        ws, nb = _workspace(hca_dense_attn_workspace_size(B, T, H, D, nc, window), q, workspace)
        rc = lib().hca_dense_attn_paged(
            B, T, H, D, m, window, scale, _p(_sink(sink, H)), _p(q_pos), _p(n_cmp), _p(q),
            _p(kv_cmp), nc, pages.c() if pages is not None else None, _p(kv_raw), rcap,
            _p(raw_base), raw_pages.c() if raw_pages is not None else None, _DT[q.dtype], _p(out),
            _p(lse), _p(ws), nb, _stream(q))
        _check("hca_dense_attn_paged", rc)
        return out, lse
    ws, nb = _workspace(hca_dense_attn_workspace_size(B, T, H, D, kv_cmp.shape[1], window), q,
                        workspace)
    rc = lib().hca_dense_attn(B, T, H, D, m, window, scale, _p(_sink(sink, H)), _p(q_pos),
                              _p(n_cmp), _p(q),
                              _p(kv_cmp), kv_cmp.shape[1], _p(kv_raw), kv_raw.shape[1],
                              _p(raw_base), _DT[q.dtype], _p(out), _p(lse), _p(ws), nb, _stream(q))
    _check("hca_dense_attn", rc)
    return out, lse


# ---------------------------------------------------------------- backward

def _bwd_outputs(q, kv_cmp, kv_raw, sink, dq, dkv_cmp, dkv_raw, dsink):
    B, T, H, D = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    if dq is None:
        dq = torch.empty(B, T, H, D, **f32)
    if dkv_cmp is None:
        dkv_cmp = torch.empty(B, kv_cmp.shape[1], 2 * D, **f32)
    if dkv_raw is None:
        dkv_raw = torch.empty(B, kv_raw.shape[1], 2 * D, **f32)
    if dsink is None and sink is not None:
        dsink = torch.empty(H, **f32)
    return dq, dkv_cmp, dkv_raw, dsink


def csa_sparse_attn_bwd(q, kv_cmp, idx, kv_raw, window, q_pos, raw_base, lse, dout,
                        scale=None, sink=None, want_mass=False, dq=None, dkv_cmp=None,
                        dkv_raw=None, dsink=None, attn_mass=None, workspace=None):
    """Gradients of csa_sparse_attn for the upstream gradient dout (bf16, like
    q); lse is the forward's.  Returns (dq, dkv_cmp, dkv_raw, dsink or
    None, attn_mass or None), all float32; attn_mass [B, T, topk] is the
    attention probability of each selected slot summed over heads."""
    _dense(q, kv_cmp, idx, kv_raw, q_pos, raw_base, lse, dout, sink)
    B, T, H, D = q.shape
    topk = idx.shape[2] if idx is not None else 0
    scale = D ** -0.5 if scale is None else float(scale)
    sink = _sink(sink, H)
    dq, dkv_cmp, dkv_raw, dsink = _bwd_outputs(q, kv_cmp, kv_raw, sink, dq, dkv_cmp, dkv_raw,
                                               dsink)
    if want_mass and attn_mass is None:
        attn_mass = torch.empty(B, T, topk, dtype=torch.float32, device=q.device)
    ws, nb = _workspace(lib().csa_sparse_attn_bwd_workspace_size(
        B, T, H, kv_cmp.shape[1], kv_raw.shape[1], window), q, workspace)
    rc = lib().csa_sparse_attn_bwd(B, T, H, D, topk, window, scale, _p(sink), _p(q_pos), _p(q),
                                   _p(kv_cmp), kv_cmp.shape[1], _p(idx), _p(kv_raw),
                                   kv_raw.shape[1], _p(raw_base), _DT[q.dtype], _p(lse), _p(dout),
                                   _p(dq), _p(dkv_cmp), _p(dkv_raw), _p(dsink), _p(attn_mass),
                                   _p(ws), nb, _stream(q))
    _check("csa_sparse_attn_bwd", rc)
    return dq, dkv_cmp, dkv_raw, dsink, attn_mass


def hca_dense_attn_bwd(q, kv_cmp, kv_raw, m, window, q_pos, n_cmp, raw_base, lse, dout,
                       scale=None, sink=None, want_mass=False, dq=None, dkv_cmp=None,
                       dkv_raw=None, dsink=None, attn_mass=None, workspace=None):
    """Gradients of hca_dense_attn; returns (dq, dkv_cmp, dkv_raw, dsink or
    None, attn_mass or None); attn_mass [B, T, Nc_cap] is the attention
    probability of each compressed entry summed over heads (0 where unseen)."""
    _dense(q, kv_cmp, kv_raw, q_pos, n_cmp, raw_base, lse, dout, sink)
    B, T, H, D = q.shape
    scale = D ** -0.5 if scale is None else float(scale)
    sink = _sink(sink, H)
    dq, dkv_cmp, dkv_raw, dsink = _bwd_outputs(q, kv_cmp, kv_raw, sink, dq, dkv_cmp, dkv_raw,
                                               dsink)
    if want_mass and attn_mass is None:
        attn_mass = torch.empty(B, T, kv_cmp.shape[1], dtype=torch.float32, device=q.device)
    ws, nb = _workspace(lib().hca_dense_attn_bwd_workspace_size(
        B, T, H, kv_cmp.shape[1], kv_raw.shape[1], window), q, workspace)
    rc = lib().hca_dense_attn_bwd(B, T, H, D, m, window, scale, _p(sink), _p(q_pos), _p(n_cmp),
                                  _p(q), _p(kv_cmp), kv_cmp.shape[1], _p(kv_raw), kv_raw.shape[1],
                                  _p(raw_base), _DT[q.dtype], _p(lse), _p(dout), _p(dq),
                                  _p(dkv_cmp), _p(dkv_raw), _p(dsink), _p(attn_mass), _p(ws), nb,
                                  _stream(q))
    _check("hca_dense_attn_bwd", rc)
    return dq, dkv_cmp, dkv_raw, dsink, attn_mass


def csa_compress_bwd(x, w_kv, w_gate, m, overlap, Nc_cap, d_out, ape=None, rotate=False,
                     want_dape=True, dx=None, dw_kv=None, dw_gate=None, dape=None,
                     workspace=None):
    """Gradients of a one-shot csa_compress call from position 0 (bf16 x
    [B, L, d_model] and weights [E, d_model]) for d_out f32 [B, Nc_cap, E].
    Returns (dx, dw_kv, dw_gate, dape or None), all float32."""
    _dense(x, w_kv, w_gate, d_out, ape)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty(B, L, d_model, **f32) if dx is None else dx
    dw_kv = torch.empty(E, d_model, **f32) if dw_kv is None else dw_kv
    dw_gate = torch.empty(E, d_model, **f32) if dw_gate is None else dw_gate
    if ape is not None and want_dape and dape is None:
        dape = torch.empty((1 + overlap) * m, E, **f32)
    ws, nb = _workspace(lib().csa_compress_bwd_workspace_size(B, L, d_model, E, m, Nc_cap), x, workspace)
    rc = lib().csa_compress_bwd(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(x), _p(w_kv),
                                _p(w_gate), _DT[x.dtype], _p(ape), Nc_cap, _p(d_out), _p(dx),
                                _p(dw_kv), _p(dw_gate), _p(dape), _p(ws), nb, _stream(x))
    _check("csa_compress_bwd", rc)
    return dx, dw_kv, dw_gate, dape


def csa_compress_bwd_ex(x, w_kv, w_gate, m, overlap, Nc_cap, d_out, ape=None, rotate=False,
                        norm_weight=None, norm_eps=1e-6, rope_dim=0, rope_offset=0,
                        rope_base=10000.0, rope_interleaved=False, want_dape=True, dx=None,
                        dw_kv=None, dw_gate=None, dape=None, d_norm_weight=None,
                        workspace=None):
    """csa_compress_bwd for entries post-processed as csa_compress does with
    the same norm_weight / norm_eps / rope_* options.  Returns (dx, dw_kv,
    dw_gate, dape or None, d_norm_weight or None), all float32."""
    _dense(x, w_kv, w_gate, d_out, ape, norm_weight)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    if norm_weight is not None and (norm_weight.dtype != torch.float32 or
                                    norm_weight.shape != (E,)):
        raise ValueError("norm_weight must be a float32 tensor of shape [E]")
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty(B, L, d_model, **f32) if dx is None else dx
    dw_kv = torch.empty(E, d_model, **f32) if dw_kv is None else dw_kv
    dw_gate = torch.empty(E, d_model, **f32) if dw_gate is None else dw_gate
    if ape is not None and want_dape and dape is None:
        dape = torch.empty((1 + overlap) * m, E, **f32)
    if norm_weight is not None and d_norm_weight is None:
        d_norm_weight = torch.empty(E, **f32)
    opts = _COpts(None if norm_weight is None else norm_weight.data_ptr(), float(norm_eps),
                  int(rope_dim), int(rope_offset), float(rope_base), int(bool(rope_interleaved)))
    ws, nb = _workspace(lib().csa_compress_bwd_workspace_size(B, L, d_model, E, m, Nc_cap), x, workspace)
    rc = lib().csa_compress_bwd_ex(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(x),
                                   _p(w_kv), _p(w_gate), _DT[x.dtype], _p(ape), Nc_cap,
                                   _p(d_out), C.byref(opts), _p(dx), _p(dw_kv), _p(dw_gate),
                                   _p(dape), _p(d_norm_weight), _p(ws), nb, _stream(x))
    _check("csa_compress_bwd_ex", rc)
    return dx, dw_kv, dw_gate, dape, (d_norm_weight if norm_weight is not None else None)


def csa_indexer_kl_bwd(q_idx, w_idx, k_idx, idx, attn_mass, grad_scale=None, loss=None,
                       dq_idx=None, dw_idx=None, dk_idx=None, workspace=None):
    """Indexer KL loss per query row and its gradients (bf16 q_idx
    [B, T, 16, 64], k_idx [B, Nc_cap, 64]; w_idx f32 [B, T, 16]; idx and
    attn_mass [B, T, topk] from csa_indexer_topk and csa_sparse_attn_bwd;
    grad_scale f32 [B, T] or None).  Returns (loss, dq_idx, dw_idx, dk_idx),
    all float32."""
    _dense(q_idx, w_idx, k_idx, idx, attn_mass, grad_scale)
    B, T, H_I, d_I = q_idx.shape
    Nc_cap, topk = k_idx.shape[1], idx.shape[2]
    f32 = dict(dtype=torch.float32, device=q_idx.device)
    loss = torch.empty(B, T, **f32) if loss is None else loss
    dq_idx = torch.empty(B, T, H_I, d_I, **f32) if dq_idx is None else dq_idx
    dw_idx = torch.empty(B, T, H_I, **f32) if dw_idx is None else dw_idx
    dk_idx = torch.empty(B, Nc_cap, d_I, **f32) if dk_idx is None else dk_idx
    ws, nb = _workspace(lib().csa_indexer_kl_bwd_workspace_size(B, T, Nc_cap, topk), q_idx,
                        workspace)
    rc = lib().csa_indexer_kl_bwd(B, T, H_I, d_I, Nc_cap, topk, _p(q_idx), _p(w_idx), _p(k_idx),
                                  _DT[q_idx.dtype], _p(idx), _p(attn_mass), _p(grad_scale),
                                  _p(loss), _p(dq_idx), _p(dw_idx), _p(dk_idx), _p(ws), nb,
                                  _stream(q_idx))
    _check("csa_indexer_kl_bwd", rc)
    return loss, dq_idx, dw_idx, dk_idx


def csa_indexer_kl_dense_bwd(q_idx, w_idx, k_idx, m, q_pos, n_cmp, attn_mass, grad_scale=None,
                             loss=None, dq_idx=None, dw_idx=None, dk_idx=None, workspace=None):
    """Dense indexer KL loss (every visible entry j < n_vis of each row) and
    its gradients: q_idx [B, T, 16, 64] and k_idx [B, Nc_cap, 64] bf16, w_idx
    f32 [B, T, 16], q_pos int64 [B], n_cmp int32 [B], attn_mass f32
    [B, T, Nc_cap] from hca_dense_attn_bwd, grad_scale f32 [B, T] or None.
    Returns (loss, dq_idx, dw_idx, dk_idx), all float32."""
    _dense(q_idx, w_idx, k_idx, q_pos, n_cmp, attn_mass, grad_scale)
    B, T, H_I, d_I = q_idx.shape
    Nc_cap = k_idx.shape[1]
    f32 = dict(dtype=torch.float32, device=q_idx.device)
    loss = torch.empty(B, T, **f32) if loss is None else loss
    dq_idx = torch.empty(B, T, H_I, d_I, **f32) if dq_idx is None else dq_idx
    dw_idx = torch.empty(B, T, H_I, **f32) if dw_idx is None else dw_idx
    dk_idx = torch.empty(B, Nc_cap, d_I, **f32) if dk_idx is None else dk_idx
    ws, nb = _workspace(lib().csa_indexer_kl_dense_bwd_workspace_size(B, T, Nc_cap), q_idx,
                        workspace)
    rc = lib().csa_indexer_kl_dense_bwd(B, T, H_I, d_I, Nc_cap, m, _p(q_pos), _p(n_cmp),
                                        _p(q_idx), _p(w_idx), _p(k_idx), _DT[q_idx.dtype],
                                        _p(attn_mass), _p(grad_scale), _p(loss), _p(dq_idx),
                                        _p(dw_idx), _p(dk_idx), _p(ws), nb, _stream(q_idx))
    _check("csa_indexer_kl_dense_bwd", rc)
    return loss, dq_idx, dw_idx, dk_idx


# ---------------------------------------------------------------- packed sequences

def _cu(t, n1):
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != n1 or not t.is_cuda:
        raise ValueError("sequence offsets must be device int32 tensors of n + 1 elements")
    return t


def csa_build_cmp_cu_seqlens(cu_seqlens, m):
    """Entry offsets of packed sequences: [0, floor(len_0 / m), ...] cumulated (device int32)."""
    n = cu_seqlens.numel() - 1
    out = torch.empty(n + 1, dtype=torch.int32, device=cu_seqlens.device)
    rc = lib().csa_build_cmp_cu_seqlens(n, _p(_cu(cu_seqlens, n + 1)), m, _p(out),
                                        _stream(cu_seqlens))
    _check("csa_build_cmp_cu_seqlens", rc)
    return out


def _opts(norm_weight, norm_eps, rope_dim, rope_offset, rope_base, rope_interleaved, E):
    if norm_weight is None and not rope_dim:
        return None
    if norm_weight is not None and (norm_weight.dtype != torch.float32 or
                                    norm_weight.shape != (E,)):
        raise ValueError("norm_weight must be a float32 tensor of shape [E]")
    return C.byref(_COpts(None if norm_weight is None else norm_weight.data_ptr(),
                          float(norm_eps), int(rope_dim), int(rope_offset), float(rope_base),
                          int(bool(rope_interleaved))))


def csa_compress_varlen(x, w_kv, w_gate, cu_seqlens, cmp_cu_seqlens, max_len, m, overlap, out,
                        out_scale=None, ape=None, state_out=None, rotate=False, workspace=None,
                        norm_weight=None, norm_eps=1e-6, rope_dim=0, rope_offset=0,
                        rope_base=10000.0, rope_interleaved=False):
    """Compressor over packed sequences (csa_compress_varlen in include/csa.h):
    x [total, d_model]; out [total entries, E] (rows from cmp_cu_seqlens)."""
    _dense(x, w_kv, w_gate, out, out_scale, ape, state_out, norm_weight)
    total, d_model = x.shape
    E = w_kv.shape[0]
    n = cu_seqlens.numel() - 1
    ws, nb = _workspace(lib().csa_compress_varlen_workspace_size(total, d_model, E, m, overlap,
                                                                 _DT[x.dtype]), x, workspace)
    rc = lib().csa_compress_varlen(n, total, int(max_len), d_model, E, m, overlap,
                                   int(bool(rotate)), _p(_cu(cu_seqlens, n + 1)),
                                   _p(_cu(cmp_cu_seqlens, n + 1)), _p(x), _p(w_kv), _p(w_gate),
                                   _DT[x.dtype], _p(ape), _p(state_out), _p(out), _p(out_scale),
                                   _DT[out.dtype],
                                   _opts(norm_weight, norm_eps, rope_dim, rope_offset, rope_base,
                                         rope_interleaved, E), _p(ws), nb, _stream(x))
    _check("csa_compress_varlen", rc)
    return out


def csa_indexer_topk_varlen(q_idx, w_idx, k_idx, cu_seqlens, cmp_cu_seqlens, max_len, max_cmp,
                            m, topk, idx_out=None, score_out=None, want_scores=False,
                            workspace=None):
    """Indexer top-k over packed sequences: q_idx [total, H_I, d_I], w_idx [total, H_I],
    k_idx [total entries, d_I]; returns (idx [total, topk] local to each sequence, scores)."""
    _dense(q_idx, w_idx, k_idx)
    total, H_I, d_I = q_idx.shape
    n = cu_seqlens.numel() - 1
    if idx_out is None:
        idx_out = torch.empty(total, topk, dtype=torch.int32, device=q_idx.device)
    if want_scores and score_out is None:
        score_out = torch.empty(total, topk, dtype=torch.float32, device=q_idx.device)
    ws, nb = _workspace(lib().csa_indexer_topk_varlen_workspace_size(total, max(1, max_cmp), topk,
                                                                     _DT[q_idx.dtype]),
                        q_idx, workspace)
    rc = lib().csa_indexer_topk_varlen(n, total, int(max_len), H_I, d_I, int(max_cmp), m, topk,
                                       _p(_cu(cu_seqlens, n + 1)), _p(_cu(cmp_cu_seqlens, n + 1)),
                                       _p(q_idx), _p(w_idx), _p(k_idx), _DT[q_idx.dtype],
                                       _p(idx_out), _p(score_out), _p(ws), nb, _stream(q_idx))
    _check("csa_indexer_topk_varlen", rc)
    return idx_out, score_out


def csa_sparse_attn_varlen(q, kv_cmp, idx, kv_raw, cu_seqlens, cmp_cu_seqlens, max_len, max_cmp,
                           window, scale=None, out=None, lse=None, want_lse=False, sink=None,
                           workspace=None):
    """CSA attention over packed sequences: q [total, H, D], kv_cmp [total entries, 2D],
    idx [total, topk] local indices, kv_raw [total, 2D]; returns (out, lse)."""
    _dense(q, kv_cmp, idx, kv_raw, sink)
    total, H, D = q.shape
    n = cu_seqlens.numel() - 1
    topk = idx.shape[1] if idx is not None else 0
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(total, H, dtype=torch.float32, device=q.device)
    ws, nb = _workspace(lib().csa_sparse_attn_varlen_workspace_size(total, H, D, topk, window), q,
                        workspace)
    rc = lib().csa_sparse_attn_varlen(n, total, int(max_len), H, D, topk, window, scale,
                                      _p(_sink(sink, H)), _p(_cu(cu_seqlens, n + 1)),
                                      _p(_cu(cmp_cu_seqlens, n + 1)), _p(q), _p(kv_cmp),
                                      int(max_cmp), _p(idx), _p(kv_raw), _DT[q.dtype], _p(out),
                                      _p(lse), _p(ws), nb, _stream(q))
    _check("csa_sparse_attn_varlen", rc)
    return out, lse
