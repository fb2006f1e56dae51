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
        L.hca_dense_attn.argtypes = [i32] * 6 + [f32, vp, vp, vp, vp, vp, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
        L.hca_dense_attn_workspace_size.argtypes = [i32] * 6
        pt = C.POINTER(_CPageTable)
        L.csa_compress_paged.argtypes = ([i32] * 7 + [vp] * 4 + [i32, vp, vp, vp, vp, vp, i32, i32,
                                         pt, vp, sz, vp])
        L.csa_indexer_topk_paged.argtypes = [i32] * 7 + [vp] * 7 + [i32, pt, vp, vp, vp, sz, vp]
        L.csa_sparse_attn_paged.argtypes = ([i32] * 6 + [f32, vp, vp, vp, vp, i32, pt, vp, vp, i32,
                                            vp, i32, vp, vp, vp, sz, vp])
        L.csa_sparse_attn_paged_workspace_size.argtypes = [i32] * 6
        L.csa_sparse_attn_paged_workspace_size.restype = C.c_size_t
        for f in (L.csa_compress, L.csa_indexer_topk, L.csa_sparse_attn, L.hca_dense_attn,
                  L.csa_compress_paged, L.csa_indexer_topk_paged, L.csa_sparse_attn_paged):
            f.restype = C.c_int
        for f in (L.csa_compress_workspace_size, L.csa_indexer_topk_workspace_size,
                  L.csa_sparse_attn_workspace_size, L.hca_dense_attn_workspace_size):
            f.restype = C.c_size_t
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
                 state_in=None, state_out=None, workspace=None, rotate=False, pages=None):
    """Gated overlapping compressor; see ``csa_compress`` in include/csa.h.

    x [B, L, d_model]; w_kv, w_gate [E, d_model]; pos0 int64 [B];
    out [B, Nc_cap, E] (f32, bf16 or float8_e4m3fn, then out_scale f32 [B, Nc_cap]),
    or float4_e2m1fn_x2 [B, Nc_cap, E / 2] with out_scale E8M0 bytes [B, Nc_cap, E / 32]
    (float8_e8m0fnu or uint8);
    ape f32 [(1+o) m, E]; state_in / state_out f32 [B, (1+o) m - 1, 2, E];
    rotate: entries times the Hadamard matrix / sqrt(E) before storage.
    pages: a PageTable; out (and out_scale) are then pools [n_pages * page_size, ...]."""
    _dense(x, w_kv, w_gate, pos0, out, out_scale, ape, state_in, state_out)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    ws, nb = _workspace(csa_compress_workspace_size(B, L, d_model, E, m, overlap, x.dtype), x,
                        workspace)
    if pages is not None:
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
                    lse=None, want_lse=False, workspace=None, sink=None, pages=None):
    """CSA attention; returns (out [B, T, H, D], lse f32 [B, T, H] or None).
    sink: f32 [H] per-head sink logits or None.  pages: a PageTable; kv_cmp is then
    the pool [n_pages * page_size, 2 D] and idx holds logical indices."""
    _dense(q, kv_cmp, idx, kv_raw, q_pos, raw_base, sink)
    B, T, H, D = q.shape
    topk = idx.shape[2] if idx is not None else 0
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    if pages is not None:
        ws, nb = _workspace(lib().csa_sparse_attn_paged_workspace_size(B, T, H, D, topk, window),
                            q, workspace)
        rc = lib().csa_sparse_attn_paged(B, T, H, D, topk, window, scale, _p(_sink(sink, H)),
                                         _p(q_pos), _p(q), _p(kv_cmp), pages.nc_cap, pages.c(),
                                         _p(idx), _p(kv_raw), kv_raw.shape[1], _p(raw_base),
                                         _DT[q.dtype], _p(out), _p(lse), _p(ws), nb, _stream(q))
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


def hca_dense_attn(q, kv_cmp, kv_raw, m, window, q_pos, n_cmp, raw_base, scale=None, out=None,
                   lse=None, want_lse=False, workspace=None, sink=None):
    """HCA attention; returns (out [B, T, H, D], lse or None).
    sink: f32 [H] per-head sink logits or None."""
    _dense(q, kv_cmp, kv_raw, q_pos, n_cmp, raw_base, sink)
    B, T, H, D = q.shape
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty(B, T, H, dtype=torch.float32, device=q.device)
    ws, nb = _workspace(hca_dense_attn_workspace_size(B, T, H, D, kv_cmp.shape[1], window), q,
                        workspace)
    rc = lib().hca_dense_attn(B, T, H, D, m, window, scale, _p(_sink(sink, H)), _p(q_pos),
                              _p(n_cmp), _p(q),
                              _p(kv_cmp), kv_cmp.shape[1], _p(kv_raw), kv_raw.shape[1],
                              _p(raw_base), _DT[q.dtype], _p(out), _p(lse), _p(ws), nb, _stream(q))
    _check("hca_dense_attn", rc)
    return out, lse
