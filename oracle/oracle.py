"""ctypes wrapper around the plain CPU oracle in ``csa_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of the benchmark.  The GPU product path never imports it.

Arrays are passed in their stored formats: fp32 as ``float32``, bf16 as the
``uint16`` bit pattern, OCP e4m3 as the ``uint8`` code, MXFP4 as packed E2M1
codes (two per byte) with E8M0 block scales (``uint8``).  Results come back as
``float64`` arrays (values before any storage rounding).

Citations follow the C file: the migration page's section 3.2 (compressor),
the DS-V4 analysis sections 1.2-1.5 (pipeline, overlap, HCA, SWA), the
article's sections 3.2 and 5.2 (mean-pool special case, entry count, window).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DT_F32, DT_BF16, DT_E4M3, DT_MXFP4 = 0, 1, 2, 3


def build() -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-o", tmp, SRC, "-lm"])
    os.replace(tmp, LIB)
    return LIB


_lib = None


class _Opts(C.Structure):
    _fields_ = [("norm_w", C.c_void_p), ("norm_eps", C.c_double), ("rope_dim", C.c_int),
                ("rope_off", C.c_int), ("rope_interleaved", C.c_int), ("rope_base", C.c_double)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = C.CDLL(LIB)
        vp, i32, i64p, dp = C.c_void_p, C.c_int, C.c_void_p, C.c_void_p
        L.orc_compress.argtypes = [i32] * 7 + [i64p, vp, vp, vp, i32, dp, dp, dp, i32, dp, vp]
        L.orc_compress_ex.argtypes = ([i32] * 7 + [i64p, vp, vp, vp, i32, dp, dp, dp, i32, dp, vp,
                                      C.POINTER(_Opts)])
        L.orc_compress_ex.restype = C.c_int
        L.orc_indexer_topk.argtypes = [i32] * 7 + [i64p, vp, vp, vp, vp, vp, vp, i32, vp, dp, dp, dp]
        L.orc_sparse_attn.argtypes = [i32] * 6 + [C.c_double, dp, i64p, vp, vp, i32, vp, vp, i32, i64p, i32, dp, dp]
        L.orc_hca_dense_attn.argtypes = [i32] * 6 + [C.c_double, dp, i64p, vp, vp, vp, i32, vp, i32, i64p, i32, dp, dp]
        for f in (L.orc_compress, L.orc_indexer_topk, L.orc_sparse_attn, L.orc_hca_dense_attn):
            f.restype = C.c_int
        L.orc_e4m3_encode.argtypes = [C.c_double]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_decode.restype = C.c_double
        L.orc_bf16_encode.argtypes = [C.c_double]
        L.orc_bf16_encode.restype = C.c_uint16
        L.orc_bf16_decode.argtypes = [C.c_uint16]
        L.orc_bf16_decode.restype = C.c_double
        L.orc_quant_rows_e4m3.argtypes = [i32, i32, dp, vp, dp]
        L.orc_quant_rows_e4m3.restype = None
        L.orc_e2m1_encode.argtypes = [C.c_double]
        L.orc_e2m1_encode.restype = C.c_uint8
        L.orc_e2m1_decode.argtypes = [C.c_uint8]
        L.orc_e2m1_decode.restype = C.c_double
        L.orc_quant_rows_mxfp4.argtypes = [i32, i32, dp, vp, vp]
        L.orc_quant_rows_mxfp4.restype = None
        L.orc_attn_bwd.argtypes = ([i32] * 6 + [C.c_double, dp, i64p, vp, vp, i32, vp, i32, vp, vp,
                                    i32, i64p, i32, dp, dp, dp, dp, dp, dp])
        L.orc_attn_bwd.restype = C.c_int
        L.orc_indexer_kl_bwd.argtypes = [i32] * 6 + [vp, vp, vp, i32, vp, dp, dp, dp, dp, dp, dp]
        L.orc_indexer_kl_bwd.restype = C.c_int
        L.orc_compress_bwd.argtypes = [i32] * 7 + [vp, vp, vp, i32, dp, i32, dp, dp, dp, dp, dp]
        L.orc_compress_bwd.restype = C.c_int
        L.orc_compress_bwd_ex.argtypes = ([i32] * 7 + [vp, vp, vp, i32, dp, i32, dp,
                                                       C.POINTER(_Opts), dp, dp, dp, dp, dp])
        L.orc_compress_bwd_ex.restype = C.c_int
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _dt(a):
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.uint8:
        return DT_E4M3
    raise TypeError("stored format must be float32, uint16 (bf16) or uint8 (e4m3): %s" % a.dtype)


def num_threads() -> int:
    return lib().orc_num_threads()


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e4m3_decode(c: int) -> float:
    return lib().orc_e4m3_decode(int(c))


def bf16_encode(v: float) -> int:
    return lib().orc_bf16_encode(float(v))


def bf16_decode(h: int) -> float:
    return lib().orc_bf16_decode(int(h))


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def e2m1_decode(c: int) -> float:
    return lib().orc_e2m1_decode(int(c))


def quant_rows_mxfp4(x):
    """MXFP4 quantisation of the last axis (a multiple of 32): returns (codes
    packed two per byte, element 2i in the low nibble; E8M0 scale codes, one
    per 32 values)."""
    x = _c(x, np.float64)
    cols = x.shape[-1]
    assert cols % 32 == 0
    rows = x.size // cols
    codes = np.zeros(x.shape[:-1] + (cols // 2,), np.uint8)
    scales = np.zeros(x.shape[:-1] + (cols // 32,), np.uint8)
    lib().orc_quant_rows_mxfp4(rows, cols, _p(x), _p(codes), _p(scales))
    return codes, scales


def mxfp4_decode(codes, scales):
    """Values of an MXFP4 store (the inverse of quant_rows_mxfp4's packing)."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    table = np.array([e2m1_decode(c) for c in range(16)], np.float64)
    lo, hi = table[codes & 15], table[codes >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (2 * codes.shape[-1],))
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return v * np.repeat(sc, 32, axis=-1)


def quant_rows_e4m3(x):
    """Per-row e4m3 quantisation (scale = amax / 448): returns (codes, scales)."""
    x = _c(x, np.float64)
    rows, cols = x.reshape(-1, x.shape[-1]).shape
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1], np.float64)
    lib().orc_quant_rows_e4m3(rows, cols, _p(x), _p(codes), _p(scales))
    return codes, scales


def compress(x, w_kv, w_gate, m, overlap, pos0, Nc_cap, ape=None, state_in=None,
             want_state=True, rotate=False, norm_weight=None, norm_eps=1e-6, rope_dim=0,
             rope_offset=0, rope_base=10000.0, rope_interleaved=False):
    """Gated overlapping compressor.

    x [B, L, d_model], w_kv / w_gate [E, d_model] (same stored format);
    ape [(1+o) m, E] float; state_in [B, (1+o) m - 1, 2, E] float or None;
    each emitted entry then goes through, in this order: an RMS norm over its
    E channels with weight norm_weight [E] (None: none), the rotary position
    embedding of channels [rope_offset, rope_offset + rope_dim) at position
    m * i (rope_dim 0: none; rotate-half pairs unless rope_interleaved), and
    rotate: the Sylvester Hadamard matrix / sqrt(E).
    Returns (out [B, Nc_cap, E] float64 with NaN in unwritten rows,
    written [B, Nc_cap] bool, state_out or None).
    """
    x, w_kv, w_gate = _c(x), _c(w_kv), _c(w_gate)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    dt = _dt(x)
    assert _dt(w_kv) == dt and _dt(w_gate) == dt
    ns = (1 + overlap) * m - 1
    pos0 = _c(np.broadcast_to(np.asarray(pos0, np.int64), (B,)), np.int64)
    ape = _c(ape, np.float64)
    state_in = _c(state_in, np.float64)
    state_out = np.zeros((B, ns, 2, E), np.float64) if want_state else None
    out = np.full((B, Nc_cap, E), np.nan, np.float64)
    written = np.zeros((B, Nc_cap), np.uint8)
    nw = _c(norm_weight, np.float64)
    opts = _Opts(None if nw is None else nw.ctypes.data, float(norm_eps), int(rope_dim),
                 int(rope_offset), int(bool(rope_interleaved)), float(rope_base))
    rc = lib().orc_compress_ex(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(pos0), _p(x),
                               _p(w_kv), _p(w_gate), dt, _p(ape), _p(state_in), _p(state_out),
                               Nc_cap, _p(out), _p(written), C.byref(opts))
    assert rc == 0
    return out, written.astype(bool), state_out


def indexer_topk(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale=None,
                 k_scale=None, want_all=False, fmt=None):
    """Lightning-indexer scores + per-row top-k.

    q_idx [B, T, H_I, d_I], w_idx [B, T, H_I] fp32, k_idx [B, Nc_cap, d_I];
    e4m3 inputs need q_scale [B, T, H_I] and k_scale [B, Nc_cap].  With
    fmt="mxfp4", q_idx [B, T, H_I, d_I / 2] and k_idx [B, Nc_cap, d_I / 2] hold
    packed E2M1 codes and q_scale [B, T, H_I, d_I / 32], k_scale
    [B, Nc_cap, d_I / 32] their E8M0 block scales (uint8).
    Returns (idx [B, T, topk] int32 ascending with -1 pads, sel_score, kth,
    all_scores or None).
    """
    q_idx, k_idx = _c(q_idx), _c(k_idx)
    w_idx = _c(w_idx, np.float32)
    B, T, H_I, d_I = q_idx.shape
    Nc_cap = k_idx.shape[1]
    if fmt == "mxfp4":
        assert q_idx.dtype == np.uint8 and k_idx.dtype == np.uint8
        dt = DT_MXFP4
        d_I *= 2
        q_scale, k_scale = _c(q_scale, np.uint8), _c(k_scale, np.uint8)
        assert q_scale.shape == (B, T, H_I, d_I // 32) and k_scale.shape == (B, Nc_cap, d_I // 32)
    else:
        dt = _dt(q_idx)
        assert _dt(k_idx) == dt
        if dt == DT_E4M3:
            q_scale, k_scale = _c(q_scale, np.float32), _c(k_scale, np.float32)
        else:
            q_scale = k_scale = None
    q_pos = _c(np.broadcast_to(np.asarray(q_pos, np.int64), (B,)), np.int64)
    n_cmp = _c(np.broadcast_to(np.asarray(n_cmp, np.int32), (B,)), np.int32)
    idx = np.zeros((B, T, topk), np.int32)
    sel = np.zeros((B, T, topk), np.float64)
    kth = np.zeros((B, T), np.float64)
    alls = np.zeros((B, T, Nc_cap), np.float64) if want_all else None
    rc = lib().orc_indexer_topk(B, T, H_I, d_I, Nc_cap, m, topk, _p(q_pos), _p(n_cmp),
                                _p(q_idx), _p(q_scale), _p(w_idx), _p(k_idx), _p(k_scale),
                                dt, _p(idx), _p(sel), _p(kth), _p(alls))
    assert rc == 0
    return idx, sel, kth, alls


def _sink(sink, H):
    if sink is None:
        return None
    return _c(np.broadcast_to(np.asarray(sink, np.float64), (H,)), np.float64)


def sparse_attn(q, kv_cmp, idx, kv_raw, window, q_pos, raw_base, scale=None, sink=None):
    """CSA attention: joint softmax over the selected compressed rows and the
    raw sliding window.  q [B, T, H, D], kv_cmp [B, Nc_cap, 2D],
    idx [B, T, topk], kv_raw [B, R_cap, 2D]; sink [H] logits or None (one
    more softmax term per head, with no value).  Returns (out, lse) float64."""
    q, kv_cmp, kv_raw = _c(q), _c(kv_cmp), _c(kv_raw)
    idx = _c(idx, np.int32)
    B, T, H, D = q.shape
    dt = _dt(q)
    assert _dt(kv_cmp) == dt and _dt(kv_raw) == dt
    topk = idx.shape[2]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q_pos = _c(np.broadcast_to(np.asarray(q_pos, np.int64), (B,)), np.int64)
    raw_base = _c(np.broadcast_to(np.asarray(raw_base, np.int64), (B,)), np.int64)
    out = np.zeros((B, T, H, D), np.float64)
    lse = np.zeros((B, T, H), np.float64)
    sk = _sink(sink, H)
    rc = lib().orc_sparse_attn(B, T, H, D, topk, window, scale, _p(sk), _p(q_pos), _p(q), _p(kv_cmp),
                               kv_cmp.shape[1], _p(idx), _p(kv_raw), kv_raw.shape[1],
                               _p(raw_base), dt, _p(out), _p(lse))
    assert rc == 0
    return out, lse


def hca_dense_attn(q, kv_cmp, kv_raw, m, window, q_pos, n_cmp, raw_base, scale=None, sink=None):
    """HCA attention: every visible compressed entry plus the raw window
    (sink as for sparse_attn)."""
    q, kv_cmp, kv_raw = _c(q), _c(kv_cmp), _c(kv_raw)
    B, T, H, D = q.shape
    dt = _dt(q)
    assert _dt(kv_cmp) == dt and _dt(kv_raw) == dt
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q_pos = _c(np.broadcast_to(np.asarray(q_pos, np.int64), (B,)), np.int64)
    n_cmp = _c(np.broadcast_to(np.asarray(n_cmp, np.int32), (B,)), np.int32)
    raw_base = _c(np.broadcast_to(np.asarray(raw_base, np.int64), (B,)), np.int64)
    out = np.zeros((B, T, H, D), np.float64)
    lse = np.zeros((B, T, H), np.float64)
    sk = _sink(sink, H)
    rc = lib().orc_hca_dense_attn(B, T, H, D, m, window, scale, _p(sk), _p(q_pos), _p(n_cmp), _p(q),
                                  _p(kv_cmp), kv_cmp.shape[1], _p(kv_raw), kv_raw.shape[1],
                                  _p(raw_base), dt, _p(out), _p(lse))
    assert rc == 0
    return out, lse


def attn_bwd(q, kv_cmp, idx, kv_raw, window, q_pos, raw_base, dout, scale=None, sink=None,
             m=None, n_cmp=None, want_mass=False):
    """Gradients of sparse_attn (idx given) or hca_dense_attn (idx None, with m
    and n_cmp) for an upstream gradient dout [B, T, H, D] of out.
    Returns (dq [B,T,H,D], dkv_cmp [B,Nc_cap,2D], dkv_raw [B,R_cap,2D],
    dsink [H] or None, attn_mass or None) in float64; attn_mass is the
    attention probability summed over heads per slot ([B,T,topk], CSA form)
    or per entry ([B,T,Nc_cap], HCA form: the dense indexer loss's target)."""
    q, kv_cmp, kv_raw = _c(q), _c(kv_cmp), _c(kv_raw)
    B, T, H, D = q.shape
    dt = _dt(q)
    assert _dt(kv_cmp) == dt and _dt(kv_raw) == dt
    dout = _c(dout, np.float64)
    assert dout.shape == (B, T, H, D)
    if idx is not None:
        idx = _c(idx, np.int32)
        topk = idx.shape[2]
        m_, ncp = 1, None
    else:
        topk = 0
        m_ = int(m)
        ncp = _c(np.broadcast_to(np.asarray(n_cmp, np.int32), (B,)), np.int32)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q_pos = _c(np.broadcast_to(np.asarray(q_pos, np.int64), (B,)), np.int64)
    raw_base = _c(np.broadcast_to(np.asarray(raw_base, np.int64), (B,)), np.int64)
    Nc_cap, R_cap = kv_cmp.shape[1], kv_raw.shape[1]
    dq = np.zeros((B, T, H, D), np.float64)
    dkc = np.zeros((B, Nc_cap, 2 * D), np.float64)
    dkr = np.zeros((B, R_cap, 2 * D), np.float64)
    sk = _sink(sink, H)
    dsink = np.zeros(H, np.float64) if sk is not None else None
    mass = None
    if want_mass:
        mass = np.zeros((B, T, topk if idx is not None else Nc_cap), np.float64)
    rc = lib().orc_attn_bwd(B, T, H, D, topk, window, scale, _p(sk), _p(q_pos), _p(q),
                            _p(kv_cmp), Nc_cap, _p(idx), m_, _p(ncp), _p(kv_raw), R_cap,
                            _p(raw_base), dt, _p(dout), _p(dq), _p(dkc), _p(dkr), _p(dsink),
                            _p(mass))
    assert rc == 0
    return dq, dkc, dkr, dsink, mass


def indexer_kl_dense_bwd(q_idx, w_idx, k_idx, m, q_pos, n_cmp, mass, grad_scale=None):
    """Dense indexer KL loss: the sparse form (indexer_kl_bwd) over every
    visible entry of each row - slots 0 .. n_vis - 1 in order, n_vis as for
    the indexer (m, q_pos, n_cmp) - with mass [B,T,Nc_cap] the dense
    attention's per-entry mass (attn_bwd's HCA form).  Returns (loss, dq_idx,
    dw_idx, dk_idx) in float64."""
    B, T = np.asarray(mass).shape[:2]
    Nc_cap = np.asarray(k_idx).shape[1]
    q_pos = np.broadcast_to(np.asarray(q_pos, np.int64), (B,))
    n_cmp = np.broadcast_to(np.asarray(n_cmp, np.int64), (B,))
    idx = np.full((B, T, Nc_cap), -1, np.int32)
    for b in range(B):
        for t in range(T):
            nv = min(int(q_pos[b] + t + 1) // int(m), int(n_cmp[b]), Nc_cap)
            idx[b, t, :nv] = np.arange(nv, dtype=np.int32)
    return indexer_kl_bwd(q_idx, w_idx, k_idx, idx, mass, grad_scale)


def indexer_kl_bwd(q_idx, w_idx, k_idx, idx, mass, grad_scale=None):
    """Sparse indexer KL loss per query row and its gradients (see the C
    file): q_idx [B,T,H_I,d_I], w_idx [B,T,H_I] fp32, k_idx [B,Nc_cap,d_I]
    (fp32 or bf16 bits), idx [B,T,topk], mass [B,T,topk] (attention mass per
    slot), grad_scale [B,T] or None (1).  Returns (loss [B,T], dq_idx, dw_idx,
    dk_idx) in float64."""
    q_idx, k_idx = _c(q_idx), _c(k_idx)
    w_idx = _c(w_idx, np.float32)
    idx = _c(idx, np.int32)
    mass = _c(mass, np.float64)
    B, T, H_I, d_I = q_idx.shape
    Nc_cap = k_idx.shape[1]
    topk = idx.shape[2]
    dt = _dt(q_idx)
    assert _dt(k_idx) == dt and dt in (DT_F32, DT_BF16)
    gs = None if grad_scale is None else _c(np.broadcast_to(np.asarray(grad_scale, np.float64),
                                                            (B, T)), np.float64)
    loss = np.zeros((B, T), np.float64)
    dq = np.zeros((B, T, H_I, d_I), np.float64)
    dw = np.zeros((B, T, H_I), np.float64)
    dk = np.zeros((B, Nc_cap, d_I), np.float64)
    rc = lib().orc_indexer_kl_bwd(B, T, H_I, d_I, Nc_cap, topk, _p(q_idx), _p(w_idx), _p(k_idx),
                                  dt, _p(idx), _p(mass), _p(gs), _p(loss), _p(dq), _p(dw), _p(dk))
    assert rc == 0
    return loss, dq, dw, dk


def compress_bwd(x, w_kv, w_gate, m, overlap, Nc_cap, dC, ape=None, rotate=False):
    """Gradients of a one-shot compress call from position 0 (no state) for
    an upstream gradient dC [B, Nc_cap, E] of its entries.  Returns (dx
    [B,L,d_model], dw_kv [E,d_model], dw_gate [E,d_model], dape or None)."""
    x, w_kv, w_gate = _c(x), _c(w_kv), _c(w_gate)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    dt = _dt(x)
    assert _dt(w_kv) == dt and _dt(w_gate) == dt
    dC = _c(dC, np.float64)
    assert dC.shape == (B, Nc_cap, E)
    ape = _c(ape, np.float64)
    dx = np.zeros((B, L, d_model), np.float64)
    dwk = np.zeros((E, d_model), np.float64)
    dwg = np.zeros((E, d_model), np.float64)
    dape = np.zeros(((1 + overlap) * m, E), np.float64) if ape is not None else None
    rc = lib().orc_compress_bwd(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(x), _p(w_kv),
                                _p(w_gate), dt, _p(ape), Nc_cap, _p(dC), _p(dx), _p(dwk),
                                _p(dwg), _p(dape))
    assert rc == 0
    return dx, dwk, dwg, dape


def compress_bwd_ex(x, w_kv, w_gate, m, overlap, Nc_cap, dC, ape=None, rotate=False,
                    norm_weight=None, norm_eps=1e-6, rope_dim=0, rope_offset=0,
                    rope_base=10000.0, rope_interleaved=False):
    """compress_bwd for entries post-processed as compress does with the same
    norm / rotary options.  Returns (dx, dw_kv, dw_gate, dape or None,
    dnorm_weight [E] or None)."""
    x, w_kv, w_gate = _c(x), _c(w_kv), _c(w_gate)
    B, L, d_model = x.shape
    E = w_kv.shape[0]
    dt = _dt(x)
    assert _dt(w_kv) == dt and _dt(w_gate) == dt
    dC = _c(dC, np.float64)
    assert dC.shape == (B, Nc_cap, E)
    ape = _c(ape, np.float64)
    dx = np.zeros((B, L, d_model), np.float64)
    dwk = np.zeros((E, d_model), np.float64)
    dwg = np.zeros((E, d_model), np.float64)
    dape = np.zeros(((1 + overlap) * m, E), np.float64) if ape is not None else None
    nw = _c(norm_weight, np.float64)
    dnw = np.zeros(E, np.float64) if nw is not None else None
    opts = _Opts(None if nw is None else nw.ctypes.data, float(norm_eps), int(rope_dim),
                 int(rope_offset), int(bool(rope_interleaved)), float(rope_base))
    rc = lib().orc_compress_bwd_ex(B, L, d_model, E, m, overlap, int(bool(rotate)), _p(x),
                                   _p(w_kv), _p(w_gate), dt, _p(ape), Nc_cap, _p(dC),
                                   C.byref(opts), _p(dx), _p(dwk), _p(dwg), _p(dape), _p(dnw))
    assert rc == 0
    return dx, dwk, dwg, dape, dnw
