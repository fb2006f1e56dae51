"""Seeded synthetic inputs for the compressed sparse attention path.

This module holds no step of the method: it only draws random tensors, puts
them in their storage formats (fp32, bf16, OCP e4m3 codes with per-row
scales) and describes the workload shapes.  Both the GPU path's tests and the
CPU oracle consume what it produces.

Recipe: ``torch.Generator`` seeded with ``1000 + config number`` (or the
seed a test passes), tensors drawn in the order listed by each builder.
Weights are N(0, 1/fan_in); activations, caches and indexer head weights are
N(0, 1).  bf16 storage uses torch's round-to-nearest-even conversion; e4m3
storage divides each row by ``amax / 448`` and converts with torch's
``float8_e4m3fn`` cast.  MXFP4 storage (OCP: E2M1 codes two per byte, one
E8M0 exponent per 32 values) is drawn directly: code bytes uniform over
0..255 and block exponents uniform over -3..3 (E8M0 bytes 124..130).  Small inputs are drawn on the CPU (identical on
every machine); the multi-GiB decode caches are drawn on the device they are
used on, and the checks copy the sampled rows back to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

F32, BF16, FP8, MXFP4 = "f32", "bf16", "fp8", "mxfp4"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload (sizes as the pages' DeepSeek-V4 shapes)."""
    name: str
    kind: str            # "csa_prefill" | "csa_train_bwd" | "csa_decode" | "hca_prefill"
    B: int
    ctx: int             # tokens of context per sequence
    T: int               # query tokens per sequence in the call
    H: int               # query heads (one shared KV head)
    D: int               # head dim
    m: int               # compression ratio
    overlap: int         # 1: windows of 2m tokens, 0: m tokens
    window: int          # sliding window W over raw KV
    topk: int = 0
    H_I: int = 0         # indexer heads
    d_I: int = 0         # indexer head dim
    d_model: int = 0     # compressor input width (0: caches are given)
    dt: str = BF16       # q / kv / compressor storage
    idx_dt: str = BF16   # indexer q / k storage
    tail: int = 0        # tokens streamed into the compressor state before the step
    n_cmp: int = 0       # compressed entries held in the cache for the step
    seed: int = 1000
    page: int = 0        # paged compressed caches: entries per page (0: unpaged)


WORKLOADS = {
    # tiny CSA prefill, everything fp32
    "csa_prefill_tiny_f32": Workload("csa_prefill_tiny_f32", "csa_prefill", B=1, ctx=256, T=256,
                                     H=8, D=64, m=4, overlap=1, window=32, topk=16, H_I=4,
                                     d_I=32, d_model=256, dt=F32, idx_dt=F32, n_cmp=64, seed=1001),
    # CSA prefill 8K, bf16
    "csa_prefill_8k_bf16": Workload("csa_prefill_8k_bf16", "csa_prefill", B=1, ctx=8192, T=8192,
                                    H=64, D=128, m=4, overlap=1, window=512, topk=512, H_I=16,
                                    d_I=64, d_model=4096, dt=BF16, idx_dt=BF16, n_cmp=2048, seed=1002),
    # the backward of the 8K bf16 prefill step (training): attention
    # gradients, the indexer KL loss and its gradients, both compressors'
    # gradients; the forward shapes above
    "csa_train_bwd_8k_bf16": Workload("csa_train_bwd_8k_bf16", "csa_train_bwd", B=1, ctx=8192,
                                      T=8192, H=64, D=128, m=4, overlap=1, window=512, topk=512,
                                      H_I=16, d_I=64, d_model=4096, dt=BF16, idx_dt=BF16,
                                      n_cmp=2048, seed=1007),
    # CSA decode at 128K context, batch 32, fp8 indexer
    "csa_decode_128k_b32": Workload("csa_decode_128k_b32", "csa_decode", B=32, ctx=131072, T=1,
                                    H=64, D=128, m=4, overlap=1, window=512, topk=2048, H_I=16,
                                    d_I=64, dt=BF16, idx_dt=FP8, n_cmp=32768, seed=1003),
    # the same decode with MXFP4 indexer keys and queries (FP4 indexer)
    "csa_decode_128k_b32_mxfp4": Workload("csa_decode_128k_b32_mxfp4", "csa_decode", B=32,
                                          ctx=131072, T=1, H=64, D=128, m=4, overlap=1,
                                          window=512, topk=2048, H_I=16, d_I=64, dt=BF16,
                                          idx_dt=MXFP4, n_cmp=32768, seed=1006),
    # the e4m3 128K decode with paged compressed caches (256-entry pages,
    # shuffled over the pool)
    "csa_decode_128k_b32_paged": Workload("csa_decode_128k_b32_paged", "csa_decode", B=32,
                                          ctx=131072, T=1, H=64, D=128, m=4, overlap=1,
                                          window=512, topk=2048, H_I=16, d_I=64, dt=BF16,
                                          idx_dt=FP8, n_cmp=32768, seed=1003, page=256),
    # HCA prefill chunk of 4096 tokens at the tail of a 1M context
    "hca_prefill_1m_chunk4k": Workload("hca_prefill_1m_chunk4k", "hca_prefill", B=1, ctx=1 << 20,
                                       T=4096, H=64, D=128, m=128, overlap=0, window=512,
                                       dt=BF16, n_cmp=8192, seed=1004),
    # CSA decode at 1M context, batch 8, fp8 indexer, streaming compressor update
    "csa_decode_1m_b8_stream": Workload("csa_decode_1m_b8_stream", "csa_decode", B=8, ctx=1 << 20,
                                        T=1, H=64, D=128, m=4, overlap=1, window=512, topk=2048,
                                        H_I=16, d_I=64, d_model=4096, dt=BF16, idx_dt=FP8,
                                        tail=7, n_cmp=262144, seed=1005),
}


def torch_dtype(fmt: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.float8_e4m3fn,
            MXFP4: torch.float4_e2m1fn_x2}[fmt]


class Draw:
    """A seeded stream of N(0, sigma^2) tensors."""

    def __init__(self, seed: int, device="cpu"):
        self.device = torch.device(device)
        self.g = torch.Generator(device=self.device)
        self.g.manual_seed(seed)

    def normal(self, *shape, std: float = 1.0) -> torch.Tensor:
        t = torch.randn(*shape, generator=self.g, device=self.device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t

    def ints(self, lo: int, hi: int, *shape) -> torch.Tensor:
        return torch.randint(lo, hi, shape, generator=self.g, device=self.device)


def store(t: torch.Tensor, fmt: str) -> torch.Tensor:
    """fp32 values -> storage format (fp32 or bf16; e4m3 goes through store_fp8)."""
    if fmt == F32:
        return t.float().contiguous()
    if fmt == BF16:
        return t.to(torch.bfloat16).contiguous()
    raise ValueError(fmt)


def store_fp8(t: torch.Tensor):
    """Per-row e4m3 storage: scale = amax(row) / 448 (1 for a zero row).

    Returns (codes as float8_e4m3fn, scales float32 of shape t.shape[:-1])."""
    t = t.float()
    amax = t.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (t / scale.unsqueeze(-1)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.contiguous(), scale.contiguous()


def host_bits(t: torch.Tensor):
    """A tensor's stored bits as a numpy array: float32, uint16 (bf16) or uint8 (e4m3)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.float8_e4m3fn, torch.float4_e2m1fn_x2, torch.float8_e8m0fnu,
                   torch.uint8):
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    raise TypeError(t.dtype)


# --------------------------------------------------------------------------
# stage inputs


def compressor_weights(d: Draw, d_model: int, E: int, fmt: str):
    """w_kv, w_gate in [E, d_model] (output-major) layout, N(0, 1/d_model)."""
    std = 1.0 / math.sqrt(d_model)
    w_kv = store(d.normal(E, d_model, std=std), fmt)
    w_gate = store(d.normal(E, d_model, std=std), fmt)
    return w_kv, w_gate


def mxfp4_random(d: Draw, *shape_n):
    """Random MXFP4 rows of n values (n a multiple of 32): (codes as
    float4_e2m1fn_x2 [..., n / 2], E8M0 scale bytes uint8 [..., n / 32])."""
    *lead, n = shape_n
    codes = d.ints(0, 256, *lead, n // 2).to(torch.uint8).view(torch.float4_e2m1fn_x2)
    scales = d.ints(124, 131, *lead, n // 32).to(torch.uint8)
    return codes.contiguous(), scales.contiguous()


def indexer_query(d: Draw, B: int, T: int, H_I: int, d_I: int, fmt: str):
    """q_idx [B,T,H_I,d_I] (+ per-(t,h) scales when e4m3; MXFP4: codes
    [B,T,H_I,d_I/2] and E8M0 block scales [B,T,H_I,d_I/32]) and w_idx [B,T,H_I]."""
    if fmt == MXFP4:
        q_idx, q_scale = mxfp4_random(d, B, T, H_I, d_I)
        return q_idx, q_scale, d.normal(B, T, H_I)
    q = d.normal(B, T, H_I, d_I)
    if fmt == FP8:
        q_idx, q_scale = store_fp8(q)
    else:
        q_idx, q_scale = store(q, fmt), None
    w_idx = d.normal(B, T, H_I)
    return q_idx, q_scale, w_idx


def indexer_keys(d: Draw, B: int, Nc: int, d_I: int, fmt: str):
    if fmt == MXFP4:
        return mxfp4_random(d, B, Nc, d_I)
    k = d.normal(B, Nc, d_I)
    if fmt == FP8:
        return store_fp8(k)
    return store(k, fmt), None


def prefill_inputs(w: Workload, device="cpu", seed: Optional[int] = None):
    """All inputs of a CSA prefill step, in the documented draw order:
    x, w_kv, w_gate, w_ikv, w_igate, q, kv_raw, q_idx(+scale), w_idx."""
    d = Draw(w.seed if seed is None else seed, device)
    B, S = w.B, w.T
    x = store(d.normal(B, S, w.d_model), w.dt)
    w_kv, w_gate = compressor_weights(d, w.d_model, 2 * w.D, w.dt)
    w_ikv, w_igate = compressor_weights(d, w.d_model, w.d_I, w.dt)
    q = store(d.normal(B, S, w.H, w.D), w.dt)
    kv_raw = store(d.normal(B, S, 2 * w.D), w.dt)
    q_idx, q_scale, w_idx = indexer_query(d, B, S, w.H_I, w.d_I, w.idx_dt)
    return dict(x=x, w_kv=w_kv, w_gate=w_gate, w_ikv=w_ikv, w_igate=w_igate, q=q,
                kv_raw=kv_raw, q_idx=q_idx, q_scale=q_scale, w_idx=w_idx)


def decode_inputs(w: Workload, device="cpu", seed: Optional[int] = None, n_cmp: Optional[int] = None):
    """Inputs of a CSA decode step with precomputed caches, draw order:
    kv_cmp, k_idx(+scale), kv_raw, q, q_idx(+scale), w_idx, then (streaming
    workloads) w_kv, w_gate, w_ikv, w_igate, x_tail, x_new.

    The query is the last context token (position ctx - 1); kv_raw holds the
    last ``window`` tokens.  For a streaming workload the caches hold entries
    [0, ctx/m - 1) and the step itself emits the last one."""
    d = Draw(w.seed if seed is None else seed, device)
    B, Nc = w.B, (w.n_cmp if n_cmp is None else n_cmp)
    kv_cmp = store(d.normal(B, Nc, 2 * w.D), w.dt)
    k_idx, k_scale = indexer_keys(d, B, Nc, w.d_I, w.idx_dt)
    kv_raw = store(d.normal(B, w.window, 2 * w.D), w.dt)
    q = store(d.normal(B, 1, w.H, w.D), w.dt)
    q_idx, q_scale, w_idx = indexer_query(d, B, 1, w.H_I, w.d_I, w.idx_dt)
    out = dict(kv_cmp=kv_cmp, k_idx=k_idx, k_scale=k_scale, kv_raw=kv_raw, q=q,
               q_idx=q_idx, q_scale=q_scale, w_idx=w_idx)
    if w.d_model:
        w_kv, w_gate = compressor_weights(d, w.d_model, 2 * w.D, w.dt)
        w_ikv, w_igate = compressor_weights(d, w.d_model, w.d_I, w.dt)
        out.update(w_kv=w_kv, w_gate=w_gate, w_ikv=w_ikv, w_igate=w_igate,
                   x_tail=store(d.normal(B, w.tail, w.d_model), w.dt),
                   x_new=store(d.normal(B, 1, w.d_model), w.dt))
    return out


def hca_inputs(w: Workload, device="cpu", seed: Optional[int] = None):
    """HCA prefill chunk: kv_cmp [B, ctx/m, 2D], q [B, T, H, D] for the last T
    tokens, kv_raw covering [ctx - T - W + 1, ctx) (draw order kv_cmp, q, kv_raw)."""
    d = Draw(w.seed if seed is None else seed, device)
    B = w.B
    kv_cmp = store(d.normal(B, w.n_cmp, 2 * w.D), w.dt)
    q = store(d.normal(B, w.T, w.H, w.D), w.dt)
    R = w.T + w.window - 1
    kv_raw = store(d.normal(B, R, 2 * w.D), w.dt)
    return dict(kv_cmp=kv_cmp, q=q, kv_raw=kv_raw)


def random_index_sets(d: Draw, B: int, T: int, topk: int, n_vis, pad_frac: float = 0.0):
    """Per-row random distinct indices in [0, n_vis[b, t]) (ascending, -1 padded).

    n_vis: int tensor [B, T].  pad_frac drops that fraction of each row's
    slots to -1 (tests of padded rows)."""
    idx = torch.full((B, T, topk), -1, dtype=torch.int32)
    for b in range(B):
        for t in range(T):
            n = int(n_vis[b, t])
            k = min(topk, n)
            if k <= 0:
                continue
            perm = torch.randperm(n, generator=d.g if d.device.type == "cpu" else None)[:k]
            if pad_frac > 0:
                keep = int(round(k * (1 - pad_frac)))
                perm = perm[:keep]
            idx[b, t, :perm.numel()] = perm.sort().values.to(torch.int32)
    return idx
