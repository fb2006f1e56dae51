"""Benchmark of the compressed sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  * csa_prefill_8k_bf16 (the line's `value`): compress (main and indexer) ->
    indexer top-k -> sparse attention for 8192 tokens;
  * reported in the same line: csa_train_bwd_8k_bf16 ("train_bwd_8k": the
    backward of that step for training: attention gradients with the
    per-entry attention mass, the indexer KL loss and its gradients, both
    compressors' gradients), csa_decode_128k_b32 ("decode_128k": indexer
    top-k -> sparse attention for 32 sequences at 131072 tokens of context,
    caches resident in HBM), hca_prefill_1m_chunk4k ("hca_1m_chunk4k": dense
    compressed attention of a 4096-token chunk at 1M context) and
    csa_decode_1m_b8_stream ("decode_1m_stream": streaming compressor step,
    indexer top-k and sparse attention for 8 sequences at 1M context);
  * --workload selects any workload instead.
Timing uses HIP events on the stream the library launches on.  Every step
runs with the L2 and the 256 MB last-level cache flushed (a 1 GiB write)
before it, outside the timed events, so cache-resident reuse across steps
does not pass for HBM bandwidth.  Each record gives the mean, median and p90
step time.

The CPU baseline times the oracle (test infrastructure under oracle/) on a
bounded sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import compressed_sparse_attention_overlapped_amd as csa  # noqa: E402
from compressed_sparse_attention_overlapped_amd import inputs as gen  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3
DEV = "cuda"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the stored counter
    runs (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel calibration), or
    None when none is stored or the kernel's source changed since."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            entries = json.load(f)["entries"]
    except (OSError, ValueError, KeyError):
        return None
    for e in entries:
        if e.get("kernel") != kernel or e.get("workload") != workload:
            continue
        try:
            with open(os.path.join(ROOT, e["source"]), "rb") as f:
                digest = hashlib.sha256(f.read()).hexdigest()
        except OSError:
            return None
        return e["bytes_per_launch"] if digest == e.get("source_sha256") else None
    return None


def i64(v):
    return torch.tensor(np.asarray(v, np.int64).reshape(-1), dtype=torch.int64, device=DEV)


def i32(v):
    return torch.tensor(np.asarray(v, np.int32).reshape(-1), dtype=torch.int32, device=DEV)


def n_vis(t, ncmp, m):
    return min(ncmp, (t + 1) // m)


# ---------------------------------------------------------------- work counts

def csa_counts(w: gen.Workload, q_pos0: int, T: int, ncmp: int):
    """(indexer pairs, attention key visits) summed over query rows."""
    t = np.arange(q_pos0, q_pos0 + T, dtype=np.int64)
    nv = np.minimum(ncmp, (t + 1) // w.m)
    pairs = int(nv.sum())
    visits = int(np.minimum(w.topk, nv).sum() + np.minimum(w.window, t + 1).sum())
    return pairs, visits


def hca_visits(w: gen.Workload, q_pos0: int):
    t = np.arange(q_pos0, q_pos0 + w.T, dtype=np.int64)
    nv = np.minimum(w.n_cmp, (t + 1) // w.m)
    return int(nv.sum() + np.minimum(w.window, t + 1).sum())


# ---------------------------------------------------------------- timing

class Timer:
    """Per-stage HIP-event timing of one step on the current stream."""

    def __init__(self, names):
        self.names = names
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]

    def mark(self, i):
        self.ev[i].record()

    def stage_ms(self):
        return [self.ev[i].elapsed_time(self.ev[i + 1]) for i in range(len(self.names))]


def flush_caches(buf):
    buf.fill_(1.0)       # 1 GiB write: evicts L2 and the last-level cache


def run_steps(step_fn, names, steps, warmup, flush):
    buf = torch.empty(1 << 28, dtype=torch.float32, device=DEV) if flush else None
    for _ in range(warmup):
        if flush:
            flush_caches(buf)
        step_fn(Timer(names))
    torch.cuda.synchronize()
    timers = []
    wall0 = time.perf_counter()
    for _ in range(steps):
        if flush:
            flush_caches(buf)
        tm = Timer(names)
        step_fn(tm)
        timers.append(tm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = np.array([tm.stage_ms() for tm in timers])          # steps x stages
    step_ms = per.sum(axis=1)
    return {
        "step_ms_mean": float(step_ms.mean()),
        "step_ms_median": float(np.median(step_ms)),
        "step_ms_p90": float(np.percentile(step_ms, 90)),
        "stage_ms": {n: float(per[:, i].mean()) for i, n in enumerate(names)},
        "wall_s": wall,
    }


class NullTimer:
    def mark(self, i):
        pass


def run_graph(step_fn, steps, warmup, flush):
    """The step captured once as a HIP graph and replayed: per-launch host work
    leaves the timed region.  Every output and workspace is preallocated, and
    the library issues no memset, so the captured step is the eager step."""
    buf = torch.empty(1 << 28, dtype=torch.float32, device=DEV) if flush else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step_fn(NullTimer())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_fn(NullTimer())
    for _ in range(warmup):
        if flush:
            flush_caches(buf)
        g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        if flush:
            flush_caches(buf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        ms.append((e0, e1))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ms])
    del g
    return {"step_ms_mean": float(t.mean()), "step_ms_median": float(np.median(t)),
            "step_ms_p90": float(np.percentile(t, 90))}


# ---------------------------------------------------------------- workloads

def setup_prefill(w):
    inp = gen.prefill_inputs(w, device=DEV)
    B, S = w.B, w.T
    dt = gen.torch_dtype(w.dt)
    st = dict(inp)
    st["kv_cmp"] = torch.empty(B, w.n_cmp, 2 * w.D, device=DEV, dtype=dt)
    st["k_idx"] = torch.empty(B, w.n_cmp, w.d_I, device=DEV, dtype=dt)
    st["pos0"] = i64([0] * B)
    st["ncmp"] = i32([w.n_cmp] * B)
    st["raw_base"] = i64([0] * B)
    st["idx"] = torch.empty(B, S, w.topk, dtype=torch.int32, device=DEV)
    st["out"] = torch.empty(B, S, w.H, w.D, device=DEV, dtype=dt)
    st["ws_c1"] = torch.empty(max(1, csa.csa_compress_workspace_size(B, S, w.d_model, 2 * w.D, w.m, w.overlap, dt)), dtype=torch.uint8, device=DEV)
    st["ws_c2"] = torch.empty(max(1, csa.csa_compress_workspace_size(B, S, w.d_model, w.d_I, w.m, w.overlap, dt)), dtype=torch.uint8, device=DEV)
    st["ws_i"] = torch.empty(max(1, csa.csa_indexer_topk_workspace_size(B, S, w.H_I, w.d_I, w.n_cmp, w.topk, dt)), dtype=torch.uint8, device=DEV)
    st["ws_a"] = torch.empty(max(1, csa.csa_sparse_attn_workspace_size(B, S, w.H, w.D, w.topk, w.window)), dtype=torch.uint8, device=DEV)
    return st


def step_prefill(w, st):
    # The main compressor feeds only the attention, the indexer compressor only
    # the indexer: the main one runs on a second stream (default priority)
    # beside the indexer compressor and the indexer, joined before the
    # attention.  Stages on the step's stream: the indexer compressor; the
    # indexer, up to the join with the main compressor; the attention alone.
    side = st.setdefault("side_stream", torch.cuda.Stream())

    def fn(tm):
        cur = torch.cuda.current_stream()
        tm.mark(0)
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            csa.csa_compress(st["x"], st["w_kv"], st["w_gate"], st["pos0"], w.m, w.overlap,
                             st["kv_cmp"], workspace=st["ws_c1"])
        csa.csa_compress(st["x"], st["w_ikv"], st["w_igate"], st["pos0"], w.m, w.overlap,
                         st["k_idx"], workspace=st["ws_c2"])
        tm.mark(1)
        csa.csa_indexer_topk(st["q_idx"], st["w_idx"], st["k_idx"], w.m, w.topk, st["pos0"],
                             st["ncmp"], q_scale=st["q_scale"], idx_out=st["idx"],
                             workspace=st["ws_i"])
        cur.wait_stream(side)
        tm.mark(2)
        csa.csa_sparse_attn(st["q"], st["kv_cmp"], st["idx"], st["kv_raw"], w.window, st["pos0"],
                            st["raw_base"], out=st["out"], workspace=st["ws_a"])
        tm.mark(3)
    return fn, ["indexer_compress", "indexer_topk_and_main_compress", "sparse_attn"]


def setup_train_bwd(w):
    """The forward of the 8K prefill step once (untimed), through the
    library, then every buffer of its backward."""
    st = setup_prefill(w)
    B, S, dt = w.B, w.T, gen.torch_dtype(w.dt)
    d = gen.Draw(w.seed + 7, DEV)
    # each compressor's two weights (and their gradients below) in one
    # [2E, d_model] buffer, as a fused projection keeps them
    for wk, wg in (("w_kv", "w_gate"), ("w_ikv", "w_igate")):
        E = st[wk].shape[0]
        cat = torch.cat([st[wk], st[wg]]).contiguous()
        st[wk], st[wg] = cat[:E], cat[E:]
    csa.csa_compress(st["x"], st["w_kv"], st["w_gate"], st["pos0"], w.m, w.overlap, st["kv_cmp"],
                     workspace=st["ws_c1"])
    csa.csa_compress(st["x"], st["w_ikv"], st["w_igate"], st["pos0"], w.m, w.overlap, st["k_idx"],
                     workspace=st["ws_c2"])
    csa.csa_indexer_topk(st["q_idx"], st["w_idx"], st["k_idx"], w.m, w.topk, st["pos0"],
                         st["ncmp"], q_scale=st["q_scale"], idx_out=st["idx"], workspace=st["ws_i"])
    _, st["lse"] = csa.csa_sparse_attn(st["q"], st["kv_cmp"], st["idx"], st["kv_raw"], w.window,
                                       st["pos0"], st["raw_base"], out=st["out"], want_lse=True,
                                       workspace=st["ws_a"])
    st["dout"] = gen.store(d.normal(B, S, w.H, w.D), w.dt)
    f32 = dict(dtype=torch.float32, device=DEV)
    st["dq"] = torch.empty(B, S, w.H, w.D, **f32)
    st["dkv_cmp"] = torch.empty(B, w.n_cmp, 2 * w.D, **f32)
    st["dkv_raw"] = torch.empty(B, S, 2 * w.D, **f32)
    st["mass"] = torch.empty(B, S, w.topk, **f32)
    st["loss"] = torch.empty(B, S, **f32)
    st["dq_idx"] = torch.empty(B, S, w.H_I, w.d_I, **f32)
    st["dw_idx"] = torch.empty(B, S, w.H_I, **f32)
    st["dk_idx"] = torch.empty(B, w.n_cmp, w.d_I, **f32)
    for k, E in (("c1", 2 * w.D), ("c2", w.d_I)):
        st["dx_" + k] = torch.empty(B, S, w.d_model, **f32)
        dwcat = torch.empty(2 * E, w.d_model, **f32)
        st["dwk_" + k], st["dwg_" + k] = dwcat[:E], dwcat[E:]
        st["wsb_" + k] = torch.empty(csa.lib().csa_compress_bwd_workspace_size(B, S, w.d_model, E, w.m, w.n_cmp),
                                     dtype=torch.uint8, device=DEV)
    st["wsb_a"] = torch.empty(csa.lib().csa_sparse_attn_bwd_workspace_size(
        B, S, w.H, w.n_cmp, S, w.window), dtype=torch.uint8, device=DEV)
    st["wsb_i"] = torch.empty(csa.lib().csa_indexer_kl_bwd_workspace_size(B, S, w.n_cmp, w.topk),
                              dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    return st


def step_train_bwd(w, st):
    def fn(tm):
        tm.mark(0)
        csa.csa_sparse_attn_bwd(st["q"], st["kv_cmp"], st["idx"], st["kv_raw"], w.window,
                                st["pos0"], st["raw_base"], st["lse"], st["dout"], dq=st["dq"],
                                dkv_cmp=st["dkv_cmp"], dkv_raw=st["dkv_raw"],
                                attn_mass=st["mass"], workspace=st["wsb_a"])
        tm.mark(1)
        csa.csa_indexer_kl_bwd(st["q_idx"], st["w_idx"], st["k_idx"], st["idx"], st["mass"],
                               loss=st["loss"], dq_idx=st["dq_idx"], dw_idx=st["dw_idx"],
                               dk_idx=st["dk_idx"], workspace=st["wsb_i"])
        tm.mark(2)
        for k, wk, wg, dc in (("c1", "w_kv", "w_gate", "dkv_cmp"), ("c2", "w_ikv", "w_igate", "dk_idx")):
            csa.csa_compress_bwd(st["x"], st[wk], st[wg], w.m, w.overlap, w.n_cmp, st[dc],
                                 dx=st["dx_" + k], dw_kv=st["dwk_" + k], dw_gate=st["dwg_" + k],
                                 workspace=st["wsb_" + k])
        tm.mark(3)
    return fn, ["attn_bwd", "indexer_kl_bwd", "compress_bwd"]


def setup_decode(w):
    stream = w.d_model > 0
    # the streaming step emits the last entry itself
    inp = gen.decode_inputs(w, device=DEV)
    B = w.B
    st = dict(inp)
    T = w.ctx
    st["q_pos"] = i64([T - 1] * B)
    st["ncmp"] = i32([w.n_cmp] * B)
    st["raw_base"] = i64([T - w.window] * B)
    st["idx"] = torch.empty(B, 1, w.topk, dtype=torch.int32, device=DEV)
    st["out"] = torch.empty(B, 1, w.H, w.D, device=DEV, dtype=torch.bfloat16)
    st["ws_i"] = torch.empty(max(1, csa.csa_indexer_topk_workspace_size(B, 1, w.H_I, w.d_I, w.n_cmp, w.topk, torch.float8_e4m3fn)), dtype=torch.uint8, device=DEV)
    st["ws_a"] = torch.empty(max(1, csa.csa_sparse_attn_workspace_size(B, 1, w.H, w.D, w.topk, w.window)), dtype=torch.uint8, device=DEV)
    st["pages"] = None
    # the attention in two halves: the window half on a side stream beside
    # the compressors and the indexer, the selected half after top-k
    nb = csa.csa_sparse_attn_split_workspace_size(B, 1, w.H, w.D, w.topk, w.window)
    st["split"] = False
    st["can_split"] = nb > 0 and not w.page
    if st["can_split"]:
        st["ws_s"] = torch.empty(nb, dtype=torch.uint8, device=DEV)
        st["side"] = torch.cuda.Stream()
    if w.page:
        # paged compressed caches: every sequence's pages shuffled over one
        # pool (untimed setup); the step reads them through the block table
        P, n = w.page, -(-w.n_cmp // w.page)
        n_pages = B * n
        table = torch.randperm(n_pages, generator=torch.Generator().manual_seed(w.seed))
        table = table.to(torch.int32).view(B, n).to(DEV)
        j = torch.arange(w.n_cmp, device=DEV)
        rows = (table[:, j // P].long() * P + j % P).reshape(-1)
        for k in ("kv_cmp", "k_idx", "k_scale"):
            t = st[k]
            feat = tuple(t.shape[2:]) or (1,)
            pool = torch.empty((n_pages * P,) + feat, dtype=t.dtype, device=DEV)
            pool.view(torch.uint8)[rows] = t.reshape((-1,) + feat).view(torch.uint8)
            st[k] = pool if t.dim() > 2 else pool.view(-1)
            del t
        st["pages"] = csa.PageTable(table, P, n_pages, nc_cap=w.n_cmp)
        st["ws_a"] = torch.empty(csa.lib().csa_sparse_attn_paged_workspace_size(B, 1, w.H, w.D, w.topk, w.window), dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
    if stream:
        ns = 2 * w.m - 1
        for k, E in (("main", 2 * w.D), ("idx", w.d_I)):
            st["s0_" + k] = torch.empty(B, ns, 2, E, device=DEV)
            st["s1_" + k] = torch.empty(B, ns, 2, E, device=DEV)
            st["ws_" + k] = torch.empty(max(1, csa.csa_compress_workspace_size(B, w.tail, w.d_model, E, w.m, w.overlap, torch.bfloat16)), dtype=torch.uint8, device=DEV)
        # untimed: stream the 7-token tail (positions T-8 .. T-2) into the state
        p_tail = i64([T - 1 - w.tail] * B)
        csa.csa_compress(st["x_tail"], st["w_kv"], st["w_gate"], p_tail, w.m, w.overlap,
                         st["kv_cmp"], state_out=st["s0_main"], workspace=st["ws_main"])
        csa.csa_compress(st["x_tail"], st["w_ikv"], st["w_igate"], p_tail, w.m, w.overlap,
                         st["k_idx"], out_scale=st["k_scale"], state_out=st["s0_idx"],
                         workspace=st["ws_idx"])
        torch.cuda.synchronize()
    return st


def step_decode(w, st):
    stream = w.d_model > 0

    def fn(tm):
        tm.mark(0)
        i = 0
        main = torch.cuda.current_stream()
        if st["split"]:
            st["side"].wait_stream(main)
            with torch.cuda.stream(st["side"]):
                csa.csa_sparse_attn_window_half(st["q"], st["kv_raw"], w.window, st["q_pos"],
                                                st["raw_base"], w.topk, st["ws_s"])
        if stream:
            csa.csa_compress(st["x_new"], st["w_kv"], st["w_gate"], st["q_pos"], w.m, w.overlap,
                             st["kv_cmp"], state_in=st["s0_main"], state_out=st["s1_main"],
                             workspace=st["ws_main"])
            csa.csa_compress(st["x_new"], st["w_ikv"], st["w_igate"], st["q_pos"], w.m, w.overlap,
                             st["k_idx"], out_scale=st["k_scale"], state_in=st["s0_idx"],
                             state_out=st["s1_idx"], workspace=st["ws_idx"])
            i += 1
            tm.mark(i)
        csa.csa_indexer_topk(st["q_idx"], st["w_idx"], st["k_idx"], w.m, w.topk, st["q_pos"],
                             st["ncmp"], q_scale=st["q_scale"], k_scale=st["k_scale"],
                             idx_out=st["idx"], workspace=st["ws_i"], pages=st["pages"])
        i += 1
        tm.mark(i)
        if st["split"]:
            main.wait_stream(st["side"])
            csa.csa_sparse_attn_selected_half(st["q"], st["kv_cmp"], st["idx"], st["kv_raw"],
                                              w.window, st["q_pos"], st["raw_base"], st["ws_s"],
                                              out=st["out"])
        else:
            csa.csa_sparse_attn(st["q"], st["kv_cmp"], st["idx"], st["kv_raw"], w.window,
                                st["q_pos"], st["raw_base"], out=st["out"], workspace=st["ws_a"],
                                pages=st["pages"])
        i += 1
        tm.mark(i)
    names = (["compress"] if stream else []) + ["indexer_topk", "sparse_attn"]
    return fn, names


def setup_hca(w):
    st = gen.hca_inputs(w, device=DEV)
    q0 = w.ctx - w.T
    st["q_pos"] = i64([q0] * w.B)
    st["ncmp"] = i32([w.n_cmp] * w.B)
    st["raw_base"] = i64([q0 - w.window + 1] * w.B)
    st["out"] = torch.empty_like(st["q"])
    st["ws"] = torch.empty(max(1, csa.hca_dense_attn_workspace_size(w.B, w.T, w.H, w.D, w.n_cmp, w.window)), dtype=torch.uint8, device=DEV)
    return st


def step_hca(w, st):
    def fn(tm):
        tm.mark(0)
        csa.hca_dense_attn(st["q"], st["kv_cmp"], st["kv_raw"], w.m, w.window, st["q_pos"],
                           st["ncmp"], st["raw_base"], out=st["out"], workspace=st["ws"])
        tm.mark(1)
    return fn, ["hca_dense_attn"]


# ---------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s=12.0):
    """Time the oracle on a bounded sample of the workload on the host cores.

    The oracle parallelises over query rows (and over tokens inside the
    compressor), so samples are batched: 16 consecutive query rows per call
    for prefill, 8 sequences per call for decode."""
    from oracle import oracle as orc
    cores = orc.num_threads()
    rng = np.random.default_rng(0)
    d = gen.Draw(w.seed + 999)
    if w.kind == "csa_prefill":
        dm, S, blk = w.d_model, w.T, 16
        wk, wg = (gen.host_bits(t) for t in gen.compressor_weights(d, dm, 2 * w.D, w.dt))
        wik, wig = (gen.host_bits(t) for t in gen.compressor_weights(d, dm, w.d_I, w.dt))
        kv_cmp = gen.host_bits(gen.store(d.normal(1, w.n_cmp, 2 * w.D), w.dt))
        kv_raw = gen.host_bits(gen.store(d.normal(1, S, 2 * w.D), w.dt))
        k_idx = gen.host_bits(gen.store(d.normal(1, w.n_cmp, w.d_I), w.idx_dt))
        n_tok, tot = 0, 0.0
        while tot < budget_s:
            s0 = int(rng.integers(0, S - blk + 1))
            x = gen.host_bits(gen.store(d.normal(1, blk, dm), w.dt))
            q_idx = gen.host_bits(gen.store(d.normal(1, blk, w.H_I, w.d_I), w.idx_dt))
            w_idx = d.normal(1, blk, w.H_I).numpy()
            q = gen.host_bits(gen.store(d.normal(1, blk, w.H, w.D), w.dt))
            a = time.perf_counter()
            # the block's share of both compressors (blk / m entries each) ...
            orc.compress(x, wk, wg, w.m, w.overlap, s0, w.n_cmp, want_state=False)
            orc.compress(x, wik, wig, w.m, w.overlap, s0, w.n_cmp, want_state=False)
            # ... its indexer rows and attention rows
            idx = orc.indexer_topk(q_idx, w_idx, k_idx, w.m, w.topk, s0, w.n_cmp)[0]
            orc.sparse_attn(q, kv_cmp, idx, kv_raw, w.window, s0, 0)
            tot += time.perf_counter() - a
            n_tok += blk
        return {"value": n_tok / tot, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": "%d query tokens in blocks of %d consecutive positions drawn uniformly "
                          "from the %d-token prefill; per block both compressors over the block, "
                          "its indexer rows and its attention rows" % (n_tok, blk, S)}
    if w.kind == "csa_train_bwd":
        dm, S, blk = w.d_model, w.T, 16
        wk, wg = (gen.host_bits(t) for t in gen.compressor_weights(d, dm, 2 * w.D, w.dt))
        wik, wig = (gen.host_bits(t) for t in gen.compressor_weights(d, dm, w.d_I, w.dt))
        kv_cmp = gen.host_bits(gen.store(d.normal(1, w.n_cmp, 2 * w.D), w.dt))
        kv_raw = gen.host_bits(gen.store(d.normal(1, S, 2 * w.D), w.dt))
        k_idx = gen.host_bits(gen.store(d.normal(1, w.n_cmp, w.d_I), w.idx_dt))
        n_tok, tot = 0, 0.0
        while tot < budget_s:
            s0 = 4 * int(rng.integers(0, (S - blk) // 4 + 1))
            x = gen.host_bits(gen.store(d.normal(1, blk, dm), w.dt))
            q_idx = gen.host_bits(gen.store(d.normal(1, blk, w.H_I, w.d_I), w.idx_dt))
            w_idx = d.normal(1, blk, w.H_I).numpy()
            q = gen.host_bits(gen.store(d.normal(1, blk, w.H, w.D), w.dt))
            dout = d.normal(1, blk, w.H, w.D).double().numpy()
            nv = np.minimum((s0 + np.arange(blk) + 1) // w.m, w.n_cmp)
            idx = np.full((1, blk, w.topk), -1, np.int32)
            for r in range(blk):
                k = min(w.topk, int(nv[r]))
                idx[0, r, :k] = np.sort(rng.choice(int(nv[r]), k, replace=False))
            dc1 = d.normal(1, blk // w.m, 2 * w.D).double().numpy()
            dc2 = d.normal(1, blk // w.m, w.d_I).double().numpy()
            a = time.perf_counter()
            # the block's attention rows, their indexer loss rows, and both
            # compressors over the block's tokens
            _, _, _, _, mass = orc.attn_bwd(q, kv_cmp, idx, kv_raw, w.window, s0, 0, dout,
                                            want_mass=True)
            orc.indexer_kl_bwd(q_idx, w_idx, k_idx, idx, mass)
            orc.compress_bwd(x, wk, wg, w.m, w.overlap, blk // w.m, dc1)
            orc.compress_bwd(x, wik, wig, w.m, w.overlap, blk // w.m, dc2)
            tot += time.perf_counter() - a
            n_tok += blk
        return {"value": n_tok / tot, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": "%d tokens in blocks of %d consecutive positions drawn uniformly from "
                          "the %d-token chunk; per block the attention backward of its rows, their "
                          "indexer KL loss and gradients, and both compressors' backward over "
                          "the block" % (n_tok, blk, S)}
    if w.kind == "csa_decode":
        Bs = 8
        Ns = min(w.n_cmp, 65536)
        k_idx, k_scale = gen.indexer_keys(d, Bs, w.n_cmp, w.d_I, w.idx_dt)
        q_idx, q_scale, w_idx = gen.indexer_query(d, Bs, 1, w.H_I, w.d_I, w.idx_dt)
        kv_cmp = gen.host_bits(gen.store(d.normal(Bs, Ns, 2 * w.D), w.dt))
        kv_raw = gen.host_bits(gen.store(d.normal(Bs, w.window, 2 * w.D), w.dt))
        q = gen.host_bits(gen.store(d.normal(Bs, 1, w.H, w.D), w.dt))
        kb, ks = gen.host_bits(k_idx), gen.host_bits(k_scale)
        qb, qs, wb = gen.host_bits(q_idx), gen.host_bits(q_scale), w_idx.numpy()
        n_q, tot = 0, 0.0
        while tot < budget_s:
            a = time.perf_counter()
            idx = orc.indexer_topk(qb, wb, kb, w.m, w.topk, w.ctx - 1, w.n_cmp, q_scale=qs,
                                   k_scale=ks, fmt="mxfp4" if w.idx_dt == gen.MXFP4 else None)[0]
            idx = np.where(idx >= Ns, idx % Ns, idx)
            orc.sparse_attn(q, kv_cmp, idx, kv_raw, w.window, w.ctx - 1, w.ctx - w.window)
            tot += time.perf_counter() - a
            n_q += Bs
        return {"value": n_q / tot, "unit": "queries/s", "cores": cores, "kind": "oracle",
                "sample": "%d decode queries, %d sequences per oracle call: indexer over all %d "
                          "entries, top-%d, attention over %d keys (the selected rows are read "
                          "from a %d-entry cache sample)" % (n_q, Bs, w.n_cmp, w.topk,
                                                             w.topk + w.window, Ns)}
    if w.kind == "hca_prefill":
        kv_cmp = gen.host_bits(gen.store(d.normal(1, w.n_cmp, 2 * w.D), w.dt))
        kv_raw = gen.host_bits(gen.store(d.normal(1, w.T + w.window - 1, 2 * w.D), w.dt))
        q0 = w.ctx - w.T
        n_tok, tot, Ts = 0, 0.0, 16
        while tot < budget_s:
            t = int(rng.integers(0, w.T - Ts))
            q = gen.host_bits(gen.store(d.normal(1, Ts, w.H, w.D), w.dt))
            a = time.perf_counter()
            orc.hca_dense_attn(q, kv_cmp, kv_raw, w.m, w.window, q0 + t, w.n_cmp, q0 - w.window + 1)
            tot += time.perf_counter() - a
            n_tok += Ts
        return {"value": n_tok / tot, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": "%d query tokens of the %d-token chunk, %d consecutive per oracle call"
                          % (n_tok, w.T, Ts)}
    return None


# ---------------------------------------------------------------- driver

def measure(name, steps, warmup, with_cpu, graph=True):
    w = gen.WORKLOADS[name]
    flush = True   # every workload: L2 and the last-level cache flushed before each step
    if w.kind == "csa_prefill":
        st = setup_prefill(w)
        fn, names = step_prefill(w, st)
        pairs, visits = csa_counts(w, 0, w.T, w.n_cmp)
        attn_flops = visits * w.H * w.D * 4
        idx_flops = pairs * w.H_I * w.d_I * 2
        comp_flops = 2 * w.B * w.T * w.d_model * 2 * (2 * w.D + w.d_I)
        unit_items, unit = w.B * w.T, "tokens/s"
    elif w.kind == "csa_train_bwd":
        st = setup_train_bwd(w)
        fn, names = step_train_bwd(w, st)
        pairs, visits = csa_counts(w, 0, w.T, w.n_cmp)
        sel = int(np.minimum(w.topk, np.minimum(w.n_cmp, (np.arange(w.T) + 1) // w.m)).sum())
        # S (recomputed), dP, dQ, dK, dV per key visit; the indexer loss: the
        # scores twice, dq and dk; each compressor: the projection recomputed,
        # dx and dW
        attn_flops = visits * w.H * w.D * 2 * 5
        idx_flops = sel * w.H_I * w.d_I * 2 * 4
        comp_flops = 3 * 2 * w.B * w.T * w.d_model * 2 * (2 * w.D + w.d_I)
        unit_items, unit = w.B * w.T, "tokens/s"
    elif w.kind == "csa_decode":
        st = setup_decode(w)
        fn, names = step_decode(w, st)
        unit_items, unit = w.B, "queries/s"
    else:
        st = setup_hca(w)
        fn, names = step_hca(w, st)
        unit_items, unit = w.B * w.T, "tokens/s"
    r = run_steps(fn, names, steps, warmup, flush)
    step_s = r["step_ms_mean"] / 1e3
    res = {"workload": name, "value": unit_items / step_s, "unit": unit,
           "ms_per_step": r["step_ms_mean"], "ms_median": r["step_ms_median"],
           "ms_p90": r["step_ms_p90"], "stage_ms": r["stage_ms"],
           "cache": "L2 + last-level cache flushed before every step (outside the timed events)"}
    if w.kind == "csa_decode" and st["can_split"]:
        # the attention in two halves, the window half on a side stream beside
        # the indexer, timed for comparison (on this stack the join of the two
        # streams costs more than the overlap saves)
        st["split"] = True
        res["ms_per_step_split"] = run_steps(fn, names, steps, warmup, flush)["step_ms_mean"]
        st["split"] = False
    if w.kind == "csa_decode" and graph:
        # the same step captured as a HIP graph and replayed, for comparison
        # (on this stack the replay is not faster than the eager launches)
        gr = run_graph(fn, steps, warmup, flush)
        res["ms_per_step_graph"] = gr["step_ms_mean"]
    sm = r["stage_ms"]
    if w.kind == "csa_prefill":
        if w.dt == gen.BF16:
            ach = attn_flops / (sm["sparse_attn"] / 1e3) / 1e12
            res["roofline"] = {"bound": "mfma", "kernel": "attn_pf_kernel",
                               "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                               "traffic": measured_traffic("attn_pf_kernel", name)}
        else:
            ach = attn_flops / (sm["sparse_attn"] / 1e3) / 1e12
            res["roofline"] = {"bound": "alu", "kernel": "attn_f32_kernel", "achieved": ach,
                               "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": ach / FP32_VECTOR_PEAK_TFLOPS, "traffic": None}
        res["work"] = {"attn_gflop": attn_flops / 1e9, "indexer_gflop": idx_flops / 1e9,
                       "compress_gflop": comp_flops / 1e9,
                       "step_mfma_frac": (attn_flops + idx_flops + comp_flops) / step_s / 1e12
                       / MFMA_BF16_PEAK_TFLOPS}
    elif w.kind == "csa_train_bwd":
        ach = attn_flops / (sm["attn_bwd"] / 1e3) / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": "attention backward (attn_bwd_dq_kernel + "
                           "attn_bwd_dkv_kernel)", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                           "traffic": measured_traffic("attn_bwd", name)}
        res["work"] = {"attn_bwd_gflop": attn_flops / 1e9, "indexer_kl_gflop": idx_flops / 1e9,
                       "compress_bwd_gflop": comp_flops / 1e9,
                       "step_mfma_frac": (attn_flops + idx_flops + comp_flops) / step_s / 1e12
                       / MFMA_BF16_PEAK_TFLOPS}
    elif w.kind == "csa_decode":
        B, Nc = w.B, w.n_cmp
        # per entry: e4m3 codes + an fp32 scale, or MXFP4 codes + E8M0 block scales
        key_bytes = B * Nc * ((w.d_I // 2 + w.d_I // 32) if w.idx_dt == gen.MXFP4 else (w.d_I + 4))
        gather = B * (w.topk + w.window) * 4 * w.D
        small = B * (2 * w.H * w.D * 2 + 2 * w.topk * 4 + w.H_I * w.d_I + w.H_I * 8)
        total = key_bytes + gather + small
        if w.d_model:
            total += 2 * (2 * w.D + w.d_I) * w.d_model * 2       # compressor weights (bf16)
            total += B * (w.d_model * 2 + 2 * 7 * 2 * (2 * w.D + w.d_I) * 4)
        ach = key_bytes / (sm["indexer_topk"] / 1e3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "indexer_topk (score_fp8_kernel + select)",
                           "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS,
                           "traffic": measured_traffic("indexer_topk", name)}
        res["work"] = {"step_bytes": total, "indexer_key_bytes": key_bytes,
                       "attn_gather_bytes": gather,
                       "step_hbm_frac": total / step_s / 1e9 / HBM_PEAK_GBS,
                       "attn_gbs": gather / (sm["sparse_attn"] / 1e3) / 1e9}
    else:
        visits = hca_visits(w, w.ctx - w.T)
        flops = visits * w.H * w.D * 4
        ach = flops / step_s / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": "attn_pf_kernel (dense)", "achieved": ach,
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                           "traffic": measured_traffic("attn_pf_kernel", name)}
        res["work"] = {"attn_gflop": flops / 1e9}
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
        if res["cpu_baseline"] is not None:
            res["cpu_baseline"]["cpu_model"] = cpu_model()
    del st
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device to device three times (the reference "
                         "kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the path shards by sequence across "
              "GPUs by design, but no multi-GPU run is implemented); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device=DEV)
        dst = torch.empty_like(src)
        flush = torch.empty(1 << 28, dtype=torch.float32, device=DEV)
        for _ in range(3):
            flush_caches(flush)
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return
    csa.lib()
    if args.workload == "all":
        for name in gen.WORKLOADS:
            r = measure(name, args.steps, args.warmup, not args.no_cpu)
            print(json.dumps(r), flush=True)
        return
    if args.workload != "default":
        print(json.dumps(measure(args.workload, args.steps, args.warmup, not args.no_cpu)), flush=True)
        return
    prim = measure("csa_prefill_8k_bf16", args.steps, args.warmup, not args.no_cpu)
    sub = {}
    for key, wl, graph in (("train_bwd_8k", "csa_train_bwd_8k_bf16", False),
                           ("decode_128k", "csa_decode_128k_b32", True),
                           ("hca_1m_chunk4k", "hca_prefill_1m_chunk4k", False),
                           ("decode_1m_stream", "csa_decode_1m_b8_stream", False)):
        r = measure(wl, args.steps, args.warmup, not args.no_cpu, graph=graph)
        sub[key] = {k: r[k] for k in ("workload", "value", "unit", "ms_per_step", "ms_median",
                                      "ms_p90", "stage_ms", "roofline", "work", "cache")
                    if k in r}
        for k in ("ms_per_step_graph", "ms_per_step_split"):
            if k in r:
                sub[key][k] = r[k]
        sub[key]["cpu_baseline"] = r.get("cpu_baseline")
    line = {
        "metric": "CSA prefill tokens/s + decode queries/s at 128K ctx; % of HBM/MFMA peak",
        "value": prim["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": prim["ms_per_step"],
        "ms_median": prim["ms_median"], "ms_p90": prim["ms_p90"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "csa_prefill_8k_bf16", "batch": 1, "seq_len": 8192,
                   "d_model": 4096, "m": 4, "overlap": 1, "heads": 64, "head_dim": 128,
                   "indexer": "16x64 bf16", "topk": 512, "window": 512, "parallelism": "none"},
        "roofline": prim["roofline"],
        "cpu_baseline": prim.get("cpu_baseline"),
        "stage_ms": prim["stage_ms"], "work": prim["work"], "cache": prim["cache"],
    }
    line.update(sub)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
