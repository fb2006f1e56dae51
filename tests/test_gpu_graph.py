"""The decode step (indexer top-k on long rows, split-key sparse attention)
and a backward slice (attention backward of both forms with the mass, the
sparse and dense indexer losses) captured as HIP graphs and replayed give the
eager result on every replay.

bench.py times decode steps as graph replays; this checks that capture adds
nothing and drops nothing: all library launches are kernels (no memset), and
every buffer is preallocated.  Replays are separated by eager work and host
synchronisations, and each one is compared bit for bit with the eager run."""
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _paged(B, Nc, P, tensors):
    """Shuffled page table and pools of the given [B, Nc, ...] caches."""
    n = -(-Nc // P)
    table = torch.randperm(B * n, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    table = table.view(B, n).to(DEV)
    j = torch.arange(Nc, device=DEV)
    rows = (table[:, j // P].long() * P + j % P).reshape(-1)
    pools = []
    for t in tensors:
        feat = tuple(t.shape[2:]) or (1,)
        pool = torch.zeros((B * n * P,) + feat, dtype=t.dtype, device=DEV)
        pool.view(torch.uint8)[rows] = t.reshape((-1,) + feat).view(torch.uint8)
        pools.append(pool if t.dim() > 2 else pool.view(-1))
    return csa.PageTable(table, P, B * n, nc_cap=Nc), pools


@pytest.mark.parametrize("paged", [False, True])
def test_decode_step_graph_replays_match_eager(paged):
    d = gen.Draw(31, DEV)
    B, Nc, m, topk, W, H, D = 4, 20000, 4, 512, 64, 64, 128
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.FP8)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 1, 16, 64, gen.FP8)
    kv = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kvr = gen.store(d.normal(B, W, 2 * D), gen.BF16)
    q = gen.store(d.normal(B, 1, H, D), gen.BF16)
    ctx = [4 * Nc, 4 * Nc - 9, 4 * 15000 + 2, 4 * 3000]      # ragged visibility
    q_pos = torch.tensor([c - 1 for c in ctx], dtype=torch.int64, device=DEV)
    n_cmp = torch.tensor([Nc] * B, dtype=torch.int32, device=DEV)
    raw_base = torch.tensor([c - W for c in ctx], dtype=torch.int64, device=DEV)
    idx = torch.empty(B, 1, topk, dtype=torch.int32, device=DEV)
    out = torch.empty(B, 1, H, D, dtype=torch.bfloat16, device=DEV)
    ws_i = torch.empty(csa.csa_indexer_topk_workspace_size(B, 1, 16, 64, Nc, topk, torch.float8_e4m3fn),
                       dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(max(1, csa.csa_sparse_attn_workspace_size(B, 1, H, D, topk, W)),
                       dtype=torch.uint8, device=DEV)
    pages = None

    def step():
        csa.csa_indexer_topk(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale=q_scale,
                             k_scale=k_scale, idx_out=idx, workspace=ws_i, pages=pages)
        csa.csa_sparse_attn(q, kv, idx, kvr, W, q_pos, raw_base, out=out, workspace=ws_a,
                            pages=pages)

    step()
    torch.cuda.synchronize()
    ref_idx, ref_out = idx.clone(), out.clone()
    if paged:
        # the same step on paged caches: bit-exact with the unpaged one, and
        # captured and replayed below
        pages, (k_idx, k_scale, kv) = _paged(B, Nc, 64, (k_idx, k_scale, kv))
        ws_a = torch.empty(csa.lib().csa_sparse_attn_paged_workspace_size(B, 1, H, D, topk, W),
                           dtype=torch.uint8, device=DEV)
        step()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        idx.fill_(-7)
        out.fill_(float("nan"))
        ws_i.fill_(0xA5)                 # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), "replay %d: indices differ" % rep
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "replay %d" % rep
        step()                           # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx) and torch.equal(out.view(torch.int16), ref_out.view(torch.int16))


def test_backward_graph_replays_match_eager():
    # one training-step backward slice captured as a graph: the CSA attention
    # backward with the per-slot mass and the sparse indexer loss on it, the
    # HCA-form backward with the per-entry mass and the dense indexer loss on
    # it.  Everything is compared bit for bit except dk_idx, whose rows are
    # summed with fp32 atomics (order-dependent last bits).
    d = gen.Draw(33)
    B, T, H, D, Nc, R, W, m, topk = 1, 200, 64, 128, 300, 300, 64, 4, 64
    qp, rb = 100, 0
    q = gen.store(d.normal(B, T, H, D), gen.BF16).to(DEV)
    kv = gen.store(d.normal(B, Nc, 2 * D), gen.BF16).to(DEV)
    kvr = gen.store(d.normal(B, R, 2 * D), gen.BF16).to(DEV)
    dout = gen.store(d.normal(B, T, H, D), gen.BF16).to(DEV)
    qi = gen.store(d.normal(B, T, 16, 64), gen.BF16).to(DEV)
    wi = d.normal(B, T, 16).float().contiguous().to(DEV)
    ki = gen.store(d.normal(B, Nc, 64), gen.BF16).to(DEV)
    nv = torch.tensor([[min(Nc, (qp + t + 1) // m) for t in range(T)]])
    idx = gen.random_index_sets(d, B, T, topk, nv).to(DEV)
    q_pos = torch.tensor([qp], dtype=torch.int64, device=DEV)
    n_cmp = torch.tensor([Nc], dtype=torch.int32, device=DEV)
    raw_base = torch.tensor([rb], dtype=torch.int64, device=DEV)
    _, lse = csa.csa_sparse_attn(q, kv, idx, kvr, W, q_pos, raw_base, want_lse=True)
    _, lse_h = csa.hca_dense_attn(q, kv, kvr, m, W, q_pos, n_cmp, raw_base, want_lse=True)
    L = csa.lib()
    wsz = [L.csa_sparse_attn_bwd_workspace_size(B, T, H, Nc, R, W),
           L.csa_indexer_kl_bwd_workspace_size(B, T, Nc, topk),
           L.hca_dense_attn_bwd_workspace_size(B, T, H, Nc, R, W),
           L.csa_indexer_kl_dense_bwd_workspace_size(B, T, Nc)]
    ws = [torch.empty(n, dtype=torch.uint8, device=DEV) for n in wsz]
    # outputs allocated by one eager call, then reused
    a = csa.csa_sparse_attn_bwd(q, kv, idx, kvr, W, q_pos, raw_base, lse, dout, want_mass=True,
                                workspace=ws[0])
    k1 = csa.csa_indexer_kl_bwd(qi, wi, ki, idx, a[4], workspace=ws[1])
    h = csa.hca_dense_attn_bwd(q, kv, kvr, m, W, q_pos, n_cmp, raw_base, lse_h, dout,
                               want_mass=True, workspace=ws[2])
    k2 = csa.csa_indexer_kl_dense_bwd(qi, wi, ki, m, q_pos, n_cmp, h[4], workspace=ws[3])

    def step():
        csa.csa_sparse_attn_bwd(q, kv, idx, kvr, W, q_pos, raw_base, lse, dout, dq=a[0],
                                dkv_cmp=a[1], dkv_raw=a[2], attn_mass=a[4], workspace=ws[0])
        csa.csa_indexer_kl_bwd(qi, wi, ki, idx, a[4], loss=k1[0], dq_idx=k1[1], dw_idx=k1[2],
                               dk_idx=k1[3], workspace=ws[1])
        csa.hca_dense_attn_bwd(q, kv, kvr, m, W, q_pos, n_cmp, raw_base, lse_h, dout, dq=h[0],
                               dkv_cmp=h[1], dkv_raw=h[2], attn_mass=h[4], workspace=ws[2])
        csa.csa_indexer_kl_dense_bwd(qi, wi, ki, m, q_pos, n_cmp, h[4], loss=k2[0],
                                     dq_idx=k2[1], dw_idx=k2[2], dk_idx=k2[3], workspace=ws[3])

    exact = [a[0], a[1], a[2], a[4], k1[0], k1[1], k1[2], h[0], h[1], h[2], h[4], k2[0], k2[1],
             k2[2]]
    summed = [k1[3], k2[3]]
    step()
    torch.cuda.synchronize()
    ref_x = [t.clone() for t in exact]
    ref_s = [t.clone() for t in summed]

    def check(what):
        for i, (t, r) in enumerate(zip(exact, ref_x)):
            assert torch.equal(t.view(torch.int32), r.view(torch.int32)), "%s: output %d" % (what, i)
        for t, r in zip(summed, ref_s):
            err = (t - r).abs().amax(-1)
            assert (err <= 1e-5 * r.abs().amax(-1) + 1e-30).all(), what + ": dk_idx"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in exact + summed:
            t.fill_(float("nan"))
        for w in ws:
            w.fill_(0xA5)                # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check("replay %d" % rep)
        step()                           # eager work between replays
        torch.cuda.synchronize()
        check("eager after replay %d" % rep)
