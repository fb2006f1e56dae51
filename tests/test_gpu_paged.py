"""GPU parity of the paged compressed caches.  Each paged call is checked
against the same call on the unpaged layout, bit for bit (the kernels do the
same arithmetic on rows found through the block table), and against the
oracle on the logical caches."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import dev_i32, dev_i64
from tests.test_gpu_attn import _check as attn_check, _n_vis, _rand_idx
from tests.test_gpu_indexer import _compare, _oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pages(B, nc_cap, P, seed, spare=3):
    """A shuffled block table over a pool with a few spare pages."""
    max_pages = -(-nc_cap // P)
    n_pages = B * max_pages + spare
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(n_pages, generator=g)[:B * max_pages].to(torch.int32)
    table = table.view(B, max_pages)
    return csa.PageTable(table.to(DEV), P, n_pages, nc_cap=nc_cap), table


def _rows(table, P, nc_cap):
    """Pool row of every logical entry, [B, nc_cap]."""
    j = torch.arange(nc_cap)
    return table[:, j // P].long() * P + j % P


def _bytes(t):
    x = t.detach().cpu()
    if x.dim() == 2:
        x = x.unsqueeze(-1)
    return x.contiguous().view(torch.uint8)


def _to_pool(t, rows, n_rows, fill=0):
    """Logical [B, Nc, ...] to a pool [n_rows, ...]; unmapped rows hold `fill` bytes."""
    xb = _bytes(t)
    pool = torch.full((n_rows, xb.shape[-1]), fill, dtype=torch.uint8)
    pool[rows.reshape(-1)] = xb.reshape(-1, xb.shape[-1])
    pool = pool.view(t.dtype)
    return (pool.squeeze(-1) if t.dim() == 2 else pool).to(DEV)


def _same_bits(a, b, what):
    assert torch.equal(_bytes(a), _bytes(b)), what


@pytest.mark.parametrize("fmt", [gen.BF16, gen.FP8, gen.MXFP4])
@pytest.mark.parametrize("P", [16, 256])
@pytest.mark.parametrize("Nc,T", [(3000, 3), (20000, 1)])
def test_paged_indexer_matches_unpaged_and_oracle(fmt, P, Nc, T):
    d = gen.Draw(40 + P + T, "cpu")
    B, m, topk = 3, 4, 300
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, fmt)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, T, 16, 64, fmt)
    q_pos = [4 * Nc, 4 * (Nc // 3) + 1, 4 * 200]
    n_cmp = [Nc, Nc - 9, Nc]
    args = (dev_i64(q_pos), dev_i32(n_cmp))
    dev = lambda t: None if t is None else t.to(DEV)
    iu, su = csa.csa_indexer_topk(q_idx.to(DEV), w_idx.to(DEV), k_idx.to(DEV), m, topk, *args,
                                  q_scale=dev(q_scale), k_scale=dev(k_scale), want_scores=True)
    pt, table = _pages(B, Nc, P, seed=P + Nc)
    rows = _rows(table, P, Nc)
    n_rows = pt.n_pages * P
    ip, sp = csa.csa_indexer_topk(q_idx.to(DEV), w_idx.to(DEV), _to_pool(k_idx, rows, n_rows), m,
                                  topk, *args, q_scale=dev(q_scale),
                                  k_scale=None if k_scale is None else _to_pool(k_scale, rows,
                                                                                 n_rows),
                                  want_scores=True, pages=pt)
    torch.cuda.synchronize()
    _same_bits(ip, iu, "paged indexer indices")
    _same_bits(sp, su, "paged indexer scores")
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    _compare(ip.cpu().numpy(), sp.cpu().numpy(), o[3], m, topk, q_pos, n_cmp, Nc,
             "paged indexer %s P=%d" % (fmt, P))


@pytest.mark.parametrize("dt", [gen.BF16, gen.F32])
@pytest.mark.parametrize("B,T,topk", [(4, 1, 512), (2, 40, 64)])
def test_paged_sparse_attn_matches_unpaged_and_oracle(dt, B, T, topk):
    d = gen.Draw(50 + T)
    H, D, Nc, R, W, m, P = 64, 128, 3000, 700, 128, 4, 64
    q = gen.store(d.normal(B, T, H, D), dt)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), dt)
    kv_raw = gen.store(d.normal(B, R, 2 * D), dt)
    q_pos = [4 * Nc - T - 5 - 40 * b for b in range(B)]
    raw_base = [p + T - R for p in q_pos]
    idx = _rand_idx(d, B, T, topk, lambda b, t: _n_vis(q_pos[b] + t, Nc, m, Nc), 0.1)
    common = (W, dev_i64(q_pos), dev_i64(raw_base))
    ou, lu = csa.csa_sparse_attn(q.to(DEV), kv_cmp.to(DEV), idx.to(DEV), kv_raw.to(DEV), *common,
                                 want_lse=True)
    pt, table = _pages(B, Nc, P, seed=T + topk)
    pool = _to_pool(kv_cmp, _rows(table, P, Nc), pt.n_pages * P)
    op, lp = csa.csa_sparse_attn(q.to(DEV), pool, idx.to(DEV), kv_raw.to(DEV), *common,
                                 want_lse=True, pages=pt)
    torch.cuda.synchronize()
    _same_bits(op, ou, "paged attention out")
    _same_bits(lp, lu, "paged attention lse")
    ref, rl = orc.sparse_attn(gen.host_bits(q), gen.host_bits(kv_cmp), idx.numpy(),
                              gen.host_bits(kv_raw), W, q_pos, raw_base)
    attn_check(op, lp, ref, rl, q.dtype, "paged sparse attention %s T=%d" % (dt, T))


@pytest.mark.parametrize("out_fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("L", [37, 1])
def test_paged_compress_matches_unpaged(out_fmt, L):
    # a chunk (the tiled projection) and a one-token step (the few-row
    # projection with split partials), each carrying a state in
    d = gen.Draw(60 + L)
    B, d_model, E, m, o, P = 3, 512, 64, 4, 1, 16
    Nc = 160
    wk, wg = (w.to(DEV) for w in gen.compressor_weights(d, d_model, E, gen.BF16))
    x = gen.store(d.normal(B, L, d_model), gen.BF16).to(DEV)
    pos0 = dev_i64([3, 100 - L, 600 - L])
    ns = (1 + o) * m - 1
    state_in = d.normal(B, ns, 2, E).to(DEV)
    state_in[:, :, 1, :] = d.normal(B, ns, E).to(DEV)
    pt, table = _pages(B, Nc, P, seed=L)
    n_rows = pt.n_pages * P

    def buffers(shape_rows):
        if out_fmt == "bf16":
            return torch.zeros(*shape_rows, E, dtype=torch.bfloat16, device=DEV), None
        if out_fmt == "fp8":
            return (torch.zeros(*shape_rows, E, dtype=torch.uint8, device=DEV)
                    .view(torch.float8_e4m3fn), torch.zeros(*shape_rows, device=DEV))
        return (torch.zeros(*shape_rows, E // 2, dtype=torch.uint8, device=DEV)
                .view(torch.float4_e2m1fn_x2),
                torch.zeros(*shape_rows, E // 32, dtype=torch.uint8, device=DEV))

    out_u, sc_u = buffers((B, Nc))
    su = torch.zeros(B, ns, 2, E, device=DEV)
    csa.csa_compress(x, wk, wg, pos0, m, o, out_u, out_scale=sc_u, state_in=state_in,
                     state_out=su)
    out_p, sc_p = buffers((n_rows,))
    sp = torch.zeros(B, ns, 2, E, device=DEV)
    csa.csa_compress(x, wk, wg, pos0, m, o, out_p, out_scale=sc_p, state_in=state_in,
                     state_out=sp, pages=pt)
    torch.cuda.synchronize()
    rows = _rows(table, P, Nc).reshape(-1)
    # every logical row (written or untouched) reads the same through the table
    pb = out_p.cpu().contiguous().view(torch.uint8)
    ub = out_u.cpu().contiguous().view(torch.uint8)
    assert torch.equal(pb[rows].view(ub.shape), ub), "paged store " + out_fmt
    if out_fmt == "fp8":
        assert torch.equal(sc_p.cpu()[rows].view(B, Nc).view(torch.int32),
                           sc_u.cpu().view(torch.int32)), "paged fp8 scales"
    elif out_fmt == "mxfp4":
        assert torch.equal(sc_p.cpu()[rows].view(sc_u.shape), sc_u.cpu()), "paged mxfp4 scales"
    _same_bits(sp, su, "carried state")
    # the spare pages are never written
    used = torch.zeros(n_rows, dtype=torch.bool)
    used[rows] = True
    assert not pb[~used].any()
