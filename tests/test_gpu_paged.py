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


def test_paged_compress_fused_chunk_matches_unpaged():
    # a 260-token chunk through the fused projection + pool, storing each
    # entry at its pool row, bit-exact against the unpaged call
    d = gen.Draw(66)
    B, d_model, E, m, o, P = 2, 512, 128, 4, 1, 16
    L, Nc = 260, 160
    wk, wg = (w.to(DEV) for w in gen.compressor_weights(d, d_model, E, gen.BF16))
    x = gen.store(d.normal(B, L, d_model), gen.BF16).to(DEV)
    pos0 = dev_i64([3, 300])
    ns = (1 + o) * m - 1
    state_in = d.normal(B, ns, 2, E).to(DEV)
    pt, table = _pages(B, Nc, P, seed=9)
    n_rows = pt.n_pages * P
    out_u = torch.zeros(B, Nc, E, dtype=torch.bfloat16, device=DEV)
    su = torch.zeros(B, ns, 2, E, device=DEV)
    csa.csa_compress(x, wk, wg, pos0, m, o, out_u, state_in=state_in, state_out=su)
    out_p = torch.zeros(n_rows, E, dtype=torch.bfloat16, device=DEV)
    sp = torch.zeros(B, ns, 2, E, device=DEV)
    csa.csa_compress(x, wk, wg, pos0, m, o, out_p, state_in=state_in, state_out=sp, pages=pt)
    torch.cuda.synchronize()
    rows = _rows(table, P, Nc).reshape(-1)
    pb = out_p.cpu().contiguous().view(torch.uint8)
    ub = out_u.cpu().contiguous().view(torch.uint8)
    assert torch.equal(pb[rows].view(ub.shape), ub), "paged fused store"
    # the entries of each call were written (positions 3 .. 262 and 300 .. 559)
    ue = ub.view(B, Nc, E * 2)
    assert ue[0, 1:65].any(dim=1).all() and ue[1, 75:140].any(dim=1).all()
    _same_bits(sp, su, "carried state")
    used = torch.zeros(n_rows, dtype=torch.bool)
    used[rows] = True
    assert not pb[~used].any()


def _absent(table, n_pages, P, nc_cap):
    """Marks one page of sequence 0 with -1 and one of the last sequence with
    an id past the pool; returns the table, and the logical entries that the
    two pages held, per sequence."""
    t = table.clone()
    B, max_pages = t.shape
    gone = {}
    for b, pg, bad in ((0, 1, -1), (B - 1, max_pages // 2, n_pages + 5)):
        t[b, pg] = bad
        gone[b] = np.union1d(gone.get(b, np.zeros(0, np.int64)),
                             np.arange(pg * P, min((pg + 1) * P, nc_cap)))
    return t, gone


@pytest.mark.parametrize("fmt", [gen.BF16, gen.FP8])
def test_paged_indexer_absent_pages_score_minus_inf(fmt):
    # an out-of-range page id marks its entries absent: score -inf, so they
    # lose to every present entry, and no pool row is read for them
    d = gen.Draw(70)
    B, T, Nc, m, topk, P = 3, 2, 3000, 4, 300, 64
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, fmt)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, T, 16, 64, fmt)
    q_pos, n_cmp = [4 * Nc, 4 * Nc - 10, 4 * 1500], [Nc, Nc, Nc]
    pt, table = _pages(B, Nc, P, seed=7)
    rows = _rows(table, P, Nc)
    n_rows = pt.n_pages * P
    bad_table, gone = _absent(table, pt.n_pages, P, Nc)
    pt_bad = csa.PageTable(bad_table.to(DEV), P, pt.n_pages, nc_cap=Nc)
    dev = lambda t: None if t is None else t.to(DEV)
    ip, sp = csa.csa_indexer_topk(q_idx.to(DEV), w_idx.to(DEV), _to_pool(k_idx, rows, n_rows), m,
                                  topk, dev_i64(q_pos), dev_i32(n_cmp), q_scale=dev(q_scale),
                                  k_scale=None if k_scale is None else _to_pool(k_scale, rows,
                                                                                 n_rows),
                                  want_scores=True, pages=pt_bad)
    torch.cuda.synchronize()
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    alls = o[3].copy()
    for b, js in gone.items():
        alls[b, :, js] = -np.inf
    g_idx = ip.cpu().numpy()
    for b, js in gone.items():
        assert not np.isin(g_idx[b], js).any(), "an absent entry was selected"
    _compare(g_idx, sp.cpu().numpy(), alls, m, topk, q_pos, n_cmp, Nc, "absent pages " + fmt)


@pytest.mark.parametrize("B,T", [(4, 1), (1, 1100)])
def test_paged_sparse_attn_absent_pages_are_skipped(B, T):
    # (4, 1): the decode kernel maps indices while staging them; (1, 1100):
    # the translation launch feeds the prefill kernel
    d = gen.Draw(71 + T)
    H, D, Nc, R, W, m, P, topk = 64, 128, 3000, 1300, 128, 4, 64, 64
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    q_pos = [4 * Nc - T - 5 - 40 * b for b in range(B)]
    raw_base = [p + T - R for p in q_pos]
    # indices crowd into the first pages so that the absent ones are hit
    nv = torch.tensor([[min(_n_vis(q_pos[b] + t, Nc, m, Nc), 400) for t in range(T)]
                       for b in range(B)])
    idx = gen.random_index_sets(d, B, T, topk, nv, 0.1)
    pt, table = _pages(B, Nc, P, seed=T)
    bad_table, gone = _absent(table, pt.n_pages, P, Nc)
    pt_bad = csa.PageTable(bad_table.to(DEV), P, pt.n_pages, nc_cap=Nc)
    pool = _to_pool(kv_cmp, _rows(table, P, Nc), pt.n_pages * P)
    op, lp = csa.csa_sparse_attn(q.to(DEV), pool, idx.to(DEV), kv_raw.to(DEV), W,
                                 dev_i64(q_pos), dev_i64(raw_base), want_lse=True, pages=pt_bad)
    torch.cuda.synchronize()
    ref_idx = idx.numpy().copy()
    hit = 0
    for b, js in gone.items():
        m_ = np.isin(ref_idx[b], js)
        hit += int(m_.sum())
        ref_idx[b][m_] = -1
    assert hit > 0, "the test must name entries of an absent page"
    ref, rl = orc.sparse_attn(gen.host_bits(q), gen.host_bits(kv_cmp), ref_idx,
                              gen.host_bits(kv_raw), W, q_pos, raw_base)
    attn_check(op, lp, ref, rl, q.dtype, "absent pages B=%d T=%d" % (B, T))


def test_paged_sparse_attn_bf16_prefill_rows_match_unpaged():
    # 1024 or more query rows: the page translation launch, then the
    # one-row-per-wave prefill kernel over the pool
    d = gen.Draw(72)
    B, T, H, D, Nc, W, m, P, topk = 1, 1024, 64, 128, 2048, 128, 4, 64, 64
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, 4 * Nc, 2 * D), gen.BF16)
    q_pos = [4 * Nc - T]
    raw_base = [0]
    idx = _rand_idx(d, B, T, topk, lambda b, t: _n_vis(q_pos[b] + t, Nc, m, Nc), 0.1)
    common = (W, dev_i64(q_pos), dev_i64(raw_base))
    ou, lu = csa.csa_sparse_attn(q.to(DEV), kv_cmp.to(DEV), idx.to(DEV), kv_raw.to(DEV), *common,
                                 want_lse=True)
    pt, table = _pages(B, Nc, P, seed=72)
    pool = _to_pool(kv_cmp, _rows(table, P, Nc), pt.n_pages * P)
    op, lp = csa.csa_sparse_attn(q.to(DEV), pool, idx.to(DEV), kv_raw.to(DEV), *common,
                                 want_lse=True, pages=pt)
    torch.cuda.synchronize()
    _same_bits(op, ou, "paged prefill attention out")
    _same_bits(lp, lu, "paged prefill attention lse")
    rows = np.arange(0, T, 7)
    # sampled rows against the oracle (each row is independent: a one-row
    # oracle call per sampled position)
    for t in rows[:40]:
        r, l = orc.sparse_attn(gen.host_bits(q)[:, t:t + 1], gen.host_bits(kv_cmp),
                               idx.numpy()[:, t:t + 1], gen.host_bits(kv_raw), W,
                               [q_pos[0] + t], raw_base)
        attn_check(op[:, t:t + 1], lp[:, t:t + 1], r, l, q.dtype, "paged prefill row %d" % t)


def test_paged_compress_absent_page_is_not_stored():
    d = gen.Draw(73)
    B, L, d_model, E, m, o, P, Nc = 2, 128, 512, 64, 4, 1, 16, 32
    wk, wg = (w.to(DEV) for w in gen.compressor_weights(d, d_model, E, gen.BF16))
    x = gen.store(d.normal(B, L, d_model), gen.BF16).to(DEV)
    pos0 = dev_i64([0, 0])
    pt, table = _pages(B, Nc, P, seed=73, spare=2)
    n_rows = pt.n_pages * P
    bad = table.clone()
    bad[0, 1] = -1                   # entries 16..31 of sequence 0
    bad[1, 0] = pt.n_pages           # entries 0..15 of sequence 1
    out_u = torch.zeros(B, Nc, E, dtype=torch.bfloat16, device=DEV)
    csa.csa_compress(x, wk, wg, pos0, m, o, out_u)
    sentinel = torch.full((n_rows, E), 7.0, dtype=torch.bfloat16, device=DEV)
    out_p = sentinel.clone()
    csa.csa_compress(x, wk, wg, pos0, m, o, out_p,
                     pages=csa.PageTable(bad.to(DEV), P, pt.n_pages, nc_cap=Nc))
    torch.cuda.synchronize()
    rows = _rows(table, P, Nc)
    pb, ub, sb = out_p.cpu(), out_u.cpu(), sentinel.cpu()
    # present pages hold the unpaged entries
    assert torch.equal(pb[rows[0, :16]], ub[0, :16])
    assert torch.equal(pb[rows[1, 16:]], ub[1, 16:])
    # every other pool row (the absent pages' own rows and the spare pages)
    # keeps its old contents
    keep = torch.ones(n_rows, dtype=torch.bool)
    keep[rows[0, :16]] = False
    keep[rows[1, 16:]] = False
    assert torch.equal(pb[keep], sb[keep])


@pytest.mark.parametrize("dt,B,T", [(gen.BF16, 4, 1), (gen.BF16, 1, 1100), (gen.F32, 2, 30)])
@pytest.mark.parametrize("both", [False, True])
def test_paged_window_matches_unpaged_and_oracle(dt, B, T, both):
    # the raw window cache in a pool of 32-row pages (alone, or with the
    # compressed cache paged too): bit-exact with the unpaged call
    d = gen.Draw(80 + T + both)
    H, D = (64, 128) if dt == gen.BF16 else (8, 64)
    Nc, R, W, m, P, Pr, topk = 900, T + 200, 128, 4, 64, 32, 64
    q = gen.store(d.normal(B, T, H, D), dt)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), dt)
    kv_raw = gen.store(d.normal(B, R, 2 * D), dt)
    q_pos = [4 * Nc - T - 3 - 5 * b for b in range(B)]
    raw_base = [p + T - R for p in q_pos]
    idx = _rand_idx(d, B, T, topk, lambda b, t: _n_vis(q_pos[b] + t, Nc, m, Nc), 0.1)
    common = (W, dev_i64(q_pos), dev_i64(raw_base))
    ou, lu = csa.csa_sparse_attn(q.to(DEV), kv_cmp.to(DEV), idx.to(DEV), kv_raw.to(DEV), *common,
                                 want_lse=True)
    rpt, rtable = _pages(B, R, Pr, seed=11 + T)
    raw_pool = _to_pool(kv_raw, _rows(rtable, Pr, R), rpt.n_pages * Pr)
    kw = dict(raw_pages=rpt)
    cmp_in = kv_cmp.to(DEV)
    if both:
        cpt, ctable = _pages(B, Nc, P, seed=12 + T)
        cmp_in = _to_pool(kv_cmp, _rows(ctable, P, Nc), cpt.n_pages * P)
        kw["pages"] = cpt
    op, lp = csa.csa_sparse_attn(q.to(DEV), cmp_in, idx.to(DEV), raw_pool, *common, want_lse=True,
                                 **kw)
    torch.cuda.synchronize()
    _same_bits(op, ou, "paged window out")
    _same_bits(lp, lu, "paged window lse")
    rows = range(0, T, max(1, T // 12))
    for t in rows:
        r, l = orc.sparse_attn(gen.host_bits(q)[:, t:t + 1], gen.host_bits(kv_cmp),
                               idx.numpy()[:, t:t + 1], gen.host_bits(kv_raw), W,
                               [p + t for p in q_pos], raw_base)
        attn_check(op[:, t:t + 1], lp[:, t:t + 1], r, l, q.dtype, "paged window row %d" % t)


@pytest.mark.parametrize("T", [1, 1030])
def test_paged_hca_matches_unpaged(T):
    # HCA with its compressed cache and its window cache both paged: the
    # prefill kernel's shared segments and the decode kernel find every row
    # through the tables; bit-exact with the unpaged call
    d = gen.Draw(85 + T)
    B, H, D, m, W, Nc, P, Pr = 2, 64, 128, 16, 64, 300, 16, 32
    R = T + W
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    q_pos = [m * Nc - T - 1, m * 200]
    n_cmp = [Nc, 250]
    raw_base = [p - W + 1 for p in q_pos]
    args = (m, W, dev_i64(q_pos), dev_i32(n_cmp), dev_i64(raw_base))
    ou, lu = csa.hca_dense_attn(q.to(DEV), kv_cmp.to(DEV), kv_raw.to(DEV), *args, want_lse=True)
    cpt, ctable = _pages(B, Nc, P, seed=T)
    rpt, rtable = _pages(B, R, Pr, seed=T + 1)
    op, lp = csa.hca_dense_attn(q.to(DEV), _to_pool(kv_cmp, _rows(ctable, P, Nc), cpt.n_pages * P),
                                _to_pool(kv_raw, _rows(rtable, Pr, R), rpt.n_pages * Pr), *args,
                                want_lse=True, pages=cpt, raw_pages=rpt)
    torch.cuda.synchronize()
    _same_bits(op, ou, "paged hca out")
    _same_bits(lp, lu, "paged hca lse")
    for t in (0, T // 2, T - 1):
        r, l = orc.hca_dense_attn(gen.host_bits(q)[:, t:t + 1], gen.host_bits(kv_cmp),
                                  gen.host_bits(kv_raw), m, W, [p + t for p in q_pos], n_cmp,
                                  raw_base)
        attn_check(op[:, t:t + 1], lp[:, t:t + 1], r, l, q.dtype, "paged hca row %d" % t)


def test_paged_window_absent_page_rows_are_skipped():
    # a window page marked absent: its rows leave the softmax, checked
    # against the library attention with those keys masked out
    from tests import brute
    d = gen.Draw(88)
    B, T, H, D, W, Pr = 1, 3, 64, 128, 100, 16
    R = T + W
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    q_pos = [5000]
    raw_base = [q_pos[0] + T - R]
    rpt, rtable = _pages(B, R, Pr, seed=88)
    bad = rtable.clone()
    bad[0, 2] = -1                     # raw rows 32..47 absent
    raw_pool = _to_pool(kv_raw, _rows(rtable, Pr, R), rpt.n_pages * Pr)
    pt_bad = csa.PageTable(bad.to(DEV), Pr, rpt.n_pages, nc_cap=R)
    op, _ = csa.csa_sparse_attn(q.to(DEV), torch.zeros(1, 1, 2 * D, dtype=torch.bfloat16,
                                                         device=DEV), None, raw_pool, W,
                                dev_i64(q_pos), dev_i64(raw_base), raw_pages=pt_bad)
    torch.cuda.synchronize()
    kr = gen.host_bits(kv_raw)[0]
    keys = brute.decode_bits(kr[:, :D])
    vals = brute.decode_bits(kr[:, D:])
    mask = np.zeros((T, R), bool)
    for t in range(T):
        pos = q_pos[0] + t
        for tok in range(pos - W + 1, pos + 1):
            r = tok - raw_base[0]
            if 0 <= r < R and not (32 <= r < 48):
                mask[t, r] = True
    ref, _ = brute.sdpa_masked(brute.decode_bits(gen.host_bits(q)[0]), keys, vals, mask, D ** -0.5)
    from tests.helpers import assert_bf16_close
    assert_bf16_close(op[0].float().cpu().numpy(), ref, "absent window page")
