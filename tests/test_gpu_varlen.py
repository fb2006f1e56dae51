"""GPU parity of the packed variable-length prefill (csa_compress_varlen,
csa_indexer_topk_varlen, csa_sparse_attn_varlen): every packed sequence
against the oracle run on that sequence alone."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import assert_bf16_close, assert_rows_rel, check_topk_row

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _offsets(lens, m):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ccu = np.concatenate([[0], np.cumsum(np.asarray(lens) // m)]).astype(np.int32)
    return cu, ccu


@pytest.mark.parametrize("lens,dt", [([300, 7, 1030, 128], gen.BF16), ([40, 3, 100], gen.BF16),
                                     ([33, 64, 5, 77], gen.F32)])
def test_packed_prefill_matches_each_sequence_alone(lens, dt):
    d = gen.Draw(100 + len(lens) + (dt == gen.F32))
    m, o, dm = 4, 1, 256
    if dt == gen.BF16:
        H, D, H_I, d_I, topk, W = 64, 128, 16, 64, 64, 128
    else:
        H, D, H_I, d_I, topk, W = 8, 64, 4, 32, 8, 16
    n, total, max_len = len(lens), sum(lens), max(lens)
    cu, ccu = _offsets(lens, m)
    max_cmp = max(lens) // m
    x = gen.store(d.normal(total, dm), dt)
    wk, wg = gen.compressor_weights(d, dm, 2 * D, dt)
    wik, wig = gen.compressor_weights(d, dm, d_I, dt)
    q = gen.store(d.normal(total, H, D), dt)
    kv_raw = gen.store(d.normal(total, 2 * D), dt)
    q_idx = gen.store(d.normal(total, H_I, d_I), dt)
    w_idx = d.normal(total, H_I)
    tdt = gen.torch_dtype(dt)
    cu_d = torch.from_numpy(cu).to(DEV)
    ccu_d = csa.csa_build_cmp_cu_seqlens(cu_d, m)
    torch.cuda.synchronize()
    assert np.array_equal(ccu_d.cpu().numpy(), ccu), "cmp_cu_seqlens"
    n_ent = int(ccu[-1])
    kv_cmp = torch.full((n_ent, 2 * D), float("nan"), device=DEV).to(tdt)
    k_idx = torch.full((n_ent, d_I), float("nan"), device=DEV).to(tdt)
    ns = 2 * m - 1
    st_main = torch.full((n, ns, 2, 2 * D), 5.0, device=DEV)
    xg = x.to(DEV)
    csa.csa_compress_varlen(xg, wk.to(DEV), wg.to(DEV), cu_d, ccu_d, max_len, m, o, kv_cmp,
                            state_out=st_main)
    csa.csa_compress_varlen(xg, wik.to(DEV), wig.to(DEV), cu_d, ccu_d, max_len, m, o, k_idx)
    idx, sc = csa.csa_indexer_topk_varlen(q_idx.to(DEV), w_idx.to(DEV), k_idx, cu_d, ccu_d,
                                          max_len, max_cmp, m, topk, want_scores=True)
    out, lse = csa.csa_sparse_attn_varlen(q.to(DEV), kv_cmp, idx, kv_raw.to(DEV), cu_d, ccu_d,
                                          max_len, max_cmp, W, want_lse=True)
    torch.cuda.synchronize()
    g_kv, g_k = kv_cmp.float().cpu().numpy(), k_idx.float().cpu().numpy()
    g_idx, g_out = idx.cpu().numpy(), out.float().cpu().numpy()
    g_lse, g_st = lse.cpu().numpy(), st_main.cpu().numpy()
    hb = lambda t: gen.host_bits(t)
    for b in range(n):
        t0, t1, e0, e1 = cu[b], cu[b + 1], ccu[b], ccu[b + 1]
        L, Nc = t1 - t0, e1 - e0
        what = "seq %d (len %d)" % (b, L)
        ref_kv, wr, st_ref = orc.compress(hb(x[None, t0:t1]), hb(wk), hb(wg), m, o, 0, max(Nc, 1))
        ref_k, _, _ = orc.compress(hb(x[None, t0:t1]), hb(wik), hb(wig), m, o, 0, max(Nc, 1))
        assert wr[0, :Nc].all()
        if dt == gen.F32:
            assert_rows_rel(g_kv[e0:e1], ref_kv[0, :Nc], 1e-5, "main entries " + what)
            assert_rows_rel(g_k[e0:e1], ref_k[0, :Nc], 1e-5, "indexer entries " + what)
        else:
            assert_bf16_close(g_kv[e0:e1], ref_kv[0, :Nc], "main entries " + what)
            assert_bf16_close(g_k[e0:e1], ref_k[0, :Nc], "indexer entries " + what)
        np.testing.assert_allclose(g_st[b, :, 0], st_ref[0, :, 0], rtol=2e-5, atol=2e-5)
        # the selection, scored by the oracle on the device's own keys
        if Nc > 0:
            kb = hb(k_idx[e0:e1].cpu())[None]
            _, _, _, alls = orc.indexer_topk(hb(q_idx[None, t0:t1]), w_idx[None, t0:t1].numpy(), kb,
                                             m, topk, 0, Nc, want_all=True)
        for t in range(L):
            nv = min(Nc, (t + 1) // m)
            if Nc > 0:
                check_topk_row(g_idx[t0 + t], alls[0, t], topk, nv, "%s row %d" % (what, t))
            else:
                assert (g_idx[t0 + t] == -1).all()
        # attention over the device's selection
        kvc = hb(kv_cmp[e0:e1].cpu())[None] if Nc > 0 else np.zeros((1, 1, 2 * D),
                                                                        hb(kv_raw).dtype)
        r, rl = orc.sparse_attn(hb(q[None, t0:t1]), kvc, g_idx[None, t0:t1], hb(kv_raw[None, t0:t1]),
                                W, 0, 0)
        if dt == gen.F32:
            assert_rows_rel(g_out[t0:t1], r[0], 1e-5, "attention " + what)
        else:
            assert_bf16_close(g_out[t0:t1], r[0], "attention " + what)
        fin = np.isfinite(rl[0])
        np.testing.assert_allclose(g_lse[t0:t1][fin], rl[0][fin], rtol=1e-4, atol=1e-4)


def test_packed_indexer_long_sequence():
    # a packed sequence of more than 8192 entries beside short ones: every
    # row goes through the segment select with the packed offsets; sampled
    # rows of the long sequence and every row of the short ones against the
    # oracle on the sequence alone
    d = gen.Draw(120)
    m, topk = 4, 300
    lens = [33000, 50, 700]
    cu, ccu = _offsets(lens, m)
    total, max_len, max_cmp = sum(lens), max(lens), max(lens) // m
    n_ent = int(ccu[-1])
    q_idx = gen.store(d.normal(total, 16, 64), gen.BF16)
    w_idx = d.normal(total, 16)
    k_idx = gen.store(d.normal(n_ent, 64), gen.BF16)
    cu_d = torch.from_numpy(cu).to(DEV)
    ccu_d = torch.from_numpy(ccu).to(DEV)
    idx, _ = csa.csa_indexer_topk_varlen(q_idx.to(DEV), w_idx.to(DEV), k_idx.to(DEV), cu_d, ccu_d,
                                         max_len, max_cmp, m, topk)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    hb = lambda t: gen.host_bits(t)
    blocks = {0: [0, 4090, 32760, 32992], 1: [0, 8, 16, 24, 32, 40, 48], 2: list(range(0, 700, 8))}
    for b, starts in blocks.items():
        t0s, e0, e1 = cu[b], ccu[b], ccu[b + 1]
        L, Nc = cu[b + 1] - t0s, e1 - e0
        kb = hb(k_idx[e0:e1])[None]
        for s in starts:
            s1 = min(s + 8, L)
            rows = slice(t0s + s, t0s + s1)
            _, _, _, alls = orc.indexer_topk(hb(q_idx[None, rows]), w_idx[None, rows].numpy(), kb,
                                             m, topk, s, Nc, want_all=True)
            for t in range(s, s1):
                nv = min(Nc, (t + 1) // m)
                check_topk_row(g_idx[t0s + t], alls[0, t - s], topk, nv,
                               "seq %d row %d" % (b, t))
