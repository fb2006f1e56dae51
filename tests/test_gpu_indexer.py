"""GPU parity of csa_indexer_topk against the CPU oracle."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import check_topk_row, dev_i32, dev_i64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _n_vis(pos, ncmp, m, cap):
    return max(0, min(ncmp, (pos + 1) // m, cap))


def _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale=None, k_scale=None):
    idx, sc = csa.csa_indexer_topk(q_idx.to(DEV), w_idx.to(DEV), k_idx.to(DEV), m, topk,
                                   dev_i64(q_pos), dev_i32(n_cmp),
                                   q_scale=None if q_scale is None else q_scale.to(DEV),
                                   k_scale=None if k_scale is None else k_scale.to(DEV),
                                   want_scores=True)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale=None, k_scale=None):
    fmt = "mxfp4" if q_idx.dtype == torch.float4_e2m1fn_x2 else None
    return orc.indexer_topk(gen.host_bits(q_idx), gen.host_bits(w_idx), gen.host_bits(k_idx), m,
                            topk, np.asarray(q_pos), np.asarray(n_cmp),
                            q_scale=None if q_scale is None else gen.host_bits(q_scale),
                            k_scale=None if k_scale is None else gen.host_bits(k_scale),
                            want_all=True, fmt=fmt)


def _compare(g_idx, g_sc, o_all, m, topk, q_pos, n_cmp, Nc, what):
    B, T, _ = g_idx.shape
    near = 0
    for b in range(B):
        for t in range(T):
            nv = _n_vis(int(q_pos[b]) + t, int(n_cmp[b]), m, Nc)
            near += check_topk_row(g_idx[b, t], o_all[b, t], topk, nv, "%s b%d t%d" % (what, b, t))
            sel = g_idx[b, t][g_idx[b, t] >= 0]
            np.testing.assert_allclose(g_sc[b, t, :sel.size], o_all[b, t, sel], rtol=1e-4, atol=1e-4)
    return near


def test_indexer_tiny_f32_full():
    w = gen.WORKLOADS["csa_prefill_tiny_f32"]
    d = gen.Draw(21)
    q_idx, _, w_idx = gen.indexer_query(d, 1, w.T, w.H_I, w.d_I, gen.F32)
    k_idx, _ = gen.indexer_keys(d, 1, w.n_cmp, w.d_I, gen.F32)
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, w.m, w.topk, [0], [w.n_cmp])
    o = _oracle_rows(q_idx, w_idx, k_idx, w.m, w.topk, [0], [w.n_cmp])
    _compare(g_idx, g_sc, o[3], w.m, w.topk, [0], [w.n_cmp], w.n_cmp, "f32 tiny")


@pytest.mark.parametrize("topk", [16, 512])
def test_indexer_bf16_ragged_batch(topk):
    d = gen.Draw(22 + topk)
    B, T, Nc, m = 3, 70, 600, 4
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    q_pos, n_cmp = [0, 300, 2300], [Nc, 90, 550]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "bf16 ragged")


def test_indexer_bf16_exact_ties_lower_index():
    d = gen.Draw(23)
    B, T, Nc, m, topk = 1, 20, 300, 4, 40
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    k_idx[0, 100:200] = k_idx[0, 7]            # 101 identical keys -> identical scores
    k_idx[0, 250:] = k_idx[0, 3]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, [2000], [Nc])
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, [2000], [Nc])
    # exact equality must resolve exactly like the oracle (no exemption)
    for t in range(T):
        s = o[3][0, t]
        sel = set(g_idx[0, t].tolist())
        ref = set(o[0][0, t].tolist())
        diff = sel ^ ref
        tau = o[2][0, t]
        assert all(abs(s[j] - tau) <= 1e-3 for j in diff)
        # among the duplicated block, chosen members are its lowest indices
        blk = [j for j in range(100, 200) if j in sel] + ([7] if 7 in sel else [])
        if blk and len(blk) < 101:
            members = sorted([7] + list(range(100, 200)))
            assert sorted(blk) == members[:len(blk)]


def test_indexer_bf16_rows_between_2k_and_8k():
    # rows longer than the register-resident path (2048 keys) but short
    # enough for one wave's LDS slice (8192)
    d = gen.Draw(25)
    B, T, Nc, m, topk = 2, 12, 5000, 4, 512
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    k_idx[1, 1000:1300] = k_idx[1, 20]       # a block of tied scores
    q_pos, n_cmp = [20000, 3000], [Nc, 4990]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "bf16 2k-8k rows")


@pytest.mark.parametrize("kind", ["all_equal", "two_values", "one_high"])
def test_indexer_bf16_degenerate_score_rows(kind):
    # rows whose scores are all equal (keys all zero), take two values, or
    # have a single outlier: ties resolve to the lowest indices, the radix
    # passes start below the keys' common prefix
    d = gen.Draw(24)
    B, T, Nc, m, topk = 1, 6, 700, 4, 64
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    if kind == "all_equal":
        k_idx[:] = 0
    elif kind == "two_values":
        k_idx[0, 0::2] = k_idx[0, 5]
        k_idx[0, 1::2] = k_idx[0, 8]
    else:
        k_idx[0, :] = 0
        k_idx[0, 333] = k_idx[0, 333] + 1.0
    q_pos, n_cmp = [2600], [Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    for t in range(T):
        # exact equality resolves exactly like the oracle
        assert sorted(g_idx[0, t].tolist()) == sorted(o[0][0, t].tolist()), (kind, t)
    if kind == "all_equal":
        assert (g_idx[0] == np.arange(topk)[None, :]).all()


def test_indexer_prefill_8k_sampled_rows():
    w = gen.WORKLOADS["csa_prefill_8k_bf16"]
    d = gen.Draw(w.seed + 100)
    q_idx, _, w_idx = gen.indexer_query(d, 1, w.T, w.H_I, w.d_I, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, 1, w.n_cmp, w.d_I, gen.BF16)
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, w.m, w.topk, [0], [w.n_cmp])
    # blocks of 16 consecutive rows (every row of a 16-row score group, at
    # aligned and unaligned starts), through the 512-entry chunk boundaries
    # (rows 2047/2048, 4095/4096, 6143/6144) and the last rows: 288 rows
    starts = [0, 9, 1000, 2040, 3001, 4088, 4500, 5123, 6136, 6700, 7007, 7500, 7777, 7900,
              8000, 8100, 8150, 8176]
    n = 0
    for t0 in starts:
        sl = slice(t0, t0 + 16)
        o = _oracle_rows(q_idx[:, sl], w_idx[:, sl], k_idx, w.m, w.topk, [t0], [w.n_cmp])
        _compare(g_idx[:, sl], g_sc[:, sl], o[3], w.m, w.topk, [t0], [w.n_cmp], w.n_cmp,
                 "8k rows %d.." % t0)
        n += 16
    assert n >= 256


@pytest.mark.parametrize("name,rows", [("csa_decode_128k_b32", [0, 5, 13, 22, 31]),
                                       ("csa_decode_1m_b8_stream", list(range(8)))])
def test_indexer_fp8_decode_long_rows(name, rows):
    w = gen.WORKLOADS[name]
    d = gen.Draw(w.seed, DEV)
    B, Nc = w.B, w.n_cmp
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, w.d_I, gen.FP8)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 1, w.H_I, w.d_I, gen.FP8)
    q_pos = [w.ctx - 1] * B
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, w.m, w.topk, q_pos, [Nc] * B, q_scale, k_scale)
    # the sampled sequences in one oracle call (its rows run in parallel)
    sl = torch.tensor(rows)
    o = _oracle_rows(q_idx[sl], w_idx[sl], k_idx[sl], w.m, w.topk, [w.ctx - 1] * len(rows),
                     [Nc] * len(rows), q_scale[sl], k_scale[sl])
    _compare(g_idx[rows], g_sc[rows], o[3], w.m, w.topk, [w.ctx - 1] * len(rows),
             [Nc] * len(rows), Nc, name)


@pytest.mark.parametrize("name,rows", [("csa_decode_128k_b32", [0, 13, 31])])
def test_indexer_mxfp4_decode_long_rows(name, rows):
    # MXFP4 keys and queries (E2M1 codes, one E8M0 exponent per 32 values)
    # at the 128K decode shape: the long-row collect / finalize path
    w = gen.WORKLOADS[name]
    d = gen.Draw(w.seed + 7, DEV)
    B, Nc = w.B, w.n_cmp
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, w.d_I, gen.MXFP4)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 1, w.H_I, w.d_I, gen.MXFP4)
    q_pos = [w.ctx - 1] * B
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, w.m, w.topk, q_pos, [Nc] * B, q_scale, k_scale)
    for b in rows:
        sl = slice(b, b + 1)
        o = _oracle_rows(q_idx[sl], w_idx[sl], k_idx[sl], w.m, w.topk, [w.ctx - 1], [Nc],
                         q_scale[sl], k_scale[sl])
        _compare(g_idx[sl], g_sc[sl], o[3], w.m, w.topk, [w.ctx - 1], [Nc], Nc,
                 "mxfp4 %s b%d" % (name, b))


def test_indexer_mxfp4_short_rows_ragged():
    # prefill-shaped MXFP4 rows (the short-row select), ragged visibility
    d = gen.Draw(27)
    B, T, Nc, m, topk = 2, 90, 700, 4, 64
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.MXFP4)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.MXFP4)
    q_pos, n_cmp = [2500, 37], [Nc, 500]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "mxfp4 short rows")


@pytest.mark.parametrize("Nc", [20000, 40000])
def test_indexer_fp8_long_rows_heavy_ties_and_partial_visibility(Nc):
    # one repeated key: every candidate ties exactly, which overflows the LDS
    # candidate buffer and exercises the exact global path
    d = gen.Draw(24, "cpu")
    B, m, topk = 3, 4, 300
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.FP8)
    kb = k_idx.view(torch.uint8)            # edit the stored codes directly
    kb[0] = kb[0, 5].clone()
    k_scale[0] = k_scale[0, 5].clone()
    kb[1, ::2] = kb[1, 11].clone()
    k_scale[1, ::2] = k_scale[1, 11].clone()
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 2, 16, 64, gen.FP8)
    w_idx[0] = w_idx[0].abs()
    q_pos = [4 * Nc, 4 * Nc, 4 * 150]       # third sequence sees only ~150 entries
    n_cmp = [Nc, Nc - 7, Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "fp8 ties %d" % Nc)
    # all-equal row: the lowest indices win, bit-exact
    if (o[3][0, 0, :Nc] == o[3][0, 0, 0]).all():
        assert np.array_equal(g_idx[0, 0], np.arange(topk))


@pytest.mark.parametrize("Nc", [8193, 32768])
def test_indexer_bf16_long_rows_bounds_and_ragged(Nc):
    # the shortest row length past the one-wave select, and the 128K-context
    # length, over sequences whose visibility runs from a few entries (every
    # visible entry kept) to the whole row
    d = gen.Draw(30 + Nc % 7)
    B, m, topk = 3, 4, 1000
    q_idx, _, w_idx = gen.indexer_query(d, B, 1, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    k_idx[1, 4000:4500] = k_idx[1, 77]       # a block of tied scores
    q_pos, n_cmp = [4 * Nc - 2, 4 * 6000, 4 * 900], [Nc, Nc - 5, Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "bf16 long rows %d" % Nc)


@pytest.mark.parametrize("kind", ["all_equal", "two_values", "one_high"])
def test_indexer_fp8_long_rows_degenerate(kind):
    # degenerate long score rows: ties resolve to the lowest indices,
    # bit-exact against the oracle
    d = gen.Draw(31, "cpu")
    B, Nc, m, topk = 1, 24000, 4, 2048
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.FP8)
    kb = k_idx.view(torch.uint8)
    if kind == "all_equal":
        kb[0] = kb[0, 9].clone()
        k_scale[0] = k_scale[0, 9].clone()
    elif kind == "two_values":
        kb[0, 0::2] = kb[0, 5].clone()
        k_scale[0, 0::2] = k_scale[0, 5].clone()
        kb[0, 1::2] = kb[0, 8].clone()
        k_scale[0, 1::2] = k_scale[0, 8].clone()
    else:
        kb[0] = kb[0, 9].clone()
        k_scale[0] = k_scale[0, 9].clone()
        k_scale[0, 12345] = k_scale[0, 12345] * 4.0
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 1, 16, 64, gen.FP8)
    q_pos, n_cmp = [4 * Nc], [Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    assert sorted(g_idx[0, 0].tolist()) == sorted(o[0][0, 0].tolist()), kind
    assert (np.diff(g_idx[0, 0]) > 0).all()
    if kind == "all_equal":
        assert (g_idx[0, 0] == np.arange(topk)).all()


@pytest.mark.parametrize("kind", ["all_equal", "two_values", "one_high"])
def test_indexer_bf16_segment_path_degenerate(kind):
    # the same degenerate rows through the segment path (bf16 keys, two query
    # positions): one repeated key, two alternating keys, one key above a
    # repeated one; ties resolve to the lowest indices across segments
    d = gen.Draw(32, "cpu")
    B, T, Nc, m, topk = 1, 2, 24000, 4, 2048
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    if kind == "all_equal":
        k_idx[0] = k_idx[0, 9].clone()
    elif kind == "two_values":
        k_idx[0, 0::2] = k_idx[0, 5].clone()
        k_idx[0, 1::2] = k_idx[0, 8].clone()
    else:
        k_idx[0] = k_idx[0, 9].clone()
        k_idx[0, 12345] = k_idx[0, 12345] * 4.0
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    w_idx = w_idx.abs()  # positive weights: the scaled key scores higher
    q_pos, n_cmp = [4 * Nc], [Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    for t in range(T):
        assert sorted(g_idx[0, t].tolist()) == sorted(o[0][0, t].tolist()), (kind, t)
        assert (np.diff(g_idx[0, t]) > 0).all()
    if kind == "all_equal":
        assert (g_idx[0, :] == np.arange(topk)).all()


def test_indexer_edge_rows():
    d = gen.Draw(25)
    B, T, Nc, m, topk = 2, 9, 40, 4, 16
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    q_pos = [0, 60]                  # rows with n_vis = 0, 1, 2 and rows with n_vis > topk
    n_cmp = [Nc, Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    assert (g_idx[0, :3] == -1).all()        # positions 0..2 see no entry
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "edge")


def test_indexer_deterministic():
    d = gen.Draw(26, "cpu")
    B, Nc, m, topk = 2, 40000, 4, 2048
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.FP8)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 1, 16, 64, gen.FP8)
    args = (q_idx, w_idx, k_idx, m, topk, [4 * Nc] * B, [Nc] * B, q_scale, k_scale)
    a = _gpu(*args)
    for _ in range(3):
        b = _gpu(*args)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_indexer_f32_long_rows_ragged():
    # rows longer than the LDS-resident limit on the fp32 score path, several
    # query rows per sequence, with ragged visibility across the batch
    d = gen.Draw(27)
    B, T, Nc, m, topk = 2, 3, 9000, 4, 700
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 4, 32, gen.F32)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 32, gen.F32)
    q_pos = [4 * Nc, 4 * 2500 - 2]          # second sequence: ~2500 visible
    n_cmp = [Nc, Nc - 3]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "f32 long")


def test_indexer_bf16_long_row_single_query():
    d = gen.Draw(28)
    B, Nc, m, topk = 2, 12000, 4, 1024
    q_idx, _, w_idx = gen.indexer_query(d, B, 1, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    q_pos, n_cmp = [4 * Nc, 4 * 9000 + 1], [Nc, Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "bf16 long")


def test_indexer_fp8_rows_beyond_lds_bitmap():
    # 600000 entries (2.4M tokens at m = 4): the ordering bitmap of the row no
    # longer fits in LDS and lives in the workspace
    d = gen.Draw(29, "cpu")
    B, Nc, m, topk = 1, 600000, 4, 2048
    k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.FP8)
    q_idx, q_scale, w_idx = gen.indexer_query(d, B, 2, 16, 64, gen.FP8)
    q_pos, n_cmp = [4 * 550000], [Nc]        # row 0: 550000 visible, row 1: 550000
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "fp8 bitmap in workspace")


def test_indexer_bf16_long_rows_many_query_rows():
    # prefill-shaped rows (T > 1) that see more than 8192 entries: the
    # segment select over rows of one 16-row score group
    d = gen.Draw(41)
    B, T, Nc, m, topk = 2, 40, 9000, 4, 512
    q_idx, _, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    k_idx, _ = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
    q_pos, n_cmp = [4 * 8990, 4 * 8100], [Nc, 8500]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "bf16 long prefill rows")


@pytest.mark.parametrize("path", ["histogram", "segments"])
@pytest.mark.parametrize("Nc,topk", [(163841, 8192), (100000, 7), (65537, 2048), (600000, 16),
                                     (2097152, 16)])
def test_indexer_long_rows_merge_levels(Nc, topk, path):
    # the two long-row paths at row lengths with many selection segments:
    # e4m3 decode rows take the histogram path; bf16 rows of two query
    # positions take the segment path, where 163841 entries with topk 8192
    # need three merge levels (21 -> 6 -> 2 -> 1) and end in a one-entry
    # segment, as does 65537 (9 segments, two levels); 100000 with topk 7 one
    # level; 600000 and the largest row (2^21 entries, 256 segments) with
    # topk 16 two levels of 64-segment groups
    d = gen.Draw(43 + topk % 5, "cpu")
    B, m = 2, 4
    if path == "histogram":
        T = 1
        k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.FP8)
        q_idx, q_scale, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.FP8)
    else:
        T = 2
        k_idx, k_scale = gen.indexer_keys(d, B, Nc, 64, gen.BF16)
        q_idx, q_scale, w_idx = gen.indexer_query(d, B, T, 16, 64, gen.BF16)
    q_pos, n_cmp = [4 * Nc + 3, 4 * 40000], [Nc, Nc]
    g_idx, g_sc = _gpu(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    o = _oracle_rows(q_idx, w_idx, k_idx, m, topk, q_pos, n_cmp, q_scale, k_scale)
    _compare(g_idx, g_sc, o[3], m, topk, q_pos, n_cmp, Nc, "%s merge %d/%d" % (path, Nc, topk))
