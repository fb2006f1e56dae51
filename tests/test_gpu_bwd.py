"""GPU parity of the attention backward (csa_sparse_attn_bwd, hca_dense_attn_bwd)
against the CPU oracle's gradients.

The device gradients use bf16 operands for P and dS (as the forward uses
bf16 for P) with fp32 accumulation; delta = sum_j P_j dP_j is summed in fp32.  Tolerance, per row of a gradient (one head of one query for dq,
one cache row for dK / dV): max |gpu - oracle| <= GRAD_TOL * max |oracle row|
(GRAD_TOL = 1e-2: the bf16 operands P and dS carry 2^-9 relative rounding
each and their products 2^-8, while every row sums many such terms of either
sign, so the row error stays near 2^-8 of the row's scale; the cases here
measure at most 4.7e-3).  attn_mass (a sum of 64 fp32
probabilities, no bf16 rounding on its path): |gpu - oracle| <= 1e-4 + 1e-4 r.
"""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests import brute
from tests.helpers import dev_i32, dev_i64

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRAD_TOL = 1e-2


def _n_vis(pos, ncmp, m, cap):
    return max(0, min(ncmp, (pos + 1) // m, cap))


def _rows_rel(gpu, ref, what, tol=GRAD_TOL):
    """Row-relative check with a floor: a row whose exact gradient vanishes
    (a token that sees one key: P = 1 and dP = delta) is compared against
    1e-3 of the tensor's largest row, the size of the rounding noise that
    the two fp32 sums dP and delta leave."""
    g = np.asarray(gpu, np.float64).reshape(-1, np.asarray(gpu).shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, g.shape[-1])
    assert np.isfinite(g).all(), what + ": non-finite gradient"
    err = np.abs(g - r).max(axis=1)
    scale = np.maximum(np.abs(r).max(axis=1), 1e-3 * np.abs(r).max())
    rel = err / np.maximum(scale, 1e-30)
    worst = np.argsort(-rel)[:3]
    print("%s: worst row-relative error %.3e over %d rows; worst rows %s (err %s, scale %s)"
          % (what, rel.max(), rel.size, worst.tolist(), err[worst].tolist(),
             np.abs(r).max(axis=1)[worst].tolist()))
    bad = rel > tol
    assert not bad.any(), "%s: %d rows over %.1e; worst %.3e (row %d)" % (
        what, bad.sum(), tol, rel.max(), int(np.argmax(rel)))


def _dec(t):
    return t.float().cpu().numpy().astype(np.float64)


def _sink_vec(d, H):
    z = (d.normal(H) * 2.0).float()
    z[0] = -math.inf          # no sink for head 0
    z[1] = 12.0               # a sink above every logit
    return z


def _run_sparse(d, B, T, H, Nc, R, topk, W, q_pos, raw_base, sink=False, pad=0.2):
    D = 128
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    dout = gen.store(d.normal(B, T, H, D), gen.BF16)
    nv = torch.tensor([[_n_vis(q_pos[b] + t, Nc, 4, Nc) for t in range(T)] for b in range(B)])
    idx = gen.random_index_sets(d, B, T, topk, nv, pad)
    z = _sink_vec(d, H) if sink else None
    zd = z.to(DEV) if sink else None
    args = (q.to(DEV), kv_cmp.to(DEV), idx.to(DEV), kv_raw.to(DEV), W, dev_i64(q_pos),
            dev_i64(raw_base))
    out, lse = csa.csa_sparse_attn(*args, want_lse=True, sink=zd)
    dq, dkc, dkr, ds, mass = csa.csa_sparse_attn_bwd(*args, lse, dout.to(DEV), sink=zd,
                                                     want_mass=True)
    torch.cuda.synchronize()
    host = dict(q=gen.host_bits(q), kv_cmp=gen.host_bits(kv_cmp), kv_raw=gen.host_bits(kv_raw),
                idx=idx.numpy(), dout=_dec(dout), sink=None if z is None else z.double().numpy())
    return (dq, dkc, dkr, ds, mass), host


@pytest.mark.parametrize("H,sink", [(64, False), (64, True), (32, False)])
def test_csa_attn_bwd_ragged_matches_oracle(H, sink):
    # ragged everywhere: 77 rows (two 64-row chunks), 150 entries and 260 raw
    # rows (partial 128-key tiles), rows with no compressed entry, a sequence
    # whose early window rows are absent, padded index rows
    d = gen.Draw(500 + H + 7 * sink)
    B, T, Nc, R, topk, W = 2, 77, 150, 260, 40, 45
    q_pos, raw_base = [0, 480], [0, 470]
    (dq, dkc, dkr, ds, mass), h = _run_sparse(d, B, T, H, Nc, R, topk, W, q_pos, raw_base, sink)
    rq, rc, rr, rs, rm = orc.attn_bwd(h["q"], h["kv_cmp"], h["idx"], h["kv_raw"], W, q_pos,
                                      raw_base, h["dout"], sink=h["sink"], want_mass=True)
    _rows_rel(_dec(dq), rq, "dq H=%d" % H)
    _rows_rel(_dec(dkc), rc, "dkv_cmp H=%d" % H)
    _rows_rel(_dec(dkr), rr, "dkv_raw H=%d" % H)
    m = _dec(mass)
    assert np.all(np.abs(m - rm) <= 1e-4 + 1e-4 * np.abs(rm)), np.abs(m - rm).max()
    # rows no token attends stay exactly zero
    assert (_dec(dkc)[rc == 0] == 0).all() and (_dec(dkr)[rr == 0] == 0).all()
    if sink:
        g = _dec(ds)
        np.testing.assert_allclose(g, rs, rtol=GRAD_TOL, atol=GRAD_TOL * np.abs(rs).max())
        assert g[0] == 0  # head 0 has no sink


def test_csa_attn_bwd_window_only_and_empty_rows():
    # topk = 0 (the sliding-window layer) and a second call with every index
    # slot padded: both reduce to the window's gradients
    d = gen.Draw(520)
    B, T, H, Nc, R, W = 1, 70, 64, 40, 70, 30
    for topk, pad in ((0, 0.0), (16, 1.0)):
        (dq, dkc, dkr, _, _), h = _run_sparse(d, B, T, H, Nc, R, topk, W, [0], [0], pad=pad)
        rq, rc, rr, _, _ = orc.attn_bwd(h["q"], h["kv_cmp"], h["idx"], h["kv_raw"], W, 0, 0,
                                        h["dout"])
        _rows_rel(_dec(dq), rq, "dq topk=%d" % topk)
        _rows_rel(_dec(dkr), rr, "dkv_raw topk=%d" % topk)
        assert (_dec(dkc) == 0).all()


@pytest.mark.parametrize("H", [64, 32])
def test_hca_attn_bwd_matches_oracle(H):
    d = gen.Draw(530 + H)
    B, T, D, m, Nc, R, W = 2, 90, 128, 4, 300, 200, 37
    q_pos, n_cmp, raw_base = [300, 0], [Nc, 17], [250, 0]
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    dout = gen.store(d.normal(B, T, H, D), gen.BF16)
    z = _sink_vec(d, H).to(DEV)
    args = (q.to(DEV), kv_cmp.to(DEV), kv_raw.to(DEV), m, W, dev_i64(q_pos), dev_i32(n_cmp),
            dev_i64(raw_base))
    out, lse = csa.hca_dense_attn(*args, want_lse=True, sink=z)
    dq, dkc, dkr, ds, mass = csa.hca_dense_attn_bwd(*args, lse, dout.to(DEV), sink=z,
                                                    want_mass=True)
    torch.cuda.synchronize()
    rq, rc, rr, rs, rm = orc.attn_bwd(gen.host_bits(q), gen.host_bits(kv_cmp), None,
                                      gen.host_bits(kv_raw), W, q_pos, raw_base, _dec(dout),
                                      sink=z.double().cpu().numpy(), m=m, n_cmp=n_cmp,
                                      want_mass=True)
    # per-entry mass, exactly zero for entries a row does not see
    mg = _dec(mass)
    assert np.all(np.abs(mg - rm) <= 1e-4 + 1e-4 * np.abs(rm)), np.abs(mg - rm).max()
    assert (mg[rm == 0] == 0).all()
    _rows_rel(_dec(dq), rq, "hca dq H=%d" % H)
    _rows_rel(_dec(dkc), rc, "hca dkv_cmp H=%d" % H)
    _rows_rel(_dec(dkr), rr, "hca dkv_raw H=%d" % H)
    np.testing.assert_allclose(_dec(ds), rs, rtol=GRAD_TOL, atol=GRAD_TOL * np.abs(rs).max())


def test_csa_attn_bwd_full_8k_prefill():
    # the 8K prefill shape (T = 8192, H = 64, topk = 512, W = 512, 2048
    # entries): dq and attention mass of sampled rows (every row index mod 64,
    # the dK/dV row chunk, and both ends), dK/dV of the entries and raw rows
    # that only the last 40 rows attend (exact from those rows), and for the
    # whole call the identities sum dV = sum dout, sum dK = 0 (no sink) and
    # sum q . dq = sum K . dK
    w = gen.WORKLOADS["csa_prefill_8k_bf16"]
    d = gen.Draw(540, DEV)
    T, H, D, Nc, topk, W = w.T, w.H, w.D, w.n_cmp, w.topk, w.window
    q = gen.store(d.normal(1, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(1, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(1, T, 2 * D), gen.BF16)
    dout = gen.store(d.normal(1, T, H, D), gen.BF16)
    t = torch.arange(T, device=DEV)
    nv = torch.clamp((t + 1) // 4, max=Nc)
    sc = torch.rand(T, Nc, device=DEV, generator=d.g)
    sc[torch.arange(Nc, device=DEV)[None, :] >= nv[:, None]] = -1
    top = sc.topk(topk, dim=1)
    big = torch.full_like(top.indices, 1 << 30)
    idx = torch.where(top.values >= 0, top.indices, big).sort(dim=1).values
    idx = torch.where(idx == (1 << 30), torch.full_like(idx, -1), idx).to(torch.int32)
    idx = idx.view(1, T, topk).contiguous()
    zero = dev_i64([0])
    out, lse = csa.csa_sparse_attn(q, kv_cmp, idx, kv_raw, W, zero, zero, want_lse=True)
    dq, dkc, dkr, _, mass = csa.csa_sparse_attn_bwd(q, kv_cmp, idx, kv_raw, W, zero, zero, lse,
                                                    dout, want_mass=True)
    torch.cuda.synchronize()
    hq, hc, hr = gen.host_bits(q), gen.host_bits(kv_cmp), gen.host_bits(kv_raw)
    hi, hd = idx.cpu().numpy(), _dec(dout)
    rows = sorted(set([0, 1, 63, 64, 4095, 4096] + list(range(5, T, 131)) + [T - 1]))
    rows = sorted(set(rows + [64 * k + (k % 64) for k in range(T // 64)][::2]))
    gq, gm = _dec(dq), _dec(mass)
    for i in range(0, len(rows), 48):
        part = rows[i:i + 48]
        rq = np.zeros((1, len(part), H, D))
        rm = np.zeros((1, len(part), topk))
        for k, r in enumerate(part):
            a, _, _, _, b = orc.attn_bwd(hq[:, r:r + 1], hc, hi[:, r:r + 1], hr, W, r, 0,
                                         hd[:, r:r + 1], want_mass=True)
            rq[:, k], rm[:, k] = a[:, 0], b[:, 0]
        _rows_rel(gq[:, part], rq, "8k dq rows %d..%d" % (part[0], part[-1]))
        assert np.all(np.abs(gm[:, part] - rm) <= 1e-4 + 1e-4 * np.abs(rm))
    t0 = T - 40
    _, rc, rr, _, _ = orc.attn_bwd(hq[:, t0:], hc, hi[:, t0:], hr, W, t0, 0, hd[:, t0:])
    jc = (t0 + 1) // 4 + 1          # entries no row before t0 can see
    _rows_rel(_dec(dkc)[0, jc:], rc[0, jc:], "8k dkv_cmp tail entries")
    _rows_rel(_dec(dkr)[0, t0:], rr[0, t0:], "8k dkv_raw tail rows")
    # identities over the whole call (fp32 sums of fp32 gradients)
    gc, gr = _dec(dkc), _dec(dkr)
    sdv = gc[0, :, D:].sum(0) + gr[0, :, D:].sum(0)
    sdo = hd[0].sum((0, 1))
    e_dv = np.abs(sdv - sdo).max() / np.abs(sdo).max()
    sdk = gc[0, :, :D].sum(0) + gr[0, :, :D].sum(0)
    e_dk = np.abs(sdk).max() / (np.abs(gc[0, :, :D]).sum(0) + np.abs(gr[0, :, :D]).sum(0)).max()
    qv, kc, kr = brute.decode_bits(hq), brute.decode_bits(hc), brute.decode_bits(hr)
    lhs = (qv * gq).sum()
    rhs = (kc[0, :, :D] * gc[0, :, :D]).sum() + (kr[0, :, :D] * gr[0, :, :D]).sum()
    e_bl = abs(lhs - rhs) / np.abs(qv * gq).sum()
    print("8k identities: sum dV %.2e, sum dK %.2e, q.dq vs K.dK %.2e" % (e_dv, e_dk, e_bl))
    assert e_dv <= 1e-2 and e_dk <= 1e-2 and e_bl <= 1e-2


def test_hca_attn_bwd_1m_chunk_shape():
    # the 1M-context HCA chunk (T = 4096 at position 1M - 4096, 8192 entries of
    # m = 128, W = 512): dq and the per-entry mass of three runs of rows (the
    # first 16, 16 in the middle, the last 40), dK/dV of the entry and the raw
    # rows only the last 40 rows see (exact from those rows), and the identities
    # sum dV = sum dout, sum dK = 0 and sum q . dq = sum K . dK over the call
    w = gen.WORKLOADS["hca_prefill_1m_chunk4k"]
    d = gen.Draw(630, DEV)
    T, H, D, Nc, W, m = w.T, w.H, w.D, w.n_cmp, w.window, w.m
    qp, R = w.ctx - T, w.T + w.window - 1
    rbase = qp - (W - 1)
    q = gen.store(d.normal(1, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(1, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(1, R, 2 * D), gen.BF16)
    dout = gen.store(d.normal(1, T, H, D), gen.BF16)
    args = (q, kv_cmp, kv_raw, m, W, dev_i64([qp]), dev_i32([Nc]), dev_i64([rbase]))
    out, lse = csa.hca_dense_attn(*args, want_lse=True)
    dq, dkc, dkr, _, mass = csa.hca_dense_attn_bwd(*args, lse, dout, want_mass=True)
    torch.cuda.synchronize()
    hq, hc, hr, hd = gen.host_bits(q), gen.host_bits(kv_cmp), gen.host_bits(kv_raw), _dec(dout)
    gq, gm, gc, gr = _dec(dq), _dec(mass), _dec(dkc), _dec(dkr)
    t0 = T - 40
    for a, n in ((0, 16), (T // 2 - 8, 16), (t0, 40)):
        rq, rc, rr, _, rm = orc.attn_bwd(hq[:, a:a + n], hc, None, hr, W, qp + a, rbase,
                                         hd[:, a:a + n], m=m, n_cmp=Nc, want_mass=True)
        _rows_rel(gq[:, a:a + n], rq, "1m hca dq rows %d.." % a)
        assert np.all(np.abs(gm[:, a:a + n] - rm) <= 1e-4 + 1e-4 * np.abs(rm))
    # rc, rr: from the last 40 rows; an entry first seen at row m (j + 1) - 1 - qp
    jc = -(-(t0 + 1 + qp) // m) - 1
    ic = t0 + qp - rbase            # raw rows no row before t0 sees
    _rows_rel(gc[0, jc:], rc[0, jc:], "1m hca dkv_cmp tail entries")
    _rows_rel(gr[0, ic:], rr[0, ic:], "1m hca dkv_raw tail rows")
    sdv = gc[0, :, D:].sum(0) + gr[0, :, D:].sum(0)
    sdo = hd[0].sum((0, 1))
    e_dv = np.abs(sdv - sdo).max() / np.abs(sdo).max()
    sdk = gc[0, :, :D].sum(0) + gr[0, :, :D].sum(0)
    e_dk = np.abs(sdk).max() / (np.abs(gc[0, :, :D]).sum(0) + np.abs(gr[0, :, :D]).sum(0)).max()
    qv, kc, kr = brute.decode_bits(hq), brute.decode_bits(hc), brute.decode_bits(hr)
    lhs = (qv * gq).sum()
    rhs = (kc[0, :, :D] * gc[0, :, :D]).sum() + (kr[0, :, :D] * gr[0, :, :D]).sum()
    e_bl = abs(lhs - rhs) / np.abs(qv * gq).sum()
    print("1m hca identities: sum dV %.2e, sum dK %.2e, q.dq vs K.dK %.2e" % (e_dv, e_dk, e_bl))
    assert e_dv <= 1e-2 and e_dk <= 1e-2 and e_bl <= 1e-2
    # every row sees at least 8160 entries: the mass of a row sums to its
    # non-window probability, at most the head count
    assert (gm.sum(-1) <= H * (1 + 1e-5)).all()


# ---------------------------------------------------------------- indexer KL loss
# loss: fp32 scores (bf16 inputs, fp32 MFMA accumulation) and fp32 softmax:
# |gpu - oracle| <= 1e-4 (1 + |oracle|); dw (fp32 sums): row-relative 1e-4;
# dq and dk (the coefficients dI w [v > 0] rounded to bf16 for the MFMA):
# row-relative GRAD_TOL as above.

def _kl_inputs(d, B, T, Nc, topk, q_pos):
    qi = gen.store(d.normal(B, T, 16, 64), gen.BF16)
    wi = d.normal(B, T, 16).float().contiguous()
    ki = gen.store(d.normal(B, Nc, 64), gen.BF16)
    nv = torch.tensor([[_n_vis(q_pos[b] + t, Nc, 4, Nc) for t in range(T)] for b in range(B)])
    idx = gen.random_index_sets(d, B, T, topk, nv, 0.15)
    mass = (torch.rand(B, T, topk, generator=d.g) * (idx >= 0)).float()
    return qi, wi, ki, idx, mass


def _kl_check(res, ref, what, with_dk=True):
    loss, dq, dw = (_dec(x) for x in res[:3])
    rl, rq, rw = ref[:3]
    assert np.all(np.abs(loss - rl) <= 1e-4 * (1 + np.abs(rl))), (what, np.abs(loss - rl).max())
    _rows_rel(dw, rw, what + " dw", tol=1e-4)
    _rows_rel(dq, rq, what + " dq")
    if with_dk:
        _rows_rel(_dec(res[3]), ref[3], what + " dk")


@pytest.mark.parametrize("Nc,topk,pos1", [(300, 100, 900), (700, 600, 2800)])
def test_indexer_kl_bwd_ragged_matches_oracle(Nc, topk, pos1):
    # 100 slots (a partial 16-slot tile and a partial 32-slot step of the dq
    # product), rows without a selected entry, a row whose mass is zero, a
    # per-row gradient scale, 300 entries (a partial 128-entry dk tile); 600
    # slots take the row kernel's variant for more than 512 slots (three
    # 256-slot dq chunks, the last partial)
    d = gen.Draw(560 + topk)
    B, T = 2, 70
    q_pos = [0, pos1]  # (the second sequence sees every entry at pos1 = 2800)
    qi, wi, ki, idx, mass = _kl_inputs(d, B, T, Nc, topk, q_pos)
    idx[1, 5] = -1
    mass[1, 6] = 0.0
    gs = (torch.rand(B, T, generator=d.g) + 0.5).float()
    res = csa.csa_indexer_kl_bwd(qi.to(DEV), wi.to(DEV), ki.to(DEV), idx.to(DEV), mass.to(DEV),
                                 gs.to(DEV))
    torch.cuda.synchronize()
    ref = orc.indexer_kl_bwd(gen.host_bits(qi), wi.numpy(), gen.host_bits(ki), idx.numpy(),
                             mass.double().numpy(), gs.double().numpy())
    _kl_check(res, ref, "kl ragged")
    assert float(res[0][1, 5]) == 0.0 and float(res[0][1, 6]) == 0.0
    assert (_dec(res[1])[1, 5] == 0).all() and (_dec(res[2])[1, 6] == 0).all()


def test_indexer_kl_bwd_8k_prefill_shape():
    # T = 8192, 2048 entries, topk = 512: loss, dq, dw of sampled rows (both
    # ends, every 131st row) and dk of the entries only the last 40 rows see
    d = gen.Draw(570)
    B, T, Nc, topk = 1, 8192, 2048, 512
    qi, wi, ki, idx, mass = _kl_inputs(d, B, T, Nc, topk, [0])
    res = csa.csa_indexer_kl_bwd(qi.to(DEV), wi.to(DEV), ki.to(DEV), idx.to(DEV), mass.to(DEV))
    torch.cuda.synchronize()
    hq, hk, hi, hm, hw = (gen.host_bits(qi), gen.host_bits(ki), idx.numpy(),
                          mass.double().numpy(), wi.numpy())
    rows = sorted(set([0, 1, 4095, 4096] + list(range(5, T, 131)) + [T - 1]))
    loss, dq, dw, _ = (_dec(x) for x in res)
    rl, rq, rw, _ = orc.indexer_kl_bwd(hq[:, rows], hw[:, rows], hk, hi[:, rows], hm[:, rows])
    _kl_check((res[0][:, rows], res[1][:, rows], res[2][:, rows]), (rl, rq, rw), "kl 8k rows",
              with_dk=False)
    t0 = T - 40
    _, _, _, rk = orc.indexer_kl_bwd(hq[:, t0:], hw[:, t0:], hk, hi[:, t0:], hm[:, t0:])
    jc = (t0 + 1) // 4 + 1
    _rows_rel(_dec(res[3])[0, jc:], rk[0, jc:], "kl 8k dk tail entries")


# dense form: the same tolerances; the selected set of a row is every visible
# entry, the target the dense attention's mass per entry [B, T, Nc_cap]

def _dense_kl_inputs(d, B, T, Nc, m, q_pos, n_cmp):
    qi = gen.store(d.normal(B, T, 16, 64), gen.BF16)
    wi = d.normal(B, T, 16).float().contiguous()
    ki = gen.store(d.normal(B, Nc, 64), gen.BF16)
    nv = torch.tensor([[_n_vis(q_pos[b] + t, n_cmp[b], m, Nc) for t in range(T)]
                       for b in range(B)])
    seen = torch.arange(Nc)[None, None, :] < nv[:, :, None]
    mass = (torch.rand(B, T, Nc, generator=d.g) * seen).float()
    return qi, wi, ki, mass, seen


def _dense_rows_ref(hq, hw, hk, hm_rows, rows, nv):
    """The oracle's dense loss for chosen rows of batch 0 (hm_rows: their
    mass): the sparse form over each row's visible entries, as the dense
    form is defined."""
    Nc = hk.shape[1]
    idx = np.full((1, len(rows), Nc), -1, np.int32)
    for i, t in enumerate(rows):
        idx[0, i, :nv[t]] = np.arange(nv[t], dtype=np.int32)
    return orc.indexer_kl_bwd(hq[:, rows], hw[:, rows], hk, idx, hm_rows)


def test_indexer_kl_dense_bwd_ragged_matches_oracle():
    # 300 entries (a partial 128-entry dk tile), the second sequence seeing
    # 275 .. 290 entries (two 256-entry chunks, the second partial, and a
    # partial 16-entry tile), rows of the first that see no entry, a row
    # whose mass is zero, a per-row gradient scale; the mass past n_vis and
    # the key rows past n_cmp hold NaN, which must not be read
    d = gen.Draw(600)
    B, T, Nc, m = 2, 70, 300, 4
    q_pos, n_cmp = [0, 1100], [300, 290]
    qi, wi, ki, mass, seen = _dense_kl_inputs(d, B, T, Nc, m, q_pos, n_cmp)
    mass[1, 6] = 0.0
    gs = (torch.rand(B, T, generator=d.g) + 0.5).float()
    mg = torch.where(seen, mass, torch.full_like(mass, float("nan")))
    kg = ki.clone()
    kg[1, n_cmp[1]:] = float("nan")
    res = csa.csa_indexer_kl_dense_bwd(qi.to(DEV), wi.to(DEV), kg.to(DEV), m, dev_i64(q_pos),
                                       dev_i32(n_cmp), mg.to(DEV), gs.to(DEV))
    torch.cuda.synchronize()
    ref = orc.indexer_kl_dense_bwd(gen.host_bits(qi), wi.numpy(), gen.host_bits(ki), m, q_pos,
                                   n_cmp, mass.double().numpy(), gs.double().numpy())
    _kl_check(res, ref, "kl dense ragged")
    for t in (0, 1, 2):  # no visible entry
        assert float(res[0][0, t]) == 0.0 and (_dec(res[1])[0, t] == 0).all()
    assert float(res[0][1, 6]) == 0.0 and (_dec(res[2])[1, 6] == 0).all()
    assert (_dec(res[3])[1, n_cmp[1]:] == 0).all()


def test_indexer_kl_dense_bwd_without_entries():
    # an empty cache (Nc_cap = 0): every row has loss 0 and no gradient, and
    # neither the mass nor the keys are read
    d = gen.Draw(605)
    B, T = 2, 9
    qi = gen.store(d.normal(B, T, 16, 64), gen.BF16).to(DEV)
    wi = d.normal(B, T, 16).float().contiguous().to(DEV)
    ki = torch.empty(B, 0, 64, dtype=torch.bfloat16, device=DEV)
    mass = torch.empty(B, T, 0, dtype=torch.float32, device=DEV)
    loss, dq, dw, dk = csa.csa_indexer_kl_dense_bwd(qi, wi, ki, 4, dev_i64([0, 100]),
                                                    dev_i32([0, 0]), mass)
    torch.cuda.synchronize()
    assert (_dec(loss) == 0).all() and (_dec(dq) == 0).all() and (_dec(dw) == 0).all()
    assert dk.shape == (B, 0, 64)


def test_indexer_kl_dense_bwd_8k_shape():
    # T = 8192 and 2048 entries of the m = 4 cache: loss, dq, dw of sampled
    # rows (both ends, every 131st row) and dk of the entries only the last
    # 40 rows see
    d = gen.Draw(610, DEV)
    B, T, Nc, m = 1, 8192, 2048, 4
    qi = gen.store(d.normal(B, T, 16, 64), gen.BF16)
    wi = d.normal(B, T, 16).float().contiguous()
    ki = gen.store(d.normal(B, Nc, 64), gen.BF16)
    nv = [_n_vis(t, Nc, m, Nc) for t in range(T)]
    seen = torch.arange(Nc, device=DEV)[None, :] < torch.tensor(nv, device=DEV)[:, None]
    mass = (torch.rand(B, T, Nc, device=DEV, generator=d.g) * seen).float()
    zero = dev_i64([0])
    res = csa.csa_indexer_kl_dense_bwd(qi, wi, ki, m, zero, dev_i32([Nc]), mass)
    torch.cuda.synchronize()
    hq, hk, hw = gen.host_bits(qi), gen.host_bits(ki), wi.cpu().numpy()
    rows = sorted(set([0, 1, 3, 4, 1023, 1024, 4095, 4096] + list(range(5, T, 131)) + [T - 1]))
    rl, rq, rw, _ = _dense_rows_ref(hq, hw, hk, mass[:, rows].double().cpu().numpy(), rows, nv)
    _kl_check((res[0][:, rows], res[1][:, rows], res[2][:, rows]), (rl, rq, rw),
              "kl dense 8k rows", with_dk=False)
    t0 = T - 40
    _, _, _, rk = orc.indexer_kl_dense_bwd(hq[:, t0:], hw[:, t0:], hk, m, [t0], [Nc],
                                           mass[:, t0:].double().cpu().numpy())
    jc = (t0 + 1) // m + 1
    _rows_rel(_dec(res[3])[0, jc:], rk[0, jc:], "kl dense 8k dk tail entries")


def test_dense_indexer_loss_on_the_dense_attention_mass():
    # the chain of the dense form: the HCA-form attention backward's per-entry
    # mass as the target of the dense indexer loss, on the device and in the
    # oracle (each side from its own mass)
    d = gen.Draw(620)
    B, T, H, D, m, Nc, R, W = 1, 96, 64, 128, 4, 40, 96, 16
    q_pos, n_cmp, raw_base = [60], [Nc], [0]
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    dout = gen.store(d.normal(B, T, H, D), gen.BF16)
    qi = gen.store(d.normal(B, T, 16, 64), gen.BF16)
    wi = d.normal(B, T, 16).float().contiguous()
    ki = gen.store(d.normal(B, Nc, 64), gen.BF16)
    args = (q.to(DEV), kv_cmp.to(DEV), kv_raw.to(DEV), m, W, dev_i64(q_pos), dev_i32(n_cmp),
            dev_i64(raw_base))
    out, lse = csa.hca_dense_attn(*args, want_lse=True)
    mass = csa.hca_dense_attn_bwd(*args, lse, dout.to(DEV), want_mass=True)[4]
    res = csa.csa_indexer_kl_dense_bwd(qi.to(DEV), wi.to(DEV), ki.to(DEV), m, dev_i64(q_pos),
                                       dev_i32(n_cmp), mass)
    torch.cuda.synchronize()
    rm = orc.attn_bwd(gen.host_bits(q), gen.host_bits(kv_cmp), None, gen.host_bits(kv_raw), W,
                      q_pos, raw_base, _dec(dout), m=m, n_cmp=n_cmp, want_mass=True)[4]
    ref = orc.indexer_kl_dense_bwd(gen.host_bits(qi), wi.numpy(), gen.host_bits(ki), m, q_pos,
                                   n_cmp, rm)
    _kl_check(res, ref, "kl dense on hca mass")


# ---------------------------------------------------------------- compressor
# dP and dG enter the two products as bf16 (fp32 accumulation): dx, dW row-
# relative GRAD_TOL; dape (fp32 sums): row-relative 1e-4.

def _cmp_inputs(d, B, L, dm, E, m, o, ape=True):
    x = gen.store(d.normal(B, L, dm), gen.BF16)
    wk = gen.store(d.normal(E, dm, std=dm ** -0.5), gen.BF16)
    wg = gen.store(d.normal(E, dm, std=dm ** -0.5), gen.BF16)
    ap = (d.normal((1 + o) * m, E) * 0.3).float().contiguous() if ape else None
    return x, wk, wg, ap


@pytest.mark.parametrize("m,o,rotate,E,Nc", [(4, 1, False, 128, 30), (4, 1, True, 64, 12),
                                            (3, 0, False, 128, 40)])
def test_compress_bwd_matches_oracle(m, o, rotate, E, Nc):
    # L = 75 is no multiple of m (trailing tokens without an entry); Nc = 12
    # keeps fewer entries than L / m (the rest get no gradient)
    d = gen.Draw(580 + m + 3 * rotate)
    B, L, dm = 2, 75, 128
    x, wk, wg, ap = _cmp_inputs(d, B, L, dm, E, m, o)
    dC = d.normal(B, Nc, E).float().contiguous()
    dx, dwk, dwg, dape = csa.csa_compress_bwd(x.to(DEV), wk.to(DEV), wg.to(DEV), m, o, Nc,
                                              dC.to(DEV), ape=ap.to(DEV), rotate=rotate)
    torch.cuda.synchronize()
    rx, rk, rg, ra = orc.compress_bwd(gen.host_bits(x), gen.host_bits(wk), gen.host_bits(wg), m,
                                      o, Nc, dC.double().numpy(), ape=ap.double().numpy(),
                                      rotate=rotate)
    _rows_rel(_dec(dx), rx, "cmp dx")
    _rows_rel(_dec(dwk), rk, "cmp dw_kv")
    _rows_rel(_dec(dwg), rg, "cmp dw_gate")
    _rows_rel(_dec(dape), ra, "cmp dape", tol=1e-4)
    n_ent = min(L // m, Nc)
    assert (_dec(dx)[:, n_ent * m:] == 0).all()  # tokens of no entry


@pytest.mark.parametrize("rotate,interleaved,E", [(False, False, 128), (True, False, 64),
                                                   (False, True, 96)])
def test_compress_bwd_with_norm_and_rope_matches_oracle(rotate, interleaved, E):
    # entries RMS-normed and rotated on a channel slice at their positions
    # m i (base 100: sizeable angles), optionally Hadamard-rotated; L = 75 is
    # no multiple of m; E = 96 is no power of two (the entry kernel's block
    # sums over any width); the norm weight's gradient to fp32 accuracy
    d = gen.Draw(600 + E + rotate)
    m, o, Nc = 4, 1, 16
    B, L, dm = 2, 75, 128
    x, wk, wg, ap = _cmp_inputs(d, B, L, dm, E, m, o)
    nw = (1.0 + 0.3 * d.normal(E)).float().contiguous()
    dC = d.normal(B, Nc, E).float().contiguous()
    opt = dict(norm_eps=1e-5, rope_dim=32, rope_offset=8, rope_base=100.0,
               rope_interleaved=interleaved)
    dx, dwk, dwg, dape, dnw = csa.csa_compress_bwd_ex(
        x.to(DEV), wk.to(DEV), wg.to(DEV), m, o, Nc, dC.to(DEV), ape=ap.to(DEV), rotate=rotate,
        norm_weight=nw.to(DEV), **opt)
    torch.cuda.synchronize()
    rx, rk, rg, ra, rn = orc.compress_bwd_ex(
        gen.host_bits(x), gen.host_bits(wk), gen.host_bits(wg), m, o, Nc, dC.double().numpy(),
        ape=ap.double().numpy(), rotate=rotate, norm_weight=nw.double().numpy(), **opt)
    _rows_rel(_dec(dx), rx, "cmp+norm dx")
    _rows_rel(_dec(dwk), rk, "cmp+norm dw_kv")
    _rows_rel(_dec(dwg), rg, "cmp+norm dw_gate")
    _rows_rel(_dec(dape), ra, "cmp+norm dape", tol=1e-4)
    _rows_rel(_dec(dnw)[None], rn[None], "cmp+norm dnorm_w", tol=1e-4)
    # the same call without options is csa_compress_bwd's
    a = csa.csa_compress_bwd(x.to(DEV), wk.to(DEV), wg.to(DEV), m, o, Nc, dC.to(DEV),
                             ape=ap.to(DEV), rotate=rotate)
    b_ = csa.csa_compress_bwd_ex(x.to(DEV), wk.to(DEV), wg.to(DEV), m, o, Nc, dC.to(DEV),
                                 ape=ap.to(DEV), rotate=rotate)
    torch.cuda.synchronize()
    for u, v, name in zip(a, b_[:4], ("dx", "dw_kv", "dw_gate", "dape")):
        assert torch.equal(u, v), name
    assert b_[4] is None


def test_compress_bwd_with_norm_and_rope_main_width():
    # the main compressor's width (E = 256: [K | V], the rotary slice the
    # key's first 64 channels, the usual base) on 1024 tokens of a 1024-wide
    # model: every output against the oracle
    d = gen.Draw(610, DEV)
    B, L, dm, E, m, o = 1, 1024, 1024, 256, 4, 1
    Nc = L // m
    x, wk, wg, ap = _cmp_inputs(d, B, L, dm, E, m, o)
    nw = (1.0 + 0.3 * d.normal(E)).float().contiguous()
    dC = d.normal(B, Nc, E).float().contiguous()
    opt = dict(norm_eps=1e-6, rope_dim=64, rope_offset=0, rope_base=10000.0)
    dx, dwk, dwg, dape, dnw = csa.csa_compress_bwd_ex(x, wk, wg, m, o, Nc, dC, ape=ap,
                                                      norm_weight=nw, **opt)
    torch.cuda.synchronize()
    rx, rk, rg, ra, rn = orc.compress_bwd_ex(
        gen.host_bits(x), gen.host_bits(wk), gen.host_bits(wg), m, o, Nc,
        dC.double().cpu().numpy(), ape=ap.double().cpu().numpy(),
        norm_weight=nw.double().cpu().numpy(), **opt)
    _rows_rel(_dec(dx), rx, "main-width dx")
    _rows_rel(_dec(dwk), rk, "main-width dw_kv")
    _rows_rel(_dec(dwg), rg, "main-width dw_gate")
    _rows_rel(_dec(dape), ra, "main-width dape", tol=1e-4)
    _rows_rel(_dec(dnw)[None], rn[None], "main-width dnorm_w", tol=1e-4)


def test_compress_bwd_stacked_weights_in_place():
    # weights kept as one [2E, d_model] buffer (w_gate right after w_kv) and
    # weight gradients likewise are used in place: the same products as the
    # stacking copies of separate buffers, so the results are bit-identical
    d = gen.Draw(585)
    B, L, dm, E, m, o, Nc = 2, 75, 128, 64, 4, 1, 18
    x, wk, wg, ap = _cmp_inputs(d, B, L, dm, E, m, o)
    dC = d.normal(B, Nc, E).float().contiguous().to(DEV)
    x, wk, wg, ap = x.to(DEV), wk.to(DEV), wg.to(DEV), ap.to(DEV)
    sep = csa.csa_compress_bwd(x, wk.clone(), wg.clone(), m, o, Nc, dC, ape=ap)
    wcat = torch.cat([wk, wg]).contiguous()
    dwcat = torch.full((2 * E, dm), float("nan"), device=DEV)
    st = csa.csa_compress_bwd(x, wcat[:E], wcat[E:], m, o, Nc, dC, ape=ap,
                              dw_kv=dwcat[:E], dw_gate=dwcat[E:])
    torch.cuda.synchronize()
    for a, b_, name in zip(sep, st, ("dx", "dw_kv", "dw_gate", "dape")):
        assert torch.equal(a, b_), name
    assert torch.equal(dwcat, torch.cat([sep[1], sep[2]]))


@pytest.mark.parametrize("E", [256, 64])
def test_compress_bwd_8k_main_compressor(E):
    # the 8K prefill chunk's compressors (L = 8192, d_model = 4096, m = 4 with
    # overlap; E = 256 the main one, E = 64 the indexer's, whose weight
    # gradient is summed from four token-range partial products): dW rows of
    # sampled channels (the pool is per channel, so a one-channel oracle call
    # gives them exactly), dx of sampled tokens from a local slice (a token's
    # gradient depends on the two windows that hold it), and for everything
    # the bilinear identity
    # sum_j x_j . dx_j = sum W_kv . dW_kv + sum W_gate . dW_gate
    d = gen.Draw(590 + E, DEV)
    B, L, dm, m, o = 1, 8192, 4096, 4, 1
    Nc = L // m
    x, wk, wg, ap = _cmp_inputs(d, B, L, dm, E, m, o)
    dC = d.normal(B, Nc, E).float().contiguous()
    dx, dwk, dwg, dape = csa.csa_compress_bwd(x, wk, wg, m, o, Nc, dC, ape=ap)
    torch.cuda.synchronize()
    hx, hk, hg, ha, hd = (gen.host_bits(x), gen.host_bits(wk), gen.host_bits(wg),
                          ap.double().cpu().numpy(), dC.double().cpu().numpy())
    for e in ((0, 1, 63, 64, 129, 255) if E == 256 else (0, 1, 31, 32, 63)):
        _, rk, rg, ra = orc.compress_bwd(hx, hk[e:e + 1], hg[e:e + 1], m, o, Nc,
                                         hd[:, :, e:e + 1], ape=ha[:, e:e + 1])
        _rows_rel(_dec(dwk[e:e + 1]), rk, "8k dw_kv channel %d" % e)
        _rows_rel(_dec(dwg[e:e + 1]), rg, "8k dw_gate channel %d" % e)
        np.testing.assert_allclose(_dec(dape)[:, e], ra[:, 0], rtol=1e-4,
                                   atol=1e-4 * np.abs(ra).max())
    for q0 in (0, 1000, 2047 - 16):
        j0 = 4 * q0
        sl = slice(j0, j0 + 64)
        rx, _, _, _ = orc.compress_bwd(hx[:, sl], hk, hg, m, o, 16, hd[:, q0:q0 + 16],
                                       ape=ha)
        lo = 0 if q0 == 0 else 4   # a slice's first block lacks its previous block
        _rows_rel(_dec(dx)[0, j0 + lo:j0 + 56], rx[0, lo:56], "8k dx tokens %d.." % j0)
    xv, wkv, wgv = (brute.decode_bits(a) for a in (hx, hk, hg))
    lhs = (xv * _dec(dx)).sum()
    rhs = (wkv * _dec(dwk)).sum() + (wgv * _dec(dwg)).sum()
    print("8k compressor identity: %.3e vs %.3e" % (lhs, rhs))
    assert abs(lhs - rhs) <= 1e-3 * (np.abs(xv * _dec(dx)).sum())


def test_training_step_end_to_end_small():
    # forward (both compressors, the indexer, the attention) and backward
    # (attention, indexer KL loss, both compressors) on the device, against
    # the oracle's own chain (its entries rounded to the bf16 the caches
    # store): the index sets agree exactly, then the losses, and the input and
    # weight gradients within the gradient tolerance (errors compound over
    # the chain: 2 GRAD_TOL)
    d = gen.Draw(600)
    B, T, dm, H, D, HI, dI, m, o, topk, W = 1, 128, 128, 64, 128, 16, 64, 4, 1, 8, 16
    Nc = T // m
    x = gen.store(d.normal(B, T, dm), gen.BF16)
    wk, wg = gen.compressor_weights(d, dm, 2 * D, gen.BF16)
    wik, wig = gen.compressor_weights(d, dm, dI, gen.BF16)
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_raw = gen.store(d.normal(B, T, 2 * D), gen.BF16)
    qi = gen.store(d.normal(B, T, HI, dI), gen.BF16)
    wi = d.normal(B, T, HI).float().contiguous()
    dout = gen.store(d.normal(B, T, H, D), gen.BF16)
    z = dev_i64([0])
    dv = lambda t: t.to(DEV)
    kv_cmp = torch.empty(B, Nc, 2 * D, dtype=torch.bfloat16, device=DEV)
    k_idx = torch.empty(B, Nc, dI, dtype=torch.bfloat16, device=DEV)
    csa.csa_compress(dv(x), dv(wk), dv(wg), z, m, o, kv_cmp)
    csa.csa_compress(dv(x), dv(wik), dv(wig), z, m, o, k_idx)
    idx, _ = csa.csa_indexer_topk(dv(qi), dv(wi), k_idx, m, topk, z, dev_i32([Nc]))
    out, lse = csa.csa_sparse_attn(dv(q), kv_cmp, idx, dv(kv_raw), W, z, z, want_lse=True)
    dq, dkc, dkr, _, mass = csa.csa_sparse_attn_bwd(dv(q), kv_cmp, idx, dv(kv_raw), W, z, z, lse,
                                                    dv(dout), want_mass=True)
    loss, dqi, dwi, dki = csa.csa_indexer_kl_bwd(dv(qi), dv(wi), k_idx, idx, mass)
    dx1, dwk, dwg, _ = csa.csa_compress_bwd(dv(x), dv(wk), dv(wg), m, o, Nc, dkc)
    dx2, dwik, dwig, _ = csa.csa_compress_bwd(dv(x), dv(wik), dv(wig), m, o, Nc, dki)
    torch.cuda.synchronize()
    # the oracle's chain
    hx, hwk, hwg, hwik, hwig = (gen.host_bits(t) for t in (x, wk, wg, wik, wig))
    c1, _, _ = orc.compress(hx, hwk, hwg, m, o, 0, Nc, want_state=False)
    c2, _, _ = orc.compress(hx, hwik, hwig, m, o, 0, Nc, want_state=False)
    enc = np.vectorize(orc.bf16_encode, otypes=[np.uint16])
    r_kv, r_k = enc(c1), enc(c2)
    r_idx = orc.indexer_topk(gen.host_bits(qi), wi.numpy(), r_k, m, topk, 0, Nc)[0]
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    hdo = _dec(dout)
    _, rkc, rkr, _, rmass = orc.attn_bwd(gen.host_bits(q), r_kv, r_idx, gen.host_bits(kv_raw), W,
                                         0, 0, hdo, want_mass=True)
    rl, rqi, rwi, rki = orc.indexer_kl_bwd(gen.host_bits(qi), wi.numpy(), r_k, r_idx, rmass)
    rx1, rwk, rwg, _ = orc.compress_bwd(hx, hwk, hwg, m, o, Nc, rkc)
    rx2, rwik, rwig, _ = orc.compress_bwd(hx, hwik, hwig, m, o, Nc, rki)
    assert np.all(np.abs(_dec(loss) - rl) <= 1e-3 * (1 + np.abs(rl)))
    tol = 2 * GRAD_TOL
    _rows_rel(_dec(dqi), rqi, "e2e dq_idx", tol)
    _rows_rel(_dec(dwi), rwi, "e2e dw_idx", tol)
    _rows_rel(_dec(dx1) + _dec(dx2), rx1 + rx2, "e2e dx", tol)
    _rows_rel(_dec(dwk), rwk, "e2e dw_kv", tol)
    _rows_rel(_dec(dwg), rwg, "e2e dw_gate", tol)
    _rows_rel(_dec(dwik), rwik, "e2e indexer dw_kv", tol)
    _rows_rel(_dec(dwig), rwig, "e2e indexer dw_gate", tol)
