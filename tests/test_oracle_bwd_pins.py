"""CPU pins of the oracle's backward functions (attention, indexer KL loss,
compressor).

Each gradient is checked against something other than the oracle's own
formulas: torch autograd through a library attention (scaled dot-product
attention with an explicit mask, float64) or through torch's KL divergence,
central finite differences of the oracle's forward functions (themselves
pinned in test_oracle_pins.py), and identities the chain rule fixes exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as orc
from tests import brute


def rng(seed):
    return np.random.default_rng(seed)


def _case(seed, B=2, T=7, H=3, D=8, Nc=10, R=16, topk=4, dt=np.float32):
    r = rng(seed)
    q = r.normal(0, 1, (B, T, H, D)).astype(dt)
    kv_cmp = r.normal(0, 1, (B, Nc, 2 * D)).astype(dt)
    kv_raw = r.normal(0, 1, (B, R, 2 * D)).astype(dt)
    idx = np.full((B, T, topk), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = r.integers(0, topk + 1)
            idx[b, t, :n] = np.sort(r.choice(Nc, n, replace=False))
    dout = r.normal(0, 1, (B, T, H, D))
    return q, kv_cmp, kv_raw, idx, dout


def _autograd_attention(q, kv_cmp, kv_raw, masks, dout, scale, sink=None):
    """Gradients of sum(dout * out) through a library attention over the
    concatenated [compressed | raw] rows with a boolean mask per batch."""
    B, T, H, D = q.shape
    Nc = kv_cmp.shape[1]
    qt = torch.tensor(brute.decode_bits(q), requires_grad=True)
    kc = torch.tensor(brute.decode_bits(kv_cmp), requires_grad=True)
    kr = torch.tensor(brute.decode_bits(kv_raw), requires_grad=True)
    zs = torch.tensor(np.asarray(sink, np.float64), requires_grad=True) if sink is not None else None
    total = 0
    for b in range(B):
        rows = torch.cat([kc[b], kr[b]])
        m = torch.as_tensor(masks[b])
        qh = qt[b].permute(1, 0, 2)                                   # H, T, D
        k = rows[:, :D].unsqueeze(0).expand(H, -1, -1)
        v = rows[:, D:].unsqueeze(0).expand(H, -1, -1)
        if zs is None:
            # rows with an empty key set give out = 0 (SDPA would give NaN)
            live = m.any(-1)
            mm = m.clone()
            mm[~live, 0] = True
            out = F.scaled_dot_product_attention(qh, k, v, attn_mask=mm.unsqueeze(0), scale=scale)
            out = out * live[None, :, None]
        else:
            logits = torch.matmul(qh, k.transpose(1, 2).contiguous()) * scale
            logits = logits.masked_fill(~m.unsqueeze(0), float("-inf"))
            z = zs[:, None, None].expand(H, T, 1)
            p = torch.softmax(torch.cat([logits, z], -1), -1)[..., :-1]
            out = torch.matmul(p, v)
        total = total + (out.permute(1, 0, 2) * torch.as_tensor(dout[b])).sum()
    total.backward()
    return (qt.grad.numpy(), kc.grad.numpy(), kr.grad.numpy(),
            None if zs is None else zs.grad.numpy())


@pytest.mark.parametrize("with_sink", [False, True])
@pytest.mark.parametrize("dt", [np.float32, np.uint16])
def test_csa_attn_bwd_matches_autograd(with_sink, dt):
    q, kv_cmp, kv_raw, idx, dout = _case(40)
    if dt == np.uint16:
        q, kv_cmp, kv_raw = (np.array([orc.bf16_encode(v) for v in a.ravel()], np.uint16)
                             .reshape(a.shape) for a in (q, kv_cmp, kv_raw))
    B, T, H, D = q.shape
    Nc, R, W = kv_cmp.shape[1], kv_raw.shape[1], 5
    q_pos, raw_base = np.array([9, 2]), np.array([3, 0])
    sink = np.linspace(-1.0, 2.0, H) if with_sink else None
    dq, dkc, dkr, ds, _ = orc.attn_bwd(q, kv_cmp, idx, kv_raw, W, q_pos, raw_base, dout, sink=sink)
    masks = [brute.csa_mask(T, q_pos[b], idx[b], Nc, R, raw_base[b], W) for b in range(B)]
    gq, gc, gr, gs = _autograd_attention(q, kv_cmp, kv_raw, masks, dout, 1 / math.sqrt(D), sink)
    np.testing.assert_allclose(dq, gq, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dkc, gc, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dkr, gr, rtol=1e-9, atol=1e-12)
    if with_sink:
        np.testing.assert_allclose(ds, gs, rtol=1e-9, atol=1e-12)


def test_hca_attn_bwd_matches_autograd():
    r = rng(41)
    B, T, H, D, m, Nc, R, W = 2, 10, 2, 8, 4, 6, 24, 4
    q = r.normal(0, 1, (B, T, H, D)).astype(np.float32)
    kv_cmp = r.normal(0, 1, (B, Nc, 2 * D)).astype(np.float32)
    kv_raw = r.normal(0, 1, (B, R, 2 * D)).astype(np.float32)
    dout = r.normal(0, 1, (B, T, H, D))
    q_pos, n_cmp, raw_base = np.array([13, 1]), np.array([Nc, 2]), np.array([2, 0])
    dq, dkc, dkr, _, _ = orc.attn_bwd(q, kv_cmp, None, kv_raw, W, q_pos, raw_base, dout, m=m,
                                      n_cmp=n_cmp)
    masks = []
    for b in range(B):
        vis = [list(range(max(0, min((q_pos[b] + t + 1) // m, n_cmp[b], Nc)))) for t in range(T)]
        masks.append(brute.csa_mask(T, q_pos[b], vis, Nc, R, raw_base[b], W))
    gq, gc, gr, _ = _autograd_attention(q, kv_cmp, kv_raw, masks, dout, 1 / math.sqrt(D))
    np.testing.assert_allclose(dq, gq, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dkc, gc, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dkr, gr, rtol=1e-9, atol=1e-12)


def test_attn_bwd_finite_differences_of_the_forward():
    # central differences of sum(dout * out) through the oracle's forward
    q, kv_cmp, kv_raw, idx, dout = _case(42, B=1, T=5, H=2, D=4, Nc=6, R=8, topk=3)
    q = q.astype(np.float64).astype(np.float32)
    W, q_pos, raw_base = 3, 4, 1
    sink = np.array([0.3, -0.7])
    dq, dkc, dkr, ds, _ = orc.attn_bwd(q, kv_cmp, idx, kv_raw, W, q_pos, raw_base, dout, sink=sink)

    def f(q_, kc_, kr_, s_):
        out, _ = orc.sparse_attn(q_, kc_, idx, kr_, W, q_pos, raw_base, sink=s_)
        return float((out * dout).sum())

    r = rng(43)
    h = 1e-3
    for name, arr, grad in (("q", q, dq), ("kv_cmp", kv_cmp, dkc), ("kv_raw", kv_raw, dkr)):
        for _ in range(6):
            i = tuple(r.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            step = float(ap[i]) - float(am[i])         # the representable step
            args_p = {"q": (ap, kv_cmp, kv_raw), "kv_cmp": (q, ap, kv_raw),
                      "kv_raw": (q, kv_cmp, ap)}[name]
            args_m = {"q": (am, kv_cmp, kv_raw), "kv_cmp": (q, am, kv_raw),
                      "kv_raw": (q, kv_cmp, am)}[name]
            fd = (f(*args_p, sink) - f(*args_m, sink)) / step
            assert abs(fd - grad[i]) <= 2e-5 * max(1.0, abs(grad[i])), (name, i, fd, grad[i])
    for hh in range(2):
        sp, sm = sink.copy(), sink.copy()
        sp[hh] += 1e-5
        sm[hh] -= 1e-5
        fd = (f(q, kv_cmp, kv_raw, sp) - f(q, kv_cmp, kv_raw, sm)) / 2e-5
        assert abs(fd - ds[hh]) <= 1e-6 * max(1.0, abs(ds[hh]))


def test_attn_bwd_identities_and_mass():
    # Without a sink every nonempty row's probabilities sum to 1, so
    # sum_rows dV = sum of dO over (token, head) with a nonempty key set and
    # sum_rows dK = scale * sum q * sum_j dl_j = 0; by bilinearity
    # sum q . dq = sum_rows K . dK.  The attention mass per slot equals the
    # library softmax's probability summed over heads.
    q, kv_cmp, kv_raw, idx, dout = _case(44, T=9, H=4, Nc=12, R=20, topk=5)
    B, T, H, D = q.shape
    Nc, R, W = kv_cmp.shape[1], kv_raw.shape[1], 4
    q_pos, raw_base = np.array([11, 0]), np.array([2, 0])
    idx[1, 0] = -1                                      # an empty key set (token 0, window 4 keeps 1)
    dq, dkc, dkr, _, mass = orc.attn_bwd(q, kv_cmp, idx, kv_raw, W, q_pos, raw_base, dout,
                                         want_mass=True)
    live = np.zeros((B, T), bool)
    for b in range(B):
        live[b] = brute.csa_mask(T, q_pos[b], idx[b], Nc, R, raw_base[b], W).any(-1)
    dV = dkc[..., D:].sum((0, 1)) + dkr[..., D:].sum((0, 1))
    np.testing.assert_allclose(dV, (dout * live[..., None, None]).sum((0, 1, 2)), rtol=1e-10,
                               atol=1e-10)
    dK = dkc[..., :D].sum((0, 1)) + dkr[..., :D].sum((0, 1))
    np.testing.assert_allclose(dK, 0, atol=1e-10)
    lhs = (q.astype(np.float64) * dq).sum()
    rhs = (kv_cmp[..., :D] * dkc[..., :D]).sum() + (kv_raw[..., :D] * dkr[..., :D]).sum()
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10)
    for b in range(B):
        mask = torch.as_tensor(brute.csa_mask(T, q_pos[b], idx[b], Nc, R, raw_base[b], W))
        rows = torch.as_tensor(np.concatenate([kv_cmp[b], kv_raw[b]]).astype(np.float64))
        logits = torch.einsum("thd,nd->thn", torch.as_tensor(q[b].astype(np.float64)),
                              rows[:, :D]) / math.sqrt(D)
        p = torch.softmax(logits.masked_fill(~mask[:, None, :], float("-inf")), -1)
        p = torch.nan_to_num(p).sum(1).numpy()          # [T, Nc + R]
        for t in range(T):
            for k in range(idx.shape[2]):
                j = idx[b, t, k]
                want = p[t, j] if j >= 0 else 0.0
                assert abs(mass[b, t, k] - want) <= 1e-12


def test_hca_attn_mass_per_entry_is_the_library_softmax():
    # the HCA form's mass per compressed entry (the dense indexer loss's
    # target): the library softmax over the row's keys (visible entries and
    # window) summed over heads, zero past the visible entries
    r = rng(45)
    B, T, H, D, m, Nc, R, W = 2, 10, 3, 8, 4, 6, 24, 4
    q = r.normal(0, 1, (B, T, H, D)).astype(np.float32)
    kv_cmp = r.normal(0, 1, (B, Nc, 2 * D)).astype(np.float32)
    kv_raw = r.normal(0, 1, (B, R, 2 * D)).astype(np.float32)
    dout = r.normal(0, 1, (B, T, H, D))
    q_pos, n_cmp, raw_base = np.array([13, 1]), np.array([Nc, 2]), np.array([2, 0])
    *_, mass = orc.attn_bwd(q, kv_cmp, None, kv_raw, W, q_pos, raw_base, dout, m=m, n_cmp=n_cmp,
                            want_mass=True)
    assert mass.shape == (B, T, Nc)
    for b in range(B):
        vis = [list(range(max(0, min((q_pos[b] + t + 1) // m, n_cmp[b], Nc)))) for t in range(T)]
        mask = torch.as_tensor(brute.csa_mask(T, q_pos[b], vis, Nc, R, raw_base[b], W))
        rows = torch.as_tensor(np.concatenate([kv_cmp[b], kv_raw[b]]).astype(np.float64))
        logits = torch.einsum("thd,nd->thn", torch.as_tensor(q[b].astype(np.float64)),
                              rows[:, :D]) / math.sqrt(D)
        p = torch.softmax(logits.masked_fill(~mask[:, None, :], float("-inf")), -1)
        p = torch.nan_to_num(p).sum(1).numpy()          # [T, Nc + R]
        for t in range(T):
            nv = len(vis[t])
            np.testing.assert_allclose(mass[b, t, :nv], p[t, :nv], rtol=1e-12, atol=1e-14)
            assert (mass[b, t, nv:] == 0).all()


def test_indexer_kl_dense_matches_autograd_over_every_visible_entry():
    # the dense form: KL of the normalised per-entry mass against the softmax
    # of the indexer scores over every visible entry, through torch's kl_div
    r = rng(52)
    B, T, HI, dI, Nc, m = 2, 9, 3, 8, 7, 4
    qi = r.normal(0, 1, (B, T, HI, dI)).astype(np.float32)
    wi = r.normal(0, 1, (B, T, HI)).astype(np.float32)
    ki = r.normal(0, 1, (B, Nc, dI)).astype(np.float32)
    q_pos, n_cmp = np.array([3, 20]), np.array([Nc, 5])
    nvis = [[min((q_pos[b] + t + 1) // m, n_cmp[b], Nc) for t in range(T)] for b in range(B)]
    mass = r.uniform(0.0, 2.0, (B, T, Nc))
    for b in range(B):
        for t in range(T):
            mass[b, t, nvis[b][t]:] = 0.0
    gs = r.uniform(0.5, 2.0, (B, T))
    loss, dq, dw, dk = orc.indexer_kl_dense_bwd(qi, wi, ki, m, q_pos, n_cmp, mass, gs)
    qt = torch.tensor(qi.astype(np.float64), requires_grad=True)
    wt = torch.tensor(wi.astype(np.float64), requires_grad=True)
    kt = torch.tensor(ki.astype(np.float64), requires_grad=True)
    total = 0
    for b in range(B):
        for t in range(T):
            nv = nvis[b][t]
            if nv == 0:
                assert loss[b, t] == 0 and (dq[b, t] == 0).all()
                continue
            v = torch.relu(torch.matmul(kt[b, :nv], qt[b, t].T))        # [nv, HI]
            scores = (v * wt[b, t]).sum(-1)
            p = torch.as_tensor(mass[b, t, :nv])
            p = p / p.sum()
            kl = F.kl_div(torch.log_softmax(scores, 0), p, reduction="sum")
            assert abs(kl.item() - loss[b, t]) <= 1e-12 * max(1.0, kl.item())
            total = total + gs[b, t] * kl
    total.backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-13)


def _kl_case(seed, B=2, T=6, HI=3, dI=8, Nc=9, topk=4):
    r = rng(seed)
    qi = r.normal(0, 1, (B, T, HI, dI)).astype(np.float32)
    wi = r.normal(0, 1, (B, T, HI)).astype(np.float32)
    ki = r.normal(0, 1, (B, Nc, dI)).astype(np.float32)
    idx = np.full((B, T, topk), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = r.integers(1, topk + 1)
            idx[b, t, :n] = np.sort(r.choice(Nc, n, replace=False))
    mass = r.uniform(0.0, 2.0, (B, T, topk)) * (idx >= 0)
    return qi, wi, ki, idx, mass


def test_indexer_kl_matches_autograd_of_library_kl():
    qi, wi, ki, idx, mass = _kl_case(50)
    B, T, HI, dI = qi.shape
    gs = rng(51).uniform(0.5, 2.0, (B, T))
    loss, dq, dw, dk = orc.indexer_kl_bwd(qi, wi, ki, idx, mass, gs)
    qt = torch.tensor(qi.astype(np.float64), requires_grad=True)
    wt = torch.tensor(wi.astype(np.float64), requires_grad=True)
    kt = torch.tensor(ki.astype(np.float64), requires_grad=True)
    total = 0
    for b in range(B):
        for t in range(T):
            sel = idx[b, t][idx[b, t] >= 0]
            v = torch.relu(torch.matmul(kt[b, sel], qt[b, t].T))        # [n, HI]
            scores = (v * wt[b, t]).sum(-1)
            p = torch.as_tensor(mass[b, t][idx[b, t] >= 0])
            p = p / p.sum()
            kl = F.kl_div(torch.log_softmax(scores, 0), p, reduction="sum")
            klv = kl.item()
            assert abs(klv - loss[b, t]) <= 1e-12 * max(1.0, klv)
            total = total + gs[b, t] * kl
    total.backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_indexer_kl_closed_forms():
    # KL >= 0; KL = 0 and no gradient when the target equals the indexer's
    # own softmax; rows with no selection or no mass carry nothing; the
    # gradient is linear in grad_scale.
    qi, wi, ki, idx, mass = _kl_case(52)
    loss, dq, dw, dk = orc.indexer_kl_bwd(qi, wi, ki, idx, mass)
    assert (loss >= -1e-15).all() and (loss > 0).any()
    _, _, _, alls = orc.indexer_topk(qi, wi, ki, 1, 1, 10 ** 6, ki.shape[1], want_all=True)
    own = np.zeros_like(mass)
    for b in range(idx.shape[0]):
        for t in range(idx.shape[1]):
            for k, j in enumerate(idx[b, t]):
                if j >= 0:
                    own[b, t, k] = math.exp(alls[b, t, j] - 3.0)
    l0, q0, w0, k0 = orc.indexer_kl_bwd(qi, wi, ki, idx, own)
    np.testing.assert_allclose(l0, 0, atol=1e-12)
    for g in (q0, w0, k0):
        np.testing.assert_allclose(g, 0, atol=1e-12)
    idx2, mass2 = idx.copy(), mass.copy()
    idx2[0, 0] = -1
    mass2[1, 1] = 0
    l2, q2, w2, _ = orc.indexer_kl_bwd(qi, wi, ki, idx2, mass2)
    assert l2[0, 0] == 0 and l2[1, 1] == 0
    assert (q2[0, 0] == 0).all() and (w2[1, 1] == 0).all()
    l3, q3, w3, k3 = orc.indexer_kl_bwd(qi, wi, ki, idx, mass, np.full(loss.shape, 2.5))
    np.testing.assert_allclose(l3, loss, rtol=1e-15)
    np.testing.assert_allclose(q3, 2.5 * dq, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(k3, 2.5 * dk, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("m,overlap,rotate", [(4, 1, False), (4, 1, True), (3, 0, False)])
def test_compress_bwd_finite_differences_of_the_forward(m, overlap, rotate):
    r = rng(60 + m)
    B, L, dm, E = 2, 4 * m + 1, 6, 8
    Nc = L // m + 1
    x = r.normal(0, 1, (B, L, dm)).astype(np.float32)
    wk = r.normal(0, 0.5, (E, dm)).astype(np.float32)
    wg = r.normal(0, 0.5, (E, dm)).astype(np.float32)
    ape = r.normal(0, 0.3, ((1 + overlap) * m, E))
    dC = r.normal(0, 1, (B, Nc, E))
    dx, dwk, dwg, dape = orc.compress_bwd(x, wk, wg, m, overlap, Nc, dC, ape=ape, rotate=rotate)

    def f(x_, wk_, wg_, ape_):
        out, written, _ = orc.compress(x_, wk_, wg_, m, overlap, 0, Nc, ape=ape_,
                                       want_state=False, rotate=rotate)
        return float(np.where(written[..., None], out * dC, 0.0).sum())

    h = 1e-3
    for name, arr, grad in (("x", x, dx), ("wk", wk, dwk), ("wg", wg, dwg)):
        for _ in range(8):
            i = tuple(r.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            step = float(ap[i]) - float(am[i])
            sub = {"x": lambda a: (a, wk, wg, ape), "wk": lambda a: (x, a, wg, ape),
                   "wg": lambda a: (x, wk, a, ape)}[name]
            fd = (f(*sub(ap)) - f(*sub(am))) / step
            assert abs(fd - grad[i]) <= 5e-5 * max(1.0, abs(grad[i])), (name, i, fd, grad[i])
    for _ in range(6):
        i = tuple(r.integers(0, s) for s in ape.shape)
        ap, am = ape.copy(), ape.copy()
        ap[i] += 1e-5
        am[i] -= 1e-5
        fd = (f(x, wk, wg, ap) - f(x, wk, wg, am)) / 2e-5
        assert abs(fd - dape[i]) <= 1e-6 * max(1.0, abs(dape[i]))


@pytest.mark.parametrize("rotate,interleaved", [(False, False), (True, False), (False, True)])
def test_compress_bwd_with_norm_and_rope_finite_differences(rotate, interleaved):
    # entries RMS-normed, rotated on channels [2, 6) at their positions m i
    # (base 10: angles well away from 0) and optionally Hadamard-rotated: the
    # gradients of x, both weights, ape and the norm weight against central
    # differences of the oracle's own forward with the same options
    r = rng(80 + 2 * rotate + interleaved)
    m, overlap = 4, 1
    B, L, dm, E = 2, 4 * m + 3, 6, 8
    Nc = L // m + 1
    x = r.normal(0, 1, (B, L, dm)).astype(np.float32)
    wk = r.normal(0, 0.5, (E, dm)).astype(np.float32)
    wg = r.normal(0, 0.5, (E, dm)).astype(np.float32)
    ape = r.normal(0, 0.3, ((1 + overlap) * m, E))
    nw = r.normal(1, 0.3, E)
    dC = r.normal(0, 1, (B, Nc, E))
    opt = dict(norm_eps=1e-3, rope_dim=4, rope_offset=2, rope_base=10.0,
               rope_interleaved=interleaved)
    dx, dwk, dwg, dape, dnw = orc.compress_bwd_ex(x, wk, wg, m, overlap, Nc, dC, ape=ape,
                                                  rotate=rotate, norm_weight=nw, **opt)

    def f(x_, wk_, wg_, ape_, nw_):
        out, written, _ = orc.compress(x_, wk_, wg_, m, overlap, 0, Nc, ape=ape_,
                                       want_state=False, rotate=rotate, norm_weight=nw_, **opt)
        return float(np.where(written[..., None], out * dC, 0.0).sum())

    h = 1e-3
    args = {"x": x, "wk": wk, "wg": wg}
    for name, grad in (("x", dx), ("wk", dwk), ("wg", dwg)):
        arr = args[name]
        for _ in range(8):
            i = tuple(r.integers(0, s_) for s_ in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            step = float(ap[i]) - float(am[i])
            kp = dict(args, **{name: ap})
            km = dict(args, **{name: am})
            fd = (f(kp["x"], kp["wk"], kp["wg"], ape, nw) - f(km["x"], km["wk"], km["wg"], ape, nw)) / step
            assert abs(fd - grad[i]) <= 1e-4 * max(1.0, abs(grad[i])), (name, i, fd, grad[i])
    for arr, grad, which in ((ape, dape, "ape"), (nw, dnw, "nw")):
        for _ in range(6):
            i = tuple(r.integers(0, s_) for s_ in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[i] += 1e-5
            am[i] -= 1e-5
            if which == "ape":
                fd = (f(x, wk, wg, ap, nw) - f(x, wk, wg, am, nw)) / 2e-5
            else:
                fd = (f(x, wk, wg, ape, ap) - f(x, wk, wg, ape, am)) / 2e-5
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(grad[i])), (which, i, fd, grad[i])
    # no options: the plain entry point (to rounding: the oracle sums token rows
    # shared by two entries with atomics, in thread order)
    a = orc.compress_bwd(x, wk, wg, m, overlap, Nc, dC, ape=ape, rotate=rotate)
    b_ = orc.compress_bwd_ex(x, wk, wg, m, overlap, Nc, dC, ape=ape, rotate=rotate)
    for u, v in zip(a, b_[:4]):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-14)
    assert b_[4] is None


def test_compress_bwd_mean_pool_closed_form():
    # uniform gates (zero gate weights, no ape) and no overlap: each entry is
    # the mean of its m projected tokens, so dP_j = dC_i / m for the entry i
    # that holds token j, dG_j = (P_j - C_i) dC_i / m, dx = W_kv^T dP (the
    # gate weights are zero) and dW = sum_j d_j x_j^T for both projections.
    r = rng(70)
    B, m, L, dm, E = 1, 4, 16, 5, 6
    Nc = L // m
    x = r.normal(0, 1, (B, L, dm)).astype(np.float32)
    wk = r.normal(0, 1, (E, dm)).astype(np.float32)
    wg = np.zeros((E, dm), np.float32)
    dC = r.normal(0, 1, (B, Nc, E))
    dx, dwk, dwg, _ = orc.compress_bwd(x, wk, wg, m, 0, Nc, dC)
    X = x[0].astype(np.float64)
    P = X @ wk.T.astype(np.float64)
    dP = np.repeat(dC[0], m, axis=0) / m
    C = P.reshape(Nc, m, E).mean(1)
    dG = (P - np.repeat(C, m, axis=0)) * dP
    np.testing.assert_allclose(dx[0], dP @ wk.astype(np.float64), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dwk, dP.T @ X, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dwg, dG.T @ X, rtol=1e-10, atol=1e-12)
