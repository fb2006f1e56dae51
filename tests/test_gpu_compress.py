"""GPU parity of csa_compress against the CPU oracle (called through the C ABI)."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import assert_bf16_close, assert_rows_rel, dev_i64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(x, w_kv, w_gate, pos0, m, o, Nc_cap, out_dtype, ape=None, state_in=None, want_state=True,
         rotate=False):
    B = x.shape[0]
    E = w_kv.shape[0]
    out = torch.full((B, Nc_cap, E), float("nan"), device=DEV).to(out_dtype)
    out_scale = torch.zeros(B, Nc_cap, device=DEV) if out_dtype == torch.float8_e4m3fn else None
    ns = (1 + o) * m - 1
    state_out = torch.full((B, ns, 2, E), 7.0, device=DEV) if want_state else None
    csa.csa_compress(x, w_kv, w_gate, dev_i64(pos0), m, o, out, out_scale=out_scale,
                     ape=ape, state_in=state_in, state_out=state_out, rotate=rotate)
    torch.cuda.synchronize()
    return out, out_scale, state_out


def _oracle(x, w_kv, w_gate, pos0, m, o, Nc_cap, ape=None, state_in=None, rotate=False):
    return orc.compress(gen.host_bits(x), gen.host_bits(w_kv), gen.host_bits(w_gate), m, o,
                        np.asarray(pos0), Nc_cap,
                        ape=None if ape is None else ape.cpu().numpy(),
                        state_in=None if state_in is None else state_in.cpu().numpy(),
                        rotate=rotate)


@pytest.mark.parametrize("E", [128, 32])
def test_compress_tiny_f32(E):
    w = gen.WORKLOADS["csa_prefill_tiny_f32"]
    d = gen.Draw(7 + E)
    x = gen.store(d.normal(1, w.T, w.d_model), gen.F32)
    w_kv, w_gate = gen.compressor_weights(d, w.d_model, E, gen.F32)
    out, _, st = _run(x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), [0], w.m, w.overlap, w.n_cmp,
                      torch.float32)
    ref, written, st_ref = _oracle(x, w_kv, w_gate, [0], w.m, w.overlap, w.n_cmp)
    assert written.all()
    assert_rows_rel(out.cpu().numpy()[0], ref[0], 1e-5, "compress f32")
    np.testing.assert_allclose(st.cpu().numpy()[:, :, 0], st_ref[:, :, 0], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("out_kind,rotate", [("bf16", False), ("fp8", False), ("f32", False),
                                             ("bf16", True), ("fp8", True), ("f32", True)])
def test_compress_bf16_ragged_with_ape(out_kind, rotate):
    d = gen.Draw(11)
    B, L, dm, E, m, o = 3, 61, 256, 64, 4, 1
    x = gen.store(d.normal(B, L, dm), gen.BF16)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    ape = d.normal(2 * m, E)
    pos0 = [0, 5, 130]          # ragged starts; tokens before pos0 absent (no state)
    Nc = 64
    odt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "f32": torch.float32}[out_kind]
    out, osc, st = _run(x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), pos0, m, o, Nc, odt,
                        ape=ape.to(DEV), rotate=rotate)
    ref, written, st_ref = _oracle(x, w_kv, w_gate, pos0, m, o, Nc, ape=ape, rotate=rotate)
    if out_kind == "fp8":
        codes, scales = orc.quant_rows_e4m3(np.nan_to_num(ref))
        g_codes = gen.host_bits(out)
        g_sc = osc.cpu().numpy()
        for b in range(B):
            for i in np.nonzero(written[b])[0]:
                np.testing.assert_allclose(g_sc[b, i], scales[b, i], rtol=1e-5)
                # within one e4m3 step: compare decoded values by code distance
                gv = np.array([orc.e4m3_decode(c) for c in g_codes[b, i]])
                rv = np.array([orc.e4m3_decode(c) for c in codes[b, i]])
                step = np.maximum(np.abs(rv), 2.0 ** -6) * 2.0 ** -3
                assert (np.abs(gv - rv) <= step + 1e-12).all(), (b, i)
    else:
        g = out.float().cpu().numpy()
        for b in range(B):
            wr = written[b]
            assert np.isnan(g[b, ~wr]).all(), "rows not completed must be untouched"
            if out_kind == "f32":
                assert_rows_rel(g[b, wr], ref[b, wr], 1e-5, "compress bf16->f32")
            else:
                assert_bf16_close(g[b, wr], ref[b, wr], "compress bf16->bf16")
    np.testing.assert_allclose(st.cpu().numpy()[:, :, 0], st_ref[:, :, 0], rtol=2e-5, atol=2e-5)
    assert np.array_equal(np.isneginf(st.cpu().numpy()[:, :, 1]), np.isneginf(st_ref[:, :, 1]))


def _mxfp4_step(r, x):
    """One E2M1 step at magnitude r in a block of shared exponent x."""
    u = np.abs(r) / 2.0 ** x
    return np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0)) * 2.0 ** x


def check_mxfp4_rows(g_codes, g_scales, ref_rows, what):
    """GPU MXFP4 rows against the oracle's quantisation of its own entries:
    block exponents equal (or one apart where the block maximum lies within
    fp32 rounding of a power of two) and values within one E2M1 step."""
    codes, scales = orc.quant_rows_mxfp4(ref_rows)
    xo = scales.astype(np.int64) - 127
    xg = g_scales.astype(np.int64) - 127
    amax = np.abs(ref_rows).reshape(ref_rows.shape[:-1] + (-1, 32)).max(-1)
    near = np.abs(np.log2(np.maximum(amax, 1e-300)) - np.round(np.log2(np.maximum(amax, 1e-300)))) < 1e-5
    assert ((xo == xg) | ((np.abs(xo - xg) == 1) & near)).all(), what + " block exponents"
    gv = orc.mxfp4_decode(g_codes, g_scales)
    rv = orc.mxfp4_decode(codes, scales)
    x = np.repeat(np.minimum(xo, xg), 32, axis=-1)
    assert (np.abs(gv - rv) <= _mxfp4_step(rv, x) + 1e-30).all(), what + " values"
    same = (xo == xg)
    frac = (np.repeat(same, 16, axis=-1) & (g_codes == codes)).mean()
    assert frac > 0.99, "%s: only %.4f of the code bytes agree" % (what, frac)


@pytest.mark.parametrize("E,rotate", [(64, False), (64, True), (256, False)])
def test_compress_mxfp4_output(E, rotate):
    # OCP MXFP4 entries (E2M1 codes, one E8M0 exponent per 32 channels):
    # ragged starts with ape, as the bf16/fp8 test above
    d = gen.Draw(13 + E + rotate)
    B, L, dm, m, o = 3, 61, 256, 4, 1
    x = gen.store(d.normal(B, L, dm), gen.BF16)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    ape = d.normal(2 * m, E)
    pos0 = [0, 5, 130]
    Nc = 64
    out = torch.full((B, Nc, E // 2), 0xAB, dtype=torch.uint8, device=DEV)
    osc = torch.full((B, Nc, E // 32), 0xCD, dtype=torch.uint8, device=DEV)
    csa.csa_compress(x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), dev_i64(pos0), m, o,
                     out.view(torch.float4_e2m1fn_x2), out_scale=osc, ape=ape.to(DEV),
                     rotate=rotate)
    torch.cuda.synchronize()
    ref, written, _ = _oracle(x, w_kv, w_gate, pos0, m, o, Nc, ape=ape, rotate=rotate)
    g_codes, g_sc = out.cpu().numpy(), osc.cpu().numpy()
    for b in range(B):
        wr = written[b]
        assert (g_codes[b, ~wr] == 0xAB).all() and (g_sc[b, ~wr] == 0xCD).all(), \
            "rows not completed must be untouched"
        check_mxfp4_rows(g_codes[b, wr], g_sc[b, wr], ref[b, wr], "mxfp4 E=%d b=%d" % (E, b))


def test_compress_decode_step_mxfp4():
    # the indexer compressor's decode step (few-row projection, pool from the
    # carried state) with an MXFP4 store
    w = gen.WORKLOADS["csa_decode_1m_b8_stream"]
    d = gen.Draw(15)
    B, dm, m, o, E = w.B, w.d_model, w.m, w.overlap, w.d_I
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    x_tail = gen.store(d.normal(B, 7, dm), gen.BF16)
    x_new = gen.store(d.normal(B, 1, dm), gen.BF16)
    T = w.ctx
    Nc = T // m
    pos_tail = [T - 8] * B
    _, _, st1 = _oracle(x_tail, w_kv, w_gate, pos_tail, m, o, Nc)
    ref2, wr2, _ = _oracle(x_new, w_kv, w_gate, [T - 1] * B, m, o, Nc,
                           state_in=torch.from_numpy(st1))
    assert wr2[:, Nc - 1].all()
    wk, wg = w_kv.to(DEV), w_gate.to(DEV)
    s0 = torch.zeros(B, 2 * m - 1, 2, E, device=DEV)
    s1 = torch.zeros(B, 2 * m - 1, 2, E, device=DEV)
    out = torch.zeros(B, Nc, E // 2, dtype=torch.uint8, device=DEV)
    osc = torch.zeros(B, Nc, E // 32, dtype=torch.uint8, device=DEV)
    o4 = out.view(torch.float4_e2m1fn_x2)
    csa.csa_compress(x_tail.to(DEV), wk, wg, dev_i64(pos_tail), m, o, o4, out_scale=osc,
                     state_out=s0)
    csa.csa_compress(x_new.to(DEV), wk, wg, dev_i64([T - 1] * B), m, o, o4, out_scale=osc,
                     state_in=s0, state_out=s1)
    torch.cuda.synchronize()
    check_mxfp4_rows(out[:, Nc - 1].cpu().numpy(), osc[:, Nc - 1].cpu().numpy(),
                     ref2[:, Nc - 1], "mxfp4 decode entry")


@pytest.mark.parametrize("m,o", [(4, 1), (128, 0), (3, 1)])
def test_compress_chunked_with_state_equals_one_shot(m, o):
    d = gen.Draw(12 + m)
    B, S, dm, E = 2, 3 * m + 37, 64, 48
    x = gen.store(d.normal(B, S, dm), gen.F32)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.F32)
    ape = d.normal((1 + o) * m, E)
    Nc = S // m + 1
    ref, written, st_ref = _oracle(x, w_kv, w_gate, [0] * B, m, o, Nc, ape=ape)
    xg, wk, wg, ag = x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), ape.to(DEV)
    ns = (1 + o) * m - 1
    out = torch.full((B, Nc, E), float("nan"), device=DEV)
    st = [torch.zeros(B, ns, 2, E, device=DEV), torch.zeros(B, ns, 2, E, device=DEV)]
    st_in, p, k = None, 0, 0
    for L in [1, 5, 1, m + 3, 2, S]:
        L = min(L, S - p)
        if L <= 0:
            break
        csa.csa_compress(xg[:, p:p + L].contiguous(), wk, wg, dev_i64([p] * B), m, o, out,
                         ape=ag, state_in=st_in, state_out=st[k])
        st_in = st[k]
        k ^= 1
        p += L
    assert p == S
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    for b in range(B):
        assert_rows_rel(g[b, written[b]], ref[b, written[b]], 1e-5, "chunked compress")
    np.testing.assert_allclose(st_in.cpu().numpy()[:, :, 0], st_ref[:, :, 0], rtol=1e-5, atol=1e-5)


def test_compress_decode_step_splits_k():
    # one token per sequence at 4096-wide input: the projection splits K over
    # many workgroups; the emitted entry must match the oracle's streaming step
    w = gen.WORKLOADS["csa_decode_1m_b8_stream"]
    d = gen.Draw(13)
    B, dm, E, m, o = 4, w.d_model, 2 * w.D, w.m, w.overlap
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    x_tail = gen.store(d.normal(B, 7, dm), gen.BF16)
    x_new = gen.store(d.normal(B, 1, dm), gen.BF16)
    T = 1 << 16                     # position of the new token: T - 1
    Nc = T // m
    pos_tail = [T - 8] * B
    ref1, _, st1 = _oracle(x_tail, w_kv, w_gate, pos_tail, m, o, Nc)
    ref2, wr2, _ = _oracle(x_new, w_kv, w_gate, [T - 1] * B, m, o, Nc,
                           state_in=torch.from_numpy(st1))
    assert wr2[:, Nc - 1].all()
    wk, wg = w_kv.to(DEV), w_gate.to(DEV)
    ns = 2 * m - 1
    s0 = torch.zeros(B, ns, 2, E, device=DEV)
    s1 = torch.zeros(B, ns, 2, E, device=DEV)
    out = torch.zeros(B, Nc, E, device=DEV, dtype=torch.bfloat16)
    csa.csa_compress(x_tail.to(DEV), wk, wg, dev_i64(pos_tail), m, o, out, state_out=s0)
    csa.csa_compress(x_new.to(DEV), wk, wg, dev_i64([T - 1] * B), m, o, out, state_in=s0,
                     state_out=s1)
    torch.cuda.synchronize()
    assert_bf16_close(out[:, Nc - 1].float().cpu().numpy(), ref2[:, Nc - 1], "decode entry")


@pytest.mark.parametrize("E,out_kind,rotate", [(256, "bf16", False), (64, "fp8", False),
                                               (64, "fp8", True)])
def test_compress_decode_step_main_and_indexer_widths(E, out_kind, rotate):
    # the decode step of both compressors of the streaming decode workload
    # (main: 2D channels to bf16; indexer: d_I channels to e4m3 with a row
    # scale): few-row projection over all of K, pool from the carried state
    w = gen.WORKLOADS["csa_decode_1m_b8_stream"]
    d = gen.Draw(14 + E)
    B, dm, m, o = w.B, w.d_model, w.m, w.overlap
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    x_tail = gen.store(d.normal(B, 7, dm), gen.BF16)
    x_new = gen.store(d.normal(B, 1, dm), gen.BF16)
    T = w.ctx
    Nc = T // m
    pos_tail = [T - 8] * B
    _, _, st1 = _oracle(x_tail, w_kv, w_gate, pos_tail, m, o, Nc)
    ref2, wr2, st2 = _oracle(x_new, w_kv, w_gate, [T - 1] * B, m, o, Nc,
                             state_in=torch.from_numpy(st1), rotate=rotate)
    assert wr2[:, Nc - 1].all()
    wk, wg = w_kv.to(DEV), w_gate.to(DEV)
    ns = 2 * m - 1
    s0 = torch.zeros(B, ns, 2, E, device=DEV)
    odt = torch.bfloat16 if out_kind == "bf16" else torch.float8_e4m3fn
    out, osc, s1 = None, None, None
    tmp = torch.zeros(B, Nc, E, device=DEV, dtype=odt)
    tsc = torch.zeros(B, Nc, device=DEV) if out_kind == "fp8" else None
    csa.csa_compress(x_tail.to(DEV), wk, wg, dev_i64(pos_tail), m, o, tmp, out_scale=tsc,
                     state_out=s0, rotate=rotate)
    out, osc, s1 = _run(x_new.to(DEV), wk, wg, [T - 1] * B, m, o, Nc, odt, state_in=s0,
                        rotate=rotate)
    np.testing.assert_allclose(s1.cpu().numpy()[:, :, 0], st2[:, :, 0], rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(s1.cpu().numpy()[:, :, 1], st2[:, :, 1], rtol=2e-5, atol=2e-5)
    if out_kind == "bf16":
        assert_bf16_close(out[:, Nc - 1].float().cpu().numpy(), ref2[:, Nc - 1], "decode entry")
        return
    codes, scales = orc.quant_rows_e4m3(np.nan_to_num(ref2[:, Nc - 1:Nc]))
    g_codes = gen.host_bits(out[:, Nc - 1:Nc])
    np.testing.assert_allclose(osc[:, Nc - 1].cpu().numpy(), scales[:, 0], rtol=1e-5)
    for b in range(B):
        gv = np.array([orc.e4m3_decode(c) for c in g_codes[b, 0]])
        rv = np.array([orc.e4m3_decode(c) for c in codes[b, 0]])
        step = np.maximum(np.abs(rv), 2.0 ** -6) * 2.0 ** -3
        assert (np.abs(gv - rv) <= step + 1e-12).all(), b


def test_compress_few_rows_chunks_ragged_k():
    # 15-row chunks (the few-row projection) with K = 512 (no full unrolled
    # k block per wave), 2E = 88 columns (a partial 16-column group), ragged
    # starts, a carried state between the chunks and an ape
    d = gen.Draw(21)
    B, L, dm, E, m, o = 3, 5, 512, 44, 4, 1
    x = gen.store(d.normal(B, 2 * L, dm), gen.BF16)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    ape = d.normal(2 * m, E)
    pos0 = [0, 6, 13]
    Nc = 8
    ref, written, st_ref = _oracle(x, w_kv, w_gate, pos0, m, o, Nc, ape=ape)
    xg, wk, wg, ag = x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), ape.to(DEV)
    out = torch.full((B, Nc, E), float("nan"), device=DEV)
    ns = 2 * m - 1
    s0 = torch.full((B, ns, 2, E), 7.0, device=DEV)
    s1 = torch.full((B, ns, 2, E), 7.0, device=DEV)
    csa.csa_compress(xg[:, :L].contiguous(), wk, wg, dev_i64(pos0), m, o, out, ape=ag,
                     state_out=s0)
    csa.csa_compress(xg[:, L:].contiguous(), wk, wg, dev_i64([p + L for p in pos0]), m, o, out,
                     ape=ag, state_in=s0, state_out=s1)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    for b in range(B):
        wr = written[b]
        assert wr.any()
        assert np.isnan(g[b, ~wr]).all()
        assert_rows_rel(g[b, wr], ref[b, wr], 1e-5, "few-row chunks")
    np.testing.assert_allclose(s1.cpu().numpy()[:, :, 0], st_ref[:, :, 0], rtol=2e-5, atol=2e-5)
    assert np.array_equal(np.isneginf(s1.cpu().numpy()[:, :, 1]), np.isneginf(st_ref[:, :, 1]))


def test_compress_prefill_8k_sampled_entries():
    w = gen.WORKLOADS["csa_prefill_8k_bf16"]
    inp = gen.prefill_inputs(w, device="cpu")
    x = inp["x"]
    out = torch.empty(w.B, w.n_cmp, 2 * w.D, device=DEV, dtype=torch.bfloat16)
    kidx = torch.empty(w.B, w.n_cmp, w.d_I, device=DEV, dtype=torch.bfloat16)
    xg = x.to(DEV)
    pos0 = dev_i64([0])
    csa.csa_compress(xg, inp["w_kv"].to(DEV), inp["w_gate"].to(DEV), pos0, w.m, w.overlap, out)
    csa.csa_compress(xg, inp["w_ikv"].to(DEV), inp["w_igate"].to(DEV), pos0, w.m, w.overlap, kidx)
    torch.cuda.synchronize()
    g_main, g_idx = out.float().cpu().numpy(), kidx.float().cpu().numpy()
    # blocks of 16 consecutive entries (136 in all): the first entries, blocks
    # across the projection's 128-token tile boundaries (entries 31/32, 63/64)
    # and the last entries; each block's oracle call starts at the block's
    # first window token
    checked = 0
    for i0 in (0, 24, 56, 500, 1017, 1530, 1777, 2032):
        i1 = min(i0 + 16, w.n_cmp)
        lo = max(0, w.m * (i0 - 1))
        xs = x[:, lo:w.m * i1]
        for wk, wg, g in ((inp["w_kv"], inp["w_gate"], g_main), (inp["w_ikv"], inp["w_igate"], g_idx)):
            ref, wr, _ = _oracle(xs, wk, wg, [lo], w.m, w.overlap, i1)
            assert wr[0, i0:i1].all()
            assert_bf16_close(g[0, i0:i1], ref[0, i0:i1], "prefill entries %d..%d" % (i0, i1 - 1))
        checked += i1 - i0
    assert checked >= 128


@pytest.mark.parametrize("E,out_kind", [(128, "f32"), (128, "bf16"), (256, "f32"), (64, "bf16")])
def test_compress_fused_prefill_chunks_with_state(E, out_kind):
    # chunks of at least 128 tokens with E >= 128 take the fused projection +
    # pool (the windows pooled out of LDS, 31 entries per 128-token tile, 4
    # halo tokens); the short chunk in between, and E = 64, take the
    # two-kernel path; chunk
    # starts off the block boundary (307, 507), two sequences, ape, and the
    # carried state across the calls, against the oracle run in one shot
    d = gen.Draw(140 + E)
    B, dm, m, o = 2, 256, 4, 1
    S = 700
    x = gen.store(d.normal(B, S, dm), gen.BF16)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    ape = d.normal((1 + o) * m, E)
    Nc = S // m + 1
    ref, written, st_ref = _oracle(x, w_kv, w_gate, [0] * B, m, o, Nc, ape=ape)
    xg, wk, wg, ag = x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), ape.to(DEV)
    ns = (1 + o) * m - 1
    odt = torch.float32 if out_kind == "f32" else torch.bfloat16
    out = torch.full((B, Nc, E), float("nan"), device=DEV).to(odt)
    st = [torch.zeros(B, ns, 2, E, device=DEV), torch.zeros(B, ns, 2, E, device=DEV)]
    st_in, p, k = None, 0, 0
    for L in (301, 6, 200, 193):
        csa.csa_compress(xg[:, p:p + L].contiguous(), wk, wg, dev_i64([p] * B), m, o, out,
                         ape=ag, state_in=st_in, state_out=st[k])
        st_in = st[k]
        k ^= 1
        p += L
    assert p == S
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    for b in range(B):
        wr = written[b]
        assert wr.all() or np.isnan(g[b, ~wr]).all()
        if out_kind == "f32":
            assert_rows_rel(g[b, wr], ref[b, wr], 1e-5, "fused chunks")
        else:
            assert_bf16_close(g[b, wr], ref[b, wr], "fused chunks")
    np.testing.assert_allclose(st_in.cpu().numpy()[:, :, 0], st_ref[:, :, 0], rtol=2e-5, atol=2e-5)
    assert np.array_equal(np.isneginf(st_in.cpu().numpy()[:, :, 1]), np.isneginf(st_ref[:, :, 1]))


def test_compress_bf16_ragged_tiles_and_split_k():
    # output width 2E = 80 (a partial 128-column tile), 300 rows (a partial
    # 128-row tile) and d_model 1024 so that the projection splits K and the
    # pool sums the split partials
    d = gen.Draw(19)
    B, L, dm, E, m, o = 2, 150, 1024, 40, 4, 1
    x = gen.store(d.normal(B, L, dm), gen.BF16)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    pos0 = [3, 0]
    Nc = 40
    out, _, st = _run(x.to(DEV), w_kv.to(DEV), w_gate.to(DEV), pos0, m, o, Nc, torch.float32)
    ref, written, st_ref = _oracle(x, w_kv, w_gate, pos0, m, o, Nc)
    g = out.cpu().numpy()
    for b in range(B):
        wr = written[b]
        assert wr.any()
        assert np.isnan(g[b, ~wr]).all()
        assert_rows_rel(g[b, wr], ref[b, wr], 1e-5, "compress bf16 ragged tiles")
    np.testing.assert_allclose(st.cpu().numpy()[:, :, 0], st_ref[:, :, 0], rtol=2e-5, atol=2e-5)


def _run_opts(x, w_kv, w_gate, pos0, m, o, Nc_cap, out_dtype, state_in=None, **opts):
    B, E = x.shape[0], w_kv.shape[0]
    out = torch.full((B, Nc_cap, E), float("nan"), device=DEV).to(out_dtype)
    out_scale = torch.zeros(B, Nc_cap, device=DEV) if out_dtype == torch.float8_e4m3fn else None
    ns = (1 + o) * m - 1
    state_out = torch.zeros(B, ns, 2, E, device=DEV)
    csa.csa_compress(x, w_kv, w_gate, dev_i64(pos0), m, o, out, out_scale=out_scale,
                     state_in=state_in, state_out=state_out, **opts)
    torch.cuda.synchronize()
    return out, out_scale, state_out


@pytest.mark.parametrize("out_kind,interleaved,rotate", [("f32", False, False), ("f32", True, False),
                                                          ("bf16", False, True), ("fp8", False, False)])
def test_compress_norm_and_rope_chunks(out_kind, interleaved, rotate):
    # RMS norm + rotary embedding of a slice of the K half (E = 2 D, D = 64:
    # channels 32..63), ragged starts, a carried state between two chunks;
    # positions reach past 2^18 tokens
    d = gen.Draw(90 + interleaved + 2 * rotate)
    B, L, dm, E, m, o = 3, 45, 256, 128, 4, 1
    x = gen.store(d.normal(B, 2 * L, dm), gen.BF16)
    w_kv, w_gate = gen.compressor_weights(d, dm, E, gen.BF16)
    g = 1.0 + 0.2 * d.normal(E)
    pos0 = [0, 13, (1 << 18) + 3]
    Nc = ((1 << 18) + 3 + 2 * L) // m + 1
    opts = dict(norm_weight=g, norm_eps=1e-6, rope_dim=32, rope_offset=32, rope_base=10000.0,
                rope_interleaved=interleaved)
    odt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "f32": torch.float32}[out_kind]
    xg, wk, wg = x.to(DEV), w_kv.to(DEV), w_gate.to(DEV)
    gopts = dict(opts, norm_weight=g.to(DEV))
    # two chunks: the second starts where the first ended and takes its state
    out1, sc1, st1 = _run_opts(xg[:, :L].contiguous(), wk, wg, pos0, m, o, Nc, odt, rotate=rotate,
                               **gopts)
    out2, sc2, _ = _run_opts(xg[:, L:].contiguous(), wk, wg, [p + L for p in pos0], m, o, Nc, odt,
                             state_in=st1, rotate=rotate, **gopts)
    oo = dict(opts, norm_weight=g.numpy())
    r1, w1, s1 = orc.compress(gen.host_bits(x[:, :L]), gen.host_bits(w_kv), gen.host_bits(w_gate),
                              m, o, np.asarray(pos0), Nc, rotate=rotate, **oo)
    r2, w2, _ = orc.compress(gen.host_bits(x[:, L:]), gen.host_bits(w_kv), gen.host_bits(w_gate),
                             m, o, np.asarray(pos0) + L, Nc, state_in=s1, rotate=rotate, **oo)
    for out, sc, ref, wr in ((out1, sc1, r1, w1), (out2, sc2, r2, w2)):
        for b in range(B):
            rows = np.nonzero(wr[b])[0]
            assert rows.size > 0
            if out_kind == "f32":
                assert_rows_rel(out[b, rows].cpu().numpy(), ref[b, rows], 1e-5, "norm+rope f32")
            elif out_kind == "bf16":
                assert_bf16_close(out[b, rows].float().cpu().numpy(), ref[b, rows], "norm+rope bf16")
            else:
                codes, scales = orc.quant_rows_e4m3(ref[b, rows])
                np.testing.assert_allclose(sc[b, rows].cpu().numpy(), scales, rtol=1e-5)
                gv = (gen.host_bits(out[b, rows]).astype(np.int64))
                gvv = np.vectorize(orc.e4m3_decode)(gv)
                rv = np.vectorize(orc.e4m3_decode)(codes)
                step = np.maximum(np.abs(rv), 2.0 ** -6) * 2.0 ** -3
                assert (np.abs(gvv - rv) <= step + 1e-12).all()


def test_compress_rope_decode_step_at_1m():
    # the one-token decode step (few-row projection with split partials)
    # emitting entry 262143 at position 2^20 - 4, RMS norm + RoPE, fp32 store
    d = gen.Draw(95)
    B, dm, E, m, o = 8, 4096, 256, 4, 1
    wk, wg = gen.compressor_weights(d, dm, E, gen.BF16)
    x_tail = gen.store(d.normal(B, 7, dm), gen.BF16)
    x_new = gen.store(d.normal(B, 1, dm), gen.BF16)
    g = 1.0 + 0.1 * d.normal(E)
    T = 1 << 20
    Nc = T // m
    opts = dict(norm_weight=g.to(DEV), norm_eps=1e-6, rope_dim=64, rope_offset=64)
    _, _, st = _run_opts(x_tail.to(DEV), wk.to(DEV), wg.to(DEV), [T - 8] * B, m, o, Nc,
                         torch.float32, **opts)
    out, _, _ = _run_opts(x_new.to(DEV), wk.to(DEV), wg.to(DEV), [T - 1] * B, m, o, Nc,
                          torch.float32, state_in=st, **opts)
    oo = dict(norm_weight=g.numpy(), norm_eps=1e-6, rope_dim=64, rope_offset=64)
    _, _, s_ref = orc.compress(gen.host_bits(x_tail), gen.host_bits(wk), gen.host_bits(wg), m, o,
                               np.full(B, T - 8), Nc, **oo)
    ref, wr, _ = orc.compress(gen.host_bits(x_new), gen.host_bits(wk), gen.host_bits(wg), m, o,
                              np.full(B, T - 1), Nc, state_in=s_ref, **oo)
    assert wr[:, Nc - 1].all()
    assert_rows_rel(out[:, Nc - 1].cpu().numpy(), ref[:, Nc - 1], 1e-5, "decode rope at 1M")
