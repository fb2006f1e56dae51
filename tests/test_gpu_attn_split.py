"""CSA attention taken in two halves (csa_sparse_attn_window_half on a side
stream while other work runs, then csa_sparse_attn_selected_half): parity with
the oracle's joint softmax over the selected entries and the window (DS-V4
analysis section 1.2), and agreement with the one-call csa_sparse_attn."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import assert_bf16_close, dev_i64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _split_call(q, kv_cmp, idx, kv_raw, W, q_pos, raw_base, sink=None, busy=None):
    """Window half on a second stream (beside `busy`, a callable that queues other
    work on the current stream), the selected half after an event."""
    B, T, H, D = q.shape
    topk = idx.shape[2]
    nb = csa.csa_sparse_attn_split_workspace_size(B, T, H, D, topk, W)
    assert nb > 0
    # poisoned workspace: every partial the merge reads must have been written
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)
    qp, rb = dev_i64(q_pos), dev_i64(raw_base)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        csa.csa_sparse_attn_window_half(q, kv_raw, W, qp, rb, topk, ws)
    if busy is not None:
        busy()
    main.wait_stream(side)
    out, lse = csa.csa_sparse_attn_selected_half(q, kv_cmp, idx, kv_raw, W, qp, rb, ws,
                                                 want_lse=True, sink=sink)
    torch.cuda.synchronize()
    return out, lse


def _check(out, lse, ref, ref_lse, what):
    assert_bf16_close(out.float().cpu().numpy(), ref, what)
    gl = lse.cpu().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin), what + " lse finiteness"
    np.testing.assert_allclose(gl[fin], ref_lse[fin], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("with_sink", [False, True])
def test_split_ragged(H, with_sink):
    """Ragged: topk not a multiple of the 64-key tile, absent slots, rows whose window
    is cut by position 0, two query rows per sequence."""
    d = gen.Draw(710 + H + with_sink)
    B, T, D, topk, W, Nc, R = 3, 2, 128, 200, 130, 700, 400
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    nv = torch.tensor([[Nc, Nc], [37, 38], [Nc, Nc]])
    idx = gen.random_index_sets(gen.Draw(720 + H), B, T, topk, nv, 0.2)
    q_pos, raw_base = [R - 2, 5, 300], [0, 0, 0]
    sink = (torch.linspace(-1.0, 2.0, H, dtype=torch.float32) if with_sink else None)
    qd, kcd, krd, idd = q.to(DEV), kv_cmp.to(DEV), kv_raw.to(DEV), idx.to(DEV)
    sd = sink.to(DEV) if sink is not None else None
    scratch = torch.randn(4096, 4096, device=DEV)
    out, lse = _split_call(qd, kcd, idd, krd, W, q_pos, raw_base, sink=sd,
                           busy=lambda: scratch.mul_(1.0001))
    ref, rl = orc.sparse_attn(gen.host_bits(q), gen.host_bits(kv_cmp), idx.numpy(),
                              gen.host_bits(kv_raw), W, q_pos, raw_base,
                              sink=sink.numpy().astype(np.float64) if sink is not None else None)
    _check(out, lse, ref, rl, "split ragged H=%d sink=%s" % (H, with_sink))
    one, one_lse = csa.csa_sparse_attn(qd, kcd, idd, krd, W, dev_i64(q_pos), dev_i64(raw_base),
                                       want_lse=True, sink=sd)
    torch.cuda.synchronize()
    # the one-call form merges different split partials: equal up to fp32 order
    assert_bf16_close(out.float().cpu().numpy(), one.float().cpu().numpy().astype(np.float64),
                      "split vs one call")
    np.testing.assert_allclose(lse.cpu().numpy(), one_lse.cpu().numpy(), rtol=1e-5, atol=1e-5)


def test_split_no_selected_entries():
    """topk = 0: the selected half only merges the window's partials."""
    d = gen.Draw(731)
    B, T, H, D, W, R = 2, 1, 64, 128, 64, 100
    q = gen.store(d.normal(B, T, H, D), gen.BF16)
    kv_raw = gen.store(d.normal(B, R, 2 * D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, 4, 2 * D), gen.BF16)
    idx = torch.empty(B, T, 0, dtype=torch.int32)
    q_pos, raw_base = [R - 1, 20], [0, 0]
    out, lse = _split_call(q.to(DEV), kv_cmp.to(DEV), idx.to(DEV), kv_raw.to(DEV), W, q_pos,
                           raw_base)
    ref, rl = orc.sparse_attn(gen.host_bits(q), gen.host_bits(kv_cmp), idx.numpy(),
                              gen.host_bits(kv_raw), W, q_pos, raw_base)
    _check(out, lse, ref, rl, "split topk=0")


@pytest.mark.parametrize("name", ["csa_decode_128k_b32", "csa_decode_1m_b8_stream"])
def test_split_decode_full_size(name):
    """The decode workloads' shapes, indices spanning the whole compressed cache."""
    w = gen.WORKLOADS[name]
    d = gen.Draw(w.seed + 740, DEV)
    B, Nc = w.B, w.n_cmp
    kv_cmp = gen.store(d.normal(B, Nc, 2 * w.D), gen.BF16)
    kv_raw = gen.store(d.normal(B, w.window, 2 * w.D), gen.BF16)
    q = gen.store(d.normal(B, 1, w.H, w.D), gen.BF16)
    nv = torch.full((B, 1), Nc)
    idx = gen.random_index_sets(gen.Draw(w.seed + 741), B, 1, w.topk, nv, 0.0)
    q_pos = [w.ctx - 1] * B
    raw_base = [w.ctx - w.window] * B
    out, lse = _split_call(q, kv_cmp, idx.to(DEV), kv_raw, w.window, q_pos, raw_base)
    ref, rl = orc.sparse_attn(gen.host_bits(q), gen.host_bits(kv_cmp), idx.numpy(),
                              gen.host_bits(kv_raw), w.window, q_pos, raw_base)
    _check(out, lse, ref, rl, name + " split")


def test_split_rejects_unsupported():
    """Prefill-sized calls, f32 and a short workspace are refused before any launch."""
    B, T, H, D, topk, W = 1, 1024, 64, 128, 64, 64
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16, device=DEV)
    kv_raw = torch.zeros(B, 8, 2 * D, dtype=torch.bfloat16, device=DEV)
    assert csa.csa_sparse_attn_split_workspace_size(B, T, H, D, topk, W) == 0
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError):
        csa.csa_sparse_attn_window_half(q, kv_raw, W, dev_i64([0]), dev_i64([0]), topk, ws)
    q1 = torch.zeros(1, 1, H, D, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError):  # workspace too small
        csa.csa_sparse_attn_window_half(q1, kv_raw, W, dev_i64([7]), dev_i64([0]), topk, ws)
    q32 = torch.zeros(1, 1, H, D, dtype=torch.float32, device=DEV)
    kv32 = torch.zeros(1, 8, 2 * D, dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError):
        csa.csa_sparse_attn_window_half(q32, kv32, W, dev_i64([7]), dev_i64([0]), topk, ws)
