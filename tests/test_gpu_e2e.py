"""End-to-end CSA prefill (compress x2 -> indexer top-k -> sparse attention)
on the tiny fp32 workload, GPU pipeline against the oracle pipeline."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import assert_rows_rel, check_topk_row, dev_i32, dev_i64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_csa_prefill_tiny_end_to_end():
    w = gen.WORKLOADS["csa_prefill_tiny_f32"]
    inp = gen.prefill_inputs(w)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    pos0 = dev_i64([0])
    kv_cmp = torch.empty(1, w.n_cmp, 2 * w.D, device=DEV)
    k_idx = torch.empty(1, w.n_cmp, w.d_I, device=DEV)
    csa.csa_compress(g["x"], g["w_kv"], g["w_gate"], pos0, w.m, w.overlap, kv_cmp)
    csa.csa_compress(g["x"], g["w_ikv"], g["w_igate"], pos0, w.m, w.overlap, k_idx)
    idx, sc = csa.csa_indexer_topk(g["q_idx"], g["w_idx"], k_idx, w.m, w.topk, pos0,
                                   dev_i32([w.n_cmp]), want_scores=True)
    out, lse = csa.csa_sparse_attn(g["q"], kv_cmp, idx, g["kv_raw"], w.window, pos0, dev_i64([0]),
                                   want_lse=True)
    torch.cuda.synchronize()

    hb = {k: (gen.host_bits(v) if v is not None else None) for k, v in inp.items()}
    o_kv, wr, _ = orc.compress(hb["x"], hb["w_kv"], hb["w_gate"], w.m, w.overlap, 0, w.n_cmp)
    o_k, _, _ = orc.compress(hb["x"], hb["w_ikv"], hb["w_igate"], w.m, w.overlap, 0, w.n_cmp)
    assert wr.all()
    assert_rows_rel(kv_cmp.cpu().numpy()[0], o_kv[0], 1e-5, "kv_cmp")
    assert_rows_rel(k_idx.cpu().numpy()[0], o_k[0], 1e-5, "k_idx")
    # the oracle continues from its own (fp64) compressed entries, stored fp32
    o_idx, _, _, o_all = orc.indexer_topk(hb["q_idx"], hb["w_idx"], o_k.astype(np.float32), w.m,
                                          w.topk, 0, w.n_cmp, want_all=True)
    g_idx = idx.cpu().numpy()
    same = 0
    for t in range(w.T):
        nv = max(0, min(w.n_cmp, (t + 1) // w.m))
        check_topk_row(g_idx[0, t], o_all[0, t], w.topk, nv, "e2e row %d" % t)
        same += np.array_equal(g_idx[0, t], o_idx[0, t])
    assert same >= 0.99 * w.T
    o_out, o_lse = orc.sparse_attn(hb["q"], o_kv.astype(np.float32), o_idx, hb["kv_raw"], w.window,
                                   0, 0)
    rows = [t for t in range(w.T) if np.array_equal(g_idx[0, t], o_idx[0, t])]
    assert_rows_rel(out.cpu().numpy()[0, rows], o_out[0, rows], 1e-5, "e2e out")
    np.testing.assert_allclose(lse.cpu().numpy()[0, rows], o_lse[0, rows], rtol=1e-5, atol=1e-5)
