"""csa_sparse_attn_noalloc: the attention entry point that allocates nothing
(its split-key partials live in the library's static device scratch),
checked through the C ABI against csa_sparse_attn with a workspace."""
import ctypes as C

import numpy as np
import pytest
import torch

import compressed_sparse_attention_overlapped_amd as csa
from compressed_sparse_attention_overlapped_amd import inputs as gen
from oracle import oracle as orc
from tests.helpers import assert_bf16_close, dev_i64

DEV = "cuda"


def _case(seed, B, topk, W, Nc, H=64, D=128, m=4):
    d = gen.Draw(seed)
    q = gen.store(d.normal(B, 1, H, D), gen.BF16)
    kv_cmp = gen.store(d.normal(B, Nc, 2 * D), gen.BF16)
    kv_raw = gen.store(d.normal(B, W, 2 * D), gen.BF16)
    q_pos = [m * Nc - 1 - 7 * b for b in range(B)]
    raw_base = [p + 1 - W for p in q_pos]
    nv = torch.tensor([[min(Nc, (p + 1) // m)] for p in q_pos])
    idx = gen.random_index_sets(d, B, 1, topk, nv, 0.05)
    return q, kv_cmp, kv_raw, idx, q_pos, raw_base


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    # two calls in a row on one device, the second smaller: each equals
    # csa_sparse_attn bit for bit (same kernels, partials in the static
    # scratch instead of a workspace) and the oracle within the bf16 bound
    for seed, B, topk, W, Nc in ((81, 24, 2048, 512, 40000), (82, 3, 256, 64, 3000)):
        print("noalloc case B=%d topk=%d W=%d Nc=%d" % (B, topk, W, Nc), flush=True)
        q, kv_cmp, kv_raw, idx, q_pos, raw_base = _case(seed, B, topk, W, Nc)
        assert csa.csa_sparse_attn_workspace_size(B, 1, 64, 128, topk, W) > 0   # split keys
        g = [t.to(DEV) for t in (q, kv_cmp, idx, kv_raw)]
        qp, rb = dev_i64(q_pos), dev_i64(raw_base)
        ref_out, ref_lse = csa.csa_sparse_attn(*g[:3], g[3], W, qp, rb, want_lse=True)
        out = torch.empty_like(g[0])
        lse = torch.empty(B, 1, 64, device=DEV)
        csa.csa_sparse_attn_noalloc(*g[:3], g[3], W, qp, rb, out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out, B=%d" % B
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "lse, B=%d" % B
        rows = [0, B - 1]
        r, _ = orc.sparse_attn(gen.host_bits(q)[rows], gen.host_bits(kv_cmp)[rows],
                               idx.numpy()[rows], gen.host_bits(kv_raw)[rows], W,
                               [q_pos[i] for i in rows], [raw_base[i] for i in rows])
        assert_bf16_close(out.float().cpu().numpy()[rows], r, "noalloc vs oracle B=%d" % B)


def test_noalloc_rejects_calls_beyond_the_static_scratch():
    # rejected on the host before any launch (the pointers are never used):
    # 900 decode rows of 100000 keys need far more than 16 MiB of partials
    L = csa.lib()
    p = C.c_void_p(256)
    need = L.csa_sparse_attn_workspace_size(900, 1, 64, 128, 100000, 0)
    assert need > (16 << 20)
    rc = L.csa_sparse_attn_noalloc(900, 1, 64, 128, 100000, 0, 0.1, None, p, p, p, 1 << 20, p, p,
                                   0, p, csa.DT_BF16, p, None, None)
    assert rc == 2
    assert b"static scratch" in L.csa_last_error()
