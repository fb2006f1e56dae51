"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, sizes workspaces, and rejects bad arguments before touching
the device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


@pytest.fixture(scope="module")
def L():
    import compressed_sparse_attention_overlapped_amd as csa
    if not os.path.exists(csa.LIB_PATH):
        from compressed_sparse_attention_overlapped_amd import build
        build.build()
    return csa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_\w+|hca_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["csa_compress", "csa_indexer_topk", "csa_sparse_attn", "hca_dense_attn",
              "csa_status_string", "csa_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.csa_status_string(0) == b"ok"
    assert L.csa_status_string(3) == b"workspace too small"


def test_workspace_sizes(L):
    # long rows need the score row plus chunk lists (or segment candidates);
    # short rows only scores
    a = L.csa_indexer_topk_workspace_size(8, 1, 16, 64, 262144, 2048, 2)
    assert a >= 8 * 262144 * 4 * 3
    assert L.csa_indexer_topk_workspace_size(1, 8192, 16, 64, 2048, 512, 1) == 8192 * 2048 * 4
    assert L.csa_sparse_attn_workspace_size(1, 8192, 64, 128, 512, 512) == 0   # no split
    assert L.csa_sparse_attn_workspace_size(32, 1, 64, 128, 2048, 512) > 0     # split-K partials


def test_argument_errors_are_reported_without_launch(L):
    vp = C.c_void_p
    dummy = vp(16)   # never dereferenced: validation fails first
    # B = 0
    rc = L.csa_compress(0, 1, 64, 8, 4, 1, 0, dummy, dummy, dummy, dummy, 0, None, None, None,
                        dummy, None, 0, 10, None, 0, None)
    assert rc == 1 and b"must be > 0" in L.csa_last_error()
    # overlap 2
    rc = L.csa_compress(1, 1, 64, 8, 4, 2, 0, dummy, dummy, dummy, dummy, 0, None, None, None,
                        dummy, None, 0, 10, None, 0, None)
    assert rc == 1
    # rotation of a width that is not a power of two
    rc = L.csa_compress(1, 1, 64, 6, 4, 1, 1, dummy, dummy, dummy, dummy, 0, None, None, None,
                        dummy, None, 0, 10, None, 0, None)
    assert rc == 1 and b"power of two" in L.csa_last_error()
    # fp8 output without scales
    rc = L.csa_compress(1, 1, 64, 8, 4, 1, 0, dummy, dummy, dummy, dummy, 0, None, None, None,
                        dummy, None, 2, 10, None, 0, None)
    assert rc == 1 and b"out_scale" in L.csa_last_error()
    # mxfp4 output without scales, and with a width that is not a multiple of 32
    rc = L.csa_compress(1, 1, 64, 64, 4, 1, 0, dummy, dummy, dummy, dummy, 0, None, None, None,
                        dummy, None, 3, 10, None, 0, None)
    assert rc == 1 and b"out_scale" in L.csa_last_error()
    rc = L.csa_compress(1, 1, 64, 48, 4, 1, 0, dummy, dummy, dummy, dummy, 0, None, None, None,
                        dummy, dummy, 3, 10, None, 0, None)
    assert rc == 2 and b"E % 32" in L.csa_last_error()
    # state aliasing
    rc = L.csa_compress(1, 1, 64, 8, 4, 1, 0, dummy, dummy, dummy, dummy, 0, None, dummy, dummy,
                        dummy, None, 0, 10, None, 0, None)
    assert rc == 1 and b"alias" in L.csa_last_error()
    # mxfp4 indexer inputs without their block scales
    rc = L.csa_indexer_topk(1, 1, 16, 64, 100, 4, 10, dummy, dummy, dummy, None, dummy, dummy,
                            None, 3, dummy, None, None, 0, None)
    assert rc == 1 and b"q_scale" in L.csa_last_error()
    # unsupported indexer geometry
    rc = L.csa_indexer_topk(1, 1, 8, 64, 100, 4, 10, dummy, dummy, dummy, None, dummy, dummy, None,
                            1, dummy, None, None, 0, None)
    assert rc == 2
    # workspace too small
    rc = L.csa_indexer_topk(1, 1, 16, 64, 100, 4, 10, dummy, dummy, dummy, None, dummy, dummy,
                            None, 1, dummy, None, None, 0, None)
    assert rc == 3
    # bf16 attention with an unsupported head count
    rc = L.csa_sparse_attn(1, 1, 8, 128, 4, 4, C.c_float(1.0), None, dummy, dummy, dummy, 4,
                           dummy, dummy, 4, dummy, 1, dummy, None, None, 0, None)
    assert rc == 2
    # HCA without n_cmp
    rc = L.hca_dense_attn(1, 1, 64, 128, 128, 4, C.c_float(1.0), None, dummy, None, dummy, dummy,
                          4, dummy, 4, dummy, 1, dummy, None, None, 0, None)
    assert rc == 1


def _PT(block_table, page_size, max_pages, n_pages):
    import compressed_sparse_attention_overlapped_amd as csa
    return csa._CPageTable(block_table, page_size, max_pages, n_pages)


def test_paged_entry_points_validate_the_page_table(L):
    vp = C.c_void_p
    dummy = vp(16)   # never dereferenced: validation fails first
    import compressed_sparse_attention_overlapped_amd as csa
    csa.lib()        # argtypes for the paged entry points

    def compress(pt):
        return L.csa_compress_paged(1, 1, 64, 8, 4, 1, 0, dummy, dummy, dummy, dummy, 0, None, None,
                                    None, dummy, None, 0, 100, pt, dummy, 1 << 20, None)
    rc = compress(None)
    assert rc == 1 and b"pages is required" in L.csa_last_error()
    rc = compress(C.byref(_PT(None, 64, 4, 4)))
    assert rc == 1 and b"block_table" in L.csa_last_error()
    rc = compress(C.byref(_PT(16, 24, 8, 8)))
    assert rc == 1 and b"power of two" in L.csa_last_error()
    rc = compress(C.byref(_PT(16, 8, 16, 16)))          # below the 16-row minimum
    assert rc == 1 and b"power of two" in L.csa_last_error()
    rc = compress(C.byref(_PT(16, 16, 4, 8)))           # 64 logical rows < Nc_cap 100
    assert rc == 1 and b"exceeds" in L.csa_last_error()
    # paged indexer keys must be bf16, fp8 or mxfp4 (an fp32 call is refused before launch)
    rc = L.csa_indexer_topk_paged(1, 1, 4, 32, 100, 4, 10, dummy, dummy, dummy, None, dummy,
                                  dummy, None, 0, C.byref(_PT(16, 64, 2, 2)), dummy, None, dummy,
                                  1 << 30, None)
    assert rc == 2 and b"BF16, FP8E4M3 or MXFP4" in L.csa_last_error()
    # paged attention: the workspace also holds the pool rows of the selection
    a = L.csa_sparse_attn_paged_workspace_size(2, 1, 64, 128, 512, 128)
    b = L.csa_sparse_attn_workspace_size(2, 1, 64, 128, 512, 128)
    assert a == b + 2 * 512 * 4
    rc = L.csa_sparse_attn_paged(1, 1, 64, 128, 4, 4, C.c_float(1.0), None, dummy, dummy, dummy, 64,
                                 None, dummy, dummy, 4, dummy, None, 1, dummy, None, dummy, 1 << 30,
                                 None)
    assert rc == 1 and b"pages or raw_pages is required" in L.csa_last_error()
    # a window table shorter than R_cap
    rc = L.csa_sparse_attn_paged(1, 1, 64, 128, 4, 4, C.c_float(1.0), None, dummy, dummy, dummy, 64,
                                 None, dummy, dummy, 100, dummy, C.byref(_PT(16, 16, 4, 8)), 1,
                                 dummy, None, dummy, 1 << 30, None)
    assert rc == 1 and b"exceeds" in L.csa_last_error()
    rc = L.hca_dense_attn_paged(1, 1, 64, 128, 128, 4, C.c_float(1.0), None, dummy, dummy, dummy,
                                dummy, 64, None, dummy, 4, dummy, None, 1, dummy, None, dummy,
                                1 << 30, None)
    assert rc == 1 and b"pages or raw_pages is required" in L.csa_last_error()


def test_page_table_checks_reject_bad_tables_before_any_call():
    # the C ABI sees only pointers: the binding checks what it can see
    import torch

    import compressed_sparse_attention_overlapped_amd as csa
    table = torch.zeros(2, 4, dtype=torch.int32)
    pt = csa.PageTable(table, 16, n_pages=8)
    pool = torch.zeros(8 * 16, 64)
    with pytest.raises(ValueError, match="sequences"):
        pt.check(3, pool)                       # a table row per sequence
    with pytest.raises(ValueError, match="rows"):
        pt.check(2, torch.zeros(8 * 16 - 1, 64))  # pool shorter than n_pages pages
    with pytest.raises(ValueError, match="device"):
        pt.check(2, pool)                       # a host table with the caches
    with pytest.raises(ValueError, match="int32"):
        csa.PageTable(table.long(), 16, 8)


def test_compress_ex_rejects_bad_rotary_slices(L):
    import compressed_sparse_attention_overlapped_amd as csa
    vp = C.c_void_p
    p = vp(256)
    for dim, off, base, ok in ((3, 0, 1e4, False), (16, 60, 1e4, False), (16, 0, 0.0, False),
                               (-2, 0, 1e4, False)):
        o = csa._COpts(None, 1e-6, dim, off, base, 0)
        rc = L.csa_compress_ex(1, 4, 64, 64, 4, 1, 0, p, p, p, p, 0, None, None, None, p, None, 0,
                               8, None, C.byref(o), None, 0, None)
        assert rc == 1, (dim, off, base)
        assert b"rope" in L.csa_last_error()


def test_backward_entry_points_validate_before_any_launch(L):
    vp = C.c_void_p
    d = vp(16)   # never dereferenced: validation fails first
    f = C.c_float(0.088)
    # attention backward: fp32 inputs are not supported; dsink without sink;
    # a too small workspace; too many index slots
    rc = L.csa_sparse_attn_bwd(1, 8, 64, 128, 4, 4, f, None, d, d, d, 16, d, d, 16, d, 0, d, d,
                               d, d, d, None, None, d, 10 ** 9, None)
    assert rc == 2 and b"BF16" in L.csa_last_error()
    rc = L.csa_sparse_attn_bwd(1, 8, 64, 128, 4, 4, f, None, d, d, d, 16, d, d, 16, d, 1, d, d,
                               d, d, d, d, None, d, 10 ** 9, None)
    assert rc == 1 and b"dsink needs sink" in L.csa_last_error()
    rc = L.csa_sparse_attn_bwd(1, 8, 64, 128, 4, 4, f, None, d, d, d, 16, d, d, 16, d, 1, d, d,
                               d, d, d, None, None, d, 1, None)
    assert rc == 3
    rc = L.csa_sparse_attn_bwd(1, 8, 64, 128, 5000, 4, f, None, d, d, d, 16, d, d, 16, d, 1, d,
                               d, d, d, d, None, None, d, 10 ** 9, None)
    assert rc == 2 and b"topk" in L.csa_last_error()
    rc = L.hca_dense_attn_bwd(1, 8, 48, 128, 4, 4, f, None, d, d, d, d, 16, d, 16, d, 1, d, d,
                              d, d, d, None, None, d, 10 ** 9, None)
    assert rc == 2 and b"H in {32, 64}" in L.csa_last_error()
    # indexer KL loss: geometry, topk limit, a missing mass
    rc = L.csa_indexer_kl_bwd(1, 8, 8, 64, 32, 4, d, d, d, 1, d, d, None, d, d, d, d, d,
                              10 ** 9, None)
    assert rc == 2 and b"H_I = 16" in L.csa_last_error()
    rc = L.csa_indexer_kl_bwd(1, 8, 16, 64, 32, 2048, d, d, d, 1, d, d, None, d, d, d, d, d,
                              10 ** 9, None)
    assert rc == 2 and b"topk" in L.csa_last_error()
    rc = L.csa_indexer_kl_bwd(1, 8, 16, 64, 32, 4, d, d, d, 1, d, None, None, d, d, d, d, d,
                              10 ** 9, None)
    assert rc == 1
    # dense indexer KL loss: geometry, m, a missing mass, the cache limit
    rc = L.csa_indexer_kl_dense_bwd(1, 8, 8, 64, 32, 4, d, d, d, d, d, 1, d, None, d, d, d, d,
                                    d, 10 ** 9, None)
    assert rc == 2 and b"H_I = 16" in L.csa_last_error()
    rc = L.csa_indexer_kl_dense_bwd(1, 8, 16, 64, 32, 0, d, d, d, d, d, 1, d, None, d, d, d, d,
                                    d, 10 ** 9, None)
    assert rc == 1
    rc = L.csa_indexer_kl_dense_bwd(1, 8, 16, 64, 32, 4, d, d, d, d, d, 1, None, None, d, d, d,
                                    d, d, 10 ** 9, None)
    assert rc == 1 and b"missing" in L.csa_last_error()
    rc = L.csa_indexer_kl_dense_bwd(1, 8, 16, 64, 70000, 4, d, d, d, d, d, 1, d, None, d, d, d,
                                    d, d, 10 ** 9, None)
    assert rc == 2 and b"Nc_cap" in L.csa_last_error()
    rc = L.csa_indexer_kl_dense_bwd(1, 8, 16, 64, 32, 4, d, d, d, d, d, 1, d, None, d, d, d, d,
                                    d, 16, None)
    assert rc == 3
    # compressor backward: fp32 tokens, a rotation of a width that is not a
    # power of two, dape without ape, d_model not a multiple of 64
    rc = L.csa_compress_bwd(1, 64, 128, 32, 4, 1, 0, d, d, d, 0, None, 16, d, d, d, d, None, d,
                            10 ** 9, None)
    assert rc == 2 and b"BF16" in L.csa_last_error()
    rc = L.csa_compress_bwd(1, 64, 128, 48, 4, 1, 1, d, d, d, 1, None, 16, d, d, d, d, None, d,
                            10 ** 9, None)
    assert rc == 1 and b"power of two" in L.csa_last_error()
    rc = L.csa_compress_bwd(1, 64, 128, 32, 4, 1, 0, d, d, d, 1, None, 16, d, d, d, d, d, d,
                            10 ** 9, None)
    assert rc == 1 and b"dape needs ape" in L.csa_last_error()
    rc = L.csa_compress_bwd(1, 64, 100, 32, 4, 1, 0, d, d, d, 1, None, 16, d, d, d, d, None, d,
                            10 ** 9, None)
    assert rc == 2 and b"multiple of 64" in L.csa_last_error()
    # with entry post-processing: a norm weight without its gradient's
    # output, an odd rotary slice, a slice past the entry
    import compressed_sparse_attention_overlapped_amd as csa
    o = csa._COpts(d.value, 1e-6, 0, 0, 10000.0, 0)
    rc = L.csa_compress_bwd_ex(1, 64, 128, 32, 4, 1, 0, d, d, d, 1, None, 16, d, C.byref(o), d,
                               d, d, None, None, d, 10 ** 9, None)
    assert rc == 1 and b"d_norm_weight" in L.csa_last_error()
    for dim, off in ((3, 0), (8, 28)):
        o = csa._COpts(None, 1e-6, dim, off, 10000.0, 0)
        rc = L.csa_compress_bwd_ex(1, 64, 128, 32, 4, 1, 0, d, d, d, 1, None, 16, d, C.byref(o),
                                   d, d, d, None, None, d, 10 ** 9, None)
        assert rc == 1 and b"rope" in L.csa_last_error(), (dim, off)


def test_backward_workspace_sizes(L):
    # the attention backward's workspace grows with the window rows and the
    # compressed entries, and covers the per-row terms at least
    a = L.csa_sparse_attn_bwd_workspace_size(1, 8192, 64, 2048, 8192, 512)
    assert a >= 8192 * (2 * 64 + 64) * 4 and a < 512 * 2 ** 20
    assert L.csa_sparse_attn_bwd_workspace_size(1, 8192, 64, 2048, 8192, 0) < a
    assert L.hca_dense_attn_bwd_workspace_size(1, 4096, 64, 8192, 4607, 512) > 0
    assert L.csa_indexer_kl_bwd_workspace_size(1, 8192, 2048, 512) >= 8192 * 512 * 4
    assert L.csa_indexer_kl_dense_bwd_workspace_size(1, 8192, 2048) >= 8192 * 2048 * 4
    assert L.csa_indexer_kl_dense_bwd_workspace_size(0, 8192, 2048) == 0
    assert L.csa_compress_bwd_workspace_size(1, 8192, 4096, 256, 4, 2048) >= 8192 * 512 * 6 + 512 * 4096 * 6
    assert L.csa_compress_bwd_workspace_size(1, 8192, 0, 256, 4, 2048) == 0
    assert L.csa_sparse_attn_bwd_workspace_size(0, 8, 64, 16, 16, 4) == 0
