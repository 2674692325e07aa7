"""The C ABI without a GPU: the library loads, exports every entry point that
include/dsa.h declares, and rejects invalid arguments on the host before anything
is enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def m():
    import sparse_attention_fp8_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points(m):
    names = declared_functions()
    for required in ["dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_forward"]:
        assert required in names
    assert sorted(m.EXPORTED_SYMBOLS) == names


def test_library_exports_every_declared_symbol(m):
    for name in declared_functions():
        assert hasattr(m.lib, name), name


def test_status_strings_and_version(m):
    assert m.lib.dsa_api_version() == 2
    for st in range(5):
        assert m.lib.dsa_status_string(st).decode().startswith("DSA_")


def _rows(m, R=4, B=2, N=64, max_pos=63, seq=1, pos=1):
    return m._Rows(R, B, N, max_pos, seq, pos)  # dummy non-NULL "device" addresses


def test_invalid_arguments_rejected_on_host(m):
    L = m.lib
    d = m.dims_struct(m.PRODUCTION_DIMS)
    r = _rows(m)
    p = ctypes.c_void_p(16)
    # NULL rows / dims
    assert L.dsa_topk(None, 2048, p, 64, p, None, 0, None) == m.DSA_E_INVALID
    assert L.dsa_indexer_scores(ctypes.byref(r), None, p, p, p, p, p, p, 64, None) == m.DSA_E_INVALID
    # max_pos outside [0, N)
    bad = _rows(m, max_pos=64)
    assert L.dsa_topk(ctypes.byref(bad), 2048, p, 64, p, None, 0, None) == m.DSA_E_INVALID
    # ld too small
    assert L.dsa_topk(ctypes.byref(r), 2048, p, 63, p, None, 0, None) == m.DSA_E_INVALID
    # topk out of range
    assert L.dsa_topk(ctypes.byref(r), 0, p, 64, p, None, 0, None) == m.DSA_E_UNSUPPORTED
    assert L.dsa_topk(ctypes.byref(r), 5000, p, 64, p, None, 0, None) == m.DSA_E_UNSUPPORTED
    # NULL tensors
    assert L.dsa_topk(ctypes.byref(r), 2048, None, 64, p, None, 0, None) == m.DSA_E_INVALID
    # fp8 indexer without scales
    assert L.dsa_indexer_scores(ctypes.byref(r), ctypes.byref(d), p, None, p, p, None, p, 64,
                                None) == m.DSA_E_INVALID
    assert "scale" in L.dsa_last_error().decode()
    # unsupported dims
    odd = m.dims_struct(m.Dims(32, 128, 128, 576, 512, 2048, False))
    assert L.dsa_indexer_scores(ctypes.byref(r), ctypes.byref(odd), p, p, p, p, p, p, 64,
                                None) == m.DSA_E_UNSUPPORTED
    # workspace too small
    rows_dec = _rows(m, R=32, B=32, N=32768, max_pos=32767)
    need = L.dsa_sparse_mla_attn_workspace_size(ctypes.byref(rows_dec), ctypes.byref(d))
    assert need > 0
    assert L.dsa_sparse_mla_attn(ctypes.byref(rows_dec), ctypes.byref(d), p, p, p, 0.1, p, p, p,
                                 need - 1, None) == m.DSA_E_WORKSPACE
    assert L.dsa_forward(ctypes.byref(rows_dec), ctypes.byref(d), p, p, p, p, p, p, p, 0.1, p, p,
                         None, 0, p, 16, None) == m.DSA_E_WORKSPACE
    # zero rows: nothing to do
    empty = _rows(m, R=0, seq=None, pos=None)
    assert L.dsa_topk(ctypes.byref(empty), 2048, None, 64, None, None, 0, None) == m.DSA_OK


def test_workspace_sizes(m):
    L = m.lib
    d = m.dims_struct(m.PRODUCTION_DIMS)
    dec = _rows(m, R=32, B=32, N=32768, max_pos=32767)
    attn = L.dsa_sparse_mla_attn_workspace_size(ctypes.byref(dec), ctypes.byref(d))
    assert attn == 32 * 8 * 128 * (512 * 2 + 4)   # 8 splits of bf16 partial outputs + fp32 lse
    # 8 rows (decode 128K): 16 splits of 4 stages rather than 32 of 2
    r8 = _rows(m, R=8, B=8, N=131072, max_pos=131071)
    assert L.dsa_sparse_mla_attn_workspace_size(ctypes.byref(r8), ctypes.byref(d)) == \
        8 * 16 * 128 * (512 * 2 + 4)
    fwd = L.dsa_forward_workspace_size(ctypes.byref(dec), ctypes.byref(d), 0)
    # rows of up to 32768 positions take one block each (their scores fit in the
    # block's registers): no top-k workspace, also when few rows leave CUs idle
    assert L.dsa_topk_workspace_size(ctypes.byref(dec), 2048) == 0
    assert fwd >= attn + 32 * 32768 * 4 + 32 * 2048 * 4
    assert L.dsa_topk_workspace_size(ctypes.byref(_rows(m, R=8192, B=1, N=8192, max_pos=8191)),
                                     2048) == 0
    assert L.dsa_topk_workspace_size(ctypes.byref(_rows(m, R=32, B=32, N=8192, max_pos=8191)),
                                     2048) == 0
    # few longer rows are split over several blocks each
    d128 = _rows(m, R=8, B=8, N=131072, max_pos=131071)
    tk = L.dsa_topk_workspace_size(ctypes.byref(d128), 2048)
    # candidates [8 rows, 32 chunks, 4096] of 8 bytes, their counts and the per-row counts
    assert tk == 8 * 32 * 4096 * 8 + (8 * 32 * 4 + 8 * 4 + 15) // 16 * 16
    assert L.dsa_topk_workspace_size(ctypes.byref(_rows(m, R=128, B=128, N=131072,
                                                        max_pos=131071)), 2048) == 0
    p = ctypes.c_void_p(16)
    assert L.dsa_topk(ctypes.byref(d128), 2048, p, 131072, p, p, tk - 1, None) == m.DSA_E_WORKSPACE
    pre = _rows(m, R=131072, B=1, N=131072, max_pos=131071)
    w = L.dsa_forward_workspace_size(ctypes.byref(pre), ctypes.byref(d), 8192)
    assert w >= 8192 * 131072 * 4 and w < 8192 * 131072 * 4 + 8192 * 2048 * 4 + (1 << 20)
    f32 = m.dims_struct(m.Dims(4, 32, 16, 80, 64, 64, True))
    tiny = _rows(m, R=256, B=1, N=256, max_pos=255)
    assert L.dsa_sparse_mla_attn_workspace_size(ctypes.byref(tiny), ctypes.byref(f32)) == 0
    # backward: header, per-row flags, key counts and accumulator slots of the B (max_pos + 1) keys,
    # chunk sums of dq and dw (R rows x E chunks x (64 x 128 + 64) floats, E > 1), then
    # the accumulators (4 + 1024 bytes each)
    a256 = lambda x: (x + 255) // 256 * 256
    def bwd_size(R, B, P, E, cap):
        base = 256 + a256(R * 4) + a256((B * P + 3) // 4 * 16) + a256(B * P * 4) + \
            (a256(R * E * 8256 * 4) if E > 1 else 0)
        return base + a256(cap * 4) + cap * 1024
    sz = lambda rows, k: L.dsa_indexer_backward_workspace_size(ctypes.byref(rows), ctypes.byref(d), k)
    szd = lambda rows, k: L.dsa_indexer_backward_dense_workspace_size(ctypes.byref(rows),
                                                                      ctypes.byref(d), k)
    # decode 32K: 8 chunks of 256 entries per row; at most R k / 2 keys selected twice
    assert sz(dec, 0) == bwd_size(32, 32, 32768, 8, 0)
    assert sz(dec, -1) == bwd_size(32, 32, 32768, 8, 32 * 2048 // 2)
    assert sz(dec, 100) == bwd_size(32, 32, 32768, 8, 100)
    assert szd(dec, -1) == bwd_size(32, 32, 32768, 8, 32 * 32768 // 2)
    # prefill 8K chunk: one chunk per row (no chunk sums); at most B (max_pos + 1) keys
    pre8 = _rows(m, R=8192, B=1, N=8192, max_pos=8191)
    assert sz(pre8, -1) == bwd_size(8192, 1, 8192, 1, 8192)
    assert sz(pre8, 1 << 40) == sz(pre8, -1)
    assert L.dsa_indexer_backward_workspace_size(ctypes.byref(dec), ctypes.byref(f32), -1) == 0


def test_project_append_host_checks(m):
    L = m.lib
    d = m.dims_struct(m.PRODUCTION_DIMS)
    r = _rows(m, R=32, B=32, N=32768, max_pos=32767)
    p = ctypes.c_void_p(16)
    ptrs = [p] * 11
    # d_model not a multiple of 64, too large, or zero
    for dm in (0, 100, 65600):
        assert L.dsa_project_append(ctypes.byref(r), ctypes.byref(d), dm, *ptrs, p, 1 << 30,
                                    None) == m.DSA_E_UNSUPPORTED
    # only the production indexer / latent dims have a kernel
    f32 = m.dims_struct(m.Dims(4, 32, 16, 80, 64, 64, True))
    assert L.dsa_project_append(ctypes.byref(r), ctypes.byref(f32), 7168, *ptrs, p, 1 << 30,
                                None) == m.DSA_E_UNSUPPORTED
    # a NULL output
    bad = list(ptrs)
    bad[9] = None
    assert L.dsa_project_append(ctypes.byref(r), ctypes.byref(d), 7168, *bad, p, 1 << 30,
                                None) == m.DSA_E_INVALID
    # decode-sized calls split the contraction and need the partial-sum workspace
    need = L.dsa_project_append_workspace_size(ctypes.byref(r), 7168)
    assert need == 7 * 32 * 8960 * 4
    assert L.dsa_project_append(ctypes.byref(r), ctypes.byref(d), 7168, *ptrs, p, need - 1,
                                None) == m.DSA_E_WORKSPACE
    # prefill-sized calls split nothing; zero rows do nothing
    big = _rows(m, R=8192, B=1, N=8192, max_pos=8191)
    assert L.dsa_project_append_workspace_size(ctypes.byref(big), 7168) == 0
    empty = _rows(m, R=0, seq=None, pos=None)
    assert L.dsa_project_append(ctypes.byref(empty), ctypes.byref(d), 7168, *([None] * 11), None,
                                0, None) == m.DSA_OK


def test_paged_host_checks(m):
    L = m.lib
    d = m.dims_struct(m.PRODUCTION_DIMS)
    r = _rows(m, R=32, B=32, N=32768, max_pos=32767)
    p = ctypes.c_void_p(16)

    def pages(P=64, pps=512, n=32 * 512, table=16):
        return m._Pages(P, pps, n, table)

    def idx(pg, rows=r, dims=d):
        return L.dsa_indexer_scores_paged(ctypes.byref(rows), ctypes.byref(dims),
                                          None if pg is None else ctypes.byref(pg),
                                          p, p, p, p, p, p, 32768, None)
    assert idx(None) == m.DSA_E_INVALID
    for P in (32, 96, 1 << 17):
        assert idx(pages(P=P, pps=max(1, 32768 // P))) == m.DSA_E_UNSUPPORTED
    assert idx(pages(pps=256)) == m.DSA_E_INVALID                 # max_ctx != pps * P
    assert idx(pages(table=None)) == m.DSA_E_INVALID
    assert idx(pages(n=0)) == m.DSA_E_INVALID
    f32 = m.dims_struct(m.Dims(4, 32, 16, 80, 64, 64, True))
    assert idx(pages(), dims=f32) == m.DSA_E_UNSUPPORTED
    # a latent pool past 4 GiB cannot be addressed with 32-bit offsets
    big = pages(n=(1 << 32) // (64 * 1152) + 1)
    assert L.dsa_sparse_mla_attn_paged(ctypes.byref(r), ctypes.byref(d), ctypes.byref(big), p, p,
                                       p, 0.1, p, p, p, 1 << 30, None) == m.DSA_E_UNSUPPORTED
    # the same pool size is fine for the 128-byte key rows
    empty = _rows(m, R=0, B=32, N=32768, max_pos=32767, seq=None, pos=None)
    assert idx(big, rows=empty) == m.DSA_OK
    assert L.dsa_forward_paged(ctypes.byref(r), ctypes.byref(d), ctypes.byref(pages()), p, p, p, p,
                               p, p, p, 0.1, p, p, None, 0, p, 16, None) == m.DSA_E_WORKSPACE
    assert L.dsa_project_append_paged(ctypes.byref(r), ctypes.byref(d), ctypes.byref(pages()), 100,
                                      *([p] * 11), p, 1 << 30, None) == m.DSA_E_UNSUPPORTED


def test_training_and_mha_host_checks(m):
    """The loss, backward and masked-MHA entry points reject invalid arguments on
    the host, and their workspace sizes follow the documented layouts."""
    L = m.lib
    d = m.dims_struct(m.PRODUCTION_DIMS)
    f32 = m.dims_struct(m.Dims(4, 32, 16, 80, 64, 64, True))
    p = ctypes.c_void_p(16)
    dec = _rows(m, R=32, B=32, N=32768, max_pos=32767)
    # dense warm-up loss: workspace = target [R, C * 1024] + per-chunk (max, sum) [R, C, 128]
    need = L.dsa_indexer_loss_dense_workspace_size(ctypes.byref(dec), ctypes.byref(d))
    assert need == 32 * 32 * (1024 * 4 + 128 * 8)
    assert L.dsa_indexer_loss_dense_workspace_size(ctypes.byref(dec), ctypes.byref(f32)) == 0
    dense = lambda rows, dims, ld, ws, n: L.dsa_indexer_loss_dense(
        ctypes.byref(rows), dims, p, p, 0.1, p, ld, p, p, ws, n, None)
    assert dense(dec, ctypes.byref(f32), 32768, p, need) == m.DSA_E_UNSUPPORTED
    assert dense(dec, None, 32768, p, need) == m.DSA_E_INVALID
    assert dense(dec, ctypes.byref(d), 32767, p, need) == m.DSA_E_INVALID      # ld < max_pos + 1
    assert dense(dec, ctypes.byref(d), 32768, p, need - 1) == m.DSA_E_WORKSPACE
    assert dense(dec, ctypes.byref(d), 32768, None, need) == m.DSA_E_WORKSPACE
    assert L.dsa_indexer_loss_dense(ctypes.byref(dec), ctypes.byref(d), None, p, 0.1, p, 32768, p,
                                    p, p, need, None) == m.DSA_E_INVALID
    # dense backward
    nbd = L.dsa_indexer_backward_dense_workspace_size(ctypes.byref(dec), ctypes.byref(d), 0)
    bwd = lambda ld, dq, ws, n: L.dsa_indexer_backward_dense(ctypes.byref(dec), ctypes.byref(d), p,
                                                             p, p, p, p, p, ld, dq, p, p, ws, n, None)
    assert bwd(32767, p, p, nbd) == m.DSA_E_INVALID
    assert bwd(32768, None, p, nbd) == m.DSA_E_INVALID
    assert bwd(32768, p, p, nbd - 1) == m.DSA_E_WORKSPACE
    assert bwd(32768, p, None, nbd) == m.DSA_E_WORKSPACE
    # sparse backward
    nb = L.dsa_indexer_backward_workspace_size(ctypes.byref(dec), ctypes.byref(d), 0)
    sb = lambda rows, dims, ws, n: L.dsa_indexer_backward(ctypes.byref(rows), dims, p, p, p, p, p,
                                                          p, p, p, p, p, ws, n, None)
    assert sb(dec, ctypes.byref(f32), p, nb) == m.DSA_E_UNSUPPORTED
    assert sb(dec, None, p, nb) == m.DSA_E_INVALID
    assert sb(dec, ctypes.byref(d), p, nb - 1) == m.DSA_E_WORKSPACE
    assert sb(dec, ctypes.byref(d), None, nb) == m.DSA_E_WORKSPACE
    assert L.dsa_indexer_backward(ctypes.byref(dec), ctypes.byref(d), p, p, p, p, p, None, p, p, p,
                                  p, p, nb, None) == m.DSA_E_INVALID
    # key counts of num_seqs * (max_pos + 1) >= 2^31 are refused
    big = _rows(m, R=32, B=32768, N=65536, max_pos=65535)
    assert sb(big, ctypes.byref(d), p, 1 << 50) == m.DSA_E_UNSUPPORTED
    # and rows longer than 131072 positions
    long_rows = _rows(m, R=1, B=1, N=262144, max_pos=131072)
    assert sb(long_rows, ctypes.byref(d), p, 1 << 50) == m.DSA_E_UNSUPPORTED
    # masked MHA mode: short prefill only, production dims, workspace
    pre = _rows(m, R=8192, B=1, N=8192, max_pos=8191)
    need = L.dsa_mha_prefill_workspace_size(ctypes.byref(pre), ctypes.byref(d))
    assert need == 8192 * 16384 * 2 * 2 + 8192 * (8192 // 32) * 4
    mha = lambda rows, dims, ws, n: L.dsa_mha_prefill(ctypes.byref(rows), dims, p, p, p, p, p, 0.1,
                                                     p, p, ws, n, None)
    assert mha(pre, ctypes.byref(f32), p, need) == m.DSA_E_UNSUPPORTED
    assert mha(pre, ctypes.byref(d), p, need - 1) == m.DSA_E_WORKSPACE
    long_rows = _rows(m, R=8, B=1, N=32768, max_pos=16384)                    # 16385 positions
    assert mha(long_rows, ctypes.byref(d), p, 1 << 40) == m.DSA_E_UNSUPPORTED
    assert L.dsa_mha_prefill(ctypes.byref(pre), ctypes.byref(d), None, p, p, p, p, 0.1, p, p, p,
                             need, None) == m.DSA_E_INVALID


def test_size_limits_rejected_before_enqueue(m):
    """Rows longer than the top-k kernels take (t + 1 > 131072), and contiguous
    latent caches whose per-sequence byte span does not fit the attention kernel's
    32-bit offsets, are refused on the host with DSA_E_UNSUPPORTED (the dummy
    pointers would fault if anything were launched)."""
    L = m.lib
    d = m.dims_struct(m.PRODUCTION_DIMS)
    p = ctypes.c_void_p(16)
    long_rows = _rows(m, R=1, B=1, N=262144, max_pos=131072)           # 131073 candidates
    assert L.dsa_topk(ctypes.byref(long_rows), 2048, p, 131136, p, None, 0, None) == m.DSA_E_UNSUPPORTED
    assert "131072" in L.dsa_last_error().decode()
    ok_rows = _rows(m, R=0, B=1, N=262144, max_pos=131071, seq=None, pos=None)
    assert L.dsa_topk(ctypes.byref(ok_rows), 2048, None, 131072, None, None, 0, None) == m.DSA_OK
    big = 1 << 30
    assert L.dsa_forward(ctypes.byref(long_rows), ctypes.byref(d), p, p, p, p, p, p, p, 0.1, p, p,
                         None, 0, p, big, None) == m.DSA_E_UNSUPPORTED
    # 3728271 entries of 1152 bytes pass 2^32 bytes; one fewer fits
    huge = _rows(m, R=1, B=1, N=3728271, max_pos=1000)
    assert L.dsa_sparse_mla_attn(ctypes.byref(huge), ctypes.byref(d), p, p, p, 0.1, p, p, p, big,
                                 None) == m.DSA_E_UNSUPPORTED
    assert "4 GiB" in L.dsa_last_error().decode()
    assert L.dsa_forward(ctypes.byref(huge), ctypes.byref(d), p, p, p, p, p, p, p, 0.1, p, p, None,
                         0, p, big, None) == m.DSA_E_UNSUPPORTED
    fits = _rows(m, R=0, B=1, N=3728270, max_pos=1000, seq=None, pos=None)
    assert L.dsa_sparse_mla_attn(ctypes.byref(fits), ctypes.byref(d), None, None, None, 0.1, None,
                                 None, None, 0, None) == m.DSA_OK
    # the index-domain check rejects a NULL output before touching the device
    assert L.dsa_check_index_domain(None) == m.DSA_E_INVALID
