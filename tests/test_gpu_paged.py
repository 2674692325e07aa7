"""Parity of the paged-cache entry points (through the C ABI).

The pools are built from the generator's contiguous caches: the caches' pages
are scattered over a larger pool in a seeded random order, and the pool's unused
pages are filled with NaN, so that a wrong page mapping cannot go unnoticed.
Each paged call is held to the oracle's bars on sampled rows (the oracle reads
the logical caches the pools describe).  It must also match the contiguous call
bit for bit: the kernels do the same arithmetic and differ only in where they
read.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dsa_inputs as di
import oracle
from dsa_check import (HostInputs, check_attention, check_bf16_words, check_quantised,
                       check_scores, check_selection, proj_reference, to_f64)

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F      # e4m3fn NaN
NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_fp8_amd as m
    return m


_DEV = {}


def dev_inputs(name: str) -> di.Inputs:
    if name not in _DEV:
        _DEV.clear()
        torch.cuda.empty_cache()
        print(f"[gen] {name}", flush=True)
        _DEV[name] = di.make_inputs(di.CONFIGS[name], 0, device="cuda")
    return _DEV[name]


def make_pools(dsa, inp: di.Inputs, P: int, extra: int, seed: int):
    """Scatter the caches' pages over a pool of B * N / P + extra pages."""
    c = inp.cfg
    B, N = c.num_seqs, c.max_ctx
    pps = N // P
    npg = B * pps + extra
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(npg)).cuda()
    used = perm[: B * pps]
    table = used.view(B, pps).to(torch.int32).contiguous()
    k_pool = torch.full((npg, P, c.idx_dim), NAN_CODE, dtype=torch.uint8, device="cuda")
    ks_pool = torch.full((npg, P), float("nan"), dtype=torch.float32, device="cuda")
    lat_pool = torch.full((npg, P, c.qk_dim), NAN_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
    k_pool[used] = inp.k_idx.view(B * pps, P, c.idx_dim)
    ks_pool[used] = inp.k_scale.view(B * pps, P)
    lat_pool[used] = inp.latent.view(B * pps, P, c.qk_dim)
    pages = dsa.pages_struct(table, P, npg)
    print(f"[paged] {c.name}: page {P}, {npg} pages ({extra} unused)", flush=True)
    return pages, k_pool, ks_pool, lat_pool


def rows_all(dsa, inp: di.Inputs):
    c = inp.cfg
    return dsa.rows_struct(inp.row_seq, inp.row_pos, c.num_seqs, c.max_ctx, c.kv_len - 1)


def oracle_rows(dsa, name, inp, out, idx, rows):
    """C2 / C3 of sampled rows of a forward result against the oracle."""
    cfg = inp.cfg
    host = HostInputs(cfg)
    rt = torch.from_numpy(np.asarray(rows)).cuda()
    o_gpu, i_gpu = to_f64(out[rt]), idx[rt].cpu().numpy()
    for i, r in enumerate(rows):
        row = host.row(int(r))
        ref = host.scores(row)
        check_selection(i_gpu[i], ref, row.t, cfg.topk)
        n = min(cfg.topk, row.t + 1)
        o_ref, _ = host.attention(row, i_gpu[i, :n])
        check_attention(o_gpu[i], o_ref)


@pytest.mark.parametrize("P", [64, 4096])
def test_paged_decode(dsa, P):
    """Decode 32K over shuffled pages: the indexer, attention and forward calls
    equal their contiguous forms bit for bit, and the forward result meets the
    oracle's bars on 8 rows."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    pages, k_pool, ks_pool, lat_pool = make_pools(dsa, inp, P, extra=7, seed=P)
    rs = rows_all(dsa, inp)
    dims = dsa.Dims.from_config(cfg)
    ld = (cfg.kv_len + 63) // 64 * 64
    sc_c = dsa.indexer_scores(rs, dims, inp.q_idx, inp.q_scale, inp.w, inp.k_idx, inp.k_scale, ld=ld)
    sc_p = dsa.indexer_scores_paged(rs, dims, pages, inp.q_idx, inp.q_scale, inp.w, k_pool,
                                    ks_pool, ld=ld)
    torch.cuda.synchronize()
    assert torch.equal(sc_c[:, : cfg.kv_len], sc_p[:, : cfg.kv_len]), "paged scores differ"
    idx = dsa.topk(rs, cfg.topk, sc_c)
    o_c, l_c = dsa.sparse_mla_attn(rs, dims, inp.q, inp.latent, idx, cfg.scale)
    o_p, l_p = dsa.sparse_mla_attn_paged(rs, dims, pages, inp.q, lat_pool, idx, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p), "paged attention differs"
    i_f = torch.empty(cfg.num_rows, cfg.topk, dtype=torch.int32, device="cuda")
    o_f, _, _ = dsa.forward_paged(rs, dims, pages, inp.q_idx, inp.q_scale, inp.w, k_pool, ks_pool,
                                  inp.q, lat_pool, cfg.scale, indices_out=i_f)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_c) and torch.equal(i_f, idx)
    oracle_rows(dsa, "decode32k", inp, o_f, i_f, [0, 5, 11, 16, 23, 26, 30, 31])


@pytest.mark.parametrize("P", [64, 1024])
def test_paged_prefill(dsa, P):
    """Prefill 8K over shuffled pages (with 64-entry pages a 128-key group of the
    prefill indexer spans two pages): forward equals the contiguous forward bit for
    bit on every row and meets the oracle's bars on 12 sampled rows."""
    cfg = di.CONFIGS["prefill8k"]
    inp = dev_inputs("prefill8k")
    pages, k_pool, ks_pool, lat_pool = make_pools(dsa, inp, P, extra=5, seed=100 + P)
    rs = rows_all(dsa, inp)
    dims = dsa.Dims.from_config(cfg)
    R = cfg.num_rows
    i_c = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
    i_p = torch.empty_like(i_c)
    o_c, _, _ = dsa.forward(rs, dims, inp.q_idx, inp.q_scale, inp.w, inp.k_idx, inp.k_scale, inp.q,
                            inp.latent, cfg.scale, indices_out=i_c)
    o_p, _, _ = dsa.forward_paged(rs, dims, pages, inp.q_idx, inp.q_scale, inp.w, k_pool, ks_pool,
                                  inp.q, lat_pool, cfg.scale, indices_out=i_p)
    torch.cuda.synchronize()
    assert torch.equal(i_c, i_p), "paged selection differs"
    assert torch.equal(o_c, o_p), "paged output differs"
    oracle_rows(dsa, "prefill8k", inp, o_p, i_p,
                [0, 63, 64, 1000, 2047, 2048, 3333, 4096, 5000, 6543, 8000, 8191])


def test_paged_multi_sequence_tiles(dsa):
    """128 rows over four sequences with ragged positions: the prefill indexer's
    tiles hold rows of several sequences and take the per-row path, paged."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    pages, k_pool, ks_pool, _ = make_pools(dsa, inp, 64, extra=3, seed=7)
    R = 128
    seq = np.arange(R) % 4
    pos = (1000 + 211 * np.arange(R)) % cfg.max_ctx
    src = np.arange(R) % 32                         # query rows reused
    rs = dsa.rows_struct(torch.from_numpy(seq.astype(np.int32)).cuda(),
                         torch.from_numpy(pos.astype(np.int32)).cuda(), cfg.num_seqs,
                         cfg.max_ctx, int(pos.max()))
    sel = torch.from_numpy(src).cuda()
    q_idx, q_scale, w = (inp.q_idx[sel].contiguous(), inp.q_scale[sel].contiguous(),
                         inp.w[sel].contiguous())
    dims = dsa.Dims.from_config(cfg)
    sc_c = dsa.indexer_scores(rs, dims, q_idx, q_scale, w, inp.k_idx, inp.k_scale)
    sc_p = dsa.indexer_scores_paged(rs, dims, pages, q_idx, q_scale, w, k_pool, ks_pool)
    torch.cuda.synchronize()
    host = HostInputs(cfg)
    got = sc_p.cpu().numpy()
    ref_c = sc_c.cpu().numpy()
    for r in range(R):
        t = int(pos[r])
        assert np.array_equal(got[r, : t + 1], ref_c[r, : t + 1])
    for r in (0, 1, 2, 3, 77, 127):
        row = host.row(int(src[r]))
        row.b, row.t = int(seq[r]), int(pos[r])
        check_scores(got[r, : row.t + 1], host.scores(row))


def test_paged_long_rows_forward(dsa):
    """Rows longer than the top-k's register-resident length in chunks of 128: the
    paged forward (whose tiled indexer passes each row's score extremes to the
    top-k) equals the contiguous forward bit for bit, on tiles spanning two
    sequences and tiles of one sequence."""
    cfg = di.CONFIGS["decode128k"]
    inp = dev_inputs("decode128k")
    pages, k_pool, ks_pool, lat_pool = make_pools(dsa, inp, 64, extra=5, seed=11)
    R, CH = 256, 128
    seq = np.zeros(R, dtype=np.int32)
    pos = np.zeros(R, dtype=np.int32)
    for i in range(CH):
        seq[i] = i & 1
        pos[i] = 40000 + 7 * i if i & 1 == 0 else 131071 - 11 * i
    for i in range(CH, R):
        j = i - CH
        seq[i] = 2 + ((j >> 4) & 1)
        pos[i] = 70000 + 13 * j if seq[i] == 2 else 100000 + 3 * j
    pos[7], pos[CH + 1] = 500, 32768
    rs = dsa.rows_struct(torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                         cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    sel = torch.arange(R, device="cuda") % cfg.num_rows
    q_idx, q_scale, w, q = (inp.q_idx[sel].contiguous(), inp.q_scale[sel].contiguous(),
                            inp.w[sel].contiguous(), inp.q[sel].contiguous())
    dims = dsa.Dims.from_config(cfg)
    i_c = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
    i_p = torch.empty_like(i_c)
    o_c, _, _ = dsa.forward(rs, dims, q_idx, q_scale, w, inp.k_idx, inp.k_scale, q, inp.latent,
                            cfg.scale, indices_out=i_c, chunk_rows=CH)
    o_p, _, _ = dsa.forward_paged(rs, dims, pages, q_idx, q_scale, w, k_pool, ks_pool, q,
                                  lat_pool, cfg.scale, indices_out=i_p, chunk_rows=CH)
    torch.cuda.synchronize()
    assert torch.equal(i_c, i_p), "paged selection differs"
    assert torch.equal(o_c, o_p), "paged output differs"


def test_paged_table_entries_out_of_range(dsa):
    """Block-table entries outside the pool are read as page 0: the call completes
    and every score stays finite (its value is unspecified)."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    pages, k_pool, ks_pool, _ = make_pools(dsa, inp, 1024, extra=0, seed=9)
    table = pages._keep.clone()
    table[0, 3] = -5
    table[1, 7] = pages.num_pages + 10
    bad = dsa.pages_struct(table, 1024, pages.num_pages)
    rs = rows_all(dsa, inp)
    sc = dsa.indexer_scores_paged(rs, dsa.Dims.from_config(cfg), bad, inp.q_idx, inp.q_scale,
                                  inp.w, k_pool, ks_pool)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sc[:, : cfg.kv_len]).all())


def test_paged_project_append(dsa):
    """Projections appended into shuffled pages land at the pool rows the table
    names (C4 against the oracle), equal the contiguous append bit for bit, and
    leave every other pool row untouched."""
    R, d, B, P, pps = 37, 512, 3, 64, 2
    N = P * pps
    npg = B * pps + 2
    g = di.ProjGenerator(6, d)
    h = g.h(0, R, device="cuda")
    wts = g.weights(device="cuda")
    seq = np.array([r % B for r in range(R)], dtype=np.int32)
    pos = np.array([(5 * r) % N for r in range(R)], dtype=np.int32)
    seq[4] = B                                     # no cache row for this token
    perm = np.random.default_rng(3).permutation(npg)
    table = torch.from_numpy(perm[: B * pps].reshape(B, pps).astype(np.int32)).cuda()
    pages = dsa.pages_struct(table, P, npg)
    dev = torch.device("cuda")
    k_pool = torch.full((npg, P, 128), 0x5A, dtype=torch.uint8, device=dev)
    ks_pool = torch.full((npg, P), -7.0, dtype=torch.float32, device=dev)
    lat_pool = torch.full((npg, P, 576), 0x3F80, dtype=torch.int16, device=dev).view(torch.bfloat16)
    rs = dsa.rows_struct(torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev), B, N, N - 1)
    q_p, qs_p, w_p = dsa.project_append_paged(rs, pages, h, *wts, k_pool, ks_pool, lat_pool)
    k_c = torch.zeros(B, N, 128, dtype=torch.uint8, device=dev)
    ks_c = torch.zeros(B, N, dtype=torch.float32, device=dev)
    lat_c = torch.zeros(B, N, 576, dtype=torch.bfloat16, device=dev)
    q_c, qs_c, w_c = dsa.project_append(rs, h, *wts, k_c, ks_c, lat_c)
    torch.cuda.synchronize()
    assert torch.equal(q_p, q_c) and torch.equal(qs_p, qs_c) and torch.equal(w_p, w_c)
    # pool rows of the valid tokens, through the block table (host copy)
    tab = table.cpu().numpy()
    valid = [r for r in range(R) if seq[r] < B]
    prow = [(int(tab[seq[r], pos[r] // P]), int(pos[r] % P)) for r in valid]
    pi = torch.tensor([a for a, _ in prow], device=dev)
    pj = torch.tensor([b for _, b in prow], device=dev)
    vt = torch.tensor(valid, device=dev)
    sq, ps = torch.from_numpy(seq[valid].astype(np.int64)).to(dev), torch.from_numpy(pos[valid].astype(np.int64)).to(dev)
    assert torch.equal(k_pool[pi, pj], k_c[sq, ps])
    assert torch.equal(ks_pool[pi, pj], ks_c[sq, ps])
    assert torch.equal(lat_pool[pi, pj], lat_c[sq, ps])
    ref = proj_reference(di.bf16_bits(g.h(0, R)), [di.bf16_bits(x) for x in g.weights()], 64)
    vi = np.array(valid)
    check_quantised(k_pool[pi, pj].cpu().numpy(), ks_pool[pi, pj].cpu().numpy(),
                    ref["y_k"][vi], ref["err_k"][vi])
    check_bf16_words(di.bf16_bits(lat_pool[pi, pj]), ref["y_c"][vi], ref["err_c"][vi])
    written = torch.zeros(npg, P, dtype=torch.bool, device=dev)
    written[pi, pj] = True
    assert bool((k_pool[~written] == 0x5A).all()) and bool((ks_pool[~written] == -7.0).all())
    assert bool((lat_pool.view(torch.int16)[~written] == 0x3F80).all())
