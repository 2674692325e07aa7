"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Every GPU input comes from the seeded generator on the device; every oracle input
is regenerated on the host from the same generator.  Workloads are the five
configurations of the hot path; the 128K ones are checked on a seeded sample of
256 rows, as are the rows of the 8K prefill.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dsa_inputs as di
import oracle
from dsa_check import (HostInputs, attn_errors, check_attention, check_scores,
                       check_selection, to_f64, ATTN_MAX_ABS, ATTN_MEAN_ABS)

pytestmark = pytest.mark.gpu

CFGS = ["tiny", "decode32k", "prefill8k", "decode128k", "prefill128k", "prefill2k"]


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_fp8_amd as m
    return m


_DEV = {}


def dev_inputs(name: str, set_id: int = 0) -> di.Inputs:
    key = (name, set_id)
    if key not in _DEV:
        _DEV.clear()
        torch.cuda.empty_cache()
        print(f"[gen] {name} set {set_id}", flush=True)
        _DEV[key] = di.make_inputs(di.CONFIGS[name], set_id, device="cuda")
    return _DEV[key]


def sample(cfg: di.Config) -> np.ndarray:
    if cfg.name in ("prefill8k", "prefill2k"):
        return di.sample_rows(cfg, 64)
    return di.sample_rows(cfg, 256)


def chunks(cfg: di.Config):
    R = cfg.num_rows
    CH = cfg.chunk_rows if cfg.chunk_rows > 0 else R
    return [(a, min(R, a + CH)) for a in range(0, R, CH)]


def rows_of(m, inp: di.Inputs, a: int, b: int):
    c = inp.cfg
    return m.rows_struct(inp.row_seq[a:b], inp.row_pos[a:b], c.num_seqs, c.max_ctx,
                         c.kv_len - 1)


# ---------------------------------------------------------------- generator

@pytest.mark.parametrize("name", ["tiny", "decode32k"])
def test_generator_device_matches_host(name):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    g = di.Generator(cfg)
    b = cfg.num_seqs - 1
    n = min(512, cfg.max_ctx)
    codes, sc = g.k_idx(b, 0, n)
    assert torch.equal(inp.k_idx[b, :n].cpu(), codes)
    assert torch.equal(inp.k_scale[b, :n].cpu(), sc)
    assert torch.equal(inp.latent[b, 100:164].cpu(), g.latent(b, 100, 164))
    r = cfg.num_rows - 1
    qc, qs = g.q_idx(r, r + 1)
    assert torch.equal(inp.q_idx[r:r + 1].cpu(), qc)
    assert torch.equal(inp.q_scale[r:r + 1].cpu(), qs)
    assert torch.equal(inp.w[r:r + 1].cpu(), g.w(r, r + 1))
    assert torch.equal(inp.q[r:r + 1].cpu(), g.q(r, r + 1))


# ---------------------------------------------------------------- step 1

@pytest.mark.parametrize("name", CFGS)
def test_indexer_parity(dsa, name):
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    rows = sample(cfg)
    dims = dsa.Dims.from_config(cfg)
    ld = (cfg.kv_len + 63) // 64 * 64
    worst, rel_row = 0.0, 0.0
    for a, b in chunks(cfg):
        want = rows[(rows >= a) & (rows < b)]
        if want.size == 0:
            continue
        rs = rows_of(dsa, inp, a, b)
        print(f"[indexer] {name} rows {a}..{b}", flush=True)
        sc = dsa.indexer_scores(rs, dims, inp.q_idx[a:b], None if cfg.fp32 else inp.q_scale[a:b],
                                inp.w[a:b], inp.k_idx, None if cfg.fp32 else inp.k_scale, ld=ld)
        torch.cuda.synchronize()
        got = sc[torch.from_numpy(want - a).cuda()].cpu().numpy()
        for i, r in enumerate(want):
            row = host.row(int(r))
            ref = host.scores(row)
            worst = max(worst, check_scores(got[i, : row.t + 1], ref))
            rel_row = max(rel_row, float(np.max(np.abs(got[i, : row.t + 1] - ref))
                                         / max(np.max(np.abs(ref)), 1e-30)))
    print(f"[indexer] {name}: worst error / allowed = {worst:.3e}, "
          f"worst |error| / max|score| of its row = {rel_row:.3e}")


# ---------------------------------------------------------------- step 2

def _synthetic_score_rows():
    """(t, scores[0..t]) rows covering value patterns and the kernel's size regimes."""
    rng = np.random.default_rng(1234)
    out = []
    for t in [0, 1, 63, 64, 100, 2046, 2047, 2048, 2049, 5000, 8191, 8192, 20000, 32767,
              32768, 50000, 131071]:
        L = t + 1
        out.append((t, rng.standard_normal(L).astype(np.float32) * 8))
    L = 40000
    out.append((L - 1, rng.integers(-3, 4, size=L).astype(np.float32)))          # heavy ties
    out.append((L - 1, np.zeros(L, dtype=np.float32)))                          # ReLU-zero row
    z = np.zeros(L, dtype=np.float32)
    z[rng.choice(L, 700, replace=False)] = rng.random(700).astype(np.float32) + 0.5
    out.append((L - 1, z))                                                      # few positives
    s = (rng.integers(0, 2, size=L) * 2 - 1).astype(np.float32) * 0.0           # +-0.0 mix
    s[rng.choice(L, 100, replace=False)] = 1.0
    out.append((L - 1, s))
    out.append((L - 1, -np.abs(rng.standard_normal(L)).astype(np.float32) - 3))  # negatives
    out.append((L - 1, (rng.standard_normal(L) * 1e30).astype(np.float32)))      # huge range
    base = np.float32(1.0)
    tiny = np.nextafter(base, np.float32(2.0), dtype=np.float32) - base
    out.append((L - 1, (base + tiny * rng.integers(0, 5, size=L)).astype(np.float32)))  # ulp ties
    out.append((3000, rng.standard_normal(3001).astype(np.float32)))
    return out


@pytest.mark.parametrize("k,copies", [(2048, 1), (64, 1), (1, 1), (4096, 1), (2048, 6)])
def test_topk_exact(dsa, k, copies):
    """Selection is integer work: the GPU set must equal the oracle's bit for bit
    on the same float32 scores (synthetic rows, not produced by the HIP path).
    One copy of the rows is few enough that each row is split over several
    blocks; six copies (162 rows) run one block per row."""
    rows = _synthetic_score_rows() * copies
    maxt = max(t for t, _ in rows)
    ld = maxt + 1
    R = len(rows)
    host = np.full((R, ld), np.nan, dtype=np.float32)
    for i, (t, s) in enumerate(rows):
        host[i, : t + 1] = s
    scores = torch.from_numpy(host).cuda()
    pos = torch.tensor([t for t, _ in rows], dtype=torch.int32, device="cuda")
    seq = torch.zeros(R, dtype=torch.int32, device="cuda")
    rs = dsa.rows_struct(seq, pos, 1, ld, maxt)
    idx = dsa.topk(rs, k, scores).cpu().numpy()
    for i, (t, s) in enumerate(rows):
        n = min(k, t + 1)
        want = oracle.select_topk(s.astype(np.float64), n)
        assert np.array_equal(idx[i, :n], want), f"row {i} (t={t}) differs"
        assert np.all(idx[i, n:] == -1)


def test_topk_single_regime_per_launch(dsa):
    """Rows of one launch share the register-cached regime chosen from max_pos:
    a launch whose longest row is short uses the cached kernels."""
    rng = np.random.default_rng(7)
    for L in [3000, 8192, 8193, 32768]:
        R = 16
        host = (rng.standard_normal((R, L)) * 4).astype(np.float32)
        pos = rng.integers(0, L, size=R).astype(np.int32)
        pos[0] = L - 1
        rs = dsa.rows_struct(torch.zeros(R, dtype=torch.int32, device="cuda"),
                             torch.from_numpy(pos).cuda(), 1, L, L - 1)
        idx = dsa.topk(rs, 2048, torch.from_numpy(host).cuda()).cpu().numpy()
        for i in range(R):
            t = int(pos[i])
            n = min(2048, t + 1)
            want = oracle.select_topk(host[i, : t + 1].astype(np.float64), n)
            assert np.array_equal(idx[i, :n], want), (
                f"L={L} row {i} t={t}: {np.sum(idx[i, :n] != want)} slots differ; "
                f"first gpu {idx[i, :6]} want {want[:6]}")


# ---------------------------------------------------------------- step 3

def _synthetic_selection(cfg: di.Config, t: int, rng) -> np.ndarray:
    n = min(cfg.topk, t + 1)
    sel = np.sort(rng.choice(t + 1, size=n, replace=False)).astype(np.int32)
    return np.concatenate([sel, np.full(cfg.topk - n, -1, dtype=np.int32)])


@pytest.mark.parametrize("name", ["tiny", "decode32k", "prefill8k", "decode128k"])
def test_attention_parity(dsa, name):
    """Attention alone on a given selection (synthetic position sets, padded)."""
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    rng = np.random.default_rng(cfg.cfg_id)
    R = cfg.num_rows
    pos = inp.row_pos.cpu().numpy()
    sel = np.stack([_synthetic_selection(cfg, int(pos[r]), rng) for r in range(R)])
    idx = torch.from_numpy(sel).cuda()
    dims = dsa.Dims.from_config(cfg)
    rs = rows_of(dsa, inp, 0, R)
    print(f"[attn] {name}", flush=True)
    out, lse = dsa.sparse_mla_attn(rs, dims, inp.q, inp.latent, idx, cfg.scale)
    torch.cuda.synchronize()
    rows = sample(cfg)
    o_gpu = to_f64(out[torch.from_numpy(rows).cuda()])
    l_gpu = to_f64(lse[torch.from_numpy(rows).cuda()])
    errs, lerr = [], 0.0
    for i, r in enumerate(rows):
        row = host.row(int(r))
        s = sel[r][sel[r] >= 0]
        o_ref, l_ref = host.attention(row, s)
        errs.append(np.abs(o_gpu[i] - o_ref))
        lerr = max(lerr, float(np.max(np.abs(l_gpu[i] - l_ref))))
    d = np.concatenate([e.ravel() for e in errs])
    print(f"[attn] {name}: max {d.max():.3e} mean {d.mean():.3e} lse max {lerr:.3e}")
    assert np.all(np.isfinite(o_gpu))
    assert d.max() <= ATTN_MAX_ABS and d.mean() <= ATTN_MEAN_ABS
    assert lerr <= 1e-2


def test_attention_edge_rows(dsa):
    """Row t=0 (one entry: out is that entry exactly), all-padding splits, padding
    in the middle of the list, and an out-of-range position treated as padding."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    host = HostInputs(cfg)
    R = cfg.num_rows
    sel = np.full((R, cfg.topk), -1, dtype=np.int32)
    sel[0, 0] = 0                                   # single entry
    sel[1, :5] = [7, 3, 1000, 31000, 32767]         # 5 entries, unsorted
    sel[2, ::2] = np.arange(0, cfg.topk, 2) * 7     # padding interleaved
    sel[3, :2048] = np.arange(2048) + 100
    sel[3, 10] = cfg.max_ctx + 5                    # out of range -> padding
    for r in range(4, R):
        sel[r, :3] = [r, r + 1, r + 2]
    idx = torch.from_numpy(sel).cuda()
    rs = rows_of(dsa, inp, 0, R)
    out, lse = dsa.sparse_mla_attn(rs, dsa.Dims.from_config(cfg), inp.q, inp.latent, idx, cfg.scale)
    torch.cuda.synchronize()
    o = out.cpu()
    # t = 0 style row: a single entry gives exactly that entry's value part
    assert torch.equal(o[0], inp.latent[0, 0, :512].cpu().unsqueeze(0).expand(128, 512))
    for r in range(R):
        s = sel[r][(sel[r] >= 0) & (sel[r] < cfg.max_ctx)]
        row = host.row(r)
        o_ref, _ = host.attention(row, s)
        check_attention(to_f64(out[r]), o_ref)


def test_attention_future_positions_are_padding(dsa):
    """The causal rule of the selection (S_t holds positions s <= t): an index entry
    past its row's position is padding, exactly as -1 is, in the bf16 and fp32
    attention and in the sparse-stage loss; it also raises the device's
    index-domain flag, which a clean call leaves clear."""
    assert dsa.check_index_domain() in (False, True)   # clear whatever earlier tests left
    for name, rows in (("prefill8k", [0, 100, 5000, 8190]), ("tiny", [0, 3, 64, 200])):
        cfg = di.CONFIGS[name]
        inp = dev_inputs(name)
        host = HostInputs(cfg)
        dims = dsa.Dims.from_config(cfg)
        rng = np.random.default_rng(21)
        R = len(rows)
        ridx = torch.tensor(rows, device="cuda")
        seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
        rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
        clean = np.full((R, cfg.topk), -1, dtype=np.int32)
        dirty = clean.copy()
        for i, r in enumerate(rows):
            t = int(host.row(r).t)
            n = min(cfg.topk // 2, t + 1)
            s = np.sort(rng.choice(t + 1, n, replace=False)).astype(np.int32)
            clean[i, :n] = s
            dirty[i, :n] = s
            fut = np.arange(t + 1, cfg.max_ctx)
            if fut.size:  # future positions in the free slots, some beyond the last row
                f = rng.choice(fut, min(fut.size, cfg.topk - n), replace=False)
                dirty[i, n:n + f.size] = f
        q = inp.q[ridx].contiguous()
        o_c, l_c = dsa.sparse_mla_attn(rs, dims, q, inp.latent, torch.from_numpy(clean).cuda(), cfg.scale)
        torch.cuda.synchronize()
        assert dsa.check_index_domain() is False, name
        o_d, l_d = dsa.sparse_mla_attn(rs, dims, q, inp.latent, torch.from_numpy(dirty).cuda(), cfg.scale)
        torch.cuda.synchronize()
        assert dsa.check_index_domain() is True, name
        assert dsa.check_index_domain() is False, name   # read-and-clear
        for i, r in enumerate(rows):
            o_ref, _ = host.attention(host.row(r), clean[i][clean[i] >= 0])
            check_attention(to_f64(o_d[i]), o_ref)
        if not cfg.fp32:
            # the padding of both lists lands in the same slots, but a split's slice
            # can hold different numbers of valid entries, so compare under C3 too
            check_attention(to_f64(o_d), to_f64(o_c))
            # the sparse-stage loss ignores the future entries as it ignores -1
            ld = (cfg.kv_len + 63) // 64 * 64
            sc = torch.randn(R, ld, device="cuda")
            l1, g1 = dsa.indexer_loss(rs, q, inp.latent, torch.from_numpy(clean).cuda(), l_c,
                                      cfg.scale, sc)
            l2, g2 = dsa.indexer_loss(rs, q, inp.latent, torch.from_numpy(dirty).cuda(), l_c,
                                      cfg.scale, sc)
            torch.cuda.synchronize()
            assert torch.equal(l1, l2) and torch.equal(g1, g2)
        print(f"[future] {name}: future entries treated as padding, flag raised", flush=True)


# ---------------------------------------------------------------- whole path

def _forward(dsa, name, inp, set_chunk=True):
    cfg = inp.cfg
    R = cfg.num_rows
    rs = rows_of(dsa, inp, 0, R)
    idx = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.forward(rs, dsa.Dims.from_config(cfg), inp.q_idx,
                              None if cfg.fp32 else inp.q_scale, inp.w, inp.k_idx,
                              None if cfg.fp32 else inp.k_scale, inp.q, inp.latent, cfg.scale,
                              indices_out=idx, chunk_rows=cfg.chunk_rows if set_chunk else 0)
    return out, lse, idx


@pytest.mark.parametrize("name", CFGS)
def test_forward_parity(dsa, name):
    """dsa_forward end to end: selection under C2 against the oracle's scores,
    output under C3.  Where the GPU set equals the oracle's (the usual case) the
    output is compared with the oracle's attention on the oracle's set; where it
    differs inside the tie band (both are correct selections) it is compared with
    the oracle's attention on the GPU's set."""
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    print(f"[forward] {name}", flush=True)
    out, lse, idx = _forward(dsa, name, inp)
    torch.cuda.synchronize()
    rows = sample(cfg)
    rt = torch.from_numpy(rows).cuda()
    o_gpu, i_gpu = to_f64(out[rt]), idx[rt].cpu().numpy()
    errs, differing, band_total = [], 0, 0
    for i, r in enumerate(rows):
        row = host.row(int(r))
        ref_scores = host.scores(row)
        band_total += check_selection(i_gpu[i], ref_scores, row.t, cfg.topk)
        n = min(cfg.topk, row.t + 1)
        s_ref = oracle.select_topk(ref_scores, n)
        s_gpu = i_gpu[i, :n]
        same = np.array_equal(s_gpu, s_ref)
        differing += (not same)
        o_ref, _ = host.attention(row, s_ref if same else s_gpu)
        errs.append(np.abs(o_gpu[i] - o_ref).ravel())
    d = np.concatenate(errs)
    print(f"[forward] {name}: rows {len(rows)} set-differs {differing} band {band_total} "
          f"max {d.max():.3e} mean {d.mean():.3e}")
    assert np.all(np.isfinite(o_gpu))
    assert d.max() <= ATTN_MAX_ABS and d.mean() <= ATTN_MEAN_ABS


def test_forward_rows_below_k_are_dense(dsa):
    """Rows t < k of the 8K prefill select every prior position: their selection is
    exactly 0..t and their output is dense causal attention."""
    cfg = di.CONFIGS["prefill8k"]
    inp = dev_inputs("prefill8k")
    host = HostInputs(cfg)
    out, _, idx = _forward(dsa, "prefill8k", inp)
    torch.cuda.synchronize()
    for r in [0, 1, 17, 1000, 2046, 2047]:
        got = idx[r].cpu().numpy()
        assert np.array_equal(got[: r + 1], np.arange(r + 1)) and np.all(got[r + 1:] == -1)
        row = host.row(r)
        o_ref, _ = host.attention(row, np.arange(r + 1))
        check_attention(to_f64(out[r]), o_ref)
    # row 0 attends to itself only: out is exactly the latent part of entry 0
    assert torch.equal(out[0].cpu(), inp.latent[0, 0, :512].cpu().unsqueeze(0).expand(128, 512))


def _assert_isolated(scores, s):
    """No other score within 1e-5 relative of scores[s], so GPU rounding cannot
    reorder the boundary against its neighbours."""
    d = np.abs(scores - scores[s])
    d[s] = np.inf
    assert d.min() > 1e-5 * abs(scores[s])


def test_forward_relu_zero_and_exact_ties(dsa):
    """A row whose indexer query is zero scores 0 everywhere and selects 0..n-1;
    two positions with identical keys straddling the cut keep the lower one."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k", set_id=3)
    host = HostInputs(cfg, set_id=3)
    q_idx = inp.q_idx.clone()
    q_idx[0].zero_()
    k_idx = inp.k_idx.clone()
    k_scale = inp.k_scale.clone()
    # tie: copy the boundary key of row 1 (n-th selected) to a later position
    row1 = host.row(1)
    ref1 = host.scores(row1)
    s_ref1 = oracle.select_topk(ref1, cfg.topk)
    boundary = int(s_ref1[np.argmin(ref1[s_ref1])])
    _assert_isolated(ref1, boundary)
    later = next(s for s in range(boundary + 1, cfg.max_ctx) if s not in set(s_ref1.tolist()))
    k_idx[1, later] = k_idx[1, boundary]
    k_scale[1, later] = k_scale[1, boundary]
    # and an earlier copy for row 2: the earlier position wins over the boundary
    row2 = host.row(2)
    ref2 = host.scores(row2)
    s_ref2 = oracle.select_topk(ref2, cfg.topk)
    boundary2 = int(s_ref2[np.argmin(ref2[s_ref2])])
    _assert_isolated(ref2, boundary2)
    earlier = next(s for s in range(0, boundary2) if s not in set(s_ref2.tolist()))
    k_idx[2, earlier] = k_idx[2, boundary2]
    k_scale[2, earlier] = k_scale[2, boundary2]
    R = cfg.num_rows
    rs = rows_of(dsa, inp, 0, R)
    idx = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
    dsa.forward(rs, dsa.Dims.from_config(cfg), q_idx, inp.q_scale, inp.w, k_idx, k_scale,
                inp.q, inp.latent, cfg.scale, indices_out=idx)
    got = idx.cpu().numpy()
    assert np.array_equal(got[0], np.arange(cfg.topk))
    s1 = set(got[1].tolist())
    assert boundary in s1 and later not in s1
    s2 = set(got[2].tolist())
    assert earlier in s2 and boundary2 not in s2


def test_forward_ragged_decode(dsa):
    """Sequences of one decode batch at different lengths (including t+1 < k and
    t = 0), through the split-k decode path."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    host = HostInputs(cfg)
    lens = [32768, 20000, 2048, 2049, 1, 100, 4097, 31000]
    R = len(lens)
    rows_g = np.arange(R) * 3           # decode: global row r belongs to sequence r
    seq = torch.from_numpy(rows_g.astype(np.int32)).cuda()
    pos = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device="cuda")
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, max(lens) - 1)
    qsel = torch.from_numpy(rows_g).cuda()
    idx = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.forward(rs, dsa.Dims.from_config(cfg), inp.q_idx[qsel].contiguous(),
                              inp.q_scale[qsel].contiguous(), inp.w[qsel].contiguous(), inp.k_idx,
                              inp.k_scale, inp.q[qsel].contiguous(), inp.latent, cfg.scale,
                              indices_out=idx)
    torch.cuda.synchronize()
    o_all = to_f64(out)
    for i in range(R):
        r = int(rows_g[i])
        row = host.row(r)
        row.t = lens[i] - 1
        ref = host.scores(row)
        check_selection(idx[i].cpu().numpy(), ref, row.t, cfg.topk)
        n = min(cfg.topk, row.t + 1)
        s_gpu = idx[i, :n].cpu().numpy()
        o_ref, _ = host.attention(row, s_gpu)
        check_attention(o_all[i], o_ref)


def test_forward_long_rows_match_separate_calls(dsa):
    """Long-context chunks pass each row's score extremes from the tiled indexer to
    the streamed top-k, which then skips its min / max pass.  The selections must be
    the same bits as the separate indexer and top-k calls on the same rows: two
    chunks of 128 rows (the second reuses the words the first left at zero), tiles
    spanning two sequences (the indexer's per-row path) and tiles of one sequence,
    rows shorter and longer than the top-k's register-resident length."""
    cfg = di.CONFIGS["decode128k"]
    inp = dev_inputs("decode128k")
    R, CH = 256, 128
    seq = np.zeros(R, dtype=np.int32)
    pos = np.zeros(R, dtype=np.int32)
    for i in range(CH):                      # chunk 0: sequences 0 and 1 alternate
        seq[i] = i & 1
        pos[i] = 40000 + 7 * i if i & 1 == 0 else 131071 - 11 * i
    pos[5], pos[9], pos[12] = 1000, 0, 32768
    for i in range(CH, R):                   # chunk 1: 16-row tiles of sequences 2 / 3
        j = i - CH
        seq[i] = 2 + ((j >> 4) & 1)
        pos[i] = 70000 + 13 * j if seq[i] == 2 else 100000 + 3 * j
    pos[CH + 3], pos[CH + 20] = 32767, 32768
    seq_t, pos_t = torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda()
    rs = dsa.rows_struct(seq_t, pos_t, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    qsel = torch.arange(R, device="cuda") % cfg.num_rows
    q_idx, q_scale = inp.q_idx[qsel].contiguous(), inp.q_scale[qsel].contiguous()
    w, q = inp.w[qsel].contiguous(), inp.q[qsel].contiguous()
    dims = dsa.Dims.from_config(cfg)
    # second pass: NaN key codes give NaN scores (read as -inf by the top-k) in rows of
    # both chunks
    k_nan = inp.k_idx.clone()
    k_nan[0, 5000:5040, 0] = 0x7F
    k_nan[1, 90000:90100, 7] = 0x7F
    k_nan[3, 40000:40064, 1] = 0xFF
    for k_idx, what in ((inp.k_idx, "finite"), (k_nan, "NaN keys")):
        idx_f = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
        dsa.forward(rs, dims, q_idx, q_scale, w, k_idx, inp.k_scale, q, inp.latent, cfg.scale,
                    indices_out=idx_f, chunk_rows=CH)
        for a in range(0, R, CH):
            rc = dsa.rows_struct(seq_t[a:a + CH], pos_t[a:a + CH], cfg.num_seqs, cfg.max_ctx,
                                 cfg.kv_len - 1)
            sc = dsa.indexer_scores(rc, dims, q_idx[a:a + CH], q_scale[a:a + CH], w[a:a + CH],
                                    k_idx, inp.k_scale, ld=cfg.kv_len)
            idx_s = dsa.topk(rc, cfg.topk, sc)
            torch.cuda.synchronize()
            same = (idx_f[a:a + CH] == idx_s).all(dim=1).cpu().numpy()
            assert same.all(), f"{what}, chunk at {a}: rows {np.nonzero(~same)[0][:8]} differ"
        print(f"[forward] long rows ({what}): fused extremes give the separate calls' "
              f"selections", flush=True)


def test_forward_long_rows_graph_replays(dsa):
    """The long-row forward (a fill kernel clears the extremes words, every top-k
    block clears its row's words again) captured in a HIP graph: three replays, with
    eager calls of the same forward between them, each give the eager call's bits."""
    cfg = di.CONFIGS["decode128k"]
    inp = dev_inputs("decode128k")
    R, CH = 256, 128
    pos = torch.tensor([40000 + 97 * i for i in range(R)], dtype=torch.int32, device="cuda")
    pos[3], pos[200] = 20000, 0
    seq = (torch.arange(R, device="cuda") // 64).to(torch.int32)
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    sel = torch.arange(R, device="cuda") % cfg.num_rows
    q_idx, q_scale = inp.q_idx[sel].contiguous(), inp.q_scale[sel].contiguous()
    w, q = inp.w[sel].contiguous(), inp.q[sel].contiguous()
    dims = dsa.Dims.from_config(cfg)
    out = torch.empty(R, cfg.n_heads, cfg.v_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(R, cfg.n_heads, dtype=torch.float32, device="cuda")
    idx = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.forward_workspace_size(rs, dims, CH), dtype=torch.uint8, device="cuda")

    def run():
        dsa.forward(rs, dims, q_idx, q_scale, w, inp.k_idx, inp.k_scale, q, inp.latent,
                    cfg.scale, out=out, lse=lse, indices_out=idx, chunk_rows=CH, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), idx.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_(); idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(idx, ref[2]), \
            f"replay {rep} differs from the eager call"
        run()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[2]), f"eager call after replay {rep} differs"
    print("[forward] long rows: graph replays equal the eager call", flush=True)


def test_forward_deterministic(dsa):
    """Two runs give bitwise-identical outputs, and a NaN-filled workspace does not
    leak into them (catches races and reads of uninitialised scratch)."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    R = cfg.num_rows
    rs = rows_of(dsa, inp, 0, R)
    dims = dsa.Dims.from_config(cfg)
    need = dsa.forward_workspace_size(rs, dims, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    res = []
    for fill in (0, 0xFF):
        ws.fill_(fill)  # 0xFF bytes are NaN floats and -1 ints
        idx = torch.empty(R, cfg.topk, dtype=torch.int32, device="cuda")
        out, lse, _ = dsa.forward(rs, dims, inp.q_idx, inp.q_scale, inp.w, inp.k_idx, inp.k_scale,
                                  inp.q, inp.latent, cfg.scale, indices_out=idx, workspace=ws)
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone(), idx.clone()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
