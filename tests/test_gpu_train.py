"""Parity of the indexer training loss and its backward (through the C ABI) with
the float64 oracle.

Each kernel is checked on oracle inputs, so that only its own arithmetic is
measured.  The loss is fed the oracle's scores (rounded to fp32) and the oracle's
selection; it uses the attention lse that the library computes for that
selection.  The backward is fed a seeded gradient.  The bars follow the
arithmetic:
* target and softmax run in fp32 over 576-term bf16 dots and 2048-entry sums, so
  p and softmax carry relative errors near 1e-5: |d dI_i| <= 1e-3 (p_i +
  softmax_i) + 1e-7 and |d loss| <= 1e-3 |loss| + 1e-6;
* the backward's dots are the forward's fp8 MFMA sums, off by at most
  GROUP_EPS per unit of each 8-product group's largest product plus SUM_EPS of
  sum_d |q_d k_d| (tests/test_gpu_fp8_accumulation.py), so a ReLU mask may flip
  where a dot lies within (GROUP_EPS + SUM_EPS) sum_d |q_d k_d| of zero.  Such a
  pair may add its whole term, and it is allowed for.  The fp32 sums add 1e-5 of
  the absolute sum of the terms.
A composed run (the GPU's own scores and selection) is held to C2 plus a bar on
the loss that accounts for the indexer's own C1 error.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dsa_inputs as di
import oracle
from dsa_check import GROUP_EPS, SUM_EPS, HostInputs

pytestmark = pytest.mark.gpu

# bound on |MFMA dot - exact dot| per unit of sum_d |q_d k_d| (each group's largest
# product is at most the group's share of that sum)
DOT_EPS = GROUP_EPS + SUM_EPS


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


def _oracle_setup(cfg, host, rows):
    """Per sampled row: oracle scores, oracle selection (padded to k), dequantised
    q, keys and latent entries of the selection."""
    out = []
    for r in rows:
        row = host.row(int(r))
        I = host.scores(row)
        n = min(cfg.topk, row.t + 1)
        S = oracle.select_topk(I, n)
        out.append((row, I, S))
    return out


@pytest.mark.parametrize("name,rows", [("decode32k", [0, 9, 17, 31]),
                                       ("prefill8k", [5, 2047, 2048, 4100, 8191])])
def test_indexer_loss_parity(dsa, name, rows):
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    print(f"[loss] {name} rows {rows}", flush=True)
    setup = _oracle_setup(cfg, host, rows)
    R = len(rows)
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    dims = dsa.Dims.from_config(cfg)
    ld = (cfg.kv_len + 63) // 64 * 64
    sc = np.zeros((R, ld), dtype=np.float32)
    idx = np.full((R, cfg.topk), -1, dtype=np.int32)
    for i, (row, I, S) in enumerate(setup):
        sc[i, : row.t + 1] = I.astype(np.float32)
        idx[i, : S.size] = S
    sc_d, idx_d = torch.from_numpy(sc).cuda(), torch.from_numpy(idx).cuda()
    q = inp.q[ridx].contiguous()
    _, lse = dsa.sparse_mla_attn(rs, dims, q, inp.latent, idx_d, cfg.scale)
    loss, dsc = dsa.indexer_loss(rs, q, inp.latent, idx_d, lse, cfg.scale, sc_d)
    torch.cuda.synchronize()
    loss, dsc = loss.cpu().numpy(), dsc.cpu().numpy()
    for i, (row, I, S) in enumerate(setup):
        ent = host.latent_rows(row.b, S)
        p = oracle.attention_target(oracle.decode_bf16(row.q), oracle.decode_bf16(ent), cfg.scale)
        Is = sc[i, S].astype(np.float64)      # the fp32 scores the kernel read
        l_ref, g_ref = oracle.indexer_kl(p, Is)
        sm = np.exp(Is - Is.max())
        sm /= sm.sum()
        assert abs(loss[i] - l_ref) <= 1e-3 * abs(l_ref) + 1e-6, (loss[i], l_ref)
        err = np.abs(dsc[i, : S.size] - g_ref)
        assert np.all(err <= 1e-3 * (p + sm) + 1e-7), float(err.max())
        assert np.all(dsc[i, S.size:] == 0.0)
        print(f"[loss] row {int(rows[i])}: loss {loss[i]:.6f} ref {l_ref:.6f}, "
              f"max |d dI| {err.max():.2e}", flush=True)


@pytest.mark.parametrize("name,rows", [("decode32k", [0, 31]),
                                       ("prefill8k", [0, 5, 2047, 2048, 5000, 8191])])
def test_indexer_loss_dense_parity(dsa, name, rows):
    """The dense warm-up loss over every s <= t, fed the oracle's scores (as fp32):
    against the oracle's target over all t + 1 entries and its KL, under the same
    bars as the sparse loss (the sums now run over up to 32768 terms)."""
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    print(f"[dense loss] {name} rows {rows}", flush=True)
    R = len(rows)
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    ld = (cfg.kv_len + 63) // 64 * 64
    sc = np.full((R, ld), np.nan, dtype=np.float32)  # past t: never read
    hrows = [host.row(int(r)) for r in rows]
    for i, row in enumerate(hrows):
        sc[i, : row.t + 1] = host.scores(row).astype(np.float32)
    q = inp.q[ridx].contiguous()
    loss, dsc = dsa.indexer_loss_dense(rs, q, inp.latent, cfg.scale, torch.from_numpy(sc).cuda())
    torch.cuda.synchronize()
    loss, dsc = loss.cpu().numpy(), dsc.cpu().numpy()
    for i, row in enumerate(hrows):
        n = row.t + 1
        ent = host.latent_rows(row.b, np.arange(n))
        p = oracle.attention_target(oracle.decode_bf16(row.q), oracle.decode_bf16(ent), cfg.scale)
        Is = sc[i, :n].astype(np.float64)
        l_ref, g_ref = oracle.indexer_kl(p, Is)
        sm = np.exp(Is - Is.max())
        sm /= sm.sum()
        assert abs(loss[i] - l_ref) <= 1e-3 * abs(l_ref) + 1e-6, (rows[i], loss[i], l_ref)
        err = np.abs(dsc[i, :n] - g_ref)
        assert np.all(err <= 1e-3 * (p + sm) + 1e-7), (rows[i], float(err.max()))
        assert np.all(dsc[i, n:] == 0.0)
        print(f"[dense loss] row {int(rows[i])} (t = {row.t}): loss {loss[i]:.6f} ref {l_ref:.6f}, "
              f"max |d dI| {err.max():.2e}", flush=True)


def test_indexer_loss_composed(dsa):
    """The whole forward on the GPU (scores, top-k, attention, loss): the loss is
    finite and non-negative, dscores sum to ~0 per row, and the loss agrees with the
    oracle's on its own selection within the indexer's score error."""
    cfg = di.CONFIGS["decode32k"]
    inp = dev_inputs("decode32k")
    host = HostInputs(cfg)
    R = cfg.num_rows
    rs = dsa.rows_struct(inp.row_seq, inp.row_pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    dims = dsa.Dims.from_config(cfg)
    sc = dsa.indexer_scores(rs, dims, inp.q_idx, inp.q_scale, inp.w, inp.k_idx, inp.k_scale)
    idx = dsa.topk(rs, cfg.topk, sc)
    _, lse = dsa.sparse_mla_attn(rs, dims, inp.q, inp.latent, idx, cfg.scale)
    loss, dsc = dsa.indexer_loss(rs, inp.q, inp.latent, idx, lse, cfg.scale, sc)
    torch.cuda.synchronize()
    loss, dsc = loss.cpu().numpy(), dsc.cpu().numpy()
    assert np.all(np.isfinite(loss)) and np.all(loss >= -1e-6)
    assert np.all(np.abs(dsc.sum(axis=1)) < 1e-3)
    for r in (0, 31):
        row = host.row(r)
        I = host.scores(row)
        S = oracle.select_topk(I, cfg.topk)
        ent = host.latent_rows(row.b, S)
        p = oracle.attention_target(oracle.decode_bf16(row.q), oracle.decode_bf16(ent), cfg.scale)
        l_ref, _ = oracle.indexer_kl(p, I[S])
        # C1 allows score errors up to 2e-2 of the row's largest score in principle;
        # measured errors are ~1e-4 of it, which moves a KL of this size by < 5 %
        assert abs(loss[r] - l_ref) <= 0.05 * l_ref + 1e-4, (r, loss[r], l_ref)


@pytest.mark.parametrize("name,rows,mode", [("decode32k", [0, 13, 31], "full"),
                                            ("decode32k", [0, 13, 31], "dup"),
                                            ("prefill8k", list(range(4000, 4016)), "full"),
                                            ("prefill8k", list(range(4000, 4016)), "min"),
                                            ("prefill8k", list(range(4000, 4016)), "few")])
def test_indexer_backward_parity(dsa, name, rows, mode):
    """Seeded dscores on the oracle's selections; for the prefill rows the key
    gradients of rows that select the same key add up.  Modes: "full" workspace
    (every key selected more than once is summed in fixed point); "min" (no
    accumulators: such keys are added with fp32 atomics); "few" (7 accumulators, the
    rest atomics); "dup" (each row's index list holds its first 1024 selected
    positions twice, so keys repeat within a row)."""
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    print(f"[backward] {name} rows {rows[0]}..{rows[-1]} mode {mode}", flush=True)
    setup = _oracle_setup(cfg, host, rows)
    R = len(rows)
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    rng = np.random.default_rng(77)
    idx = np.full((R, cfg.topk), -1, dtype=np.int32)
    g = np.zeros((R, cfg.topk), dtype=np.float32)
    ents = []
    for i, (row, I, S) in enumerate(setup):
        ent = np.concatenate([S[:1024], S[:1024]]) if mode == "dup" else S
        ents.append(ent)
        idx[i, : ent.size] = ent
        g[i, : ent.size] = (rng.standard_normal(ent.size) * 1e-3).astype(np.float32)
    dq = torch.zeros(R, 64, 128, dtype=torch.float32, device="cuda")
    dw = torch.zeros(R, 64, dtype=torch.float32, device="cuda")
    dk = torch.zeros(cfg.num_seqs, cfg.max_ctx, 128, dtype=torch.float32, device="cuda")
    nacc = {"full": -1, "dup": -1, "min": 0, "few": 7}[mode]
    ws = torch.empty(dsa.indexer_backward_workspace_size(rs, shared_keys=nacc),
                     dtype=torch.uint8, device="cuda")
    dsa.indexer_backward(rs, inp.q_idx[ridx].contiguous(), inp.q_scale[ridx].contiguous(),
                         inp.w[ridx].contiguous(), inp.k_idx, inp.k_scale,
                         torch.from_numpy(idx).cuda(), torch.from_numpy(g).cuda(), dq, dw, dk,
                         workspace=ws)
    torch.cuda.synchronize()
    dq, dw = dq.cpu().numpy(), dw.cpu().numpy()
    dk_ref, dk_tol = {}, {}
    for i, (row, I, S) in enumerate(setup):
        S = ents[i]
        qf = oracle.decode_e4m3fn(row.q_idx) * row.q_scale[:, None]
        codes, ksc = host.keys(row.b, row.t + 1)
        kf = oracle.decode_e4m3fn(codes[S]) * ksc[S][:, None]
        gi = g[i, : S.size].astype(np.float64)
        q_ref, w_ref, k_ref = oracle.indexer_backward(qf, row.w, kf, gi)
        dots = qf @ kf.T
        amb = np.abs(dots) <= DOT_EPS * (np.abs(qf) @ np.abs(kf).T)  # mask may flip
        coef_abs = np.abs(row.w)[:, None] * np.abs(gi)[None, :]       # |w_j g_s|
        terms_q = (coef_abs * (dots > 0)) @ np.abs(kf)
        tol_q = 1e-5 * terms_q + (coef_abs * amb) @ np.abs(kf) + 1e-12
        assert np.all(np.abs(dq[i] - q_ref) <= tol_q), float(np.max(np.abs(dq[i] - q_ref) - tol_q))
        # every dot may be off by the MFMA's error bound
        tol_w = 1e-5 * (np.maximum(dots, 0) @ np.abs(gi)) + \
            (DOT_EPS * (np.abs(qf) @ np.abs(kf).T)) @ np.abs(gi) + 1e-12
        assert np.all(np.abs(dw[i] - w_ref) <= tol_w)
        tol_k = 1e-5 * ((coef_abs * (dots > 0)).T @ np.abs(qf)) + (coef_abs * amb).T @ np.abs(qf) + 1e-12
        for a, s in enumerate(S):
            key = (row.b, int(s))
            dk_ref[key] = dk_ref.get(key, 0.0) + k_ref[a]
            dk_tol[key] = dk_tol.get(key, 0.0) + tol_k[a]
    keys = list(dk_ref)
    bt = torch.tensor([k[0] for k in keys], device="cuda")
    st = torch.tensor([k[1] for k in keys], device="cuda")
    got = dk[bt, st].cpu().numpy()
    ref = np.stack([dk_ref[k] for k in keys])
    tol = np.stack([dk_tol[k] for k in keys])
    assert np.all(np.abs(got - ref) <= tol + 1e-12), float(np.max(np.abs(got - ref) - tol))
    count = {}
    for (row, I, S), ent in zip(setup, ents):
        for s_ in ent.tolist():
            count[(row.b, s_)] = count.get((row.b, s_), 0) + 1
    shared = sum(1 for k in keys if count[k] > 1)
    assert mode not in ("dup", "few") or shared > 7
    print(f"[backward] {name} {mode}: dq, dw, dk within bars; {len(keys)} keys, "
          f"{shared} selected more than once", flush=True)
    # nothing outside the selected keys is written
    mask = torch.zeros(cfg.num_seqs, cfg.max_ctx, dtype=torch.bool, device="cuda")
    mask[bt, st] = True
    assert bool((dk[~mask] == 0).all())


@pytest.mark.parametrize("name,rows", [("decode32k", [0, 13]),
                                       ("prefill8k", list(range(3000, 3008)))])
def test_indexer_backward_dense_parity(dsa, name, rows):
    """The dense backward: a seeded gradient over every position s <= t, against the
    oracle's backward over all t + 1 keys, under the sparse backward's bars; the
    prefill rows share almost all of their keys, so dk sums over rows."""
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    host = HostInputs(cfg)
    print(f"[backward dense] {name} rows {rows[0]}..{rows[-1]}", flush=True)
    R = len(rows)
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    ld = (cfg.kv_len + 63) // 64 * 64
    rng = np.random.default_rng(78)
    g = np.zeros((R, ld), dtype=np.float32)
    hrows = [host.row(int(r)) for r in rows]
    for i, row in enumerate(hrows):
        g[i, : row.t + 1] = (rng.standard_normal(row.t + 1) * 1e-4).astype(np.float32)
        g[i, row.t + 1:] = np.nan  # past t: never read
    dq = torch.zeros(R, 64, 128, dtype=torch.float32, device="cuda")
    dw = torch.zeros(R, 64, dtype=torch.float32, device="cuda")
    dk = torch.zeros(cfg.num_seqs, cfg.max_ctx, 128, dtype=torch.float32, device="cuda")
    dsa.indexer_backward_dense(rs, inp.q_idx[ridx].contiguous(), inp.q_scale[ridx].contiguous(),
                               inp.w[ridx].contiguous(), inp.k_idx, inp.k_scale,
                               torch.from_numpy(g).cuda(), dq, dw, dk)
    torch.cuda.synchronize()
    dq, dw = dq.cpu().numpy(), dw.cpu().numpy()
    dk_ref, dk_tol = {}, {}
    for i, row in enumerate(hrows):
        n = row.t + 1
        qf = oracle.decode_e4m3fn(row.q_idx) * row.q_scale[:, None]
        codes, ksc = host.keys(row.b, n)
        kf = oracle.decode_e4m3fn(codes) * ksc[:, None]
        gi = g[i, :n].astype(np.float64)
        q_ref, w_ref, k_ref = oracle.indexer_backward(qf, row.w, kf, gi)
        dots = qf @ kf.T
        absd = np.abs(qf) @ np.abs(kf).T
        amb = np.abs(dots) <= DOT_EPS * absd
        coef_abs = np.abs(row.w)[:, None] * np.abs(gi)[None, :]
        tol_q = 1e-5 * ((coef_abs * (dots > 0)) @ np.abs(kf)) + (coef_abs * amb) @ np.abs(kf) + 1e-12
        assert np.all(np.abs(dq[i] - q_ref) <= tol_q), float(np.max(np.abs(dq[i] - q_ref) - tol_q))
        tol_w = 1e-5 * (np.maximum(dots, 0) @ np.abs(gi)) + (DOT_EPS * absd) @ np.abs(gi) + 1e-12
        assert np.all(np.abs(dw[i] - w_ref) <= tol_w)
        tol_k = 1e-5 * ((coef_abs * (dots > 0)).T @ np.abs(qf)) + (coef_abs * amb).T @ np.abs(qf) + 1e-12
        for s_ in range(n):
            key = (row.b, s_)
            dk_ref[key] = dk_ref.get(key, 0.0) + k_ref[s_]
            dk_tol[key] = dk_tol.get(key, 0.0) + tol_k[s_]
    keys = list(dk_ref)
    bt = torch.tensor([k[0] for k in keys], device="cuda")
    st = torch.tensor([k[1] for k in keys], device="cuda")
    got = dk[bt, st].cpu().numpy()
    ref = np.stack([dk_ref[k] for k in keys])
    tol = np.stack([dk_tol[k] for k in keys])
    assert np.all(np.abs(got - ref) <= tol + 1e-12), float(np.max(np.abs(got - ref) - tol))
    mask = torch.zeros(cfg.num_seqs, cfg.max_ctx, dtype=torch.bool, device="cuda")
    mask[bt, st] = True
    assert bool((dk[~mask] == 0).all())
    print(f"[backward dense] {name}: dq, dw, dk within bars over {len(keys)} keys", flush=True)


def test_dense_and_sparse_loss_agree_below_k(dsa):
    """Rows with t + 1 <= k select every causal position, so the sparse-stage loss
    (selection = 0..t, lse from the attention call) and the dense warm-up loss (its
    own lse over 0..t) must agree: two entry points with separate kernels."""
    cfg = di.CONFIGS["prefill8k"]
    inp = dev_inputs("prefill8k")
    rows = [0, 1, 7, 100, 1000, 2047]
    R = len(rows)
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    dims = dsa.Dims.from_config(cfg)
    ld = (cfg.kv_len + 63) // 64 * 64
    rng = np.random.default_rng(11)
    sc = rng.standard_normal((R, ld)).astype(np.float32)
    idx = np.full((R, cfg.topk), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        t = int(inp.row_pos[r])
        idx[i, : t + 1] = np.arange(t + 1)
    sc_d, idx_d = torch.from_numpy(sc).cuda(), torch.from_numpy(idx).cuda()
    q = inp.q[ridx].contiguous()
    _, lse = dsa.sparse_mla_attn(rs, dims, q, inp.latent, idx_d, cfg.scale)
    l_s, g_s = dsa.indexer_loss(rs, q, inp.latent, idx_d, lse, cfg.scale, sc_d)
    l_d, g_d = dsa.indexer_loss_dense(rs, q, inp.latent, cfg.scale, sc_d)
    torch.cuda.synchronize()
    l_s, g_s, l_d, g_d = (x.cpu().numpy() for x in (l_s, g_s, l_d, g_d))
    for i, r in enumerate(rows):
        t = int(inp.row_pos[r])
        assert abs(l_s[i] - l_d[i]) <= 2e-3 * abs(l_d[i]) + 2e-6, (r, l_s[i], l_d[i])
        # dI: sparse by selection slot, dense by position (slot i holds position i here)
        sm = np.exp(sc[i, : t + 1] - sc[i, : t + 1].max())
        sm /= sm.sum()
        assert np.all(np.abs(g_s[i, : t + 1] - g_d[i, : t + 1]) <= 2e-3 * (sm + np.abs(g_d[i, : t + 1])) + 2e-7)
        print(f"[loss agree] row {r} (t = {t}): sparse {l_s[i]:.6f} dense {l_d[i]:.6f}", flush=True)


def test_dense_rows_past_max_pos_untouched(dsa):
    """A row at t > max_pos (still t < N) is not processed by the dense warm-up loss
    or its backward: loss 0, a zero dscores row, no gradient, and no read of another
    row's chunk partials (the row last, where such a read would pass the workspace's
    end).  The row before it is still computed as the oracle says."""
    cfg = di.CONFIGS["prefill8k"]
    inp = dev_inputs("prefill8k")
    host = HostInputs(cfg)
    rows = [100, 1500]          # max_pos 200: one 1024-position chunk; row 1500 needs two
    max_pos, ld = 200, 256
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, max_pos)
    row = host.row(rows[0])
    n = row.t + 1
    sc = np.full((2, ld), np.nan, dtype=np.float32)
    sc[0, :n] = host.scores(row).astype(np.float32)
    sc[1, :] = 1.0
    q = inp.q[ridx].contiguous()
    loss, dsc = dsa.indexer_loss_dense(rs, q, inp.latent, cfg.scale, torch.from_numpy(sc).cuda())
    g = torch.zeros(2, ld, device="cuda")
    g[0, :n] = 1e-3
    g[1, :] = 1.0
    dq = torch.zeros(2, 64, 128, device="cuda")
    dw = torch.zeros(2, 64, device="cuda")
    dk = torch.zeros(cfg.num_seqs, cfg.max_ctx, 128, device="cuda")
    dsa.indexer_backward_dense(rs, inp.q_idx[ridx].contiguous(), inp.q_scale[ridx].contiguous(),
                               inp.w[ridx].contiguous(), inp.k_idx, inp.k_scale, g, dq, dw, dk)
    torch.cuda.synchronize()
    loss, dsc = loss.cpu().numpy(), dsc.cpu().numpy()
    assert loss[1] == 0.0 and np.all(dsc[1] == 0.0)
    assert bool((dq[1] == 0).all()) and bool((dw[1] == 0).all())
    assert bool((dk[0, n:] == 0).all())           # only row 100's keys 0..100 are touched
    ent = host.latent_rows(row.b, np.arange(n))
    p = oracle.attention_target(oracle.decode_bf16(row.q), oracle.decode_bf16(ent), cfg.scale)
    l_ref, _ = oracle.indexer_kl(p, sc[0, :n].astype(np.float64))
    assert abs(loss[0] - l_ref) <= 1e-3 * abs(l_ref) + 1e-6, (loss[0], l_ref)
    print(f"[past max_pos] row {rows[1]} untouched; row {rows[0]} loss {loss[0]:.6f} ref {l_ref:.6f}",
          flush=True)


@pytest.mark.parametrize("case", ["decode32k", "prefill8k", "decode32k_dense", "prefill8k_dense"])
def test_indexer_backward_deterministic(dsa, case):
    """The backward's outputs are the same bits from run to run, whatever the
    workspace held before (it is filled with 0xFF bytes before each run): decode
    rows (one per sequence: every key has one writer) with the smallest workspace
    and with the full one, which must also agree bit for bit; prefill rows that
    share most of their keys (fixed-point sums) with the full workspace."""
    name = case.split("_")[0]
    dense = case.endswith("_dense")
    cfg = di.CONFIGS[name]
    inp = dev_inputs(name)
    rows = list(range(cfg.num_rows)) if name == "decode32k" else \
        list(range(3000, 3016)) if dense else list(range(4000, 4064))
    R = len(rows)
    ridx = torch.tensor(rows, device="cuda")
    seq, pos = inp.row_seq[ridx].contiguous(), inp.row_pos[ridx].contiguous()
    rs = dsa.rows_struct(seq, pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
    dims = dsa.Dims.from_config(cfg)
    q_idx, q_scale, w = (x[ridx].contiguous() for x in (inp.q_idx, inp.q_scale, inp.w))
    gen = torch.Generator(device="cuda").manual_seed(5)
    if dense:
        ld = (cfg.kv_len + 63) // 64 * 64
        g = torch.randn(R, ld, generator=gen, device="cuda") * 1e-4
        size = dsa.indexer_backward_dense_workspace_size
        call = lambda dq, dw, dk, ws: dsa.indexer_backward_dense(
            rs, q_idx, q_scale, w, inp.k_idx, inp.k_scale, g, dq, dw, dk, workspace=ws)
    else:
        sc = dsa.indexer_scores(rs, dims, q_idx, q_scale, w, inp.k_idx, inp.k_scale)
        idx = dsa.topk(rs, cfg.topk, sc)
        g = torch.randn(R, cfg.topk, generator=gen, device="cuda") * 1e-3
        size = dsa.indexer_backward_workspace_size
        call = lambda dq, dw, dk, ws: dsa.indexer_backward(
            rs, q_idx, q_scale, w, inp.k_idx, inp.k_scale, idx, g, dq, dw, dk, workspace=ws)
    modes = ((0, -1) if name == "decode32k" else (-1,))
    first = None
    for nacc in modes:
        ws = torch.empty(size(rs, shared_keys=nacc), dtype=torch.uint8, device="cuda")
        for run in range(3):
            ws.fill_(255)
            dq = torch.zeros(R, 64, 128, device="cuda")
            dw = torch.zeros(R, 64, device="cuda")
            dk = torch.zeros(cfg.num_seqs, cfg.max_ctx, 128, device="cuda")
            call(dq, dw, dk, ws)
            torch.cuda.synchronize()
            if first is None:
                first = (dq, dw, dk)
                assert bool(dk.abs().sum() > 0) and bool(dq.abs().sum() > 0)
                continue
            for a, b_, nm in zip(first, (dq, dw, dk), ("dq", "dw", "dk")):
                assert torch.equal(a, b_), (case, nacc, run, nm)
        del ws
    print(f"[backward determinism] {case}: {R} rows, workspaces {modes}: identical bits",
          flush=True)
