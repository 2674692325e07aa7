"""Parity of the masked MHA mode (dsa_mha_prefill, through the C ABI) with the
float64 oracle, under the attention bar C3 (max |d out| <= 2e-2, mean <= 2e-3).

A short sequence (every row dense causal) is checked against the MHA-mode oracle
itself.  For the 8192-row prefill the reference goes through the MQA-mode oracle
with the absorbed query, then the value up-projection.  The oracle pins that
identity, and it avoids decompressing 2048 entries x 128 heads per row in float64.
Selections are seeded random valid sets (all of 0..t when t + 1 <= k).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dsa_inputs as di
import oracle
from dsa_check import HostInputs, attn_errors, ATTN_MAX_ABS, ATTN_MEAN_ABS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_fp8_amd as m
    return m


def _run(dsa, cfg, L, rows_all, seed):
    """MHA mode over rows t = rows_all of one sequence of `cfg`'s latent cache."""
    g = di.Generator(cfg, 0)
    mg = di.MhaGenerator(cfg.cfg_id, 0)
    dev = torch.device("cuda")
    lat = g.latent(0, 0, L, device=dev)
    latent = torch.zeros(1, L, cfg.qk_dim, dtype=torch.bfloat16, device=dev)
    latent[0] = lat
    R = len(rows_all)
    q = mg.q(0, R, device=dev)
    w_uk, w_uv = mg.weights(device=dev)
    rng = np.random.default_rng(seed)
    idx = np.stack([di.random_selection(int(t), cfg.topk, rng) for t in rows_all])
    seq = torch.zeros(R, dtype=torch.int32, device=dev)
    pos = torch.from_numpy(np.asarray(rows_all, dtype=np.int32)).to(dev)
    rs = dsa.rows_struct(seq, pos, 1, L, int(max(rows_all)))
    dims = dsa.Dims.from_config(cfg)
    out, lse = dsa.mha_prefill(rs, q, latent, w_uk, w_uv, torch.from_numpy(idx).to(dev), cfg.scale,
                               dims=dims)
    torch.cuda.synchronize()
    return g, mg, idx, out, lse


def _check(o_gpu, o_ref, lse_gpu, lse_ref, tag):
    mx, mean = attn_errors(o_gpu, o_ref)
    dl = float(np.max(np.abs(lse_gpu - lse_ref)))
    print(f"[mha] {tag}: max {mx:.2e} mean {mean:.2e} |d lse| {dl:.2e}", flush=True)
    assert np.all(np.isfinite(o_gpu))
    assert mx <= ATTN_MAX_ABS and mean <= ATTN_MEAN_ABS
    assert dl <= 1e-2


def test_mha_short_dense(dsa):
    """A 300-token sequence: every row attends to all of 0..t (dense causal)."""
    cfg = di.CONFIGS["prefill8k"]
    L = 300
    rows_all = list(range(L))
    g, mg, idx, out, lse = _run(dsa, cfg, L, rows_all, 5)
    ent = oracle.decode_bf16(di.bf16_bits(g.latent(0, 0, L)))
    wuk, wuv = (oracle.decode_bf16(di.bf16_bits(x)) for x in mg.weights())
    k, v = oracle.mha_decompress(ent, wuk, wuv, cfg.v_dim)
    qh = oracle.decode_bf16(di.bf16_bits(mg.q(0, L)))
    for t in (0, 1, 77, 150, 299):
        z = cfg.scale * np.einsum("hd,hnd->hn", qh[t], k[:, : t + 1])
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        o_ref = np.einsum("hn,hnd->hd", e / e.sum(axis=1, keepdims=True), v[:, : t + 1])
        lse_ref = m[:, 0] + np.log(e.sum(axis=1))
        if t in (0, 150):  # the oracle's own MHA function on the same row
            o2, l2 = oracle.mha_attention(qh[t], ent[: t + 1], wuk, wuv, cfg.scale, cfg.v_dim)
            np.testing.assert_allclose(o2, o_ref, rtol=1e-10, atol=1e-12)
        _check(out[t].float().cpu().numpy().astype(np.float64), o_ref,
               lse[t].cpu().numpy().astype(np.float64), lse_ref, f"L=300 row {t}")


def test_mha_prefill8k_masked(dsa):
    """8192 rows with seeded selections of 2048 positions beyond t = 2047."""
    cfg = di.CONFIGS["prefill8k"]
    L = cfg.kv_len
    rows_all = list(range(L))
    g, mg, idx, out, lse = _run(dsa, cfg, L, rows_all, 6)
    wuk, wuv = (oracle.decode_bf16(di.bf16_bits(x)) for x in mg.weights())
    for t in (0, 2047, 2048, 5000, 8191):
        S = idx[t][idx[t] >= 0]
        ent = oracle.decode_bf16(di.bf16_bits(g.latent_rows(0, torch.from_numpy(S.astype(np.int64)))))
        qh = oracle.decode_bf16(di.bf16_bits(mg.q(t, t + 1)))[0]
        q_abs = np.concatenate([np.einsum("hdc,hd->hc", wuk, qh[:, :128]), qh[:, 128:]], axis=1)
        o_lat, lse_ref = oracle.sparse_attention(q_abs, ent, cfg.scale, cfg.v_dim)
        o_ref = np.einsum("hdc,hc->hd", wuv, o_lat)
        _check(out[t].float().cpu().numpy().astype(np.float64), o_ref,
               lse[t].cpu().numpy().astype(np.float64), lse_ref, f"8K row {t}")


def test_mha_prefill2k_batch(dsa):
    """The short-prefill workload the bench times: 4 sequences of 2048 tokens, rows
    grouped by sequence, each row selecting its whole causal set (t + 1 <= k, as
    the indexer's top-k does there); sampled rows of every sequence against the
    MQA-mode oracle with the absorbed query."""
    cfg = di.CONFIGS["prefill2k"]
    dev = torch.device("cuda")
    inp = di.make_inputs(cfg, 0, device=dev)
    R, L = cfg.num_rows, cfg.kv_len
    mg = di.MhaGenerator(cfg.cfg_id, 0)
    q = mg.q(0, R, device=dev)
    w_uk, w_uv = mg.weights(device=dev)
    seq, pos = cfg.row_seq_pos()
    idx = np.full((R, cfg.topk), -1, dtype=np.int32)
    for i, t in enumerate(pos):
        idx[i, : t + 1] = np.arange(t + 1)
    rs = dsa.rows_struct(inp.row_seq, inp.row_pos, cfg.num_seqs, cfg.max_ctx, L - 1)
    dims = dsa.Dims.from_config(cfg)
    out, lse = dsa.mha_prefill(rs, q, inp.latent, w_uk, w_uv, torch.from_numpy(idx).to(dev),
                               cfg.scale, dims=dims)
    torch.cuda.synchronize()
    g = di.Generator(cfg, 0)
    wuk, wuv = (oracle.decode_bf16(di.bf16_bits(x)) for x in mg.weights())
    for b in range(cfg.num_seqs):
        for t in (0, 63, 64, 1000, 2047):
            i = b * L + t
            S = np.arange(t + 1)
            ent = oracle.decode_bf16(di.bf16_bits(g.latent_rows(b, torch.from_numpy(S.astype(np.int64)))))
            qh = oracle.decode_bf16(di.bf16_bits(mg.q(i, i + 1)))[0]
            q_abs = np.concatenate([np.einsum("hdc,hd->hc", wuk, qh[:, :128]), qh[:, 128:]], axis=1)
            o_lat, lse_ref = oracle.sparse_attention(q_abs, ent, cfg.scale, cfg.v_dim)
            o_ref = np.einsum("hdc,hc->hd", wuv, o_lat)
            _check(out[i].float().cpu().numpy().astype(np.float64), o_ref,
                   lse[i].cpu().numpy().astype(np.float64), lse_ref, f"2K seq {b} row {t}")


def test_mha_interleaved_sequences(dsa):
    """Three sequences of 100, 250 and 180 tokens whose rows are interleaved (row
    order by position, then sequence), so every 128-row tile holds rows of all three;
    each row selects a seeded random 60 % of 0..t (the rest masked)."""
    cfg = di.CONFIGS["prefill8k"]
    lens = (100, 250, 180)
    N, B = 256, len(lens)
    g = di.Generator(cfg, 0)
    mg = di.MhaGenerator(cfg.cfg_id, 1)
    dev = torch.device("cuda")
    latent = torch.stack([g.latent(b, 0, N, device=dev) for b in range(B)]).contiguous()
    rows = [(b, t) for t in range(max(lens)) for b in range(B) if t < lens[b]]
    R = len(rows)
    rng = np.random.default_rng(9)
    idx = np.full((R, cfg.topk), -1, dtype=np.int32)
    for i, (b, t) in enumerate(rows):
        m = max(1, int(0.6 * (t + 1)))
        idx[i, :m] = np.sort(rng.choice(t + 1, size=m, replace=False))
    seq = torch.tensor([b for b, _ in rows], dtype=torch.int32, device=dev)
    pos = torch.tensor([t for _, t in rows], dtype=torch.int32, device=dev)
    rs = dsa.rows_struct(seq, pos, B, N, max(lens) - 1)
    q = mg.q(0, R, device=dev)
    w_uk, w_uv = mg.weights(device=dev)
    dims = dsa.Dims.from_config(cfg)
    out, lse = dsa.mha_prefill(rs, q, latent, w_uk, w_uv, torch.from_numpy(idx).to(dev), cfg.scale,
                               dims=dims)
    torch.cuda.synchronize()
    out_h = out.float().cpu().numpy().astype(np.float64)
    lse_h = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out_h)) and np.all(np.isfinite(lse_h))
    wuk, wuv = (oracle.decode_bf16(di.bf16_bits(x)) for x in mg.weights())
    qh_all = oracle.decode_bf16(di.bf16_bits(mg.q(0, R)))
    kv = {}
    for b in range(B):
        ent = oracle.decode_bf16(di.bf16_bits(g.latent(b, 0, lens[b])))
        kv[b] = oracle.mha_decompress(ent, wuk, wuv, cfg.v_dim)
    picks = [0, 1, 2, 150, 299, 300, 301, R - 1] + list(rng.choice(R, size=4, replace=False))
    for i in picks:
        b, t = rows[int(i)]
        S = idx[i][idx[i] >= 0]
        k, v = kv[b]
        z = cfg.scale * np.einsum("hd,hnd->hn", qh_all[i], k[:, S])
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        o_ref = np.einsum("hn,hnd->hd", e / e.sum(axis=1, keepdims=True), v[:, S])
        lse_ref = m[:, 0] + np.log(e.sum(axis=1))
        _check(out_h[i], o_ref, lse_h[i], lse_ref, f"seq {b} row t={t} ({S.size} selected)")
