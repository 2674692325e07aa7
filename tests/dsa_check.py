"""Test helpers: run the float64 oracle on host-regenerated inputs and compare the
HIP path's outputs with it.

Oracle inputs are always regenerated on the host from the seeded generator; they
never come from the GPU.  The three comparison rules follow the tolerances the
hot path is held to:

* C1 scores:  |I_gpu - I_ref| <= 2e-2 * max(|I_ref|, SCORE_FLOOR * max_s |I_ref|).
  The floor exists because w has both signs, so single scores cancel to ~0, while
  the kernel's error does not shrink with them.  Its source: the fp8 MFMA does not
  sum a 128-term dot like fp32 additions.  It forms the sum from 16 groups of 8
  products (bytes [8m, 8m + 8) of both vectors), cutting each product of a group
  toward zero at 2^-13 of the group's largest product, then adds the group sums
  with fp32 rounding (tests/test_gpu_fp8_accumulation.py pins this on the device
  against exact sums).  On the five workloads the resulting score errors reach
  3.8e-5 of the row's largest score (test_indexer_parity prints the figure per
  workload); SCORE_FLOOR = 5e-3 allows 1e-4 of it, 2.6x the measured maximum.  (The
  model's worst case, every cut product just under its unit with aligned signs,
  is ~1e-2 of the row maximum; the seeded workloads are far from it, and a bar that
  loose would pass a dropped indexer head.)
* C2 indices: the GPU set has n = min(k, t+1) unique positions in [0, t], ascending,
  -1 padded; it equals the oracle's set outside the tie band
  A = {s : |I_ref[s] - tau| <= 1e-3 |tau|}, tau = the n-th largest oracle score.
* C3 attention (bf16): max |o_gpu - o_ref| <= 2e-2 and mean <= 2e-3.
* C4 projections: the kernel accumulates y = W h in fp32, so its y differs from
  the exact one by rounding.  Each output gets the bound
  err = 16 sqrt(d) 2^-24 ||(h_k W_pk)_k||_2: the rounding errors of any summation
  order form a sum of at most d terms, each at most 2^-24 times a partial sum,
  and the partial sums of these sign-random products stay within a few
  ||x||_2 (a random-walk bound, ~4 sigma with margin).  A stored value is
  correct when it is what the oracle's encoder gives for some y' within err of
  the exact y: the fp8 scale is one of the power-of-two scales of amax +- err,
  each code lies between the codes of (y - err) / scale and (y + err) / scale,
  each bf16 word between the words of y - err and y + err, and fp32 w within
  err.  Away from rounding boundaries this is exact equality.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import dsa_inputs as di
import oracle

SCORE_RTOL = 2e-2
SCORE_FLOOR = 5e-3
# The fp8 MFMA's 128-term dot (pinned by tests/test_gpu_fp8_accumulation.py):
# 16 groups of FP8_GROUP consecutive bytes; each product cut toward zero at
# 2^-FP8_CUT_BITS of its group's largest product; group sums added in fp32.  A dot
# is off by at most GROUP_EPS per unit of each group's largest |product| plus
# SUM_EPS per unit of sum |products| (and the rounding of the result).
FP8_GROUP = 8
FP8_CUT_BITS = 13
GROUP_EPS = (FP8_GROUP - 1) * 2.0 ** -FP8_CUT_BITS
SUM_EPS = 16 * 2.0 ** -23
U32 = 2.0 ** -24
BAND = 1e-3
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3


@dataclasses.dataclass
class HostRow:
    """Raw input images of one query row, regenerated on the host."""
    r: int
    b: int
    t: int
    q_idx: np.ndarray
    q_scale: Optional[np.ndarray]
    w: np.ndarray
    q: np.ndarray


class HostInputs:
    """Lazily regenerates host copies of a workload's inputs."""

    def __init__(self, cfg: di.Config, set_id: int = 0):
        self.cfg = cfg
        self.gen = di.Generator(cfg, set_id)
        self.seq, self.pos = cfg.row_seq_pos()
        self._k: Dict[int, tuple] = {}
        self._kf: Dict[int, np.ndarray] = {}

    def row(self, r: int) -> HostRow:
        c = self.cfg
        codes, sc = self.gen.q_idx(r, r + 1)
        w = self.gen.w(r, r + 1)[0].numpy().astype(np.float64)
        q = self.gen.q(r, r + 1)[0]
        if c.fp32:
            return HostRow(r, int(self.seq[r]), int(self.pos[r]), codes[0].numpy(), None, w,
                           q.numpy())
        return HostRow(r, int(self.seq[r]), int(self.pos[r]), codes[0].numpy(),
                       sc[0].numpy().astype(np.float64), w, di.bf16_bits(q))

    def keys(self, b: int, upto: int):
        """Indexer key codes / scales of sequence b for positions [0, upto)."""
        have = self._k.get(b)
        if have is None or have[0].shape[0] < upto:
            codes, sc = self.gen.k_idx(b, 0, upto)
            self._k[b] = (codes.numpy(), None if self.cfg.fp32 else sc.numpy().astype(np.float64))
        codes, sc = self._k[b]
        return codes[:upto], (None if sc is None else sc[:upto])

    def latent_rows(self, b: int, positions: np.ndarray) -> np.ndarray:
        x = self.gen.latent_rows(b, torch.from_numpy(np.asarray(positions, dtype=np.int64)))
        return x.numpy() if self.cfg.fp32 else di.bf16_bits(x)

    def scores(self, row: HostRow) -> np.ndarray:
        """Oracle scores I[0..t] of one row.  The sequence's dequantised keys are
        cached (oracle decoder times scale, exactly what oracle.indexer_row does per
        call) so long sequences are decoded once."""
        if row.t + 1 <= 4096:
            codes, sc = self.keys(row.b, row.t + 1)
            return oracle.indexer_row(row.q_idx, row.q_scale, row.w, codes, sc, row.t,
                                      not self.cfg.fp32)
        kf = self._kf.get(row.b)
        if kf is None or kf.shape[0] < row.t + 1:
            codes, sc = self.keys(row.b, self.cfg.max_ctx)
            kf = (oracle.decode_e4m3fn(codes) * sc[:, None]) if sc is not None \
                else codes.astype(np.float64)
            self._kf[row.b] = kf
        qf = (oracle.decode_e4m3fn(row.q_idx) * row.q_scale[:, None]) if row.q_scale is not None \
            else row.q_idx.astype(np.float64)
        return oracle.indexer_scores(qf, row.w, kf[: row.t + 1])

    def attention(self, row: HostRow, positions: np.ndarray):
        ent = self.latent_rows(row.b, positions)
        return oracle.attention_row(row.q, ent, self.cfg.scale, self.cfg.v_dim, not self.cfg.fp32)


def check_scores(gpu: np.ndarray, ref: np.ndarray) -> float:
    """C1; returns the worst ratio |err| / allowed (must be <= 1)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    floor = SCORE_FLOOR * np.max(np.abs(ref)) if ref.size else 0.0
    allowed = SCORE_RTOL * np.maximum(np.abs(ref), floor)
    err = np.abs(gpu - ref)
    ok = (err <= allowed) | ((err == 0) & (allowed == 0))
    assert np.all(np.isfinite(gpu)), "non-finite GPU score"
    assert ok.all(), (f"score mismatch at {np.nonzero(~ok)[0][:8]}: gpu {gpu[~ok][:4]} "
                      f"ref {ref[~ok][:4]}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allowed > 0, err / allowed, 0.0)
    return float(ratio.max()) if ratio.size else 0.0


def check_selection(gpu_idx: np.ndarray, ref_scores: np.ndarray, t: int, k: int) -> int:
    """C2; returns the size of the tie band."""
    n = min(k, t + 1)
    g = np.asarray(gpu_idx)
    assert g.shape == (k,)
    assert np.all(g[n:] == -1), "padding must be -1"
    sel = g[:n]
    assert np.all((sel >= 0) & (sel <= t)), "selected position out of [0, t]"
    assert np.all(np.diff(sel) > 0), "selection must be strictly ascending (unique)"
    ref_sel = oracle.select_topk(ref_scores, n)
    tau = np.min(ref_scores[ref_sel])
    band = np.abs(ref_scores - tau) <= BAND * abs(tau)
    gs = set(sel.tolist())
    rs = set(ref_sel.tolist())
    outside_g = {s for s in gs if not band[s]}
    outside_r = {s for s in rs if not band[s]}
    assert outside_g == outside_r, (
        f"selection differs outside the tie band: gpu-only {sorted(outside_g - outside_r)[:8]} "
        f"ref-only {sorted(outside_r - outside_g)[:8]}")
    return int(band.sum())


def attn_errors(gpu_o: np.ndarray, ref_o: np.ndarray):
    d = np.abs(np.asarray(gpu_o, dtype=np.float64) - ref_o)
    return float(d.max()), float(d.mean())


def check_attention(gpu_o: np.ndarray, ref_o: np.ndarray):
    mx, mean = attn_errors(gpu_o, ref_o)
    assert np.all(np.isfinite(gpu_o)), "non-finite attention output"
    assert mx <= ATTN_MAX_ABS and mean <= ATTN_MEAN_ABS, (mx, mean)
    return mx, mean


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------- C4 projections

def proj_error_bound(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """C4 bound [R, P] on |fp32 projection - exact| for h [R, d], W [P, d]."""
    d = h.shape[1]
    return 16.0 * math.sqrt(d) * U32 * np.sqrt((h * h) @ (W * W).T)


def check_quantised(codes_g: np.ndarray, scale_g: np.ndarray, y: np.ndarray,
                    err: np.ndarray) -> float:
    """C4 for e4m3fn vectors along the last axis; returns the fraction of codes
    whose allowed range holds more than one code."""
    codes_g = np.asarray(codes_g)
    scale_g = np.asarray(scale_g, dtype=np.float64)
    amax_lo = np.max(np.maximum(np.abs(y) - err, 0.0), axis=-1)
    amax_hi = np.max(np.abs(y) + err, axis=-1)
    s_lo, s_hi = oracle.pow2_scale(amax_lo), oracle.pow2_scale(amax_hi)
    m, _ = np.frexp(scale_g)
    ok_s = (m == 0.5) & (scale_g >= s_lo) & (scale_g <= s_hi)
    assert ok_s.all(), (f"scale outside the allowed powers of two at {np.argwhere(~ok_s)[:4]}: "
                        f"gpu {scale_g[~ok_s][:4]} allowed [{s_lo[~ok_s][:4]}, {s_hi[~ok_s][:4]}]")
    s = scale_g[..., None]
    lo = np.clip((y - err) / s, -448.0, 448.0)
    hi = np.clip((y + err) / s, -448.0, 448.0)
    v_lo = oracle.decode_e4m3fn(oracle.encode_e4m3fn(lo))
    v_hi = oracle.decode_e4m3fn(oracle.encode_e4m3fn(hi))
    v_g = oracle.decode_e4m3fn(codes_g)
    ok = (v_g >= v_lo) & (v_g <= v_hi)
    assert np.all(~np.isnan(v_g)), "NaN code"
    assert ok.all(), (f"fp8 code outside its allowed range at {np.argwhere(~ok)[:4]}: gpu "
                      f"{v_g[~ok][:4]} allowed [{v_lo[~ok][:4]}, {v_hi[~ok][:4]}]")
    return float(np.mean(v_lo != v_hi))


def check_bf16_words(bits_g: np.ndarray, y: np.ndarray, err: np.ndarray) -> float:
    """C4 for bf16 outputs; returns the fraction with more than one allowed word."""
    v_g = oracle.decode_bf16(bits_g)
    v_lo = oracle.decode_bf16(oracle.encode_bf16(y - err))
    v_hi = oracle.decode_bf16(oracle.encode_bf16(y + err))
    ok = (v_g >= v_lo) & (v_g <= v_hi)
    assert ok.all(), (f"bf16 word outside its allowed range at {np.argwhere(~ok)[:4]}: gpu "
                      f"{v_g[~ok][:4]} allowed [{v_lo[~ok][:4]}, {v_hi[~ok][:4]}]")
    return float(np.mean(v_lo != v_hi))


def check_fp32_within(g: np.ndarray, y: np.ndarray, err: np.ndarray) -> float:
    """C4 for fp32 outputs; returns the worst |g - y| / err."""
    d = np.abs(np.asarray(g, dtype=np.float64) - y)
    ok = d <= err
    assert ok.all(), f"fp32 output off by more than the bound at {np.argwhere(~ok)[:4]}"
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(err > 0, d / err, 0.0)
    return float(ratio.max()) if ratio.size else 0.0


def proj_reference(h_bits: np.ndarray, weights_bits: Sequence[np.ndarray], n_idx_heads: int):
    """Oracle projections of the tokens in h_bits and their C4 bounds."""
    wq, wk, wc, ww = weights_bits
    ref = oracle.project_tokens(h_bits, wq, wk, wc, ww, n_idx_heads)
    h = oracle.decode_bf16(h_bits)
    R = h.shape[0]
    ref["err_q"] = proj_error_bound(h, oracle.decode_bf16(wq)).reshape(R, n_idx_heads, -1)
    ref["err_k"] = proj_error_bound(h, oracle.decode_bf16(wk))
    ref["err_c"] = proj_error_bound(h, oracle.decode_bf16(wc))
    ref["err_w"] = proj_error_bound(h, oracle.decode_bf16(ww))
    return ref
