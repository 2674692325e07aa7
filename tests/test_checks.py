"""The projection comparison rule (C4) on the CPU: it accepts what a correct
fp32-accumulating implementation stores and rejects plausible mistakes."""
import numpy as np
import pytest
import torch

import dsa_inputs as di
import oracle
from dsa_check import (check_bf16_words, check_fp32_within, check_quantised,
                       proj_reference)


def _bits(t):
    return di.bf16_bits(t)


@pytest.fixture(scope="module")
def case():
    d = 7168
    g = di.ProjGenerator(6, d)
    h = g.h(0, 32)
    wq, wk, wc, ww = (g.weight(t) for t in (di.T_WQ, di.T_WK, di.T_WC, di.T_WW))
    ref = proj_reference(_bits(h), [_bits(w) for w in (wq, wk, wc, ww)], 64)
    # an fp32 implementation: float32 matmul of the bf16 operands (another order)
    y32 = {k: (h.float() @ w.float().T).double().numpy() for k, w in
           (("q", wq), ("k", wk), ("c", wc), ("w", ww))}
    return ref, y32


def _quantise_f32(y):
    """Quantise float32 values with the oracle's encoder (scale from fp32 amax)."""
    s = oracle.pow2_scale(np.abs(y).max(axis=-1))
    return oracle.encode_e4m3fn(np.clip(y / s[..., None], -448, 448)), s


def test_fp32_projection_within_bound(case):
    ref, y32 = case
    r = check_fp32_within(y32["w"], ref["y_w"], ref["err_w"])
    assert r < 0.25, r   # the bound holds with room to spare
    r = check_fp32_within(y32["q"], ref["y_q"].reshape(32, -1), ref["err_q"].reshape(32, -1))
    assert r < 0.25, r


def test_accepts_fp32_quantisation(case):
    ref, y32 = case
    codes, s = _quantise_f32(y32["q"].reshape(32, 64, 128))
    amb = check_quantised(codes, s, ref["y_q"], ref["err_q"])
    assert amb < 0.03, amb
    kc, ks = _quantise_f32(y32["k"])
    check_quantised(kc, ks, ref["y_k"], ref["err_k"])
    amb = check_bf16_words(oracle.encode_bf16(y32["c"]), ref["y_c"], ref["err_c"])
    assert amb < 0.15, amb


def test_rejects_wrong_codes_scales_and_words(case):
    ref, y32 = case
    codes, s = _quantise_f32(y32["q"].reshape(32, 64, 128))
    bad = codes.copy()
    i = np.unravel_index(np.argmax(np.abs(ref["y_q"])), codes.shape)
    bad[i] = bad[i] - 1          # one code step toward zero on the largest element
    with pytest.raises(AssertionError):
        check_quantised(bad, s, ref["y_q"], ref["err_q"])
    with pytest.raises(AssertionError):
        check_quantised(codes, s * 2, ref["y_q"], ref["err_q"])
    words = oracle.encode_bf16(y32["c"])
    with pytest.raises(AssertionError):
        check_bf16_words(words ^ np.uint16(1), ref["y_c"], ref["err_c"])
    with pytest.raises(AssertionError):
        check_fp32_within(y32["w"] * (1 + 1e-3), ref["y_w"], ref["err_w"])
