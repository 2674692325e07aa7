"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them: a pin suite that passes a broken oracle pins nothing."""
import numpy as np
import pytest

import oracle.dsa_oracle as O
import oracle_pins

_orig = {name: getattr(O, name) for name in
         ["indexer_scores", "select_topk", "sparse_attention", "decode_e4m3fn",
          "decode_bf16", "indexer_row", "encode_e4m3fn", "encode_bf16", "pow2_scale",
         "quantize_e4m3fn", "project", "project_tokens", "paged_view", "paged_append",
         "attention_target", "indexer_kl", "indexer_backward", "mha_decompress"]}


def _no_relu(q, w, k):
    return w @ (q @ k.T)


def _relu_after_sum(q, w, k):
    return np.maximum(w @ (q @ k.T), 0.0)


def _w_per_key(q, w, k):
    return np.maximum(q @ k.T, 0.0).sum(0) * w.mean()


def _scaled_by_sqrt_d(q, w, k):
    return _orig["indexer_scores"](q, w, k) / np.sqrt(q.shape[1])


def _ties_high(scores, n):
    scores = np.asarray(scores, dtype=np.float64)
    pos = np.arange(scores.shape[0])
    order = np.lexsort((-pos, -scores))
    return np.sort(order[:n])


def _smallest(scores, n):
    return np.sort(np.argsort(scores, kind="stable")[:n])


def _unstable(scores, n):
    return np.sort(np.argsort(-np.asarray(scores), kind="quicksort")[:n][::-1])


def _value_last_cols(q, e, scale, v_dim):
    z = scale * (q @ e.T)
    m = z.max(1, keepdims=True)
    p = np.exp(z - m)
    Z = p.sum(1, keepdims=True)
    return (p / Z) @ e[:, -v_dim:], m[:, 0] + np.log(Z[:, 0])


def _no_scale(q, e, scale, v_dim):
    return _orig["sparse_attention"](q, e, 1.0, v_dim)


def _lse_no_max(q, e, scale, v_dim):
    o, lse = _orig["sparse_attention"](q, e, scale, v_dim)
    z = scale * (q @ e.T)
    return o, lse - z.max(1)


def _no_softmax_norm(q, e, scale, v_dim):
    z = scale * (q @ e.T)
    p = np.exp(z - z.max(1, keepdims=True))
    return p @ e[:, :v_dim], np.log(p.sum(1)) + z.max(1)


def _fnuz_bias(codes):
    return _orig["decode_e4m3fn"](codes) / 2.0


def _no_subnormals(codes):
    v = _orig["decode_e4m3fn"](codes)
    c = np.asarray(codes).astype(np.int64)
    return np.where(((c >> 3) & 0xF) == 0, 0.0 * v, v)


def _bf16_low_half(bits):
    b = np.asarray(bits).astype(np.uint32)
    return (b | (b << 16)).view(np.float32).astype(np.float64)


def _exclusive_causal(q_idx, q_scale, w, k_idx, k_scale, t, fp8):
    full = _orig["indexer_row"](q_idx, q_scale, w, k_idx, k_scale, t, fp8)
    return full[:t] if t > 0 else full


def _scale_ignored(q_idx, q_scale, w, k_idx, k_scale, t, fp8):
    return _orig["indexer_row"](q_idx, None, w, k_idx, None, t, fp8)


def _e4m3_ties_away(x):
    # round half away from zero instead of to even
    x = np.asarray(x, dtype=np.float64)
    table = O.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(x)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    code = np.where(a - table[lo] < table[hi] - a, lo, hi).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


def _bf16_truncate(x):
    b = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)
    return b.astype(np.uint16)


def _bf16_via_f32(x):
    # double rounding: float64 -> float32 -> bf16
    return _orig["encode_bf16"](np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64))


def _scale_amax_over_448(amax):
    amax = np.asarray(amax, dtype=np.float64)
    return np.where(amax > 0, amax / 448.0, 1.0)


def _scale_one_too_big(amax):
    return _orig["pow2_scale"](amax) * 2.0


def _scale_per_tensor(y):
    y = np.asarray(y, dtype=np.float64)
    s = O.pow2_scale(np.abs(y).max())
    return O.encode_e4m3fn(np.clip(y / s, -448, 448)), np.full(y.shape[:-1], s)


def _project_drops_last(h, W):
    return np.asarray(h, dtype=np.float64)[:, :-1] @ np.asarray(W, dtype=np.float64)[:, :-1].T


def _heads_interleaved(h_bits, wq_bits, wk_bits, wc_bits, ww_bits, n_idx_heads):
    out = _orig["project_tokens"](h_bits, wq_bits, wk_bits, wc_bits, ww_bits, n_idx_heads)
    R = out["y_q"].shape[0]
    y_q = out["y_q"].reshape(R, -1).reshape(R, -1, n_idx_heads).transpose(0, 2, 1)
    out["q_codes"], out["q_scale"] = O.quantize_e4m3fn(y_q)
    out["y_q"] = y_q
    return out


def _paged_table_transposed(pool, block_table, page_size):
    # entries taken page-major across sequences (table read in the wrong order)
    t = np.asarray(block_table)
    return _orig["paged_view"](pool, t.T.reshape(t.shape), page_size)


def _paged_offset_swapped(pool, block_table, page_size):
    pool = np.asarray(pool)
    v = pool[np.asarray(block_table)]             # [B, pps, P, ...]
    return np.swapaxes(v, 1, 2).reshape((v.shape[0], -1) + pool.shape[2:])


def _paged_append_logical_index(pool, block_table, page_size, row_seq, row_pos, values):
    # writes pool page s // P directly, ignoring the table
    out = np.array(pool, copy=True)
    for r, (b, t) in enumerate(zip(row_seq, row_pos)):
        if 0 <= b < np.asarray(block_table).shape[0] and 0 <= t < np.asarray(block_table).shape[1] * page_size:
            out[t // page_size, t % page_size] = values[r]
    return out


def _target_unnormalised_heads(q, entries, scale):
    # exp of the scores summed over heads without the per-head softmax
    z = scale * (np.asarray(q, dtype=np.float64) @ np.asarray(entries, dtype=np.float64).T)
    a = np.exp(z - z.max()).sum(axis=0)
    return a / a.sum()


def _kl_reversed(p, scores):
    # KL(softmax(I) || p) instead of KL(p || softmax(I))
    I = np.asarray(scores, dtype=np.float64)
    qd = np.exp(I - I.max())
    qd /= qd.sum()
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        loss = float(np.sum(qd * (np.log(qd) - np.log(np.maximum(p, 1e-300)))))
    return loss, _orig["indexer_kl"](p, scores)[1]


def _kl_grad_sign(p, scores):
    loss, g = _orig["indexer_kl"](p, scores)
    return loss, -g


def _bwd_no_relu_in_dw(q, w, k, g):
    dq, dw, dk = _orig["indexer_backward"](q, w, k, g)
    return dq, (np.asarray(q) @ np.asarray(k).T) @ np.asarray(g), dk


def _bwd_dq_without_w(q, w, k, g):
    return _orig["indexer_backward"](q, np.ones_like(np.asarray(w)), k, g)[0], \
        _orig["indexer_backward"](q, w, k, g)[1], _orig["indexer_backward"](q, w, k, g)[2]


def _mha_rope_dropped(entries, w_uk, w_uv, v_dim):
    k, v = _orig["mha_decompress"](entries, w_uk, w_uv, v_dim)
    k = k.copy()
    k[:, :, w_uk.shape[1]:] = 0.0
    return k, v


def _mha_value_uses_uk(entries, w_uk, w_uv, v_dim):
    k, _ = _orig["mha_decompress"](entries, w_uk, w_uv, v_dim)
    _, v = _orig["mha_decompress"](entries, w_uv, w_uk, v_dim)
    return k, v


MUTANTS = [
    ("indexer_scores", _no_relu),
    ("indexer_scores", _relu_after_sum),
    ("indexer_scores", _w_per_key),
    ("indexer_scores", _scaled_by_sqrt_d),
    ("select_topk", _ties_high),
    ("select_topk", _smallest),
    ("select_topk", _unstable),
    ("sparse_attention", _value_last_cols),
    ("sparse_attention", _no_scale),
    ("sparse_attention", _lse_no_max),
    ("sparse_attention", _no_softmax_norm),
    ("decode_e4m3fn", _fnuz_bias),
    ("decode_e4m3fn", _no_subnormals),
    ("decode_bf16", _bf16_low_half),
    ("indexer_row", _exclusive_causal),
    ("indexer_row", _scale_ignored),
    ("encode_e4m3fn", _e4m3_ties_away),
    ("encode_bf16", _bf16_truncate),
    ("encode_bf16", _bf16_via_f32),
    ("pow2_scale", _scale_amax_over_448),
    ("pow2_scale", _scale_one_too_big),
    ("quantize_e4m3fn", _scale_per_tensor),
    ("project", _project_drops_last),
    ("project_tokens", _heads_interleaved),
    ("paged_view", _paged_table_transposed),
    ("paged_view", _paged_offset_swapped),
    ("paged_append", _paged_append_logical_index),
    ("attention_target", _target_unnormalised_heads),
    ("indexer_kl", _kl_reversed),
    ("indexer_kl", _kl_grad_sign),
    ("indexer_backward", _bwd_no_relu_in_dw),
    ("indexer_backward", _bwd_dq_without_w),
    ("mha_decompress", _mha_rope_dropped),
    ("mha_decompress", _mha_value_uses_uk),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda x: getattr(x, "__name__", x))
def test_pins_catch_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:  # AssertionError or a shape error both count as caught
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mutant.__name__} in {name}"
