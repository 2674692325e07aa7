"""Pins of the float64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
hand-worked example, a published table, a library routine, a brute-force
enumeration, a closed form or an invariant.  ``test_oracle.py`` runs them as
they are; ``test_oracle_mutations.py`` plants plausible mistakes in the oracle
and checks that at least one pin fails for each.

All pins call the oracle through the module attribute ``oracle.dsa_oracle.X`` so
that a planted mistake is seen by every pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle.dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- P1 decoders

def pin_e4m3fn_golden():
    """Published OFP8 E4M3 values (tests/golden/e4m3fn_codes.txt)."""
    with open(os.path.join(GOLDEN, "e4m3fn_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code_s, val_s = line.split()
            code = int(code_s, 16)
            got = O.decode_e4m3fn(np.array([code], dtype=np.uint8))[0]
            if val_s == "nan":
                assert np.isnan(got), (hex(code), got)
            else:
                want = float(val_s)
                assert got == want and math.copysign(1, got) == math.copysign(1, want), \
                    (hex(code), got, want)


def pin_e4m3fn_library():
    """All 256 codes against torch's float8_e4m3fn decode (a library routine)."""
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(lib)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.all((ours == lib) | both_nan)
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(lib[~both_nan]))
    # strictly increasing over the non-negative finite codes
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert pos.max() == 448.0 and ours[1] == 2.0 ** -9


def pin_bf16():
    """bf16 decode: closed-form words and torch's bfloat16 (library routine)."""
    words = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x4049], dtype=np.uint16)
    got = O.decode_bf16(words)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0, 3.140625]
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w), (g, w)
    r = _rng(1).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    r = r[(r & 0x7F80) != 0x7F80]  # drop inf / nan words
    lib = torch.from_numpy(r.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.decode_bf16(r), lib)


# ---------------------------------------------------------------- P2 indexer

def pin_indexer_hand_example():
    """Hand-worked example (tests/golden/indexer_hand_example.json), float and fp8."""
    with open(os.path.join(GOLDEN, "indexer_hand_example.json")) as f:
        ex = json.load(f)
    got = O.indexer_scores(np.array(ex["q"]), np.array(ex["w"]), np.array(ex["k"]))
    assert np.array_equal(got, np.array(ex["expected"])), got
    f8 = ex["fp8_case"]
    k_codes = np.array(f8["k_codes"], dtype=np.uint8)
    got8 = O.indexer_row(np.array(f8["q_codes"], dtype=np.uint8), np.array(f8["q_scale"]),
                         np.array(ex["w"]), k_codes, np.array(f8["k_scale"]),
                         t=len(k_codes) - 1, fp8=True)
    assert np.array_equal(got8, np.array(f8["expected"])), got8


def _brute_indexer(q, w, k):
    H, d = q.shape
    out = []
    for s in range(k.shape[0]):
        acc = 0.0
        for j in range(H):
            dot = 0.0
            for i in range(d):
                dot += float(q[j, i]) * float(k[s, i])
            acc += float(w[j]) * (dot if dot > 0.0 else 0.0)
        out.append(acc)
    return np.array(out)


def pin_indexer_bruteforce():
    """Pure-Python loops on small non-square shapes (catches transposed operands)."""
    r = _rng(2)
    for H, d, n in [(3, 5, 7), (1, 4, 9), (4, 32, 11), (2, 1, 3)]:
        q = r.standard_normal((H, d))
        w = r.standard_normal(H)
        k = r.standard_normal((n, d))
        got = O.indexer_scores(q, w, k)
        assert got.shape == (n,)
        np.testing.assert_allclose(got, _brute_indexer(q, w, k), rtol=1e-12, atol=1e-12)


def pin_indexer_invariants():
    r = _rng(3)
    H, d, n = 6, 16, 40
    q = r.standard_normal((H, d))
    w = r.standard_normal(H)
    k = r.standard_normal((n, d))
    base = O.indexer_scores(q, w, k)
    # a permutation of the heads (with their weights) leaves I unchanged
    p = r.permutation(H)
    np.testing.assert_allclose(O.indexer_scores(q[p], w[p], k), base, rtol=1e-12, atol=1e-12)
    # I is linear in w
    np.testing.assert_allclose(O.indexer_scores(q, 2.5 * w, k), 2.5 * base, rtol=1e-12, atol=1e-12)
    # every q.k <= 0 gives exactly zero scores (ReLU)
    kneg = -np.abs(k)
    assert np.all(O.indexer_scores(np.abs(q), np.abs(w) + 0.1, kneg) == 0.0)
    # H_I = 1, w = 1 reduces to ReLU of a single dot product
    one = O.indexer_scores(q[:1], np.ones(1), k)
    np.testing.assert_allclose(one, np.maximum(k @ q[0], 0.0), rtol=1e-12, atol=1e-12)


def pin_indexer_row_causal_and_scales():
    """indexer_row: exactly t+1 candidates (s <= t); trading a positive constant
    between the q and k scales leaves I unchanged; keys after t do not matter."""
    r = _rng(4)
    H, d, L = 4, 8, 12
    q_codes = r.integers(0, 0x7E, size=(H, d), dtype=np.uint8) ^ (r.integers(0, 2, size=(H, d), dtype=np.uint8) << 7)
    k_codes = r.integers(0, 0x7E, size=(L, d), dtype=np.uint8) ^ (r.integers(0, 2, size=(L, d), dtype=np.uint8) << 7)
    qs = np.exp2(r.integers(-8, 2, size=H)).astype(np.float64)
    ks = np.exp2(r.integers(-8, 2, size=L)).astype(np.float64)
    w = r.standard_normal(H)
    for t in [0, 1, 5, L - 1]:
        I = O.indexer_row(q_codes, qs, w, k_codes, ks, t, fp8=True)
        assert I.shape == (t + 1,)
        k2 = k_codes.copy()
        k2[t + 1:] = 0x7E
        np.testing.assert_array_equal(O.indexer_row(q_codes, qs, w, k2, ks, t, True), I)
        I2 = O.indexer_row(q_codes, qs * 4.0, w, k_codes, ks / 4.0, t, True)
        np.testing.assert_allclose(I2, I, rtol=1e-12, atol=1e-300)
        # dequantised brute force
        qf = O.decode_e4m3fn(q_codes) * qs[:, None]
        kf = O.decode_e4m3fn(k_codes[: t + 1]) * ks[: t + 1, None]
        np.testing.assert_allclose(I, _brute_indexer(qf, w, kf), rtol=1e-12, atol=1e-300)
    # t = 0 scores the query's own position only
    I0 = O.indexer_row(q_codes, qs, w, k_codes, ks, 0, True)
    qf = O.decode_e4m3fn(q_codes) * qs[:, None]
    kf0 = O.decode_e4m3fn(k_codes[0]) * ks[0]
    assert np.isclose(I0[0], float(np.sum(w * np.maximum(qf @ kf0, 0.0))), rtol=1e-12)


# ---------------------------------------------------------------- P3 top-k

def _brute_topk(I, n):
    return sorted(sorted(range(len(I)), key=lambda s: (-I[s], s))[:n])


def pin_topk_bruteforce():
    r = _rng(5)
    for L, n in [(1, 1), (5, 3), (17, 17), (40, 7), (64, 64), (100, 10)]:
        for kind in ("normal", "dupes", "negative"):
            if kind == "normal":
                I = r.standard_normal(L)
            elif kind == "dupes":
                I = r.integers(-2, 3, size=L).astype(np.float64)
            else:
                I = -np.abs(r.standard_normal(L)) - 1.0
            got = O.select_topk(I, n)
            assert list(got) == _brute_topk(I, n), (L, n, kind)


def pin_topk_special_rows():
    # all-zero row (every ReLU zero): the n lowest positions
    assert list(O.select_topk(np.zeros(50), 8)) == list(range(8))
    # exact tie straddling the cut: the lower position wins
    I = np.array([5.0, 1.0, 3.0, 2.0, 3.0, 0.5])
    assert list(O.select_topk(I, 2)) == [0, 2]
    # only m < n positive scores: those, then the lowest-position zeros
    I = np.zeros(20)
    I[[7, 13, 19]] = [1.0, 2.0, 3.0]
    assert list(O.select_topk(I, 6)) == [0, 1, 2, 7, 13, 19]
    # n >= L selects everything
    assert list(O.select_topk(np.array([3.0, -1.0, 2.0]), 3)) == [0, 1, 2]
    # -0.0 and +0.0 are equal scores
    I = np.array([0.0, -0.0, 1.0, -0.0, 0.0])
    assert list(O.select_topk(I, 3)) == [0, 1, 2]


# ---------------------------------------------------------------- P4 attention

def pin_attention_hand_example():
    with open(os.path.join(GOLDEN, "attention_hand_example.json")) as f:
        ex = json.load(f)
    o, lse = O.sparse_attention(np.array(ex["q"]), np.array(ex["entries"]), ex["scale"],
                                ex["v_dim"])
    assert o.shape == (2, ex["v_dim"])
    np.testing.assert_allclose(o[0], ex["expected_o_head0"], rtol=1e-13)
    np.testing.assert_allclose(o[1], ex["expected_o_head1"], rtol=1e-13)
    np.testing.assert_allclose(lse, [ex["expected_lse_head0"], ex["expected_lse_head1"]],
                               rtol=1e-13)


def pin_attention_dense_equivalence():
    """Rows with t+1 <= k select every prior position, so the path must equal dense
    causal MQA attention; the dense side is torch's scaled_dot_product_attention
    in float64 (a library routine) with a causal mask."""
    r = _rng(6)
    H, Dk, Dv, L, k = 3, 10, 6, 9, 16
    q = r.standard_normal((L, H, Dk))
    c = r.standard_normal((L, Dk))
    scale = 0.37
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()          # [H, L, Dk]
    kt = torch.from_numpy(c).unsqueeze(0).expand(H, L, Dk).contiguous()
    vt = torch.from_numpy(c[:, :Dv]).unsqueeze(0).expand(H, L, Dv).contiguous()
    dense = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=scale).permute(1, 0, 2).numpy()  # [L, H, Dv]
    for t in range(L):
        S = O.select_topk(np.zeros(t + 1), min(k, t + 1))
        assert list(S) == list(range(t + 1))
        o, lse = O.sparse_attention(q[t], c[S], scale, Dv)
        np.testing.assert_allclose(o, dense[t], rtol=1e-12, atol=1e-12)
        z = scale * (q[t] @ c[: t + 1].T)
        from scipy.special import logsumexp
        np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-12, atol=1e-12)


def pin_attention_closed_forms():
    r = _rng(7)
    H, Dk, Dv = 4, 12, 8
    q = r.standard_normal((H, Dk))
    c = r.standard_normal((5, Dk))
    # single entry: o is that entry's value part, lse = scale * q.c
    o, lse = O.sparse_attention(q, c[:1], 0.3, Dv)
    assert np.array_equal(o, np.broadcast_to(c[0, :Dv], (H, Dv)))
    np.testing.assert_allclose(lse, 0.3 * (q @ c[0]), rtol=1e-14)
    # identical entries: o equals the entry
    same = np.repeat(c[2:3], 7, axis=0)
    o, lse = O.sparse_attention(q, same, 0.3, Dv)
    np.testing.assert_allclose(o, np.broadcast_to(c[2, :Dv], (H, Dv)), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, 0.3 * (q @ c[2]) + np.log(7.0), rtol=1e-13)
    # scale 0: plain mean of the values, lse = log n
    o, lse = O.sparse_attention(q, c, 0.0, Dv)
    np.testing.assert_allclose(o, np.broadcast_to(c[:, :Dv].mean(0), (H, Dv)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(5.0), rtol=1e-14)
    # convex combination: every output coordinate lies within the values' range
    o, _ = O.sparse_attention(q * 3, c, 1.0, Dv)
    lo, hi = c[:, :Dv].min(0), c[:, :Dv].max(0)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    # order of the selected entries does not matter
    p = r.permutation(5)
    o1, l1 = O.sparse_attention(q, c, 0.7, Dv)
    o2, l2 = O.sparse_attention(q, c[p], 0.7, Dv)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def pin_attention_bruteforce():
    """Softmax attention by explicit loops with math.exp on a tiny case."""
    r = _rng(8)
    H, Dk, Dv, n = 2, 3, 2, 4
    q = r.standard_normal((H, Dk))
    c = r.standard_normal((n, Dk))
    o, lse = O.sparse_attention(q, c, 0.9, Dv)
    for h in range(H):
        z = [0.9 * sum(q[h, i] * c[s, i] for i in range(Dk)) for s in range(n)]
        den = sum(math.exp(v) for v in z)
        for d in range(Dv):
            num = sum(math.exp(z[s]) * c[s, d] for s in range(n))
            assert abs(o[h, d] - num / den) < 1e-12
        assert abs(lse[h] - math.log(den)) < 1e-12


# ---------------------------------------------------------------- P5 composition

def pin_dsa_row_composition():
    """dsa_row = indexer -> top-k -> attention; with k >= t+1 the output is dense
    causal attention; with k < t+1 it is attention over the brute-force top-k."""
    r = _rng(9)
    H_I, d_I, H, Dk, Dv, L = 2, 4, 3, 6, 4, 12
    q_idx = r.standard_normal((L, H_I, d_I)).astype(np.float32)
    w = r.random((L, H_I)).astype(np.float32)
    k_idx = r.standard_normal((L, d_I)).astype(np.float32)
    q = r.standard_normal((L, H, Dk)).astype(np.float32)
    lat = r.standard_normal((L, Dk)).astype(np.float32)
    for t in range(L):
        for k in (L, 5):
            I, S, o, lse = O.dsa_row(q_idx[t], None, w[t], k_idx, None, q[t], lat, t, k,
                                     0.5, Dv, quantised=False)
            Ib = _brute_indexer(q_idx[t].astype(np.float64), w[t].astype(np.float64),
                                k_idx[: t + 1].astype(np.float64))
            np.testing.assert_allclose(I, Ib, rtol=1e-12, atol=1e-12)
            Sb = _brute_topk(list(Ib), min(k, t + 1))
            assert list(S) == Sb
            zz = 0.5 * (q[t].astype(np.float64) @ lat[Sb].astype(np.float64).T)
            ww = np.exp(zz - zz.max(1, keepdims=True))
            ww /= ww.sum(1, keepdims=True)
            np.testing.assert_allclose(o, ww @ lat[Sb, :Dv].astype(np.float64), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P6 projections
# Storage encoders, the power-of-two quantiser, the projections and the cache
# append of new tokens.

def _exact_e4m3fn_code(v: Fraction) -> int:
    """Brute force: nearest e4m3fn value to the exact rational v (|v| <= 448), ties
    to the even code, by scanning every finite code."""
    best = None
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        mag = Fraction(8 + m, 8) * Fraction(2) ** (e - 7) if e else Fraction(m, 8) * Fraction(2) ** -6
        d = abs(abs(v) - mag)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if v < 0 else 0)


def _exact_bf16_bits(v: Fraction) -> int:
    """Brute force: bf16 word nearest to the exact rational v (normal range), ties
    to the even mantissa."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128                      # 8 significant bits: integer part of a * 2^7
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    m = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else 0)
    if m == 256:
        m, e = 128, e + 1
    return sign | ((e + 127) << 7) | (m - 128)


def pin_encode_e4m3fn_roundtrip_and_ties():
    """Every finite code round-trips; a value halfway between two neighbours takes
    the even code; values off the midpoint take the nearer code; signs mirror."""
    codes = np.arange(256, dtype=np.uint8)
    vals = O.decode_e4m3fn(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(O.encode_e4m3fn(vals[fin]), codes[fin])
    pos = vals[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(O.encode_e4m3fn(mid), even.astype(np.uint8))
    assert np.array_equal(O.encode_e4m3fn(-mid), (even | 0x80).astype(np.uint8))
    gap = pos[1:] - pos[:-1]
    assert np.array_equal(O.encode_e4m3fn(mid - gap / 8), np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(O.encode_e4m3fn(mid + gap / 8), np.arange(1, 0x7F, dtype=np.uint8))


def pin_encode_e4m3fn_library():
    """Random float32 values in [-448, 448], normal and subnormal range, against
    torch's float8_e4m3fn cast (a library routine, round to nearest even)."""
    r = _rng(21)
    x = np.concatenate([r.uniform(-448, 448, 20000), r.uniform(-2 ** -5, 2 ** -5, 20000),
                        r.standard_normal(20000) * 8]).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3fn(x.astype(np.float64)), lib)


def pin_encode_bf16():
    """bf16 rounding: torch's bfloat16 cast of float32 values (library routine),
    hand-worked midpoints, and one rounding straight from float64 (a value that a
    float32 intermediate would turn into a tie)."""
    r = _rng(22)
    x = (r.standard_normal(50000) * np.exp2(r.integers(-60, 60, 50000))).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.encode_bf16(x.astype(np.float64)), lib)
    cases = [(1.0 + 2.0 ** -8, 0x3F80),             # tie -> even mantissa 0
             (1.0 + 3 * 2.0 ** -8, 0x3F82),         # tie -> even mantissa 2
             (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie
             (-(1.0 + 2.0 ** -8 - 2.0 ** -40), 0xBF80),
             (3.0, 0x4040), (-0.0, 0x8000), (0.0, 0x0000)]
    got = O.encode_bf16(np.array([c[0] for c in cases]))
    assert [int(g) for g in got] == [c[1] for c in cases], [hex(int(g)) for g in got]


def pin_pow2_scale():
    """scale = 2^e with the smallest integer e such that amax <= 448 * 2^e, found by
    an exhaustive search over e; amax = 0 gives 1."""
    r = _rng(23)
    amax = np.concatenate([np.exp2(r.uniform(-30, 30, 500)),
                           448.0 * np.exp2(np.arange(-20, 21, dtype=np.float64)),
                           np.nextafter(448.0 * np.exp2(np.arange(-20, 21, dtype=np.float64)), np.inf),
                           np.nextafter(448.0 * np.exp2(np.arange(-20, 21, dtype=np.float64)), 0)])
    got = O.pow2_scale(amax)
    for a, g in zip(amax, got):
        e = next(e for e in range(-80, 80) if a <= 448.0 * 2.0 ** e)
        assert g == 2.0 ** e, (a, g, 2.0 ** e)
    assert O.pow2_scale(np.array([0.0]))[0] == 1.0


def pin_quantize_e4m3fn():
    """Per-vector quantisation: codes equal torch's float8 cast of y / scale (exact
    for float32 y and a power-of-two scale); the largest magnitude lands in
    (224, 448]; reconstruction error within half a code spacing; a zero vector
    gives scale 1 and zero codes; each vector gets its own scale."""
    r = _rng(24)
    y = (r.standard_normal((40, 128)) * np.exp2(r.integers(-8, 8, (40, 1)))).astype(np.float32)
    y[3] = 0.0
    codes, s = O.quantize_e4m3fn(y.astype(np.float64))
    assert codes.shape == y.shape and s.shape == (40,)
    assert s[3] == 1.0 and not codes[3].any()
    ys = (y.astype(np.float64) / s[:, None]).astype(np.float32)
    lib = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, lib)
    dec = O.decode_e4m3fn(codes) * s[:, None]
    nz = np.arange(40) != 3
    top = np.abs(O.decode_e4m3fn(codes[nz])).max(axis=1)
    assert np.all((top > 224) & (top <= 448))
    err = np.abs(dec - y)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * s[:, None])
    assert np.all(err <= bound + 1e-300)


def pin_project_bruteforce():
    """y[r, p] = sum_k W[p, k] h[r, k] against pure-Python loops on a tiny case."""
    r = _rng(25)
    h = r.standard_normal((3, 7))
    W = r.standard_normal((5, 7))
    got = O.project(h, W)
    for i in range(3):
        for p in range(5):
            want = math.fsum(W[p, k] * h[i, k] for k in range(7))
            assert abs(got[i, p] - want) <= 1e-12 * (1 + abs(want))


def pin_project_tokens_exact():
    """project_tokens on tiny bf16 inputs against exact rational arithmetic: each
    projection summed as a Fraction, then rounded to bf16 or quantised with a
    brute-force code scan; heads are consecutive row blocks of w_q."""
    r = _rng(26)
    H_I, d_I, Dk, d, R = 2, 4, 3, 6, 2

    def bf(shape, scale):
        x = (r.standard_normal(shape) * scale).astype(np.float32)
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    h, wq, wk, wc, ww = bf((R, d), 1), bf((H_I * d_I, d), 0.4), bf((d_I, d), 0.4), \
        bf((Dk, d), 0.4), bf((H_I, d), 0.4)
    out = O.project_tokens(h, wq, wk, wc, ww, H_I)

    def frac(bits):
        return [Fraction(float(v)) for v in
                (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)]

    hF = [frac(h[i]) for i in range(R)]

    def dot(i, wrow):
        wF = frac(wrow)
        return sum(a * b for a, b in zip(hF[i], wF))

    def quant(vec):
        amax = max(abs(v) for v in vec)
        if amax == 0:
            return [0] * len(vec), Fraction(1)
        e = next(e for e in range(-60, 60) if amax <= 448 * Fraction(2) ** e)
        s = Fraction(2) ** e
        return [_exact_e4m3fn_code(v / s) for v in vec], s

    for i in range(R):
        for j in range(H_I):
            vec = [dot(i, wq[j * d_I + c]) for c in range(d_I)]
            codes, s = quant(vec)
            assert list(out["q_codes"][i, j]) == codes and out["q_scale"][i, j] == s
            for c in range(d_I):
                assert abs(out["y_q"][i, j, c] - float(vec[c])) <= 1e-12
        vec = [dot(i, wk[c]) for c in range(d_I)]
        codes, s = quant(vec)
        assert list(out["k_codes"][i]) == codes and out["k_scale"][i] == s
        for c in range(Dk):
            assert int(out["latent_bits"][i, c]) == _exact_bf16_bits(dot(i, wc[c]))
        for j in range(H_I):
            assert abs(out["w"][i, j] - float(dot(i, ww[j]))) <= 1e-12


def pin_append_rows():
    """Cache append: exactly the rows named by (seq, pos) change, each to its own
    token's values; out-of-range rows are skipped."""
    cache = np.arange(3 * 5 * 2, dtype=np.int64).reshape(3, 5, 2)
    vals = -np.arange(1, 9, dtype=np.int64).reshape(4, 2)
    seq = np.array([0, 2, 5, 1])
    pos = np.array([4, 0, 1, -1])
    out = O.append_rows(cache, seq, pos, vals)
    want = cache.copy()
    want[0, 4] = vals[0]
    want[2, 0] = vals[1]
    assert np.array_equal(out, want)
    assert np.array_equal(cache, np.arange(30).reshape(3, 5, 2))  # input untouched


# ---------------------------------------------------------------- P7 paged caches

def pin_paged_view_bruteforce():
    """paged_view against a loop over every (sequence, entry), for a shuffled block
    table; the identity table is a plain reshape of the pool."""
    r = _rng(31)
    P, B, pps = 4, 3, 5
    pool = r.integers(0, 1000, size=(B * pps + 2, P, 3))
    table = r.permutation(B * pps + 2)[: B * pps].reshape(B, pps)
    got = O.paged_view(pool, table, P)
    assert got.shape == (B, pps * P, 3)
    for b in range(B):
        for s in range(pps * P):
            assert np.array_equal(got[b, s], pool[table[b, s // P], s % P])
    ident = np.arange(B * pps).reshape(B, pps)
    assert np.array_equal(O.paged_view(pool[: B * pps], ident, P),
                          pool[: B * pps].reshape(B, pps * P, 3))


def pin_paged_invariants():
    """Moving pages around the pool with the table updated to match leaves every
    sequence's cache unchanged; the paged append writes exactly the entry its
    logical cache would get (compared with append_rows on the view)."""
    r = _rng(32)
    P, B, pps, npg = 8, 2, 3, 9
    pool = r.standard_normal((npg, P, 4))
    table = r.choice(npg, size=(B, pps), replace=False)
    view = O.paged_view(pool, table, P)
    perm = r.permutation(npg)            # page i moves to slot perm[i]
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    assert np.array_equal(O.paged_view(pool2, perm[table], P), view)
    seq = np.array([0, 1, 1, 2, 0])
    pos = np.array([3, 23, 9, 0, 24])     # (2, 0) and (0, 24) are out of range
    vals = r.standard_normal((5, 4))
    got = O.paged_view(O.paged_append(pool, table, P, seq, pos, vals), table, P)
    assert np.array_equal(got, O.append_rows(view, seq, pos, vals))


# ---------------------------------------------------------------- P8 indexer training loss

def pin_attention_target():
    """Target distribution: a pure-Python loop over heads and entries (per-head
    softmax, sum over heads, L1 normalisation); one head gives that head's softmax;
    identical entries give the uniform distribution."""
    r = _rng(41)
    H, n, D = 3, 5, 4
    q = r.standard_normal((H, D)) * np.array([[0.5], [2.0], [4.0]])
    e = r.standard_normal((n, D))
    got = O.attention_target(q, e, 0.7)
    agg = [0.0] * n
    for h in range(H):
        z = [0.7 * math.fsum(q[h, d] * e[s, d] for d in range(D)) for s in range(n)]
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        tot = math.fsum(ex)
        for s in range(n):
            agg[s] += ex[s] / tot
    want = np.array(agg) / math.fsum(agg)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)
    z0 = 0.7 * (q[1] @ e.T)
    np.testing.assert_allclose(O.attention_target(q[1:2], e, 0.7), np.exp(z0) / np.exp(z0).sum(),
                               rtol=1e-12)
    np.testing.assert_allclose(O.attention_target(q, np.tile(e[:1], (n, 1)), 0.7),
                               np.full(n, 1.0 / n), rtol=1e-12)


def pin_indexer_kl():
    """KL(p || softmax(I)): the hand-worked case p = (1, 0), I = (0, 0) gives log 2
    and gradient (-1/2, 1/2); p = softmax(I) gives 0; adding a constant to I changes
    nothing; the loss is non-negative; the gradient equals central differences."""
    loss, g = O.indexer_kl(np.array([1.0, 0.0]), np.array([0.0, 0.0]))
    assert abs(loss - math.log(2.0)) < 1e-15 and np.allclose(g, [-0.5, 0.5], atol=1e-15)
    r = _rng(42)
    I = r.standard_normal(7) * 3
    sm = np.exp(I - I.max())
    sm /= sm.sum()
    l0, g0 = O.indexer_kl(sm, I)
    assert abs(l0) < 1e-14 and np.abs(g0).max() < 1e-14
    p = r.random(7)
    p[2] = 0.0
    p /= p.sum()
    loss, g = O.indexer_kl(p, I)
    loss2, g2 = O.indexer_kl(p, I + 5.0)
    assert loss > 0 and abs(loss - loss2) < 1e-12 and np.allclose(g, g2, atol=1e-12)
    h = 1e-6
    for s in range(7):
        e = np.zeros(7)
        e[s] = h
        fd = (O.indexer_kl(p, I + e)[0] - O.indexer_kl(p, I - e)[0]) / (2 * h)
        assert abs(fd - g[s]) < 1e-7, (s, fd, g[s])


def pin_indexer_backward():
    """Gradients of sum_s g[s] I[s] against central differences of the oracle's own
    forward indexer_scores, away from the ReLU kinks."""
    r = _rng(43)
    H_I, d_I, n = 3, 5, 6
    q = r.standard_normal((H_I, d_I))
    w = r.standard_normal(H_I)
    k = r.standard_normal((n, d_I))
    assert np.abs(q @ k.T).min() > 1e-3
    g = r.standard_normal(n)
    dq, dw, dk = O.indexer_backward(q, w, k, g)
    F = lambda q_, w_, k_: float(g @ O.indexer_scores(q_, w_, k_))
    h = 1e-6
    for (arr, grad, name) in ((q, dq, "q"), (w, dw, "w"), (k, dk, "k")):
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1 = {"q": (a1, w, k), "w": (q, a1, k), "k": (q, w, a1)}[name]
            args2 = {"q": (a2, w, k), "w": (q, a2, k), "k": (q, w, a2)}[name]
            fd = (F(*args1) - F(*args2)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * (1 + abs(fd)), (name, idx, fd, grad[idx])


# ---------------------------------------------------------------- P9 masked MHA mode

def pin_mha_matches_mqa_absorbed():
    """MHA mode equals MQA mode with the absorbed query: sparse_attention with
    q_mqa[h] = [W_UK[h]^T q_nope[h]; q_rope[h]] gives the same lse, and W_UV[h] times
    its latent-space output is the MHA output (App. A, Fig. 4)."""
    r = _rng(51)
    H, dh, dv, lat, rope, n = 3, 4, 5, 6, 2, 7
    w_uk = r.standard_normal((H, dh, lat))
    w_uv = r.standard_normal((H, dv, lat))
    ent = r.standard_normal((n, lat + rope))
    q = r.standard_normal((H, dh + rope))
    o, lse = O.mha_attention(q, ent, w_uk, w_uv, 0.4, lat)
    q_mqa = np.concatenate([np.einsum("hdc,hd->hc", w_uk, q[:, :dh]), q[:, dh:]], axis=1)
    o_lat, lse_mqa = O.sparse_attention(q_mqa, ent, 0.4, lat)
    np.testing.assert_allclose(lse, lse_mqa, rtol=1e-12)
    np.testing.assert_allclose(o, np.einsum("hdc,hc->hd", w_uv, o_lat), rtol=1e-11, atol=1e-12)


def pin_mha_decompress_bruteforce():
    """Decompressed keys and values against loops over heads, entries and dims."""
    r = _rng(52)
    H, dh, dv, lat, rope, n = 2, 3, 2, 4, 2, 3
    w_uk = r.standard_normal((H, dh, lat))
    w_uv = r.standard_normal((H, dv, lat))
    ent = r.standard_normal((n, lat + rope))
    k, v = O.mha_decompress(ent, w_uk, w_uv, lat)
    for h in range(H):
        for s in range(n):
            for d in range(dh):
                assert abs(k[h, s, d] - math.fsum(w_uk[h, d, c] * ent[s, c] for c in range(lat))) < 1e-12
            for d in range(rope):
                assert k[h, s, dh + d] == ent[s, lat + d]
            for d in range(dv):
                assert abs(v[h, s, d] - math.fsum(w_uv[h, d, c] * ent[s, c] for c in range(lat))) < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
