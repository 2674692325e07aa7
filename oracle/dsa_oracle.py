"""Float64 CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares no code with
the HIP library and imports nothing from it.

What it computes, and where the definition comes from
------------------------------------------------------
Sources are the web pages on DeepSeek-V3.2-Exp.  "V3.2-Exp paper" below means the
full Chinese translation of the DeepSeek-V3.2-Exp paper carried on the page
"重磅！DeepSeek-V3.2-Exp 发布百万输出仅3元｜附完整论文中文翻译" (m.163.com); on that
page every equation was an image and is lost, so each step follows the paper's
prose around the lost equation.  "nsmao report" means the page
"DeepSeek-V3.2开源技术报告" (nsmao.com).

1. Indexer score (V3.2-Exp paper, §1 Architecture, "DSA prototype", Eq. 1):
   I[t,s] = sum_{j < H_I} w[t,j] * ReLU(q[t,j] . k[s]); q[t,j] and w[t,j] come from
   the query token, k[s] from a preceding token; ReLU is the activation; few heads;
   FP8 arithmetic is allowed.  Reading: no extra constant factor; "preceding" is
   inclusive, s <= t (0-indexed positions).
2. Fine-grained selection (V3.2-Exp paper, §1, text after Eq. 1, and §2.1 "sparse
   training stage"): S_t = the positions of the top-k indexer scores, k = 2048.
   Reading: exactly n = min(k, t+1) positions, equal scores broken toward the lower
   position.
3. Sparse attention (V3.2-Exp paper, §1, Eq. 2): u_t = Attn(h_t, {c_s | s in S_t}).
   Instantiated under MLA in MQA mode (§1 "Instantiate DSA under MLA"; App. A,
   Fig. 4): every selected latent entry c_s is shared by all query heads; the key is
   the whole entry (latent + rope part) and the value is its latent part (the first
   D_v columns).  Reading: plain softmax attention with a given softmax scale, no
   bias, no sink.  The nsmao report ("DSA principle") gives the cache widths: 128 per
   token for the indexer key, 512 for the latent.

4. Query and key projections with cache append (nsmao report, "DSA principle": the
   workflow's first step projects the query and the keys before indexer scoring;
   V3.2-Exp paper, §1: q[t,j] and w[t,j] are derived from the query token h_t and
   k[s] from the token h_s).  Reading: plain linear maps of h without bias or
   normalisation, stored in the formats the later steps read: the indexer query
   per (token, head) and the indexer key per token as e4m3fn codes with a
   power-of-two fp32 scale, the head weights as fp32, and the latent entry as
   bf16 (round to nearest even).  RoPE is not applied.

5. Paged ("dynamic") caches (nsmao report, "DSA principle": the serving path uses
   a dynamic KV cache).  Reading: the per-sequence caches are views of a shared
   pool of fixed-size pages through a block table: entry s of sequence b is entry
   s mod P of pool page block_table[b][s div P].  Every step computes exactly what
   it computes on the contiguous cache those views describe.

6. Indexer training loss (V3.2-Exp paper, §2.1, dense warm-up and sparse training
   stages): the main attention scores of query token t are summed over all heads
   and L1-normalised along the sequence into the target p[t,:]; the indexer is
   trained with KL(p[t,:] || Softmax(I[t,:])), in the sparse stage over the
   selected set S_t only; the indexer's inputs are detached, so the loss trains the
   indexer alone.  Reading: the "attention scores" are each head's softmax weights
   over the attended positions; gradients flow into I (p is a constant target) and
   from I into the indexer queries, weights and keys.

7. Masked MHA mode (V3.2-Exp paper, §3 "inference cost": short-sequence prefill
   runs a masked MHA mode that simulates DSA; Appendix A, Fig. 4: MLA's MHA mode,
   used for training and prefill, and its MQA mode, used for decoding).  Reading:
   each head decompresses its own key k[h,s] = [W_UK[h] c[s,:512]; c[s,512:]] and
   value v[h,s] = W_UV[h] c[s,:512] from the shared latent entry, and attends over
   the positions the indexer selected (a mask on the causal positions).  With the
   absorbed query [W_UK[h]^T q_nope[h]; q_rope[h]] the MQA mode gives the same
   weights, and W_UV[h] times its latent-space output is the MHA output.

Inputs are the exact byte images the GPU receives: e4m3fn codes with fp32 scales
(dequantised value = decode(code) * scale), bf16 bit patterns, or plain fp32.  The
oracle decodes them with its own decoders and computes every step in float64.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = [
    "decode_e4m3fn", "decode_bf16", "indexer_scores", "select_topk",
    "sparse_attention", "indexer_row", "attention_row", "dsa_row",
    "encode_e4m3fn", "encode_bf16", "pow2_scale", "quantize_e4m3fn", "project",
    "project_tokens", "append_rows", "paged_view", "paged_append", "attention_target",
    "indexer_kl", "indexer_backward", "mha_decompress", "mha_attention",
]


# ---------------------------------------------------------------------------
# O0: storage decoders
# ---------------------------------------------------------------------------

def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": finite, NaN at S.1111.111, no infinities).

    Bit layout s eeee mmm, exponent bias 7:
      e > 0: (-1)^s * 2^(e-7) * (1 + m/8)
      e = 0: (-1)^s * 2^(-6) * (m/8)           (subnormals)
      e = 15 and m = 7: NaN.
    (The pages name only "FP8"; the e4m3fn flavour is the reading adopted.)
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(e > 0, normal, subnormal)
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the bf16 word is the top half of
    an IEEE binary32 word."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# O1-O3: the three steps, on dequantised float64 operands
# ---------------------------------------------------------------------------

def indexer_scores(q: np.ndarray, w: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Lightning-indexer scores of one query token against a set of keys.

    q: [H_I, d_I] indexer queries q[t,j]; w: [H_I] head weights w[t,j];
    k: [n, d_I] indexer keys k[s].  Returns I[s] = sum_j w[j] * max(0, q[j].k[s]).
    (V3.2-Exp paper, §1, Eq. 1 prose.)
    """
    dots = q @ k.T                       # [H_I, n]: q[t,j] . k[s]
    return w @ np.maximum(dots, 0.0)     # ReLU, then the w-weighted head sum


def select_topk(scores: np.ndarray, n: int) -> np.ndarray:
    """Positions of the n largest scores, equal scores toward the lower position,
    returned in ascending position order.  (V3.2-Exp paper, §1 selection of the
    top-k key-value entries; §2.1 S_t definition and k = 2048.)"""
    scores = np.asarray(scores, dtype=np.float64)
    pos = np.arange(scores.shape[0])
    order = np.lexsort((pos, -scores))   # primary key -I ascending, then s ascending
    return np.sort(order[:n])


def sparse_attention(q: np.ndarray, entries: np.ndarray, scale: float,
                     v_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """MQA-mode attention of one query token over its selected latent entries.

    q: [H, D_k] per-head absorbed queries; entries: [n, D_k] the selected latent
    entries c_s (keys are whole entries, values their first v_dim columns).
    Returns (o [H, v_dim], lse [H]) with
      z[h,s] = scale * q[h].c_s,  o[h] = sum_s softmax_s(z[h,:]) c_s[:v_dim],
      lse[h] = log sum_s exp(z[h,s]).
    (V3.2-Exp paper, §1 Eq. 2 prose and "Instantiate DSA under MLA"; App. A.)
    """
    z = scale * (q @ entries.T)                  # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    Z = e.sum(axis=1, keepdims=True)
    o = (e / Z) @ entries[:, :v_dim]
    lse = m[:, 0] + np.log(Z[:, 0])
    return o, lse


# ---------------------------------------------------------------------------
# row drivers on raw input images
# ---------------------------------------------------------------------------

def _dequant(x: np.ndarray, scale: Optional[np.ndarray], fp8: bool) -> np.ndarray:
    v = decode_e4m3fn(x) if fp8 else np.asarray(x, dtype=np.float64)
    if scale is not None:
        v = v * np.asarray(scale, dtype=np.float64)[..., None]
    return v


def indexer_row(q_idx: np.ndarray, q_scale: Optional[np.ndarray], w: np.ndarray,
                k_idx: np.ndarray, k_scale: Optional[np.ndarray], t: int,
                fp8: bool) -> np.ndarray:
    """Scores I[0..t] of one query row at position t.

    q_idx: [H_I, d_I] (e4m3fn codes if fp8 else fp32), q_scale: [H_I] or None;
    w: [H_I]; k_idx: [>= t+1, d_I] the sequence's indexer keys, k_scale: [>= t+1]
    or None.  Only keys s <= t are candidates.
    """
    qf = _dequant(q_idx, q_scale, fp8)
    kf = _dequant(k_idx[: t + 1], None if k_scale is None else k_scale[: t + 1], fp8)
    return indexer_scores(qf, np.asarray(w, dtype=np.float64), kf)


def _decode_attn(x: np.ndarray, bf16: bool) -> np.ndarray:
    return decode_bf16(x) if bf16 else np.asarray(x, dtype=np.float64)


def attention_row(q: np.ndarray, entries: np.ndarray, scale: float, v_dim: int,
                  bf16: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for one row; q: [H, D_k], entries: [n, D_k] (bf16 bits or fp32)."""
    return sparse_attention(_decode_attn(q, bf16), _decode_attn(entries, bf16),
                            scale, v_dim)


def dsa_row(q_idx, q_scale, w, k_idx, k_scale, q, latent, t: int, topk: int,
            scale: float, v_dim: int, quantised: bool):
    """The whole path for one row at position t: scores, selected set, output.

    latent: [>= t+1, D_k] the sequence's latent cache.  Returns
    (scores [t+1], S ascending [min(topk, t+1)], o [H, v_dim], lse [H]).
    """
    I = indexer_row(q_idx, q_scale, w, k_idx, k_scale, t, quantised)
    S = select_topk(I, min(topk, t + 1))
    o, lse = attention_row(q, latent[S], scale, v_dim, quantised)
    return I, S, o, lse


# ---------------------------------------------------------------------------
# O5: projections of new tokens, storage encoders, cache append
# ---------------------------------------------------------------------------

E4M3FN_MAX = 448.0


def _e4m3fn_magnitudes() -> np.ndarray:
    """The 127 finite non-negative e4m3fn values, indexed by their code 0x00..0x7E."""
    return decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code of each value in [-448, 448] (float64 in, uint8 out).

    The magnitude is matched against the table of representable values; a value
    exactly halfway between two neighbours takes the code with the even mantissa
    (round to nearest even).  The sign bit copies the sign of x, so -0.0 -> 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3FN_MAX) or np.any(np.isnan(x)):
        raise ValueError("encode_e4m3fn expects finite values within [-448, 448]")
    table = _e4m3fn_magnitudes()
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, table.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = table[hi] - a
    d_lo = a - table[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0) & (lo != hi))
    code = np.where(take_lo, lo, hi).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), rounded once to nearest even.

    bf16 keeps 8 significant bits: x = m * 2^e with 0.5 <= |m| < 1 is rounded to a
    multiple of 2^(e-8) (2^-133 below the normal range).  The rounding is done
    directly from float64, with no intermediate float32 rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / quantum) * quantum      # x / quantum is exact (a power of two)
    bits = r.astype(np.float32).view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def pow2_scale(amax: np.ndarray) -> np.ndarray:
    """Power-of-two quantisation scale: 2^e with e the smallest integer such that
    amax <= 448 * 2^e; 1 where amax == 0.  The first guess from log2 is corrected
    with exact comparisons (448 * 2^e is exact in float64)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, E4M3FN_MAX)
    e = np.ceil(np.log2(safe / E4M3FN_MAX)).astype(np.int64)
    e = np.where(np.ldexp(E4M3FN_MAX, e) < safe, e + 1, e)
    e = np.where(np.ldexp(E4M3FN_MAX, e - 1) >= safe, e - 1, e)
    return np.where(amax > 0, np.ldexp(1.0, e), 1.0)


def quantize_e4m3fn(y: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise each vector along the last axis: (codes uint8, scale float64).
    scale = pow2_scale(max |y|), code = encode_e4m3fn(y / scale), so that
    decode(code) * scale approximates y."""
    y = np.asarray(y, dtype=np.float64)
    s = pow2_scale(np.abs(y).max(axis=-1))
    v = np.clip(y / s[..., None], -E4M3FN_MAX, E4M3FN_MAX)
    return encode_e4m3fn(v), s


def project(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Linear projection of tokens: h [R, d], W [P, d] (one output per row of W)
    -> y [R, P] with y[r, p] = sum_k W[p, k] h[r, k]."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def project_tokens(h_bits: np.ndarray, wq_bits: np.ndarray, wk_bits: np.ndarray,
                   wc_bits: np.ndarray, ww_bits: np.ndarray, n_idx_heads: int) -> dict:
    """Projections of R new tokens and their stored forms.

    h_bits [R, d] and the weights are bf16 bit patterns: wq [H_I*d_I, d] (head j =
    rows j*d_I .. j*d_I+d_I-1), wk [d_I, d], wc [D_k, d], ww [H_I, d].
    Returns the exact projections (y_q [R,H_I,d_I], y_k [R,d_I], y_c [R,D_k],
    y_w [R,H_I]) and the stored forms: q_codes/q_scale (per token and head),
    k_codes/k_scale (per token), latent_bits (bf16), w (float64).
    """
    h = decode_bf16(h_bits)
    R = h.shape[0]
    y_q = project(h, decode_bf16(wq_bits)).reshape(R, n_idx_heads, -1)
    y_k = project(h, decode_bf16(wk_bits))
    y_c = project(h, decode_bf16(wc_bits))
    y_w = project(h, decode_bf16(ww_bits))
    q_codes, q_scale = quantize_e4m3fn(y_q)
    k_codes, k_scale = quantize_e4m3fn(y_k)
    return dict(y_q=y_q, y_k=y_k, y_c=y_c, y_w=y_w, q_codes=q_codes, q_scale=q_scale,
                k_codes=k_codes, k_scale=k_scale, latent_bits=encode_bf16(y_c), w=y_w)


def append_rows(cache: np.ndarray, row_seq: np.ndarray, row_pos: np.ndarray,
                values: np.ndarray) -> np.ndarray:
    """Copy of a per-sequence cache [B, N, ...] with values[r] stored at
    (row_seq[r], row_pos[r]); rows whose sequence or position is out of range are
    skipped."""
    out = np.array(cache, copy=True)
    B, N = out.shape[0], out.shape[1]
    for r, (b, t) in enumerate(zip(np.asarray(row_seq), np.asarray(row_pos))):
        if 0 <= b < B and 0 <= t < N:
            out[b, t] = values[r]
    return out


# ---------------------------------------------------------------------------
# O6: paged caches
# ---------------------------------------------------------------------------

def paged_view(pool: np.ndarray, block_table: np.ndarray, page_size: int) -> np.ndarray:
    """The per-sequence caches a page pool describes.

    pool [num_pages, P, ...]; block_table [B, pages_per_seq] (pool page of each
    logical page).  Returns cache [B, pages_per_seq * P, ...] with
    cache[b, s] = pool[block_table[b, s // P], s % P].
    """
    pool = np.asarray(pool)
    table = np.asarray(block_table)
    if pool.shape[1] != page_size:
        raise ValueError("pool pages must hold page_size entries")
    B, pps = table.shape
    return pool[table].reshape((B, pps * page_size) + pool.shape[2:])


def paged_append(pool: np.ndarray, block_table: np.ndarray, page_size: int,
                 row_seq: np.ndarray, row_pos: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Copy of the pool with values[r] stored at logical entry (row_seq[r],
    row_pos[r]); rows outside [0, B) x [0, pages_per_seq * P) are skipped."""
    out = np.array(pool, copy=True)
    table = np.asarray(block_table)
    B, pps = table.shape
    for r, (b, t) in enumerate(zip(np.asarray(row_seq), np.asarray(row_pos))):
        if 0 <= b < B and 0 <= t < pps * page_size:
            out[table[b, t // page_size], t % page_size] = values[r]
    return out


# ---------------------------------------------------------------------------
# O7: indexer training loss and its gradients
# ---------------------------------------------------------------------------

def attention_target(q: np.ndarray, entries: np.ndarray, scale: float) -> np.ndarray:
    """Target distribution over the attended entries of one query token: each
    head's softmax weights over the entries, summed over the heads, then divided by
    their total (L1 normalisation along the sequence).  q [H, D_k], entries [n, D_k]."""
    z = scale * (np.asarray(q, dtype=np.float64) @ np.asarray(entries, dtype=np.float64).T)
    a = np.exp(z - z.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)          # per-head attention weights
    agg = a.sum(axis=0)                        # summed over heads
    return agg / agg.sum()


def indexer_kl(p: np.ndarray, scores: np.ndarray) -> Tuple[float, np.ndarray]:
    """KL(p || softmax(scores)) over one row's entries and its gradient with respect
    to the scores (p is a constant target).  Terms with p = 0 contribute 0."""
    p = np.asarray(p, dtype=np.float64)
    I = np.asarray(scores, dtype=np.float64)
    m = I.max()
    lse = m + np.log(np.exp(I - m).sum())
    logq = I - lse
    pos = p > 0
    loss = float(np.sum(p[pos] * (np.log(p[pos]) - logq[pos])))
    grad = np.exp(logq) * p.sum() - p
    return loss, grad


def indexer_backward(q: np.ndarray, w: np.ndarray, k: np.ndarray,
                     g: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of sum_s g[s] * I[s] with I[s] = sum_j w[j] ReLU(q[j] . k[s]):
    (dq [H_I, d_I], dw [H_I], dk [n, d_I]).  The ReLU's derivative is taken as 0 at
    0 (the kink)."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    dots = q @ k.T                             # [H_I, n]
    dw = np.maximum(dots, 0.0) @ g
    coef = (w[:, None] * (dots > 0)) * g[None, :]
    return coef @ k, dw, coef.T @ q


# ---------------------------------------------------------------------------
# O8: masked MHA mode
# ---------------------------------------------------------------------------

def mha_decompress(entries: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                   v_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-head keys and values of latent entries [n, D_k] (first v_dim columns
    latent, the rest rope): k [H, n, dh + D_k - v_dim] = [W_UK[h] c; c_rope] and
    v [H, n, dv] = W_UV[h] c, with w_uk [H, dh, v_dim], w_uv [H, dv, v_dim]."""
    c = np.asarray(entries, dtype=np.float64)
    lat, rope = c[:, :v_dim], c[:, v_dim:]
    k_nope = np.einsum("hdc,nc->hnd", np.asarray(w_uk, dtype=np.float64), lat)
    v = np.einsum("hdc,nc->hnd", np.asarray(w_uv, dtype=np.float64), lat)
    H = k_nope.shape[0]
    k = np.concatenate([k_nope, np.broadcast_to(rope, (H,) + rope.shape)], axis=2)
    return k, v


def mha_attention(q: np.ndarray, entries: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                  scale: float, v_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """MHA-mode attention of one query token over its selected latent entries:
    q [H, dh + rope] (per-head nope and rope parts); returns (o [H, dv], lse [H])
    with z[h,s] = scale q[h] . k[h,s] and o[h] = sum_s softmax_s(z[h]) v[h,s]."""
    k, v = mha_decompress(entries, w_uk, w_uv, v_dim)
    q = np.asarray(q, dtype=np.float64)
    z = scale * np.einsum("hd,hnd->hn", q, k)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    Z = e.sum(axis=1, keepdims=True)
    o = np.einsum("hn,hnd->hd", e / Z, v)
    return o, m[:, 0] + np.log(Z[:, 0])
