"""Seeded synthetic inputs for the DeepSeek Sparse Attention (DSA) hot path.

This module is shared by the CPU oracle side and the GPU side.  It draws random
numbers and stores them in the input formats the path consumes (fp8 e4m3fn codes
with per-vector fp32 scales, bf16, fp32).  It performs none of the method's own
arithmetic: no indexer score, no selection, no attention.

Generator
---------
Every element is a pure function of (stream key, flat element index):

    h = lowbias32(lowbias32(key ^ (i >> 32)) ^ (i & 0xffffffff))

where lowbias32 is the 32-bit integer mixer published by C. Wellons
("Prospecting for Hash Functions", 2018; constants 0x7feb352d, 0x846ca68b,
shifts 16/15/16).  From h:

* normal:  N(0,1) by inverse CDF on a 2^16-entry table of midpoint quantiles,
           ``ndtri((j + 0.5) / 2^16)`` stored as float32, indexed by ``h >> 16``.
           Only integer ops and a table lookup run per element, so the values are
           bit-identical on the host and on the GPU.
* uniform: U[0,1) as ``(h >> 8) * 2^-24`` (exact in float32).

Because values depend only on the flat index, the oracle side can regenerate any
subset (one sequence's keys, a few query rows) without materialising the rest,
while the GPU side generates multi-GB tensors directly in device memory.

Storage formats
---------------
* fp8: OCP e4m3fn codes with one power-of-two fp32 scale per 128-wide (d_I) vector:
  scale = 2^e for the smallest integer e with amax <= 448 * 2^e (amax = 0 gives
  scale 1); code = RNE_e4m3fn(x / scale).  The division is by a power of two and
  therefore exact; the only rounding is the fp8 cast.
* bf16: round-to-nearest-even cast of the float32 draw.

The workloads (shapes and distributions) are listed in ``CONFIGS``; the
projection workloads (hidden states and projection weights of new tokens) in
``PROJ_CONFIGS``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

_M32 = 0xFFFFFFFF
_TABLE_BITS = 16

# ---------------------------------------------------------------------------
# integer mixer (int64 tensors holding values in [0, 2^32); no int64 overflow)
# ---------------------------------------------------------------------------


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for 0 <= x < 2^32, computed without int64 overflow."""
    lo = x * (c & 0xFFFF)                       # < 2^48
    hi = torch.bitwise_and(x * (c >> 16), 0xFFFF)  # < 2^48 before the mask
    return torch.bitwise_and(lo + torch.bitwise_left_shift(hi, 16), _M32)


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = torch.bitwise_xor(x, torch.bitwise_right_shift(x, 16))
    x = _mul32(x, 0x7FEB352D)
    x = torch.bitwise_xor(x, torch.bitwise_right_shift(x, 15))
    x = _mul32(x, 0x846CA68B)
    x = torch.bitwise_xor(x, torch.bitwise_right_shift(x, 16))
    return x


def _lowbias32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def stream_key(*ids: int) -> int:
    """Fold a tuple of small non-negative ids into a 32-bit stream key."""
    k = 0x2545F491
    for v in ids:
        k = _lowbias32_int(k ^ _lowbias32_int(int(v) + 0x9E3779B9))
    return k


def bits32(key: int, idx: torch.Tensor) -> torch.Tensor:
    """32 random bits (as int64 in [0, 2^32)) for each flat index in ``idx``."""
    idx = idx.to(torch.int64)
    hi = torch.bitwise_right_shift(idx, 32)
    lo = torch.bitwise_and(idx, _M32)
    h = _lowbias32(torch.bitwise_xor(hi, key))
    return _lowbias32(torch.bitwise_xor(h, lo))


_TABLES: Dict[str, torch.Tensor] = {}


def normal_table(device: torch.device | str = "cpu") -> torch.Tensor:
    """2^16 equiprobable N(0,1) midpoint quantiles, float32."""
    dev = str(torch.device(device))
    t = _TABLES.get(dev)
    if t is None:
        from scipy.special import ndtri

        n = 1 << _TABLE_BITS
        q = ndtri((np.arange(n, dtype=np.float64) + 0.5) / n).astype(np.float32)
        t = torch.from_numpy(q).to(device)
        _TABLES[dev] = t
    return t


def normal(key: int, idx: torch.Tensor) -> torch.Tensor:
    h = bits32(key, idx)
    tab = normal_table(idx.device)
    return tab[torch.bitwise_right_shift(h, 32 - _TABLE_BITS)]


def uniform(key: int, idx: torch.Tensor) -> torch.Tensor:
    h = bits32(key, idx)
    return torch.bitwise_right_shift(h, 8).to(torch.float32) * (2.0 ** -24)


def _flat(start: int, count: int, device) -> torch.Tensor:
    return torch.arange(start, start + count, dtype=torch.int64, device=device)


# ---------------------------------------------------------------------------
# storage casts
# ---------------------------------------------------------------------------

FP8_MAX = 448.0


def pow2_scale_exponent(amax: torch.Tensor) -> torch.Tensor:
    """Smallest integer e with amax <= 448 * 2^e (0 where amax == 0), int32."""
    m, E = torch.frexp(amax)            # amax = m * 2^E, m in [0.5, 1)
    e = E - 9 + (m > 0.875).to(E.dtype)  # 448 = 0.875 * 2^9
    return torch.where(amax > 0, e, torch.zeros_like(e)).to(torch.int32)


def _exp2_int(e: torch.Tensor) -> torch.Tensor:
    """2^e as float32 built from its bit pattern (exact, normal range only)."""
    return torch.bitwise_left_shift((e.to(torch.int32) + 127), 23).view(torch.float32)


def quantize_fp8(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-last-dim-vector power-of-two scaled e4m3fn quantisation.

    Returns (codes uint8 same shape as x, scales float32 x.shape[:-1]).
    """
    x = x.to(torch.float32)
    e = pow2_scale_exponent(x.abs().amax(dim=-1))
    xs = x * _exp2_int(-e).unsqueeze(-1)      # exact: multiply by 2^-e
    codes = xs.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, _exp2_int(e)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    num_seqs: int          # B
    max_ctx: int           # N: per-sequence cache capacity
    q_len: int             # query rows per sequence
    kv_len: int            # cache length per sequence; row i sits at kv_len - q_len + i
    chunk_rows: int        # rows per internal chunk of dsa_forward (0 = all rows at once)
    n_idx_heads: int       # H_I
    idx_dim: int           # d_I
    n_heads: int           # H
    qk_dim: int            # D_k  (latent + rope)
    v_dim: int             # D_v  (latent)
    topk: int              # k
    scale: float           # softmax scale
    fp32: bool             # True: all inputs fp32 (no fp8 / bf16 storage)
    w_uniform: bool        # True: w ~ U(0,1); else w ~ N(0,1)/8
    description: str = ""

    @property
    def num_rows(self) -> int:
        return self.num_seqs * self.q_len

    def row_seq_pos(self) -> Tuple[np.ndarray, np.ndarray]:
        seq = np.repeat(np.arange(self.num_seqs, dtype=np.int32), self.q_len)
        pos = np.tile(np.arange(self.kv_len - self.q_len, self.kv_len, dtype=np.int32),
                      self.num_seqs)
        return seq, pos


CONFIGS: Dict[str, Config] = {
    c.name: c
    for c in [
        Config("tiny", 1, 1, 256, 256, 256, 256, 4, 32, 16, 80, 64, 64,
               1.0 / math.sqrt(80.0), True, True,
               "tiny causal prefill, fp32 throughout"),
        Config("decode32k", 2, 32, 32768, 1, 32768, 0, 64, 128, 128, 576, 512, 2048,
               1.0 / math.sqrt(192.0), False, False,
               "decode, batch 32, one query each at context 32768"),
        Config("prefill8k", 3, 1, 8192, 8192, 8192, 8192, 64, 128, 128, 576, 512, 2048,
               1.0 / math.sqrt(192.0), False, False,
               "causal prefill of one 8192-token sequence"),
        Config("decode128k", 4, 8, 131072, 1, 131072, 0, 64, 128, 128, 576, 512, 2048,
               1.0 / math.sqrt(192.0), False, False,
               "decode, batch 8, one query each at context 131072"),
        Config("prefill128k", 5, 1, 131072, 131072, 131072, 8192, 64, 128, 128, 576, 512,
               2048, 1.0 / math.sqrt(192.0), False, False,
               "causal prefill of one 131072-token sequence in 8192-row chunks"),
        Config("prefill2k", 8, 4, 2048, 2048, 2048, 8192, 64, 128, 128, 576, 512, 2048,
               1.0 / math.sqrt(192.0), False, False,
               "short causal prefill, 4 sequences of 2048 tokens (every causal set fits in k)"),
    ]
}

# tensor ids inside a config's key space
T_QIDX, T_W, T_KIDX, T_Q, T_LATENT = 1, 2, 3, 4, 5


class Generator:
    """Deterministic tensor factory for one (config, input set)."""

    def __init__(self, cfg: Config, set_id: int = 0):
        self.cfg = cfg
        self.set_id = set_id

    def key(self, tensor_id: int) -> int:
        return stream_key(self.cfg.cfg_id, self.set_id, tensor_id)

    # -- query-side tensors: global row index r in [0, num_rows) -------------
    def q_idx(self, r0: int, r1: int, device="cpu"):
        """Indexer queries of rows [r0, r1): (codes or fp32 [n,H_I,d_I], scales [n,H_I])."""
        c = self.cfg
        per = c.n_idx_heads * c.idx_dim
        x = normal(self.key(T_QIDX), _flat(r0 * per, (r1 - r0) * per, device))
        x = x.view(r1 - r0, c.n_idx_heads, c.idx_dim)
        if c.fp32:
            return x, torch.ones(r1 - r0, c.n_idx_heads, dtype=torch.float32, device=device)
        return quantize_fp8(x)

    def w(self, r0: int, r1: int, device="cpu") -> torch.Tensor:
        c = self.cfg
        per = c.n_idx_heads
        idx = _flat(r0 * per, (r1 - r0) * per, device)
        if c.w_uniform:
            v = uniform(self.key(T_W), idx)
        else:
            v = normal(self.key(T_W), idx) * 0.125
        return v.view(r1 - r0, c.n_idx_heads)

    def q(self, r0: int, r1: int, device="cpu") -> torch.Tensor:
        c = self.cfg
        per = c.n_heads * c.qk_dim
        x = normal(self.key(T_Q), _flat(r0 * per, (r1 - r0) * per, device))
        x = x.view(r1 - r0, c.n_heads, c.qk_dim)
        return x if c.fp32 else to_bf16(x)

    # -- cache-side tensors: sequence b, positions [p0, p1) -------------------
    def k_idx(self, b: int, p0: int, p1: int, device="cpu"):
        c = self.cfg
        per = c.idx_dim
        base = (b * c.max_ctx + p0) * per
        x = normal(self.key(T_KIDX), _flat(base, (p1 - p0) * per, device)).view(p1 - p0, per)
        if c.fp32:
            return x, torch.ones(p1 - p0, dtype=torch.float32, device=device)
        return quantize_fp8(x)

    def latent(self, b: int, p0: int, p1: int, device="cpu") -> torch.Tensor:
        c = self.cfg
        per = c.qk_dim
        base = (b * c.max_ctx + p0) * per
        x = normal(self.key(T_LATENT), _flat(base, (p1 - p0) * per, device)).view(p1 - p0, per)
        return x if c.fp32 else to_bf16(x)

    def latent_rows(self, b: int, positions: torch.Tensor) -> torch.Tensor:
        """Latent rows of sequence b at arbitrary positions (host)."""
        c = self.cfg
        pos = positions.to(torch.int64).view(-1, 1)
        idx = (b * c.max_ctx + pos) * c.qk_dim + torch.arange(c.qk_dim, dtype=torch.int64)
        x = normal(self.key(T_LATENT), idx.view(-1)).view(-1, c.qk_dim)
        return x if c.fp32 else to_bf16(x)


# ---------------------------------------------------------------------------
# whole-tensor materialisation (host or device), chunked to bound temporaries
# ---------------------------------------------------------------------------

_CHUNK_ELEMS = 1 << 26


def _rows_per_chunk(per_row: int) -> int:
    return max(1, _CHUNK_ELEMS // max(per_row, 1))


@dataclasses.dataclass
class Inputs:
    cfg: Config
    set_id: int
    q_idx: torch.Tensor      # uint8 [R,H_I,d_I] (fp32 for fp32 configs)
    q_scale: torch.Tensor    # f32 [R,H_I]
    w: torch.Tensor          # f32 [R,H_I]
    k_idx: torch.Tensor      # uint8 [B,N,d_I] (fp32 for fp32 configs)
    k_scale: torch.Tensor    # f32 [B,N]
    q: torch.Tensor          # bf16 [R,H,D_k] (fp32 for fp32 configs)
    latent: torch.Tensor     # bf16 [B,N,D_k] (fp32 for fp32 configs)
    row_seq: torch.Tensor    # int32 [R]
    row_pos: torch.Tensor    # int32 [R]


def make_inputs(cfg: Config, set_id: int = 0, device="cpu",
                rows: Optional[Tuple[int, int]] = None) -> Inputs:
    """Materialise every input tensor of a workload on ``device``.

    ``rows`` restricts the query-side tensors to global rows [r0, r1) (the caches
    are always whole).
    """
    g = Generator(cfg, set_id)
    c = cfg
    r0, r1 = rows if rows is not None else (0, c.num_rows)
    n = r1 - r0
    qdt = torch.float32 if c.fp32 else torch.uint8
    adt = torch.float32 if c.fp32 else torch.bfloat16

    q_idx = torch.empty(n, c.n_idx_heads, c.idx_dim, dtype=qdt, device=device)
    q_scale = torch.empty(n, c.n_idx_heads, dtype=torch.float32, device=device)
    w = torch.empty(n, c.n_idx_heads, dtype=torch.float32, device=device)
    q = torch.empty(n, c.n_heads, c.qk_dim, dtype=adt, device=device)
    step = _rows_per_chunk(c.n_heads * c.qk_dim)
    for a in range(r0, r1, step):
        b_ = min(r1, a + step)
        codes, sc = g.q_idx(a, b_, device)
        q_idx[a - r0:b_ - r0] = codes
        q_scale[a - r0:b_ - r0] = sc
        w[a - r0:b_ - r0] = g.w(a, b_, device)
        q[a - r0:b_ - r0] = g.q(a, b_, device)

    k_idx = torch.empty(c.num_seqs, c.max_ctx, c.idx_dim, dtype=qdt, device=device)
    k_scale = torch.empty(c.num_seqs, c.max_ctx, dtype=torch.float32, device=device)
    latent = torch.empty(c.num_seqs, c.max_ctx, c.qk_dim, dtype=adt, device=device)
    step = _rows_per_chunk(c.qk_dim)
    for b in range(c.num_seqs):
        for p in range(0, c.max_ctx, step):
            p1 = min(c.max_ctx, p + step)
            codes, sc = g.k_idx(b, p, p1, device)
            k_idx[b, p:p1] = codes
            k_scale[b, p:p1] = sc
            latent[b, p:p1] = g.latent(b, p, p1, device)

    seq, pos = c.row_seq_pos()
    return Inputs(c, set_id, q_idx, q_scale, w, k_idx, k_scale, q, latent,
                  torch.from_numpy(seq[r0:r1].copy()).to(device),
                  torch.from_numpy(pos[r0:r1].copy()).to(device))


# ---------------------------------------------------------------------------
# projection workloads: hidden states h of new tokens and the projection weights
# ---------------------------------------------------------------------------

T_H, T_WQ, T_WK, T_WC, T_WW = 6, 7, 8, 9, 10


@dataclasses.dataclass(frozen=True)
class ProjConfig:
    name: str
    cfg_id: int
    num_tokens: int        # R new tokens
    d_model: int           # width of h
    num_seqs: int          # B (caches [B, N, ...])
    max_ctx: int           # N
    n_idx_heads: int = 64
    idx_dim: int = 128
    qk_dim: int = 576
    description: str = ""

    def row_seq_pos(self) -> Tuple[np.ndarray, np.ndarray]:
        """Token r of a decode batch appends at the last position of sequence r; the
        tokens of a one-sequence chunk append at positions 0..R-1."""
        R = self.num_tokens
        if self.num_seqs == R:
            return (np.arange(R, dtype=np.int32),
                    np.full(R, self.max_ctx - 1, dtype=np.int32))
        return np.zeros(R, dtype=np.int32), np.arange(R, dtype=np.int32)


PROJ_CONFIGS: Dict[str, ProjConfig] = {
    c.name: c
    for c in [
        ProjConfig("proj_decode32", 6, 32, 7168, 32, 32768,
                   description="projections of 32 decode tokens, d_model 7168, "
                               "appended at position 32767 of their sequences"),
        ProjConfig("proj_prefill8k", 7, 8192, 7168, 1, 8192,
                   description="projections of an 8192-token prefill chunk, d_model 7168"),
    ]
}


class ProjGenerator:
    """h ~ N(0,1) and weights ~ N(0,1)/sqrt(d_model), both stored as bf16."""

    def __init__(self, cfg_id: int, d_model: int, set_id: int = 0,
                 n_idx_heads: int = 64, idx_dim: int = 128, qk_dim: int = 576):
        self.cfg_id, self.d, self.set_id = cfg_id, d_model, set_id
        self.shapes = {T_WQ: n_idx_heads * idx_dim, T_WK: idx_dim, T_WC: qk_dim,
                       T_WW: n_idx_heads}

    def _key(self, tensor_id: int) -> int:
        return stream_key(self.cfg_id, self.set_id, tensor_id)

    def h(self, r0: int, r1: int, device="cpu") -> torch.Tensor:
        x = normal(self._key(T_H), _flat(r0 * self.d, (r1 - r0) * self.d, device))
        return to_bf16(x.view(r1 - r0, self.d))

    def weight(self, tensor_id: int, p0: int = 0, p1: Optional[int] = None,
               device="cpu") -> torch.Tensor:
        """Rows [p0, p1) of one projection matrix (T_WQ, T_WK, T_WC or T_WW)."""
        p1 = self.shapes[tensor_id] if p1 is None else p1
        x = normal(self._key(tensor_id), _flat(p0 * self.d, (p1 - p0) * self.d, device))
        return to_bf16(x.view(p1 - p0, self.d) * (1.0 / math.sqrt(self.d)))

    def weights(self, device="cpu") -> Tuple[torch.Tensor, ...]:
        """(w_q, w_k, w_c, w_w), each materialised in row chunks."""
        out = []
        for tid in (T_WQ, T_WK, T_WC, T_WW):
            P = self.shapes[tid]
            t = torch.empty(P, self.d, dtype=torch.bfloat16, device=device)
            step = _rows_per_chunk(self.d)
            for a in range(0, P, step):
                t[a:min(P, a + step)] = self.weight(tid, a, min(P, a + step), device)
            out.append(t)
        return tuple(out)


# ---------------------------------------------------------------------------
# masked MHA mode: per-head queries and the key / value up-projections
# ---------------------------------------------------------------------------

T_QMHA, T_WUK, T_WUV = 11, 12, 13


class MhaGenerator:
    """q ~ N(0,1) [R, 128, 192] and w_uk, w_uv ~ N(0,1)/sqrt(512) [128, 128, 512],
    all bf16, for a workload's rows."""

    def __init__(self, cfg_id: int, set_id: int = 0, heads: int = 128, head_dim: int = 128,
                 rope: int = 64, latent: int = 512):
        self.cfg_id, self.set_id = cfg_id, set_id
        self.H, self.dh, self.dr, self.dl = heads, head_dim, rope, latent

    def _key(self, tensor_id: int) -> int:
        return stream_key(self.cfg_id, self.set_id, tensor_id)

    def q(self, r0: int, r1: int, device="cpu") -> torch.Tensor:
        per = self.H * (self.dh + self.dr)
        x = normal(self._key(T_QMHA), _flat(r0 * per, (r1 - r0) * per, device))
        return to_bf16(x.view(r1 - r0, self.H, self.dh + self.dr))

    def weights(self, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
        n = self.H * self.dh * self.dl
        out = []
        for tid in (T_WUK, T_WUV):
            x = normal(self._key(tid), _flat(0, n, device)) * (1.0 / math.sqrt(self.dl))
            out.append(to_bf16(x.view(self.H, self.dh, self.dl)))
        return tuple(out)


def random_selection(t: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """A valid selection for a row at position t: all of 0..t when t + 1 <= k, else
    k distinct positions drawn uniformly; ascending, padded with -1 to k."""
    n = min(k, t + 1)
    s = np.arange(t + 1) if t + 1 <= k else np.sort(rng.choice(t + 1, size=k, replace=False))
    out = np.full(k, -1, dtype=np.int32)
    out[:n] = s
    return out


def sample_rows(cfg: Config, count: int = 256, seed_offset: int = 99) -> np.ndarray:
    """Seeded sample of global row indices, always holding the first row, the rows
    at positions k-1 and k (the dense/sparse boundary) and the last row."""
    R = cfg.num_rows
    if R <= count:
        return np.arange(R)
    seq, pos = cfg.row_seq_pos()
    must = {0, R - 1}
    for p in (cfg.topk - 1, cfg.topk):
        hit = np.nonzero(pos == p)[0]
        if hit.size:
            must.add(int(hit[0]))
    rng = np.random.default_rng(cfg.cfg_id + seed_offset)
    rest = rng.choice(R, size=R, replace=False)
    out = list(sorted(must))
    for r in rest:
        if len(out) >= count:
            break
        if int(r) not in must:
            out.append(int(r))
    return np.array(sorted(out), dtype=np.int64)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def fp8_codes(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().contiguous().view(torch.uint8).numpy()
