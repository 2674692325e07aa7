"""Parity of the projection step (dsa_project_append, through the C ABI) with the
float64 oracle, under comparison rule C4 (tests/dsa_check.py).

Hidden states and weights come from the seeded generator, on the device for the
library and regenerated on the host for the oracle.  The caches start filled
with a sentinel so that every row the call must not touch can be checked.
Cases cover the three launch shapes (split contraction with a second summing
kernel, small tiles with the whole contraction, large tiles), ragged token
counts, a zero token, rows whose cache position is out of range, and the full
decode and prefill-chunk sizes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dsa_inputs as di
from dsa_check import check_bf16_words, check_fp32_within, check_quantised, proj_reference

pytestmark = pytest.mark.gpu

SENT_CODE = 0x5A
SENT_SCALE = -7.0
SENT_WORD = 0x3F80


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_fp8_amd as m
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    return di.bf16_bits(t)


def run_case(m, cfg_id, R, d, B, N, seq, pos, zero_rows=(), sample=None, set_id=0):
    print(f"[proj] R={R} d={d} B={B} N={N} zero={list(zero_rows)}", flush=True)
    g = di.ProjGenerator(cfg_id, d, set_id)
    h = g.h(0, R, device="cuda")
    for z in zero_rows:
        h[z] = 0
    weights = g.weights(device="cuda")
    dev = torch.device("cuda")
    k_idx = torch.full((B, N, 128), SENT_CODE, dtype=torch.uint8, device=dev)
    k_scale = torch.full((B, N), SENT_SCALE, dtype=torch.float32, device=dev)
    latent = torch.full((B, N, 576), SENT_WORD, dtype=torch.int16, device=dev).view(torch.bfloat16)
    seq_t = torch.from_numpy(np.asarray(seq, dtype=np.int32)).to(dev)
    pos_t = torch.from_numpy(np.asarray(pos, dtype=np.int32)).to(dev)
    rows = m.rows_struct(seq_t, pos_t, B, N, N - 1)
    q_idx, q_scale, w = m.project_append(rows, h, *weights, k_idx, k_scale, latent)
    torch.cuda.synchronize()

    sel = np.arange(R) if sample is None else np.asarray(sample)
    h_host = torch.cat([g.h(int(r), int(r) + 1) for r in sel]) if sample is not None \
        else g.h(0, R)
    for z in zero_rows:
        h_host[np.nonzero(sel == z)[0]] = 0
    ref = proj_reference(_bits(h_host), [_bits(x) for x in g.weights()], 64)

    sel_t = torch.from_numpy(sel).to(dev)
    amb_q = check_quantised(q_idx[sel_t].cpu().numpy(), q_scale[sel_t].cpu().numpy(),
                            ref["y_q"], ref["err_q"])
    ratio_w = check_fp32_within(w[sel_t].cpu().numpy(), ref["y_w"], ref["err_w"])

    seq, pos = np.asarray(seq), np.asarray(pos)
    valid = (seq[sel] >= 0) & (seq[sel] < B) & (pos[sel] >= 0) & (pos[sel] < N)
    vi = np.nonzero(valid)[0]
    amb_c = 0.0
    if vi.size:
        bs = torch.from_numpy(seq[sel][vi].astype(np.int64)).to(dev)
        ps = torch.from_numpy(pos[sel][vi].astype(np.int64)).to(dev)
        check_quantised(k_idx[bs, ps].cpu().numpy(), k_scale[bs, ps].cpu().numpy(),
                        ref["y_k"][vi], ref["err_k"][vi])
        amb_c = check_bf16_words(_bits(latent[bs, ps]), ref["y_c"][vi], ref["err_c"][vi])

    # every cache row that no valid token names keeps the sentinel
    written = torch.zeros(B, N, dtype=torch.bool, device=dev)
    ok_all = (seq >= 0) & (seq < B) & (pos >= 0) & (pos < N)
    if ok_all.any():
        written[torch.from_numpy(seq[ok_all].astype(np.int64)).to(dev),
                torch.from_numpy(pos[ok_all].astype(np.int64)).to(dev)] = True
    keep = ~written
    assert bool((k_idx[keep] == SENT_CODE).all()), "indexer-key cache row written that no token names"
    assert bool((k_scale[keep] == SENT_SCALE).all()), "key scale written that no token names"
    assert bool((latent.view(torch.int16)[keep] == SENT_WORD).all()), \
        "latent cache row written that no token names"
    print(f"[proj] ok: ambiguous fp8 {amb_q:.4f} bf16 {amb_c:.4f}, worst w error / bound "
          f"{ratio_w:.3g}", flush=True)
    return ratio_w


def test_project_split_contraction_ragged(dsa):
    """37 tokens, d 512: the contraction is split over blocks and summed by a second
    kernel; a zero token; one token with a sequence and one with a position out of
    range (q and w still written, no cache row)."""
    R, B, N = 37, 3, 50
    seq = [r % B for r in range(R)]
    pos = [(7 * r) % N for r in range(R)]
    seq[5] = B
    pos[6] = -1
    run_case(dsa, 6, R, 512, B, N, seq, pos, zero_rows=(2,))


def test_project_small_tiles_whole_contraction(dsa):
    R, B, N = 300, 4, 128
    seq = [r % B for r in range(R)]
    pos = [r // B for r in range(R)]
    run_case(dsa, 6, R, 512, B, N, seq, pos, zero_rows=(299,), set_id=1)


def test_project_large_tiles_ragged(dsa):
    """1100 tokens (8 full 128-token tiles and a partial one), d 256."""
    R, B, N = 1100, 1, 1100
    run_case(dsa, 7, R, 256, B, N, [0] * R, list(range(R)), zero_rows=(0, 1099))


def test_project_single_token(dsa):
    run_case(dsa, 6, 1, 1024, 2, 8, [1], [7], set_id=2)


def test_project_decode_full_size(dsa):
    """32 decode tokens at d_model 7168, appended at position 32767 of 32 caches of
    32768 entries."""
    c = di.PROJ_CONFIGS["proj_decode32"]
    seq, pos = c.row_seq_pos()
    run_case(dsa, c.cfg_id, c.num_tokens, c.d_model, c.num_seqs, c.max_ctx, seq, pos)


def test_project_prefill_chunk_full_size(dsa):
    """An 8192-token chunk at d_model 7168; the oracle checks a seeded sample of 64
    tokens (first and last included), the untouched-row check covers every row."""
    c = di.PROJ_CONFIGS["proj_prefill8k"]
    seq, pos = c.row_seq_pos()
    rng = np.random.default_rng(c.cfg_id + 99)
    sample = np.unique(np.concatenate([[0, c.num_tokens - 1],
                                       rng.choice(c.num_tokens, 62, replace=False)]))
    run_case(dsa, c.cfg_id, c.num_tokens, c.d_model, c.num_seqs, c.max_ctx, seq, pos,
             sample=sample)
