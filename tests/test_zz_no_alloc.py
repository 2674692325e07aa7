"""dsa_forward_noalloc (the whole path with the library's fixed scratch instead of a
workspace) against dsa_forward, the entry point whose kernels it shares: the same
seeded inputs must give the same bits, on two calls in a row, the second with a
smaller input, so that scratch left by the first call cannot leak into the second.
Also checks the host-side refusal of a call whose scratch would not fit."""
from __future__ import annotations

import pytest
import torch

import dsa_inputs as di

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_fp8_amd as m
    return m


def _both(dsa, inp, R):
    c = inp.cfg
    rows = dsa.rows_struct(inp.row_seq[:R].contiguous(), inp.row_pos[:R].contiguous(), c.num_seqs,
                           c.max_ctx, c.kv_len - 1)
    dims = dsa.Dims.from_config(c)
    args = (inp.q_idx[:R].contiguous(), inp.q_scale[:R].contiguous(), inp.w[:R].contiguous(),
            inp.k_idx, inp.k_scale, inp.q[:R].contiguous(), inp.latent, c.scale)
    out_a = torch.empty(R, c.n_heads, c.v_dim, dtype=torch.bfloat16, device="cuda")
    lse_a = torch.empty(R, c.n_heads, dtype=torch.float32, device="cuda")
    idx_a = torch.empty(R, c.topk, dtype=torch.int32, device="cuda")
    out_b, lse_b, idx_b = torch.empty_like(out_a), torch.empty_like(lse_a), torch.empty_like(idx_a)
    dsa.forward(rows, dims, *args, out=out_a, lse=lse_a, indices_out=idx_a)
    dsa.forward_noalloc(rows, dims, *args, out=out_b, lse=lse_b, indices_out=idx_b)
    torch.cuda.synchronize()
    return (out_a, lse_a, idx_a), (out_b, lse_b, idx_b)


def test_noalloc_matches_forward_twice_shrinking(dsa):
    inp = di.make_inputs(di.CONFIGS["decode32k"], 0, device="cuda")
    for R in (32, 5):      # the second call is smaller: fewer rows, more attention splits
        print(f"[noalloc] decode32k rows {R}", flush=True)
        a, b = _both(dsa, inp, R)
        assert torch.equal(a[2], b[2]), "selections differ"
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), "outputs differ"
    small = di.make_inputs(di.CONFIGS["tiny"], 0, device="cuda")
    c = small.cfg
    rows = dsa.rows_struct(small.row_seq, small.row_pos, c.num_seqs, c.max_ctx, c.kv_len - 1)
    dims = dsa.Dims.from_config(c)
    out = torch.empty(c.num_rows, c.n_heads, c.v_dim, dtype=torch.float32, device="cuda")
    lse = torch.empty(c.num_rows, c.n_heads, dtype=torch.float32, device="cuda")
    o_ref, l_ref, _ = dsa.forward(rows, dims, small.q_idx, None, small.w, small.k_idx, None,
                                  small.q, small.latent, c.scale)
    dsa.forward_noalloc(rows, dims, small.q_idx, None, small.w, small.k_idx, None, small.q,
                        small.latent, c.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
    print("[noalloc] outputs identical to dsa_forward on both calls and on the fp32 path",
          flush=True)


def test_noalloc_refuses_oversized_scratch(dsa):
    """A whole 8K prefill in one chunk needs 268 MB of scores: refused on the host,
    nothing enqueued; 64-row chunks fit."""
    c = di.CONFIGS["prefill8k"]
    dims = dsa.Dims.from_config(c)
    dev = "cuda"
    R = c.num_rows
    seq = torch.zeros(R, dtype=torch.int32, device=dev)
    pos = torch.arange(R, dtype=torch.int32, device=dev)
    rows = dsa.rows_struct(seq, pos, 1, c.max_ctx, c.kv_len - 1)
    assert dsa.forward_workspace_size(rows, dims, 0) > (64 << 20)
    assert dsa.forward_workspace_size(rows, dims, 64) <= (64 << 20)
    z8 = torch.zeros(R, 64, 128, dtype=torch.uint8, device=dev)
    f = torch.zeros(R, 64, device=dev)
    kk = torch.zeros(1, c.max_ctx, 128, dtype=torch.uint8, device=dev)
    ks = torch.ones(1, c.max_ctx, device=dev)
    q = torch.zeros(R, 128, 576, dtype=torch.bfloat16, device=dev)
    lat = torch.zeros(1, c.max_ctx, 576, dtype=torch.bfloat16, device=dev)
    out = torch.empty(R, 128, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(R, 128, device=dev)
    with pytest.raises(dsa.DSAError) as e:
        dsa.forward_noalloc(rows, dims, z8, f, f, kk, ks, q, lat, c.scale, out=out, lse=lse)
    assert e.value.status == dsa.DSA_E_WORKSPACE and str(64 << 20) in str(e.value)
