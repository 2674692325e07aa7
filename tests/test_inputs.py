"""The seeded input generator (host side): determinism, subset regeneration,
distribution sanity and the fp8 quantiser's contract."""
import numpy as np
import torch

import dsa_inputs as di
from oracle.dsa_oracle import decode_e4m3fn


def test_counter_based_subsets_match_whole():
    cfg = di.CONFIGS["decode32k"]
    g = di.Generator(cfg, set_id=1)
    whole = g.latent(3, 0, 64)
    pos = torch.tensor([5, 0, 63, 17])
    assert torch.equal(g.latent_rows(3, pos), whole[pos])
    a, sa = g.k_idx(2, 100, 164)
    b, sb = g.k_idx(2, 96, 200)
    assert torch.equal(a, b[4:68]) and torch.equal(sa, sb[4:68])


def test_sets_and_tensors_differ():
    cfg = di.CONFIGS["decode32k"]
    a = di.Generator(cfg, 0).latent(0, 0, 8)
    b = di.Generator(cfg, 1).latent(0, 0, 8)
    assert not torch.equal(a, b)
    assert di.stream_key(2, 0, 4) != di.stream_key(2, 0, 5)


def test_normal_and_uniform_moments():
    idx = torch.arange(1 << 20)
    x = di.normal(di.stream_key(9, 9, 9), idx).double()
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    u = di.uniform(di.stream_key(9, 9, 8), idx).double()
    assert 0.0 <= u.min() and u.max() < 1.0 and abs(u.mean() - 0.5) < 2e-3


def test_quantiser_contract():
    x = di.normal(di.stream_key(1, 1, 1), torch.arange(64 * 128)).view(64, 128) * 3.7
    x[5] = 0.0
    codes, scale = di.quantize_fp8(x)
    m, e = np.frexp(scale.numpy())
    assert np.all(m == 0.5)                       # powers of two
    assert scale[5] == 1.0 and torch.all(codes[5] == 0)
    dq = decode_e4m3fn(codes.numpy()) * scale.numpy()[:, None].astype(np.float64)
    amax = x.abs().amax(1).double().numpy()
    assert np.all(np.abs(dq).max(1) <= 448.0 * scale.numpy())
    # smallest exponent: halving the scale would overflow 448
    nz = amax > 0
    assert np.all(amax[nz] > 448.0 * scale.numpy()[nz] / 2)
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 on normal codes
    big = np.abs(x.double().numpy()) >= 2.0 ** -6 * scale.numpy()[:, None]
    rel = np.abs(dq - x.double().numpy())[big] / np.abs(x.double().numpy())[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_make_inputs_tiny_shapes():
    inp = di.make_inputs(di.CONFIGS["tiny"])
    c = inp.cfg
    assert inp.q_idx.shape == (256, 4, 32) and inp.q_idx.dtype == torch.float32
    assert inp.k_idx.shape == (1, 256, 32)
    assert inp.q.shape == (256, 16, 80) and inp.latent.shape == (1, 256, 80)
    assert inp.row_pos[0] == 0 and inp.row_pos[-1] == 255
    assert torch.all((inp.w >= 0) & (inp.w < 1))


def test_sample_rows_holds_boundaries():
    cfg = di.CONFIGS["prefill128k"]
    rows = di.sample_rows(cfg, 256)
    assert len(rows) == 256 and len(set(rows.tolist())) == 256
    for r in (0, cfg.topk - 1, cfg.topk, cfg.num_rows - 1):
        assert r in rows
