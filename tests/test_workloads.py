"""The seeded input generator: exact bf16 rounding, determinism, recipe."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0, -2.5, 3.0e-38, 65504.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)])
    ours = W.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_planted():
    w = W.C3.with_(seq_len=2048, heads_q=4, heads_kv=2, n_vertical_plants=8)
    a = W.generate(w)
    b = W.generate(w)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (1, 4, 2048, 128) and a["k"].shape == (1, 2, 2048, 128)
    assert a["q"].dtype == np.uint16
    for kvh in range(2):
        p = a["plants"][kvh]
        assert p[0] == 0 and len(np.unique(p)) == 8 and p.max() < 2048


def test_rotary_preserves_pair_norms():
    w = W.C1.with_(seq_len=256, n_vertical_plants=0, alpha_vertical=0.0)
    out = W.generate(w)
    q = out["q"][0, 0].astype(np.float64)
    raw = W.rng(w.seed, W.T_Q, 0).standard_normal((256, 64), dtype=np.float32).astype(np.float64)
    half = 32
    n1 = q[:, :half] ** 2 + q[:, half:] ** 2
    n0 = raw[:, :half] ** 2 + raw[:, half:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-5)
    np.testing.assert_allclose(q[0], raw[0], rtol=1e-6)  # position 0 is not rotated


def test_mixed_patterns_split():
    p = W.head_patterns(W.C4)
    assert (p == W.ASHAPE).sum() == 8 and (p == W.VSLASH).sum() == 16 and (p == W.BSPARSE).sum() == 8
