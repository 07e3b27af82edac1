"""Pins for the oracle's attention definitions (CPU only).

Each test checks the oracle against something other than itself: a library
routine (torch's scaled-dot-product attention in float64, scipy's logsumexp),
an invariant, or a brute-force formulation written differently.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import minference_oracle as O


def _rand(seed, n, d, h=1):
    g = np.random.default_rng(seed)
    return (g.standard_normal((n, d)), g.standard_normal((n, d)), g.standard_normal((n, d)))


def _sdpa(q, k, v, scale, mask=None, causal=False):
    t = lambda x: torch.from_numpy(x)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=causal, scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("n,d", [(1, 4), (37, 16), (130, 64)])
def test_dense_causal_matches_library(n, d):
    q, k, v = _rand(n * 7 + d, n, d)
    scale = 1 / np.sqrt(d)
    o, lse = O.dense_causal_attention(q, k, v, scale)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale, causal=True), rtol=0, atol=1e-12)
    s = scale * q @ k.T
    ref_lse = np.array([logsumexp(s[i, : i + 1]) for i in range(n)])
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_masked_rows_match_library_with_random_masks(seed):
    n, d = 48, 8
    q, k, v = _rand(100 + seed, n, d)
    g = np.random.default_rng(seed)
    mask = g.random((n, n)) < 0.3
    mask &= np.tril(np.ones((n, n), bool))
    mask[np.arange(n), np.arange(n)] = True  # every row keeps its own key
    scale = 0.37
    ref = _sdpa(q, k, v, scale, mask=mask)
    rows = np.arange(n)
    o, lse = O.masked_rows_attention(q, k, v, scale, rows, np.arange(n), mask)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    for i in range(n):
        oi, li = O.attention_row_gather(q, k, v, scale, i, np.nonzero(mask[i])[0])
        np.testing.assert_allclose(oi, ref[i], rtol=0, atol=1e-12)
        assert abs(li - logsumexp(scale * q[i] @ k[mask[i]].T)) < 1e-12
        assert abs(lse[i] - li) < 1e-12


def test_union_attention_with_all_keys_is_dense_causal():
    n, d = 64 * 3, 16
    q, k, v = _rand(5, n, d)
    scale = 1 / 4
    o_dense, lse_dense = O.dense_causal_attention(q, k, v, scale)
    for a in range(3):
        rows = np.arange(64 * a, 64 * a + 64)
        o, lse = O.union_attention(q, k, v, scale, rows, np.arange(n))
        np.testing.assert_allclose(o, o_dense[rows], atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, lse_dense[rows], atol=1e-12, rtol=0)


def test_softmax_rows_sum_to_one():
    n, d = 200, 8
    q, k, _ = _rand(6, n, d)
    ones = np.ones((n, 1))
    g = np.random.default_rng(1)
    union = np.unique(np.concatenate([g.choice(n, 50, replace=False), np.arange(64, 128)]))
    rows = np.arange(128, 192)
    o, _ = O.union_attention(q, k, ones, 0.5, rows, np.union1d(union, rows))
    np.testing.assert_allclose(o[:, 0], 1.0, atol=1e-12, rtol=0)


def test_causality_future_keys_do_not_matter():
    n, d = 96, 8
    q, k, v = _rand(7, n, d)
    o1, l1 = O.dense_causal_attention(q, k, v, 0.3)
    k2, v2 = k.copy(), v.copy()
    i = 40
    k2[i + 1:] += 5.0
    v2[i + 1:] -= 3.0
    o2, l2 = O.dense_causal_attention(q, k2, v2, 0.3)
    assert np.array_equal(o1[: i + 1], o2[: i + 1])
    assert np.array_equal(l1[: i + 1], l2[: i + 1])
    # same for the index form: keys above the row are excluded exactly
    rows = np.arange(0, 64)
    oa, _ = O.union_attention(q, k, v, 0.3, rows, np.arange(n))
    ob, _ = O.union_attention(q, k2, v2, 0.3, rows, np.arange(n))
    assert np.array_equal(oa[: i + 1], ob[: i + 1])


def test_gqa_mapping_matches_repeat_interleave():
    """Query head h reads kv head h // (Hq/Hkv): the grouping used by
    grouped-query attention, pinned against torch's repeat_interleave expansion."""
    hq, hkv, n, d = 8, 2, 64, 16
    g = np.random.default_rng(3)
    q = g.standard_normal((hq, n, d))
    k = g.standard_normal((hkv, n, d))
    v = g.standard_normal((hkv, n, d))
    kk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=0)[None]
    vv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], kk, vv, is_causal=True, scale=0.25)[0].numpy()
    out = O.layer_attention(q, k, v, 0.25, [O.HeadIndex(O.DENSE, n)] * hq, [0])
    for h in range(hq):
        np.testing.assert_allclose(out[h][0][0], ref[h], atol=1e-12, rtol=0)
