"""Pins for the oracle's estimates, selection and index definitions (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import minference_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":")
            out[int(key)] = [int(x) for x in vals.split()]
    return out


def _rand(seed, n, d):
    g = np.random.default_rng(seed)
    return g.standard_normal((n, d)), g.standard_normal((n, d)), g.standard_normal((n, d))


# ---------------------------------------------------------------- selection

def test_select_all_equal_takes_lowest_indices():
    assert list(O.select_topk(np.ones(10), 4)) == [0, 1, 2, 3]
    assert list(O.select_topk(np.ones(10), 4, {7})) == [0, 1, 2, 7]


def test_select_forced_members_always_present():
    s = np.arange(20, dtype=float)  # index 0 has the lowest score
    got = O.select_topk(s, 5, {0, 3})
    assert set(got) >= {0, 3}
    assert list(got) == [0, 3, 17, 18, 19]


def test_select_budget_at_least_candidates_takes_everything():
    s = np.random.default_rng(0).random(9)
    assert list(O.select_topk(s, 9)) == list(range(9))
    assert list(O.select_topk(s, 50, {4})) == list(range(9))


@pytest.mark.parametrize("seed", range(5))
def test_select_matches_python_sorted_with_ties(seed):
    g = np.random.default_rng(seed)
    m = 200
    s = g.integers(0, 12, m).astype(float)  # heavy ties
    forced = set(g.choice(m, 3, replace=False).tolist())
    k = 40
    rest = sorted((i for i in range(m) if i not in forced), key=lambda i: (-s[i], i))
    ref = sorted(forced | set(rest[: k - len(forced)]))
    assert list(O.select_topk(s, k, forced)) == ref


def test_select_rejects_more_forced_than_budget():
    with pytest.raises(ValueError):
        O.select_topk(np.ones(5), 1, {0, 1})


# ---------------------------------------------------------- VS estimate

@pytest.mark.parametrize("n,L", [(64, 64), (130, 16), (257, 64)])
def test_vs_scores_total_mass(n, L):
    q, k, _ = _rand(n + L, n, 16)
    vert, sl = O.vs_estimate(q, k, 0.25, L)
    assert abs(vert.sum() - L) < 1e-9
    assert abs(sl.sum() - L) < 1e-9
    assert (vert >= 0).all() and (sl >= 0).all()


def test_vs_scores_closed_form_equal_keys():
    """All keys equal -> each row spreads uniformly over its causal keys:
    vertical[j] = sum_r [j <= i_r]/(i_r+1), slash[o] = sum_r [o <= i_r]/(i_r+1)."""
    n, L, d = 100, 7, 8
    g = np.random.default_rng(1)
    q = g.standard_normal((n, d))
    k = np.tile(g.standard_normal((1, d)), (n, 1))
    vert, sl = O.vs_estimate(q, k, 0.3, L)
    rows = np.arange(n - L, n)
    idx = np.arange(n)
    ref = ((idx[None, :] <= rows[:, None]) / (rows[:, None] + 1.0)).sum(axis=0)
    np.testing.assert_allclose(vert, ref, atol=1e-13, rtol=0)
    np.testing.assert_allclose(sl, ref, atol=1e-13, rtol=0)


def test_vs_scores_with_all_queries_are_column_and_diagonal_sums():
    """L = N: vertical = column sums of the dense causal probability matrix,
    slash[o] = sum of its o-th subdiagonal (library softmax and trace)."""
    n, d = 90, 8
    q, k, _ = _rand(11, n, d)
    s = torch.from_numpy(0.4 * q @ k.T)
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    p = torch.softmax(s, dim=1).numpy()
    vert, sl = O.vs_estimate(q, k, 0.4, n)
    np.testing.assert_allclose(vert, p.sum(axis=0), atol=1e-12, rtol=0)
    np.testing.assert_allclose(sl, [np.trace(p, offset=-o) for o in range(n)], atol=1e-12, rtol=0)


def test_vs_scores_brute_force_loops():
    n, L, d = 23, 5, 4
    q, k, _ = _rand(12, n, d)
    vert, sl = O.vs_estimate(q, k, 0.7, L)
    bv = [0.0] * n
    bs = [0.0] * n
    for r in range(L):
        i = n - L + r
        logits = [0.7 * float(q[i] @ k[j]) for j in range(i + 1)]
        mx = max(logits)
        ex = [np.exp(x - mx) for x in logits]
        tot = sum(ex)
        for j in range(i + 1):
            bv[j] += ex[j] / tot
            bs[i - j] += ex[j] / tot
    np.testing.assert_allclose(vert, bv, atol=1e-13, rtol=0)
    np.testing.assert_allclose(sl, bs, atol=1e-13, rtol=0)


def test_vs_planted_vertical_ranks_first():
    n, d = 512, 16
    q, k, _ = _rand(13, n, d)
    k[300] += 4.0 * q[-16:].mean(axis=0)
    vert, _ = O.vs_estimate(q, k, 0.25, 16)
    assert int(np.argmax(vert[:-16])) == 300


# ---------------------------------------------------------- VS index

def test_vs_tiles_golden():
    gold = _read_golden("vs_tiles_b64.txt")
    S = [0, 1, 64, 130]
    for a, blocks in gold.items():
        assert list(O.vs_block_list(a, S, 64)) == blocks


@pytest.mark.parametrize("block", [4, 8, 64])
def test_vs_tiles_closed_form(block):
    """BL(a) = {a - floor(o/b), a - ceil(o/b) : o in S} ∩ [0, a] (the diagonal of
    offset o crosses at most two aligned key blocks per query block)."""
    g = np.random.default_rng(block)
    nb = 40
    n = nb * block
    S = np.unique(np.concatenate([[0], g.choice(n, 25, replace=False)]))
    for a in range(nb):
        ref = set()
        for o in S:
            for t in (o // block, -(-o // block)):
                if a - t >= 0:
                    ref.add(a - t)
        assert list(O.vs_block_list(a, S, block)) == sorted(ref)


def test_vs_index_full_budget_is_dense():
    n, d = 64 * 4, 8
    q, k, v = _rand(14, n, d)
    idx = O.HeadIndex(O.VSLASH, n, V=np.arange(n), S=np.arange(n))
    dense, dlse = O.dense_causal_attention(q, k, v, 0.3)
    out = O.head_attention(q, k, v, 0.3, idx, range(4))
    for a in range(4):
        np.testing.assert_allclose(out[a][0], dense[64 * a: 64 * a + 64], atol=1e-12, rtol=0)
        assert len(idx.cols(a)) == 0  # every vertical lies in a listed tile


@pytest.mark.parametrize("seed", range(3))
def test_vs_index_invariants(seed):
    g = np.random.default_rng(seed)
    n = 64 * 12
    V = np.unique(np.concatenate([[0], g.choice(n, 30, replace=False)]))
    S = np.unique(np.concatenate([[0], g.choice(n, 20, replace=False)]))
    for a in range(12):
        bl = O.vs_block_list(a, S)
        cl = O.vs_column_list(a, V, bl)
        assert a in bl  # offset 0 -> diagonal tile
        assert 0 in np.unique(np.concatenate([bl, cl // 64]))  # the sink key is reachable
        assert not np.isin(cl // 64, bl).any()  # no key counted twice
        assert np.isin(cl, V).all()
        u = O.block_union(bl, cl)
        for i in range(64 * a, 64 * a + 64):
            exact = O.vs_exact_allowed(i, V, S)
            assert np.isin(exact, u).all()  # exact VS keys are all computed
            assert i in u


# ---------------------------------------------------------- exact Vertical-Slash set

def test_vs_exact_golden():
    gold = _read_golden("vs_exact_n10_v04_s03.txt")
    assert sorted(gold) == list(range(10))
    for i, keys in gold.items():
        assert list(O.vs_exact_allowed(i, [0, 4], [0, 3])) == keys


def test_vs_exact_attention_matches_golden_rows_and_row_gather():
    """Block attention over the exact sets equals per-row gathers over the
    hand-worked key sets."""
    gold = _read_golden("vs_exact_n10_v04_s03.txt")
    q, k, v = _rand(31, 10, 6)
    o, lse = O.vs_exact_attention(q, k, v, 0.4, np.arange(10), [0, 4], [0, 3])
    for i, keys in gold.items():
        oi, li = O.attention_row_gather(q, k, v, 0.4, i, keys)
        np.testing.assert_allclose(o[i], oi, atol=1e-13, rtol=0)
        assert abs(lse[i] - li) < 1e-13


def test_vs_exact_attention_brute_force_mask():
    """Masked dense softmax with the mask written out by a double loop over
    (i, j) from the definition: j <= i and (j in V or i - j in S)."""
    n, d = 96, 8
    q, k, v = _rand(32, n, d)
    g = np.random.default_rng(33)
    V = np.unique(np.concatenate([[0], g.choice(n, 9, replace=False)]))
    S = np.unique(np.concatenate([[0], g.choice(n, 13, replace=False)]))
    Vs, Ss = set(int(x) for x in V), set(int(x) for x in S)
    mask = np.zeros((n, n), bool)
    for i in range(n):
        for j in range(i + 1):
            mask[i, j] = (j in Vs) or ((i - j) in Ss)
    s = 0.35 * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p @ v) / p.sum(axis=1, keepdims=True)
    rows = np.arange(n)
    o, _ = O.vs_exact_attention(q, k, v, 0.35, rows, V, S)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    # row sizes: |V <= i| + |S <= i| - |{o in S, o <= i : i - o in V}|
    for i in range(n):
        both = sum(1 for x in Ss if x <= i and (i - x) in Vs)
        size = sum(1 for x in Vs if x <= i) + sum(1 for x in Ss if x <= i) - both
        assert size == mask[i].sum() == len(O.vs_exact_allowed(i, V, S))


def test_vs_exact_full_sets_are_dense_and_tiles_contain_it():
    n, d = 64 * 3, 8
    q, k, v = _rand(34, n, d)
    dense, _ = O.dense_causal_attention(q, k, v, 0.3)
    full = np.arange(n)
    o, _ = O.vs_exact_attention(q, k, v, 0.3, np.arange(n), full, full)
    np.testing.assert_allclose(o, dense, atol=1e-12, rtol=0)
    # exact sets lie inside the tile covering (blocks + columns) of the same V, S
    g = np.random.default_rng(35)
    V = np.unique(np.concatenate([[0], g.choice(n, 7, replace=False)]))
    S = np.unique(np.concatenate([[0], g.choice(n, 11, replace=False)]))
    idx = O.HeadIndex(O.VSLASH_EXACT, n, V=V, S=S)
    for a in range(3):
        u = O.block_union(idx.blocks(a), idx.cols(a))
        for i in range(64 * a, 64 * a + 64):
            assert np.isin(O.vs_exact_allowed(i, V, S), u).all()


# ---------------------------------------------------------- Block-Sparse

def test_bs_block_size_one_is_per_token_topk():
    n, d = 40, 8
    q, k, _ = _rand(15, n, d)
    w, kept = O.bs_estimate(q, k, 0.5, 6, block=1)
    logits = 0.5 * q @ k.T
    for a in range(n):
        ref = O.select_topk(logits[a, : a + 1], min(6, a + 1), {0, a})
        assert list(kept[a]) == list(ref)
        np.testing.assert_allclose(w[a, : a + 1].sum(), 1.0, atol=1e-13)
        assert (w[a, a + 1:] == 0).all()


def test_bs_weights_block_size_one_equal_library_softmax():
    """Block size 1: the weights of row a are the library softmax of the
    scaled per-token logits over keys 0..a (a dropped or doubled scale fails)."""
    from scipy.special import softmax
    n, d, scale = 30, 8, 0.37
    q, k, _ = _rand(21, n, d)
    w, _ = O.bs_estimate(q, k, scale, 4, block=1)
    for a in range(n):
        ref = softmax(np.array([scale * float(np.dot(q[a], k[c])) for c in range(a + 1)]))
        np.testing.assert_allclose(w[a, : a + 1], ref, rtol=1e-12, atol=1e-15)
        assert (w[a, a + 1:] == 0).all()


def test_bs_weights_pure_python_loops():
    """Block size 64: pooled means, scaled dot products and the causal block
    softmax written out as plain Python loops with math.exp."""
    import math
    nb, d, scale = 5, 3, 0.61
    q, k, _ = _rand(22, 64 * nb, d)
    w, _ = O.bs_estimate(q, k, scale, 2)
    mean = lambda x, blk, e: sum(float(x[64 * blk + r, e]) for r in range(64)) / 64.0
    for a in range(nb):
        qb = [mean(q, a, e) for e in range(d)]
        z = [scale * sum(qb[e] * mean(k, c, e) for e in range(d)) for c in range(a + 1)]
        top = max(z)
        ex = [math.exp(x - top) for x in z]
        tot = sum(ex)
        for c in range(nb):
            ref = ex[c] / tot if c <= a else 0.0
            assert abs(w[a, c] - ref) <= 1e-13, (a, c, w[a, c], ref)


def test_bs_weights_closed_form_on_constant_blocks():
    """Constant rows per block: Qbar_a = u_a, Kbar_c = t_c exactly, so row a's
    weights are exp(s u_a.t_c) / sum_c' exp(s u_a.t_c').  With u_a = (1, 0)
    and t_c = (c, 0): w[a, c] = e^{s c} (e^s - 1) / (e^{s (a+1)} - 1)."""
    import math
    nb, s = 6, 0.25
    q = np.zeros((64 * nb, 2))
    q[:, 0] = 1.0
    k = np.zeros((64 * nb, 2))
    k[:, 0] = np.repeat(np.arange(nb, dtype=float), 64)
    w, kept = O.bs_estimate(q, k, s, 3)
    for a in range(nb):
        for c in range(a + 1):
            ref = math.exp(s * c) * (math.exp(s) - 1.0) / (math.exp(s * (a + 1)) - 1.0)
            assert abs(w[a, c] - ref) <= 1e-14, (a, c)
        # the largest weights are the latest blocks: {0, a} plus a-1
        assert list(kept[a]) == sorted({0, a} | ({a - 1} if a >= 2 else set()))


def test_bs_means_of_constant_blocks():
    d = 4
    k = np.repeat(np.arange(3 * d, dtype=float).reshape(3, d), 64, axis=0)
    np.testing.assert_array_equal(O.block_means(k), k[::64])
    x = np.arange(128 * 2, dtype=float).reshape(128, 2)
    np.testing.assert_allclose(O.block_means(x), [[63.0, 64.0], [191.0, 192.0]])


def test_bs_full_budget_is_dense():
    n, d = 64 * 5, 8
    q, k, v = _rand(16, n, d)
    _, kept = O.bs_estimate(q, k, 0.3, 100)
    idx = O.HeadIndex(O.BSPARSE, n, kept=kept)
    dense, _ = O.dense_causal_attention(q, k, v, 0.3)
    out = O.head_attention(q, k, v, 0.3, idx, range(5))
    for a in range(5):
        assert list(kept[a]) == list(range(a + 1))
        np.testing.assert_allclose(out[a][0], dense[64 * a: 64 * a + 64], atol=1e-12, rtol=0)


def test_bs_row_sizes_and_forced_blocks():
    n, d = 64 * 9, 8
    q, k, _ = _rand(17, n, d)
    _, kept = O.bs_estimate(q, k, 0.3, 4)
    for a in range(9):
        kb = kept[a]
        assert len(kb) == min(4, a + 1)
        assert 0 in kb and a in kb
        u = O.block_union(kb, [])
        for r in (0, 17, 63):
            i = 64 * a + r
            assert (u <= i).sum() == 64 * (len(kb) - 1) + r + 1


# ---------------------------------------------------------- A-shape

def test_ashape_golden():
    gold = _read_golden("ashape_n8_s2_w3.txt")
    for i, keys in gold.items():
        assert list(O.ashape_allowed(i, 2, 3)) == keys


@pytest.mark.parametrize("s,w", [(2, 3), (128, 4096), (5, 64), (0, 1)])
def test_ashape_row_sizes(s, w):
    for i in list(range(0, 300, 7)) + [5000]:
        size = len(O.ashape_allowed(i, s, w))
        assert size == (i + 1 if i + 1 <= s + w else s + w)


def test_ashape_covering_window_is_dense():
    n, d = 64 * 3, 8
    q, k, v = _rand(18, n, d)
    dense, _ = O.dense_causal_attention(q, k, v, 0.3)
    idx = O.HeadIndex(O.ASHAPE, n, sink=10, local=n - 10)
    out = O.head_attention(q, k, v, 0.3, idx, range(3))
    for a in range(3):
        np.testing.assert_allclose(out[a][0], dense[64 * a: 64 * a + 64], atol=1e-12, rtol=0)


@pytest.mark.parametrize("s,w", [(128, 4096), (100, 300), (3, 70)])
def test_ashape_block_attention_matches_row_gather(s, w):
    n, d = 64 * 10, 8
    q, k, v = _rand(19, n, d)
    for a in (0, 1, 5, 9):
        rows = np.arange(64 * a, 64 * a + 64)
        o, lse = O.ashape_attention(q, k, v, 0.3, rows, s, w)
        for r, i in enumerate(rows):
            oi, li = O.attention_row_gather(q, k, v, 0.3, i, O.ashape_allowed(i, s, w))
            np.testing.assert_allclose(o[r], oi, atol=1e-12, rtol=0)
            assert abs(lse[r] - li) < 1e-12


@pytest.mark.parametrize("s,w", [(128, 4096), (100, 300), (3, 70), (64, 64)])
def test_ashape_block_list_closed_form(s, w):
    """Key block c <= a is touched iff it holds a sink key (64c < s) or its
    nearest key pair is inside the window (64(a-c) - 63 < w)."""
    n = 64 * 80
    for a in (0, 1, 2, 10, 64, 65, 79):
        ref = [c for c in range(a + 1) if 64 * c < s or 64 * (a - c) - 63 < w]
        assert list(O.ashape_block_list(a, s, w, n)) == ref


# ----------------------------------------------------------------- antidiagonal block scoring

def _antidiag_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "antidiag_b2_n6.txt")) if l.strip() and l[0] != "#"]
    q = np.array([float(x) for x in rows[0][1:]])[:, None]
    k = np.array([float(x) for x in rows[1][1:]])[:, None]
    xs = {int(r[1]): [float(v) for v in r[3:]] for r in rows if r[0] == "x"}
    kept = {(int(r[1].split("=")[1]), int(r[2])): [int(v) for v in r[4:]] for r in rows if r[0] == "kept"}
    return q, k, xs, kept


def test_antidiag_golden():
    """Hand-worked scores: the oracle's weights are scipy's softmax of them and
    its kept lists are the worked ones (block 1 outscores block 2 in row 2 and
    is still dropped at top 2: blocks 0 and a are forced)."""
    from scipy.special import softmax
    q, k, xs, kept = _antidiag_golden()
    for top in (2, 3):
        w, kb = O.antidiag_estimate(q, k, 1.0, top, block=2)
        for a, x in xs.items():
            np.testing.assert_allclose(w[a, : a + 1], softmax(np.array(x)), rtol=1e-13)
            assert not w[a, a + 1:].any()
        for (t, a), lst in kept.items():
            if t == top:
                assert list(kb[a]) == lst, (top, a)


def test_antidiag_block_size_one_is_causal_softmax():
    """With one-token blocks the antidiagonal is the logit itself: the weights
    are the causal attention probabilities (scipy softmax at an explicit
    scale) and the lists the per-token top-k."""
    from scipy.special import softmax
    g = np.random.default_rng(41)
    n, d, sc = 23, 5, 0.43
    q, k = g.standard_normal((n, d)), g.standard_normal((n, d))
    w, kept = O.antidiag_estimate(q, k, sc, 4, block=1)
    for i in range(n):
        np.testing.assert_allclose(w[i, : i + 1], softmax(sc * (k[: i + 1] @ q[i])), rtol=1e-12)
        assert list(kept[i]) == list(O.select_topk(w[i, : i + 1], min(4, i + 1), {0, i}))


def test_antidiag_constant_blocks_match_pooled_estimate():
    """Rows constant inside each block: off the diagonal x = block * z of the
    pooled estimate (a closed form), the diagonal block sums its causal half
    (block/2 pairs); the kept lists equal the pooled estimate's."""
    g = np.random.default_rng(43)
    nb, b, d, sc = 9, 8, 6, 0.3
    qm, km = g.standard_normal((nb, d)), g.standard_normal((nb, d))
    q, k = np.repeat(qm, b, axis=0), np.repeat(km, b, axis=0)
    w, kept = O.antidiag_estimate(q, k, sc, 4, block=b)
    _, kept_pool = O.bs_estimate(q, k, sc, 4, block=b)
    for a in range(nb):
        x = np.array([b * sc * qm[a] @ km[c] for c in range(a)] + [(b // 2) * sc * qm[a] @ km[a]])
        e = np.exp(x - x.max())
        np.testing.assert_allclose(w[a, : a + 1], e / e.sum(), rtol=1e-12)
        assert list(kept[a]) == list(kept_pool[a]), a
