"""Host-side arithmetic of bench.py: the exact-pattern pair counts it reports
beside the issued tile work, checked against brute-force enumeration of the
per-element patterns on tiny layers (no GPU)."""
from types import SimpleNamespace

import numpy as np
import torch

import bench
import workloads as W


def brute(pattern, N, V=(), S=(), kept=None, sink=0, local=0):
    n = 0
    for i in range(N):
        for j in range(i + 1):
            if pattern == W.VSLASH:
                ok = j in V or (i - j) in S
            elif pattern == W.BSPARSE:
                ok = (j // 64) in kept[i // 64]
            elif pattern == W.ASHAPE:
                ok = j < sink or i - j < local
            else:
                ok = True
            n += ok
    return n


def test_exact_pairs_match_brute_force():
    N, nb = 256, 4
    rng = np.random.default_rng(0)
    V = [0, 3, 100, 255]
    S = [0, 1, 70, 129]
    vidx = torch.full((1, 4, 6), -1, dtype=torch.int32)
    sidx = torch.full((1, 4, 6), -1, dtype=torch.int32)
    vidx[0, 1, :4] = torch.tensor(V)
    sidx[0, 1, :4] = torch.tensor(S)
    kept = [sorted({0, a} | set(int(x) for x in rng.integers(0, a + 1, 2))) for a in range(nb)]
    bcnt = torch.zeros((1, 4, nb), dtype=torch.int32)
    for a in range(nb):
        bcnt[0, 2, a] = len(kept[a])
    pats = [W.ASHAPE, W.VSLASH, W.BSPARSE, W.DENSE]
    plan = SimpleNamespace(q=torch.zeros(1, 4, N, 8), pat=pats, vidx=vidx, sidx=sidx, bcnt=bcnt)
    w = SimpleNamespace(sink=16, local=40)
    got = bench.exact_pairs(plan, w)
    want = (brute(W.ASHAPE, N, sink=16, local=40) + brute(W.VSLASH, N, V=set(V), S=set(S)) +
            brute(W.BSPARSE, N, kept=kept) + brute(W.DENSE, N))
    assert got == want


def test_plant_recall_counts_planted_keys_and_hot_blocks():
    """The recall diagnostic on hand-made selections: every hot block at or
    before a query block selected gives 1; half of each kv head's planted
    keys among a Vertical-Slash head's verticals gives 0.5."""
    import types
    import torch
    w = W.WORKLOADS["c2"]
    nb, g = w.n_blocks, w.heads_q // w.heads_kv
    bidx = np.full((1, w.heads_q, nb, w.top_blocks), -1, np.int32)
    bcnt = np.zeros((1, w.heads_q, nb), np.int32)
    for h in range(w.heads_q):
        hot = W.hot_blocks(w, h // g)
        for a in range(nb):
            sel = hot[hot <= a]
            bidx[0, h, a, :len(sel)] = sel
            bcnt[0, h, a] = len(sel)
    plan = types.SimpleNamespace(pat=[W.BSPARSE] * w.heads_q, vidx=None,
                                 bidx=torch.from_numpy(bidx), bcnt=torch.from_numpy(bcnt))
    assert bench.plant_recall(plan, w)["hot_blocks"]["recall"] == 1.0
    bcnt[:] = 0  # nothing selected
    assert bench.plant_recall(plan, w)["hot_blocks"]["recall"] == 0.0
    w3 = W.WORKLOADS["c3"]
    vidx = np.full((1, w3.heads_q, w3.n_vertical), -1, np.int32)
    for h in range(w3.heads_q):
        pl = W.vertical_plants(w3, h // (w3.heads_q // w3.heads_kv))
        vidx[0, h, :len(pl) // 2] = pl[: len(pl) // 2]
    plan = types.SimpleNamespace(pat=[W.VSLASH] * w3.heads_q, vidx=torch.from_numpy(vidx), bidx=None, bcnt=None)
    r = bench.plant_recall(plan, w3)["vertical"]
    assert r["mean_recall"] == r["min_recall"] == r["max_recall"] == 0.5
