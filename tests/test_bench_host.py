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


def test_gather_hbm_reports_a_current_record_only(monkeypatch):
    """bench.py reports the gather's counter-measured HBM bytes only from a
    record taken on the current kernel sources."""
    from dynamic_sparse_attention_amd import profile_tables as P
    g = {"hbm_bytes": 6, "time_us": 3.0, "hbm_GBps": 2.0, "hbm_pct": 0.1, "staged_GBps": 5.0, "staged_pct": 0.2,
         "columns": 7, "staged_bytes": 15}
    monkeypatch.setattr(P, "current_gather_record", lambda name: {"gather": g} if name == "w" else None)
    assert bench.gather_hbm("w") == {k: g[k] for k in ("hbm_bytes", "time_us", "hbm_GBps", "hbm_pct",
                                                       "staged_GBps", "staged_pct")}
    assert bench.gather_hbm("other") is None


def test_committed_profiles_are_current():
    """The committed rocprofv3 tables (the four layers and the gather) were
    taken on the committed kernel sources: a kernel change without new
    profiles fails here."""
    from dynamic_sparse_attention_amd import profile_tables as P
    rec = P.current_gather_record(W.C3.name)
    assert rec is not None and rec["gather"]["hbm_bytes"] > 0 and rec["gather"]["staged_bytes"] > 0
    for w in (W.C2, W.C3, W.C4, W.C5):
        assert P.current_record(w.name) is not None, w.name
