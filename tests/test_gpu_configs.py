"""GPU parity at the five evaluation shapes, through the C ABI, in the same
launch configuration the benchmark times (LayerPlan: one stream, workspace
scores, index sized by index_caps).

What is compared with the oracle, per layer:
  * estimates: vertical / slash scores and block weights element by element
    (1e-3 relative) for every head at the 2K, 32K and 128K layers, for
    sampled heads at 256K and 1M; selections pass the exact gate on the GPU's
    own scores and are compared with the fp64 selection (near ties reported);
  * index lists: every query block of at least one head per pattern, and
    sampled query blocks of every other head, exactly;
  * attention rows fed the GPU's index on 16 query blocks of at least four
    heads (rows are independent given the index), always including blocks 0,
    1, nb/2 and nb-1;
  * the dense comparator (no index) on sampled rows at 128K and 1M;
  * full-size properties (ascending lists ending in the diagonal block,
    counts within caps) on every row.
The index comparison runs on a thread pool (the oracle's list arithmetic
releases the GIL); attention and estimates run serially, on the BLAS threads."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_amd as mi
import workloads as W
from oracle import minference_oracle as O
from tests.parity_util import (BF16_ATOL, F32_ATOL, assert_scores_close, check_selection,
                               gpu_index_lists, say, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mi.lib()


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pmap(fn, items):
    items = list(items)
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


def _blocks_to_check(nb, n_random, seed):
    """Query blocks 0, 1, nb/2, nb-1 plus seeded random ones (16 in total for
    n_random = 12 when nb is large)."""
    rng = np.random.default_rng(seed)
    fixed = {0, min(1, nb - 1), nb // 2, nb - 1}
    rest = np.setdiff1d(np.arange(nb), sorted(fixed))
    rnd = set(int(x) for x in rng.choice(rest, min(n_random, len(rest)), replace=False))
    return sorted(fixed | rnd)


def _run_plan(w, data):
    dev = torch.device("cuda")
    q, k, v = (to_device(data[x], w.dtype, dev) for x in ("q", "k", "v"))
    pats = [int(p) for p in data["patterns"]]
    plan = mi.LayerPlan(q, k, v, pats, last_q=w.last_q, n_vertical=w.n_vertical, n_slash=w.n_slash,
                        force_vertical=w.force_vertical, force_slash=w.force_slash,
                        top_blocks=w.top_blocks, sink=w.sink, local=w.local)
    plan.run()
    torch.cuda.synchronize()
    return plan, pats


def _ashape_blocks_closed_form(a, sink, local):
    """Key blocks of an A-shape query block: c <= a holding a sink key
    (64c < sink) or within the window of some row (64(a-c) - 63 < local).
    Pinned against the oracle's brute force in the CPU tests; used where the
    brute force (64 rows of up to N keys per block) would take minutes."""
    c = np.arange(a + 1)
    return c[(64 * c < sink) | (64 * (a - c) - 63 < local)]


def check_layer(w, *, est_heads, bs_all_rows_heads, bs_rows, full_index_heads, idx_blocks,
                att_heads, att_blocks, dense_heads=(), dense_blocks=()):
    say(f"config {w.name}: generating")
    data = W.generate(w)
    plan, pats = _run_plan(w, data)
    say(f"config {w.name}: GPU layer done")
    n, nb, g = w.seq_len, w.n_blocks, w.group
    f64 = lambda x, h: W.to_f64(x[0, h], w.dtype)
    idx = plan.index
    bc = idx.block_count[0].cpu().numpy()
    cc = idx.col_count[0].cpu().numpy()
    # full-size properties of every row of the index
    assert (bc >= 1).all() and (bc <= idx.block_cap).all() and (cc <= idx.col_cap).all()
    last = idx.block_idx[0].gather(2, (torch.from_numpy(bc).cuda().long() - 1).unsqueeze(-1))[..., 0]
    assert torch.equal(last.cpu(), torch.arange(nb, dtype=torch.int32).expand(w.heads_q, nb)), \
        "the diagonal block must be the last (largest) listed block of every row"
    oracle_index = {}
    vidx = plan.vidx[0].cpu().numpy() if plan.vidx is not None else None
    sidx = plan.sidx[0].cpu().numpy() if plan.sidx is not None else None
    for h in plan.vs_heads:
        Vh, Sh = vidx[h][vidx[h] >= 0], sidx[h][sidx[h] >= 0]
        assert np.all(np.diff(Vh) > 0) and np.all(np.diff(Sh) > 0) and Vh[0] == 0 and Sh[0] == 0
        oracle_index[h] = O.HeadIndex(O.VSLASH, n, V=Vh, S=Sh)

    # ---- Vertical-Slash estimates: one call with caller score buffers for
    # the checked heads (identical selections), scores against the oracle
    vs_est = [h for h in plan.vs_heads if h in est_heads]
    if vs_est:
        say(f"  VS estimates of {len(vs_est)} heads")
        ev, es, gv, gs = mi.vs_estimate(plan.q, plan.k, vs_est, w.last_q, w.n_vertical, w.n_slash,
                                        w.force_vertical, w.force_slash)
        torch.cuda.synchronize()
        ev, es = ev[0].cpu().numpy(), es[0].cpu().numpy()
        gv, gs = gv[0].double().cpu().numpy(), gs[0].double().cpu().numpy()

        def one(h):
            return O.vs_estimate(f64(data["q"], h), f64(data["k"], h // g), w.scale, w.last_q)

        for h, (rv, rs) in zip(vs_est, map(one, vs_est)):
            assert np.array_equal(ev[h], vidx[h]) and np.array_equal(es[h], sidx[h]), h
            assert_scores_close(gv[h], rv, f"vertical h{h}")
            assert_scores_close(gs[h], rs, f"slash h{h}")
            check_selection(vidx[h], gv[h], rv, w.n_vertical, range(w.force_vertical), f"vertical h{h}")
            check_selection(sidx[h], gs[h], rs, w.n_slash, range(w.force_slash), f"slash h{h}")
        del gv, gs

    # ---- Block-Sparse estimates
    if plan.bs_heads:
        bidx = plan.bidx[0].cpu().numpy()
        bcnt = plan.bcnt[0].cpu().numpy()
        for h in plan.bs_heads:
            oracle_index[h] = O.HeadIndex(O.BSPARSE, n, kept=[bidx[h, a, : bcnt[h, a]] for a in range(nb)])
        bs_est = [h for h in plan.bs_heads if h in est_heads]
        tri = np.tril(np.ones((nb, nb), bool))
        for h in bs_est:
            say(f"  BS estimate of head {h}")
            eb, ec, gw = mi.block_estimate(plan.q, plan.k, [h], w.top_blocks)
            torch.cuda.synchronize()
            assert np.array_equal(eb[0, h].cpu().numpy(), bidx[h])
            assert np.array_equal(ec[0, h].cpu().numpy(), bcnt[h])
            gw = gw[0, h].double().cpu().numpy()
            rw, _ = O.bs_estimate(f64(data["q"], h), f64(data["k"], h // g), w.scale, w.top_blocks)
            assert_scores_close(gw[tri], rw[tri], f"block weights h{h}")
            assert not gw[~tri].any()
            rows = range(nb) if h in bs_all_rows_heads else sorted(set(bs_rows) | {0, nb - 1})
            for a in rows:
                kk = min(w.top_blocks, a + 1)
                assert bcnt[h, a] == kk
                check_selection(bidx[h, a], gw[a, : a + 1], rw[a, : a + 1], kk, {0, a}, f"blocks h{h} a{a}")
            del gw, rw
    for h, p in enumerate(pats):
        if p == W.ASHAPE:
            oracle_index[h] = O.HeadIndex(O.ASHAPE, n, sink=w.sink, local=w.local)

    # ---- index lists, exact
    for h in range(w.heads_q):
        ih = oracle_index[h]
        full = h in full_index_heads
        blocks_here = np.arange(nb) if full else np.asarray(idx_blocks)
        sel = torch.from_numpy(blocks_here).cuda()
        bi_h = idx.block_idx[0, h].index_select(0, sel).cpu().numpy()
        ci_h = idx.col_idx[0, h].index_select(0, sel).cpu().numpy()

        def check_block(r, ih=ih, bi_h=bi_h, ci_h=ci_h, h=h, full=full, blocks_here=blocks_here):
            a = int(blocks_here[r])
            got_b = bi_h[r, : bc[h, a]]
            got_c = ci_h[r, : cc[h, a]]
            # padding: block rows of every indexed head, column rows of
            # Vertical-Slash heads (the only ones the build writes)
            if ih.pattern != O.DENSE and not np.all(bi_h[r, bc[h, a]:] == -1):
                return f"block padding h{h} a{a}"
            if ih.pattern == O.VSLASH and not np.all(ci_h[r, cc[h, a]:] == -1):
                return f"column padding h{h} a{a}"
            if ih.pattern == O.ASHAPE and full and a not in idx_blocks:
                ref_b = _ashape_blocks_closed_form(a, w.sink, w.local)
            else:
                ref_b = ih.blocks(a)
            if not np.array_equal(got_b, ref_b):
                return f"block list h{h} a{a}"
            ref_c = O.vs_column_list(a, ih.V, ref_b) if ih.pattern == O.VSLASH else np.zeros(0, np.int64)
            if not np.array_equal(got_c, ref_c):
                return f"column list h{h} a{a}"
            return None

        bad = [x for x in pmap(check_block, range(len(blocks_here))) if x]
        assert not bad, bad[:5]
        del bi_h, ci_h
        if full:
            say(f"  index of head {h} (pattern {pats[h]}): all {nb} query blocks match")
    say(f"config {w.name}: index lists match")

    # ---- attention rows fed the GPU's index
    of = plan.o[0]
    atol = F32_ATOL if w.dtype == "f32" else BF16_ATOL
    items = [(h, a) for h in att_heads for a in att_blocks]
    got_rows = {(h, a): of[h, 64 * a: 64 * a + 64].double().cpu().numpy() for h, a in items}

    def att_err(item):
        h, a = item
        qh, kh, vh = f64(data["q"], h), f64(data["k"], h // g), f64(data["v"], h // g)
        ref, _ = O.head_attention(qh, kh, vh, w.scale, oracle_index[h], [a])[a]
        return float(np.abs(got_rows[item] - ref).max())

    errs = [att_err(it) for it in items]
    worst = max(errs)
    bad = [(it, e) for it, e in zip(items, errs) if not e < atol]
    assert not bad, bad[:5]
    say(f"config {w.name}: attention max abs error {worst:.3e} over {len(att_heads)} heads x "
        f"{len(att_blocks)} blocks")

    # ---- dense comparator (same kernel, no index) on sampled rows
    if dense_heads:
        plan.attention(dense=True)
        torch.cuda.synchronize()
        items = [(h, a) for h in dense_heads for a in dense_blocks]
        got_rows = {(h, a): of[h, 64 * a: 64 * a + 64].double().cpu().numpy() for h, a in items}
        dense_idx = O.HeadIndex(O.DENSE, n)

        def dense_err(item):
            h, a = item
            qh, kh, vh = f64(data["q"], h), f64(data["k"], h // g), f64(data["v"], h // g)
            ref, _ = O.head_attention(qh, kh, vh, w.scale, dense_idx, [a])[a]
            return float(np.abs(got_rows[item] - ref).max())

        errs = [dense_err(it) for it in items]
        bad = [(it, e) for it, e in zip(items, errs) if not e < atol]
        assert not bad, bad[:5]
        say(f"config {w.name}: dense comparator max abs error {max(errs):.3e} over {len(items)} blocks")
    return plan, data, oracle_index


def test_c1_vs_single_head_fp32():
    w = W.C1
    plan, data, oidx = check_layer(w, est_heads=[0], bs_all_rows_heads=[], bs_rows=[], full_index_heads=[0],
                                   idx_blocks=range(w.n_blocks), att_heads=[0],
                                   att_blocks=list(range(w.n_blocks)), dense_heads=[0],
                                   dense_blocks=list(range(w.n_blocks)))
    # end to end against the oracle's own estimate and index (equal here
    # unless a near tie flipped a selection)
    plan.attention()
    torch.cuda.synchronize()
    q64, k64, v64 = (W.to_f64(data[x][0, 0], "f32") for x in ("q", "k", "v"))
    own, _ = O.build_head_index(O.VSLASH, q64, k64, w.scale, last_q=w.last_q, n_vertical=w.n_vertical,
                                n_slash=w.n_slash)
    res = O.head_attention(q64, k64, v64, w.scale, own, range(w.n_blocks))
    ref = np.concatenate([res[a][0] for a in range(w.n_blocks)])
    err = np.abs(plan.o[0, 0].double().cpu().numpy() - ref).max()
    say(f"C1 end to end vs the oracle's own index: max abs {err:.3e}")
    assert err < F32_ATOL


def test_c2_block_sparse_gqa():
    w = W.C2
    nb = w.n_blocks
    blocks = _blocks_to_check(nb, 12, 2)
    check_layer(w, est_heads=range(w.heads_q), bs_all_rows_heads=range(w.heads_q), bs_rows=blocks,
                full_index_heads=[0, 13], idx_blocks=blocks, att_heads=list(range(0, 32, 3)),
                att_blocks=blocks)


def test_antidiag_estimate_32k():
    """Antidiagonal block scores on the 32K block-sparse layer: the weights of
    every causal block and the list of every row of two heads (one per kv
    group of the planted hot blocks) against the fp64 oracle."""
    w = W.C2
    nb = w.n_blocks
    say(f"{w.name}: antidiagonal estimate")
    data = W.generate(w, with_v=False)
    dev = torch.device("cuda")
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k = up(data["q"]), up(data["k"])
    heads = [0, 9]
    bidx, bcnt, gw = mi.antidiag_estimate(q, k, heads, w.top_blocks)
    torch.cuda.synchronize()
    tri = np.tril(np.ones((nb, nb), bool))
    for h in heads:
        g = gw[0, h].double().cpu().numpy()
        bi, bc = bidx[0, h].cpu().numpy(), bcnt[0, h].cpu().numpy()
        rw, _ = O.antidiag_estimate(W.to_f64(data["q"][0, h], w.dtype), W.to_f64(data["k"][0, h // w.group], w.dtype),
                                    w.scale, w.top_blocks)
        assert_scores_close(g[tri], rw[tri], f"antidiagonal weights h{h}")
        for a in range(nb):
            kk = min(w.top_blocks, a + 1)
            assert bc[a] == kk
            check_selection(bi[a], g[a, : a + 1], rw[a, : a + 1], kk, {0, a}, f"antidiag h{h} a{a}")


@pytest.mark.timeout(600)
def test_split_schedule_block_sparse_256k():
    """An all-Block-Sparse layer at 256K (8 query heads, 2 kv heads, top 100:
    the split schedule with long rows): outputs bit-identical to the joint
    schedule on the same lists stored with a larger capacity, and sampled
    query blocks against the oracle fed those lists."""
    n, hq, hkv, d, top = 262144, 8, 2, 128, 100
    nb = n // 64
    say(f"split schedule, block-sparse {n // 1024}K")
    g = torch.Generator(device="cuda").manual_seed(77)
    q = torch.randn(1, hq, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
    k = torch.randn(1, hkv, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
    v = torch.randn(1, hkv, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
    pat = [W.BSPARSE] * hq
    bidx, bcnt, _ = mi.block_estimate(q, k, list(range(hq)), top, return_scores=False)
    idx = mi.build_index(q, k, pat, None, None, bidx, bcnt, top)
    assert 4 * idx.block_cap <= nb
    o1, l1 = mi.sparse_prefill(q, k, v, pat, idx, schedule=True)
    big = mi.alloc_index(1, hq, n, nb // 4 + 1, 1, "cuda")  # a capacity too large for the split
    big.block_count.copy_(idx.block_count)
    big.block_idx.fill_(-1)
    big.block_idx[..., :idx.block_cap].copy_(idx.block_idx)
    assert 4 * big.block_cap > nb
    o2, l2 = mi.sparse_prefill(q, k, v, pat, big, schedule=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    q64, k64, v64 = (t[0].double().cpu().numpy() for t in (q, k, v))
    of, lf = o1[0].double().cpu().numpy(), l1[0].double().cpu().numpy()
    for h, a in ((0, 0), (3, 1), (5, nb // 2), (7, nb - 1), (6, 2047)):
        blocks, cols = gpu_index_lists(idx, 0, h, a)
        ref, rlse = O.attention_from_index(q64[h], k64[h // 4], v64[h // 4], d ** -0.5, a, blocks, cols)
        rows = slice(64 * a, 64 * a + 64)
        assert np.abs(of[h, rows] - ref).max() < BF16_ATOL, (h, a)
        assert np.abs(lf[h, rows] - rlse).max() < 1e-3, (h, a)


@pytest.mark.timeout(600)
def test_c3_vertical_slash_128k():
    w = W.C3
    nb = w.n_blocks
    check_layer(w, est_heads=range(w.heads_q), bs_all_rows_heads=[], bs_rows=[], full_index_heads=[0, 17],
                idx_blocks=_blocks_to_check(nb, 12, 3), att_heads=[0, 9, 17, 31],
                att_blocks=_blocks_to_check(nb, 12, 33), dense_heads=[5, 30],
                dense_blocks=_blocks_to_check(nb, 4, 34))


@pytest.mark.timeout(600)
def test_c4_mixed_256k():
    w = W.C4
    nb = w.n_blocks
    pats = W.head_patterns(w)
    vs_h = [int(h) for h in np.nonzero(pats == W.VSLASH)[0]]
    bs_h = [int(h) for h in np.nonzero(pats == W.BSPARSE)[0]]
    a_h = [int(h) for h in np.nonzero(pats == W.ASHAPE)[0]]
    check_layer(w, est_heads=vs_h + bs_h[:2], bs_all_rows_heads=bs_h[:1], bs_rows=_blocks_to_check(nb, 12, 4),
                full_index_heads=[vs_h[0], bs_h[0], a_h[0]], idx_blocks=_blocks_to_check(nb, 6, 44),
                att_heads=[vs_h[0], vs_h[-1], bs_h[0], a_h[0]], att_blocks=_blocks_to_check(nb, 12, 45))


@pytest.mark.timeout(900)
def test_c5_vertical_slash_1m():
    w = W.C5
    nb = w.n_blocks
    check_layer(w, est_heads=[0, 11, 22, 31], bs_all_rows_heads=[], bs_rows=[], full_index_heads=[7],
                idx_blocks=_blocks_to_check(nb, 4, 5), att_heads=[7, 8, 20, 31],
                att_blocks=_blocks_to_check(nb, 12, 55), dense_heads=[3],
                dense_blocks=_blocks_to_check(nb, 2, 56))


def _exact_rows(q64, k64, v64, scale, a, V, S):
    """Oracle rows of query block a over the exact Vertical-Slash key sets,
    one per-row gather each (the independent per-row formulation)."""
    out = np.empty((64, q64.shape[1]))
    for r in range(64):
        i = 64 * a + r
        out[r], _ = O.attention_row_gather(q64, k64, v64, scale, i, O.vs_exact_allowed(i, V, S))
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wname", ["c3local", "c3"])
def test_exact_vertical_slash_layer(wname):
    """The element-masked (exact) Vertical-Slash variant at 128K: on the
    clustered-slash layer (5% of tiles) and on the noise-driven one (99.7% of
    tiles).  The aligned-tile plan and the exact plan share the estimate; the
    exact plan's maps equal the selected sets, its index lists equal the
    aligned ones, and its rows equal attention over the exact key sets."""
    w = W.WORKLOADS[wname]
    say(f"exact variant {w.name}: generating")
    data = W.generate(w)
    dev = torch.device("cuda")
    q, k, v = (to_device(data[x], w.dtype, dev) for x in ("q", "k", "v"))
    kw = dict(last_q=w.last_q, n_vertical=w.n_vertical, n_slash=w.n_slash, force_vertical=w.force_vertical,
              force_slash=w.force_slash)
    aligned = mi.LayerPlan(q, k, v, [W.VSLASH] * w.heads_q, **kw)
    exact = mi.LayerPlan(q, k, v, [W.VSLASH_EXACT] * w.heads_q, **kw)
    aligned.run()
    exact.run()
    torch.cuda.synchronize()
    say(f"exact variant {w.name}: GPU layers done")
    assert torch.equal(aligned.vidx, exact.vidx) and torch.equal(aligned.sidx, exact.sidx)
    assert torch.equal(aligned.index.block_count, exact.index.block_count)
    assert torch.equal(aligned.index.col_count, exact.index.col_count)
    nb, g = w.n_blocks, w.group
    density = float(exact.index.block_count.double().sum()) / (w.heads_q * nb * (nb + 1) / 2)
    say(f"  tile density {density:.4f}")
    vidx, sidx = exact.vidx[0].cpu().numpy(), exact.sidx[0].cpu().numpy()
    bits = exact.index.vs_bits[0].cpu().numpy().view(np.uint32)
    blocks = _blocks_to_check(nb, 12, 77)
    for h in range(w.heads_q):
        Vh, Sh = vidx[h][vidx[h] >= 0], sidx[h][sidx[h] >= 0]
        for m, members in ((0, Vh), (1, Sh)):
            got = np.nonzero(np.unpackbits(bits[h, m].view(np.uint8), bitorder="little"))[0] - 64
            assert np.array_equal(got, members), (h, m)
    for h in (0, 9, 22, 31):
        Vh, Sh = vidx[h][vidx[h] >= 0], sidx[h][sidx[h] >= 0]
        q64, k64, v64 = (W.to_f64(data[x][0, hh], w.dtype) for x, hh in (("q", h), ("k", h // g), ("v", h // g)))
        for a in blocks:
            got = exact.o[0, h, 64 * a: 64 * a + 64].double().cpu().numpy()
            ref = _exact_rows(q64, k64, v64, w.scale, a, Vh, Sh)
            err = float(np.abs(got - ref).max())
            assert err < BF16_ATOL, (h, a, err)
    say(f"exact variant {w.name}: rows match the exact key sets")
