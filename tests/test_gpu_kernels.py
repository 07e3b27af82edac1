"""GPU parity of each entry point against the oracle at small sizes that
still span several tiles, chunks and ragged tails, plus edge cases.

Run on the GPU: every call goes through the C ABI (libmi_sparse.so)."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_amd as mi
import workloads as W
from oracle import minference_oracle as O
from tests.parity_util import (BF16_ATOL, F32_ATOL, assert_scores_close, check_selection, f64,
                               gpu_index_lists, say, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mi.lib()


def _inputs(seed, hq, hkv, n, d, dtype, batch=1, std=1.0):
    q, k, v = W.random_qkv(seed, hq, hkv, n, d, dtype, batch=batch, scale_std=std)
    return (q, k, v), tuple(to_device(x, dtype) for x in (q, k, v)), tuple(W.to_f64(x, dtype) for x in (q, k, v))


# ----------------------------------------------------------------- dense

@pytest.mark.parametrize("dtype,d,n,hq,hkv", [("f32", 64, 256, 2, 1), ("bf16", 128, 512, 4, 2),
                                              ("bf16", 64, 192, 3, 3), ("f32", 128, 128, 2, 2),
                                              ("bf16", 128, 64, 2, 1)])  # one query block
def test_dense_attention(dtype, d, n, hq, hkv):
    say(f"dense {dtype} d={d} n={n} hq={hq} hkv={hkv}")
    _, (q, k, v), (q64, k64, v64) = _inputs(1, hq, hkv, n, d, dtype)
    o, lse = mi.sparse_prefill(q, k, v, None, None)
    torch.cuda.synchronize()
    of, lf = f64(o), f64(lse)
    g = hq // hkv
    atol = F32_ATOL if dtype == "f32" else BF16_ATOL
    for h in range(hq):
        ref, rlse = O.dense_causal_attention(q64[0, h], k64[0, h // g], v64[0, h // g], d ** -0.5)
        assert np.abs(of[0, h] - ref).max() < atol, (h, np.abs(of[0, h] - ref).max())
        assert np.abs(lf[0, h] - rlse).max() < 1e-3


def test_dense_attention_strided_batch():
    """batch 2, inputs given as [B, N, H, d] memory viewed as [B, H, N, d]."""
    say("dense strided batch")
    B, hq, hkv, n, d = 2, 4, 2, 256, 128
    g = np.random.default_rng(3)
    qn = g.standard_normal((B, n, hq, d)).astype(np.float32)
    kn = g.standard_normal((B, n, hkv, d)).astype(np.float32)
    vn = g.standard_normal((B, n, hkv, d)).astype(np.float32)
    q = torch.from_numpy(qn).cuda().to(torch.bfloat16).transpose(1, 2)
    k = torch.from_numpy(kn).cuda().to(torch.bfloat16).transpose(1, 2)
    v = torch.from_numpy(vn).cuda().to(torch.bfloat16).transpose(1, 2)
    out = torch.empty((B, n, hq, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, _ = mi.sparse_prefill(q, k, v, None, None, out=out)
    torch.cuda.synchronize()
    of = f64(o)
    for b in range(B):
        for h in range(hq):
            qq, kk, vv = (f64(t[b, hh]) for t, hh in ((q, h), (k, h // 2), (v, h // 2)))
            ref, _ = O.dense_causal_attention(qq, kk, vv, d ** -0.5)
            assert np.abs(of[b, h] - ref).max() < BF16_ATOL


# ----------------------------------------------------------------- attention from a given index

def _random_index(rng, nb, n, with_cols=True):
    lists, cols = [], []
    for a in range(nb):
        k = rng.integers(1, a + 2)
        bl = np.unique(np.concatenate([[a], rng.choice(a + 1, k, replace=True)]))
        lists.append(bl)
        if with_cols:
            cand = np.arange(64 * a + 64)
            cand = cand[~np.isin(cand // 64, bl)]
            m = min(len(cand), int(rng.integers(0, 150)))
            cols.append(np.sort(rng.choice(cand, m, replace=False)) if m else np.zeros(0, np.int64))
        else:
            cols.append(np.zeros(0, np.int64))
    return lists, cols


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_attention_given_index(dtype, d):
    """Block lists and ragged column lists chosen at random (not by an estimate)."""
    say(f"attention from a random index {dtype} d={d}")
    hq, hkv, n = 2, 1, 64 * 11
    nb = n // 64
    _, (q, k, v), (q64, k64, v64) = _inputs(5, hq, hkv, n, d, dtype)
    rng = np.random.default_rng(7)
    bcap, ccap = nb, 160
    idx = mi.alloc_index(1, hq, n, bcap, ccap, "cuda")
    ref_lists = {}
    bc = np.zeros((1, hq, nb), np.int32)
    bi = -np.ones((1, hq, nb, bcap), np.int32)
    cc = np.zeros((1, hq, nb), np.int32)
    ci = -np.ones((1, hq, nb, ccap), np.int32)
    for h in range(hq):
        lists, cols = _random_index(rng, nb, n)
        for a in range(nb):
            bc[0, h, a] = len(lists[a]); bi[0, h, a, :len(lists[a])] = lists[a]
            cc[0, h, a] = len(cols[a]); ci[0, h, a, :len(cols[a])] = cols[a]
            ref_lists[h, a] = (lists[a], cols[a])
    for t, src in ((idx.block_count, bc), (idx.block_idx, bi), (idx.col_count, cc), (idx.col_idx, ci)):
        t.copy_(torch.from_numpy(src))
    o, lse = mi.sparse_prefill(q, k, v, [W.VSLASH] * hq, idx)
    torch.cuda.synchronize()
    of, lf = f64(o), f64(lse)
    atol = F32_ATOL if dtype == "f32" else BF16_ATOL
    for h in range(hq):
        for a in range(nb):
            blocks, cols = ref_lists[h, a]
            ref, rlse = O.attention_from_index(q64[0, h], k64[0, 0], v64[0, 0], d ** -0.5, a, blocks, cols)
            rows = slice(64 * a, 64 * a + 64)
            assert np.abs(of[0, h, rows] - ref).max() < atol, (h, a)
            assert np.abs(lf[0, h, rows] - rlse).max() < 1e-3


@pytest.mark.parametrize("sink,local", [(128, 256), (0, 1), (64, 64), (100, 300), (5, 1000)])
def test_ashape_attention(sink, local):
    say(f"A-shape sink={sink} local={local}")
    hq, hkv, n, d = 2, 1, 64 * 13, 128
    _, (q, k, v), (q64, k64, v64) = _inputs(9, hq, hkv, n, d, "bf16")
    idx = mi.build_index(q, k, [W.ASHAPE] * hq, sink=sink, local=local)
    o, _ = mi.sparse_prefill(q, k, v, [W.ASHAPE] * hq, idx, sink=sink, local=local)
    torch.cuda.synchronize()
    of = f64(o)
    for h in range(hq):
        for a in range(n // 64):
            blocks, cols = gpu_index_lists(idx, 0, h, a)
            assert list(blocks) == list(O.ashape_block_list(a, sink, local, n))
            assert len(cols) == 0
            rows = np.arange(64 * a, 64 * a + 64)
            ref, _ = O.ashape_attention(q64[0, h], k64[0, 0], v64[0, 0], d ** -0.5, rows, sink, local)
            assert np.abs(of[0, h, rows] - ref).max() < BF16_ATOL, (h, a)


# ----------------------------------------------------------------- Vertical-Slash estimate

@pytest.mark.parametrize("dtype,d,n,last_q,nv,ns,fv,fs", [
    ("f32", 64, 2048, 64, 64, 128, 1, 1),
    ("bf16", 128, 64 * 37, 64, 100, 300, 1, 1),     # ragged: N not a multiple of the chunks
    ("bf16", 128, 640, 17, 40, 50, 3, 2),           # last_q < 64, wider forced sets
    ("bf16", 64, 128, 64, 500, 500, 1, 1),          # budgets above N: clamped, -1 padded
    ("f32", 128, 64, 1, 8, 8, 1, 1),                # single block, single query
])
def test_vs_estimate(dtype, d, n, last_q, nv, ns, fv, fs):
    say(f"vs_estimate {dtype} d={d} n={n} last_q={last_q} nv={nv} ns={ns}")
    hq, hkv = 4, 2
    _, (q, k, _), (q64, k64, _) = _inputs(11, hq, hkv, n, d, dtype)
    heads = [0, 1, 3]
    vidx, sidx, vsc, ssc = mi.vs_estimate(q, k, heads, last_q, nv, ns, fv, fs)
    torch.cuda.synchronize()
    vsc, ssc, vidx, sidx = f64(vsc), f64(ssc), vidx.cpu().numpy(), sidx.cpu().numpy()
    for h in heads:
        rv, rs = O.vs_estimate(q64[0, h], k64[0, h // 2], d ** -0.5, last_q)
        assert_scores_close(vsc[0, h], rv, f"vertical h{h}")
        assert_scores_close(ssc[0, h], rs, f"slash h{h}")
        check_selection(vidx[0, h], vsc[0, h], rv, nv, range(fv), f"vertical h{h}")
        check_selection(sidx[0, h], ssc[0, h], rs, ns, range(fs), f"slash h{h}")
    assert not vsc[0, 2].any() and not vidx[0, 2].any()  # unlisted head untouched


@pytest.mark.parametrize("hq,hkv,batch,heads", [
    (12, 1, 1, [0, 1, 2, 5, 7, 9, 11]),   # seven heads of one kv head: two sets
    (3, 3, 2, [0, 2]),                    # one head per kv head, batch 2
    (8, 2, 1, list(range(8))),            # full sets
])
def test_vs_estimate_head_sets(hq, hkv, batch, heads):
    """Row statistics share each staged K tile among the listed heads of one
    kv head (sets of at most four): every grouping gives the oracle's scores."""
    say(f"vs_estimate head sets hq={hq} hkv={hkv} batch={batch} heads={heads}")
    n, d, last_q, nv, ns = 64 * 21, 128, 64, 30, 50
    _, (q, k, _), (q64, k64, _) = _inputs(13, hq, hkv, n, d, "bf16", batch=batch)
    vidx, sidx, vsc, ssc = mi.vs_estimate(q, k, heads, last_q, nv, ns, 1, 1)
    torch.cuda.synchronize()
    vsc, ssc, vidx, sidx = f64(vsc), f64(ssc), vidx.cpu().numpy(), sidx.cpu().numpy()
    g = hq // hkv
    for b in range(batch):
        for h in heads:
            rv, rs = O.vs_estimate(q64[b, h], k64[b, h // g], d ** -0.5, last_q)
            assert_scores_close(vsc[b, h], rv, f"vertical b{b} h{h}")
            assert_scores_close(ssc[b, h], rs, f"slash b{b} h{h}")
            check_selection(vidx[b, h], vsc[b, h], rv, nv, range(1), f"vertical b{b} h{h}")
            check_selection(sidx[b, h], ssc[b, h], rs, ns, range(1), f"slash b{b} h{h}")


def test_vs_estimate_without_score_outputs_is_identical():
    say("vs_estimate workspace scores")
    _, (q, k, _), _ = _inputs(12, 2, 1, 1024, 128, "bf16")
    a = mi.vs_estimate(q, k, [0, 1], 64, 50, 80)
    b = mi.vs_estimate(q, k, [0, 1], 64, 50, 80, return_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------- Block-Sparse estimate

@pytest.mark.parametrize("dtype,d,n,top", [("bf16", 128, 64 * 40, 6), ("f32", 64, 64 * 9, 3),
                                           ("bf16", 128, 64 * 5, 100), ("bf16", 64, 64 * 70, 2)])
def test_block_estimate(dtype, d, n, top):
    say(f"block_estimate {dtype} d={d} n={n} top={top}")
    hq, hkv = 4, 2
    _, (q, k, _), (q64, k64, _) = _inputs(13, hq, hkv, n, d, dtype)
    heads = [1, 2]
    bidx, bcnt, w = mi.block_estimate(q, k, heads, top)
    torch.cuda.synchronize()
    bidx, bcnt, w = bidx.cpu().numpy(), bcnt.cpu().numpy(), f64(w)
    nb = n // 64
    for h in heads:
        rw, kept = O.bs_estimate(q64[0, h], k64[0, h // 2], d ** -0.5, top)
        tri = np.tril(np.ones((nb, nb), bool))
        assert_scores_close(w[0, h][tri], rw[tri], f"block weights h{h}")
        assert not w[0, h][~tri].any()
        for a in range(nb):
            kk = min(top, a + 1)
            assert bcnt[0, h, a] == kk
            check_selection(bidx[0, h, a], w[0, h, a, : a + 1], rw[a, : a + 1], kk, {0, a},
                            f"blocks h{h} a{a}")


@pytest.mark.parametrize("nb", [128, 129, 512, 513, 700, 1024, 1025, 1500, 2048, 2049, 4096, 4097, 4200])
def test_block_estimate_long_rows(nb):
    """Every row of layers whose block count sits on each side of the
    estimate's dispatch boundaries: the fused scores+select kernel (rows of up
    to 512 blocks), one wavefront per row holding 16, 32 or 64 register slots
    per lane (rows of up to 1024, 2048, 4096 blocks), and a workgroup per row
    above 4096 blocks; with and without the weights stored."""
    say(f"block_estimate long rows nb={nb}")
    n, d, top = 64 * nb, 64, 20
    _, (q, k, _), (q64, k64, _) = _inputs(14, 1, 1, n, d, "bf16")
    bidx, bcnt, w = mi.block_estimate(q, k, [0], top)
    torch.cuda.synchronize()
    bidx, bcnt, w = bidx.cpu().numpy(), bcnt.cpu().numpy(), f64(w)
    # without block_score: the weights are never stored (rows of up to 512
    # blocks keep the scores on chip too), and the lists are identical
    nb_idx, nb_cnt, none = mi.block_estimate(q, k, [0], top, return_scores=False)
    torch.cuda.synchronize()
    assert none is None
    assert np.array_equal(nb_idx.cpu().numpy(), bidx) and np.array_equal(nb_cnt.cpu().numpy(), bcnt)
    rw, _ = O.bs_estimate(q64[0, 0], k64[0, 0], d ** -0.5, top)
    tri = np.tril(np.ones((nb, nb), bool))
    assert_scores_close(w[0, 0][tri], rw[tri], "block weights")
    assert not w[0, 0][~tri].any()
    for a in range(nb):
        kk = min(top, a + 1)
        assert bcnt[0, 0, a] == kk
        check_selection(bidx[0, 0, a], w[0, 0, a, : a + 1], rw[a, : a + 1], kk, {0, a}, f"blocks a{a}")


@pytest.mark.parametrize("nb,top,const", [(1500, 200, False), (2049, 129, False), (4096, 128, False),
                                          (2049, 20, True), (700, 100, True)])
def test_block_estimate_long_rows_selection_routes(nb, top, const):
    """Rows above 512 blocks take one of three selection routes: the filter
    (survivors of the per-lane top-2 threshold, k <= 128), the radix select
    (k > 128), and the radix select again when exact ties leave more
    survivors than the filter's buffer holds (constant inputs: every weight
    of a row equal, so the lowest blocks are kept).  Every row is checked."""
    say(f"block_estimate routes nb={nb} top={top} const={const}")
    n, d = 64 * nb, 64
    if const:
        qn = np.full((1, 1, n, d), 0.25, np.float32)
        q = to_device(qn, "f32")
        k = to_device(qn.copy(), "f32")
        q64 = k64 = qn.astype(np.float64)
    else:
        _, (q, k, _), (q64, k64, _) = _inputs(19, 1, 1, n, d, "bf16")
    bidx, bcnt, w = mi.block_estimate(q, k, [0], top)
    torch.cuda.synchronize()
    bidx, bcnt, w = bidx.cpu().numpy(), bcnt.cpu().numpy(), f64(w)
    rw, _ = O.bs_estimate(q64[0, 0], k64[0, 0], d ** -0.5, top)
    tri = np.tril(np.ones((nb, nb), bool))
    assert_scores_close(w[0, 0][tri], rw[tri], "block weights")
    for a in range(nb):
        kk = min(top, a + 1)
        assert bcnt[0, 0, a] == kk
        check_selection(bidx[0, 0, a], w[0, 0, a, : a + 1], rw[a, : a + 1], kk, {0, a}, f"blocks a{a}")


# ----------------------------------------------------------------- index building

@pytest.mark.parametrize("n,nv,ns", [(64 * 23, 40, 60), (64 * 8, 600, 600), (64 * 40, 5, 1)])
def test_build_index_vs(n, nv, ns):
    say(f"build_index VS n={n} nv={nv} ns={ns}")
    hq, hkv, d = 2, 1, 128
    _, (q, k, _), _ = _inputs(17, hq, hkv, n, d, "bf16")
    vidx, sidx, _, _ = mi.vs_estimate(q, k, [0, 1], 64, nv, ns)
    idx = mi.build_index(q, k, [W.VSLASH] * hq, vidx, sidx)
    torch.cuda.synchronize()
    V, S = vidx.cpu().numpy(), sidx.cpu().numpy()
    for h in range(hq):
        Vh, Sh = V[0, h][V[0, h] >= 0], S[0, h][S[0, h] >= 0]
        for a in range(n // 64):
            blocks, cols = gpu_index_lists(idx, 0, h, a)
            rb = O.vs_block_list(a, Sh)
            assert np.array_equal(blocks, rb), (h, a)
            assert np.array_equal(cols, O.vs_column_list(a, Vh, rb)), (h, a)
        assert np.all(idx.block_idx[0, h].cpu().numpy()[np.arange(idx.block_cap)[None, :] >=
                                                        idx.block_count[0, h].cpu().numpy()[:, None]] == -1)


def test_build_index_mixed_and_dense_counts():
    say("build_index mixed")
    n, hq, hkv, d = 64 * 19, 4, 2, 128
    _, (q, k, _), _ = _inputs(19, hq, hkv, n, d, "bf16")
    pat = [W.BSPARSE, W.DENSE, W.ASHAPE, W.BSPARSE]
    bidx, bcnt, _ = mi.block_estimate(q, k, [0, 3], 5)
    idx = mi.build_index(q, k, pat, None, None, bidx, bcnt, 5, sink=70, local=200)
    torch.cuda.synchronize()
    B = bidx.cpu().numpy()
    for a in range(n // 64):
        for h in (0, 3):
            blocks, cols = gpu_index_lists(idx, 0, h, a)
            assert np.array_equal(blocks, B[0, h, a, : min(5, a + 1)]) and len(cols) == 0
        assert int(idx.block_count[0, 1, a]) == a + 1 and int(idx.col_count[0, 1, a]) == 0
        blocks, _ = gpu_index_lists(idx, 0, 2, a)
        assert list(blocks) == list(O.ashape_block_list(a, 70, 200, n))


def test_index_is_deterministic():
    say("determinism")
    n = 64 * 30
    _, (q, k, _), _ = _inputs(23, 4, 2, n, 128, "bf16")
    outs = []
    for _ in range(2):
        vidx, sidx, vs, ss = mi.vs_estimate(q, k, [0, 1, 2, 3], 64, 70, 90)
        bidx, bcnt, w = mi.block_estimate(q, k, [0, 1, 2, 3], 7)
        idx = mi.build_index(q, k, [W.VSLASH] * 4, vidx, sidx)
        outs.append([vidx, sidx, vs, ss, bidx, bcnt, w, idx.block_idx, idx.col_idx])
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("n,hq,hkv,batch", [(64 * 45, 8, 2, 2), (64 * 13, 4, 4, 1)])
def test_schedule_changes_order_not_results(n, hq, hkv, batch):
    """With the item schedule (workspace given) the attention runs its items
    in another order and on other XCDs; each item's arithmetic is unchanged,
    so O and lse must be bit-identical to the default order, for a mix of all
    four patterns with a ragged last run."""
    say(f"schedule parity n={n} hq={hq} hkv={hkv} batch={batch}")
    g = torch.Generator(device="cpu").manual_seed(7)
    q = torch.randn(batch, hq, n, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(batch, hkv, n, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(batch, hkv, n, 128, generator=g).to(torch.bfloat16).cuda()
    pat = [W.VSLASH, W.ASHAPE, W.BSPARSE, W.DENSE, W.BSPARSE, W.VSLASH, W.DENSE, W.ASHAPE][:hq]
    vs_h = [h for h, p in enumerate(pat) if p == W.VSLASH]
    bs_h = [h for h, p in enumerate(pat) if p == W.BSPARSE]
    vidx, sidx, _, _ = mi.vs_estimate(q, k, vs_h, 64, 90, 120)
    bidx, bcnt, _ = mi.block_estimate(q, k, bs_h, 9)
    idx = mi.build_index(q, k, pat, vidx, sidx, bidx, bcnt, 9, sink=100, local=700)
    o1, l1 = mi.sparse_prefill(q, k, v, pat, idx, sink=100, local=700)
    o2, l2 = mi.sparse_prefill(q, k, v, pat, idx, sink=100, local=700, schedule=True)
    o3, l3 = mi.sparse_prefill(q, k, v, None, None)
    o4, l4 = mi.sparse_prefill(q, k, v, None, None, schedule=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


@pytest.mark.parametrize("n,hq,hkv,batch,pat", [
    (64 * 45, 8, 2, 2, [1, 0, 2, 3, 2, 1, 3, 0]),
    (64 * 13, 4, 4, 1, [0, 1, 2, 3]),
    (64 * 300, 32, 8, 1, None),
    (64 * 97, 12, 3, 3, [2, 2, 0, 1, 1, 1, 1, 0, 2, 3, 3, 0]),
])
def test_device_schedule_equals_host_schedule(n, hq, hkv, batch, pat):
    """The schedule the library builds in the workspace on the device is the
    host's stable sort of the same chunks (mi_attn_schedule), entry for entry."""
    say(f"device schedule n={n} hq={hq} hkv={hkv} batch={batch}")
    q = torch.zeros(batch, hq, n, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(batch, hkv, n, 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    block_cap = 9
    idx = None
    if pat is not None:
        bcap, ccap = mi.index_caps(n, pat, 30, 40, block_cap, 100, 700)
        idx = mi.alloc_index(batch, hq, n, bcap, ccap, "cuda")
        block_cap = bcap
        # a valid (diagonal-only) index: every row lists its own block
        nb = n // 64
        idx.block_count.fill_(1)
        idx.block_idx.fill_(-1)
        idx.block_idx[..., 0] = torch.arange(nb, dtype=torch.int32, device="cuda")
    host = mi.attn_schedule(q, k, pat, 100, 700, block_cap)
    desc = mi.make_desc(q, k, v, q)
    ws = torch.full((mi.workspace_bytes(desc, mi.OP_SPARSE_PREFILL),), 0x7f, dtype=torch.uint8, device="cuda")
    mi.sparse_prefill(q, k, v, pat, idx, sink=100, local=700, workspace=ws)
    torch.cuda.synchronize()
    dev = ws[: 4 * len(host)].view(torch.int32).cpu().tolist()
    assert dev == host
    nruns = (n // 64 + 3) // 4
    items = sorted(x for x in host if x >= 0)
    assert items == list(range(batch * hq * nruns))



# ----------------------------------------------------------------- exact Vertical-Slash variant

@pytest.mark.parametrize("dtype,d,n,nv,ns", [("bf16", 128, 64 * 23, 40, 90), ("f32", 64, 64 * 13, 30, 50),
                                              ("bf16", 64, 64 * 9, 600, 600), ("f32", 128, 64 * 7, 5, 3)])
def test_exact_vertical_slash_attention(dtype, d, n, nv, ns):
    """MI_VSLASH_EXACT heads: the same tile and column lists as Vertical-Slash
    heads, membership maps equal to the selected sets, and outputs equal to
    attention over the exact key sets {j in V} u {i - o : o in S} (j <= i)."""
    say(f"exact vertical-slash {dtype} d={d} n={n} nv={nv} ns={ns}")
    hq, hkv = 3, 1
    _, (q, k, v), (q64, k64, v64) = _inputs(29, hq, hkv, n, d, dtype)
    pat = [W.VSLASH_EXACT, W.VSLASH, W.VSLASH_EXACT]
    vidx, sidx, _, _ = mi.vs_estimate(q, k, [0, 1, 2], 64, nv, ns)
    idx = mi.build_index(q, k, pat, vidx, sidx)
    o, lse = mi.sparse_prefill(q, k, v, pat, idx)
    torch.cuda.synchronize()
    of, lf = f64(o), f64(lse)
    V, S = vidx.cpu().numpy(), sidx.cpu().numpy()
    bits = idx.vs_bits.cpu().numpy().view(np.uint32)
    atol = F32_ATOL if dtype == "f32" else BF16_ATOL
    nb = n // 64
    for h in range(hq):
        Vh, Sh = V[0, h][V[0, h] >= 0], S[0, h][S[0, h] >= 0]
        for a in range(nb):
            blocks, cols = gpu_index_lists(idx, 0, h, a)
            rb = O.vs_block_list(a, Sh)
            assert np.array_equal(blocks, rb) and np.array_equal(cols, O.vs_column_list(a, Vh, rb)), (h, a)
        if pat[h] == W.VSLASH_EXACT:
            for m, members in ((0, Vh), (1, Sh)):
                got = np.nonzero(np.unpackbits(bits[0, h, m].view(np.uint8), bitorder="little"))[0] - 64
                assert np.array_equal(got, np.sort(members)), (h, m)
            res = {a: O.vs_exact_attention(q64[0, h], k64[0, 0], v64[0, 0], d ** -0.5,
                                           np.arange(64 * a, 64 * a + 64), Vh, Sh) for a in range(nb)}
        else:
            res = O.head_attention(q64[0, h], k64[0, 0], v64[0, 0], d ** -0.5, O.HeadIndex(O.VSLASH, n, V=Vh, S=Sh),
                                   range(nb))
        for a, (ref, rlse) in res.items():
            rows = slice(64 * a, 64 * a + 64)
            assert np.abs(of[0, h, rows] - ref).max() < atol, (h, a, np.abs(of[0, h, rows] - ref).max())
            assert np.abs(lf[0, h, rows] - rlse).max() < 1e-3, (h, a)


def test_exact_vertical_slash_needs_maps():
    """An exact head without membership maps is rejected before any launch."""
    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16, device="cuda")
    idx = mi.alloc_index(1, 1, 128, 4, 4, "cuda")  # no vs_bits
    with pytest.raises(mi.MiError) as e:
        mi.sparse_prefill(q, q, q, [W.VSLASH_EXACT], idx)
    assert e.value.status == 1 and "vs_bits" in str(e.value)


# ----------------------------------------------------------------- antidiagonal block scores

@pytest.mark.parametrize("dtype,d,n,top", [("bf16", 128, 64 * 40, 6), ("f32", 64, 64 * 9, 3),
                                           ("bf16", 64, 64 * 70, 2), ("bf16", 128, 64 * 33, 100),
                                           ("f32", 128, 64 * 37, 5), ("bf16", 128, 64, 3)])  # last: one block
def test_antidiag_estimate(dtype, d, n, top):
    """Weights of every causal block and every row's list against the fp64
    oracle; the lists are the same when the weights are not stored; heads
    not listed are left alone."""
    say(f"antidiag_estimate {dtype} d={d} n={n} top={top}")
    hq, hkv = 4, 2
    _, (q, k, _), (q64, k64, _) = _inputs(31, hq, hkv, n, d, dtype, std=0.5)
    heads = [1, 2]
    bidx, bcnt, w = mi.antidiag_estimate(q, k, heads, top)
    nidx, ncnt, none = mi.antidiag_estimate(q, k, heads, top, return_scores=False)
    torch.cuda.synchronize()
    assert none is None
    bidx, bcnt, w = bidx.cpu().numpy(), bcnt.cpu().numpy(), f64(w)
    assert np.array_equal(nidx.cpu().numpy(), bidx) and np.array_equal(ncnt.cpu().numpy(), bcnt)
    nb = n // 64
    tri = np.tril(np.ones((nb, nb), bool))
    for h in heads:
        rw, _ = O.antidiag_estimate(q64[0, h], k64[0, h // 2], d ** -0.5, top)
        assert_scores_close(w[0, h][tri], rw[tri], f"antidiagonal weights h{h}")
        assert not w[0, h][~tri].any()
        for a in range(nb):
            kk = min(top, a + 1)
            assert bcnt[0, h, a] == kk
            check_selection(bidx[0, h, a], w[0, h, a, : a + 1], rw[a, : a + 1], kk, {0, a}, f"antidiag h{h} a{a}")
    assert not bcnt[0, 0].any() and not bcnt[0, 3].any()


@pytest.mark.parametrize("nb", [129, 513, 1025, 2049])
def test_antidiag_long_rows(nb):
    """Every row of layers on each side of the selection's dispatch
    boundaries (register slots per lane 8, 16, 32, 64)."""
    say(f"antidiag_estimate long rows nb={nb}")
    n, d, top = 64 * nb, 64, 20
    _, (q, k, _), (q64, k64, _) = _inputs(32, 1, 1, n, d, "bf16", std=0.5)
    bidx, bcnt, w = mi.antidiag_estimate(q, k, [0], top)
    torch.cuda.synchronize()
    bidx, bcnt, w = bidx.cpu().numpy(), bcnt.cpu().numpy(), f64(w)
    rw, _ = O.antidiag_estimate(q64[0, 0], k64[0, 0], d ** -0.5, top)
    tri = np.tril(np.ones((nb, nb), bool))
    assert_scores_close(w[0, 0][tri], rw[tri], "antidiagonal weights")
    for a in range(nb):
        kk = min(top, a + 1)
        assert bcnt[0, 0, a] == kk
        check_selection(bidx[0, 0, a], w[0, 0, a, : a + 1], rw[a, : a + 1], kk, {0, a}, f"antidiag a{a}")


def test_antidiag_lists_drive_the_attention():
    """Lists from the antidiagonal estimate, used as Block-Sparse lists by the
    index and the attention, against the oracle's attention over them."""
    say("antidiag lists -> attention")
    n, hq, hkv, d, top = 64 * 24, 4, 2, 128, 5
    _, (q, k, v), (q64, k64, v64) = _inputs(33, hq, hkv, n, d, "bf16", std=0.5)
    pat = [W.BSPARSE] * hq
    bidx, bcnt, _ = mi.antidiag_estimate(q, k, list(range(hq)), top, return_scores=False)
    idx = mi.build_index(q, k, pat, None, None, bidx, bcnt, top)
    o, _ = mi.sparse_prefill(q, k, v, pat, idx)
    torch.cuda.synchronize()
    of = f64(o)
    for h in range(hq):
        for a in (0, 7, 23):
            blocks, cols = gpu_index_lists(idx, 0, h, a)
            ref, _ = O.attention_from_index(q64[0, h], k64[0, h // 2], v64[0, h // 2], d ** -0.5, a, blocks, cols)
            assert np.abs(of[0, h, 64 * a: 64 * a + 64] - ref).max() < BF16_ATOL, (h, a)


# ----------------------------------------------------------------- split schedule

@pytest.mark.parametrize("dtype,d,batch", [("bf16", 128, 1), ("f32", 64, 1), ("bf16", 64, 1), ("bf16", 128, 2)])
def test_block_sparse_split_schedule(dtype, d, batch):
    """Launches whose heads are all Block-Sparse, with lists short enough for
    two per item (4 * block_cap <= nb), run one step list per ping-pong group.
    Random lists of uneven length (group 0's blocks long, group 1's short, and
    the reverse on other heads) over a ragged number of blocks: every query
    block against the oracle, and bit for bit against the joint schedule that
    the same lists stored with a larger capacity select."""
    say(f"split schedule {dtype} d={d} batch={batch}")
    hq, hkv, n = 4, 2, 64 * 43
    nb = n // 64
    _, (q, k, v), (q64, k64, v64) = _inputs(21, hq, hkv, n, d, dtype, batch=batch)
    rng = np.random.default_rng(5)
    cap = nb // 4
    lists = {}
    for b in range(batch):
        for h in range(hq):
            for a in range(nb):
                long_grp = (a % 4) // 2 == (h + b) % 2
                kk = min(a + 1, cap if long_grp else int(rng.integers(1, 3)))
                rest = rng.choice(a, kk - 1, replace=False) if a > 0 and kk > 1 else np.zeros(0, np.int64)
                lists[b, h, a] = np.sort(np.concatenate([[a], rest])).astype(np.int64)
    outs = []
    for bcap in (cap, nb):
        assert (4 * bcap <= nb) == (bcap == cap)
        idx = mi.alloc_index(batch, hq, n, bcap, 0, "cuda")
        bc = np.zeros((batch, hq, nb), np.int32)
        bi = -np.ones((batch, hq, nb, bcap), np.int32)
        for (b, h, a), bl in lists.items():
            bc[b, h, a] = len(bl)
            bi[b, h, a, :len(bl)] = bl
        idx.block_count.copy_(torch.from_numpy(bc))
        idx.block_idx.copy_(torch.from_numpy(bi))
        outs.append(mi.sparse_prefill(q, k, v, [W.BSPARSE] * hq, idx))
    torch.cuda.synchronize()
    (o_split, l_split), (o_joint, l_joint) = outs
    assert torch.equal(o_split, o_joint) and torch.equal(l_split, l_joint)
    of, lf = f64(o_split), f64(l_split)
    atol = F32_ATOL if dtype == "f32" else BF16_ATOL
    for (b, h, a), bl in lists.items():
        ref, rlse = O.attention_from_index(q64[b, h], k64[b, h // 2], v64[b, h // 2], d ** -0.5, a, bl,
                                           np.zeros(0, np.int64))
        rows = slice(64 * a, 64 * a + 64)
        assert np.abs(of[b, h, rows] - ref).max() < atol, (b, h, a)
        assert np.abs(lf[b, h, rows] - rlse).max() < 1e-3, (b, h, a)


# ----------------------------------------------------------------- graph capture

def test_layer_plan_graph_replays_match_eager():
    """A layer's launches (estimates, index, attention) captured once in a
    HIP graph and replayed three times, with eager work that overwrites every
    output and intermediate buffer and a synchronisation between replays:
    every replay equals the eager run bit for bit."""
    say("graph capture of a layer plan")
    hq, hkv, n = 8, 2, 64 * 48
    pat = [W.VSLASH, W.ASHAPE, W.BSPARSE, W.DENSE, W.VSLASH, W.BSPARSE, W.VSLASH, W.ASHAPE]
    _, (q, k, v), _ = _inputs(41, hq, hkv, n, 128, "bf16")
    plan = mi.LayerPlan(q, k, v, pat, last_q=64, n_vertical=60, n_slash=90, top_blocks=7, sink=100,
                        local=600, with_lse=True)
    plan.run()
    torch.cuda.synchronize()
    o_ref, l_ref = plan.o.clone(), plan.lse.clone()
    bufs = [plan.vidx, plan.sidx, plan.bidx, plan.bcnt, plan.index.block_count, plan.index.block_idx,
            plan.index.col_count, plan.index.col_idx]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run()  # warm-up on the capture stream's side, as torch requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run()
    for rep in range(3):
        plan.o.fill_(float("nan"))
        plan.lse.fill_(float("nan"))
        for b in bufs:
            b.fill_(-7 - rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.o, o_ref) and torch.equal(plan.lse, l_ref), rep


def test_rows_with_no_keys():
    """Query blocks whose lists are empty (possible only through a caller's own
    index; the estimates always keep the forced keys): their rows come out
    as zeros with log-sum-exp -inf, and the other blocks are unaffected."""
    say("empty lists")
    hq, hkv, n, d = 2, 1, 64 * 9, 128
    _, (q, k, v), (q64, k64, v64) = _inputs(17, hq, hkv, n, d, "bf16")
    nb = n // 64
    idx = mi.alloc_index(1, hq, n, nb, 64, "cuda")
    bc = np.zeros((1, hq, nb), np.int32)
    bi = -np.ones((1, hq, nb, nb), np.int32)
    empty = {(0, 3), (0, 8), (1, 0), (1, 4), (1, 5), (1, 6), (1, 7)}  # head 1's second item: no steps at all
    for h in range(hq):
        for a in range(nb):
            if (h, a) not in empty:
                bc[0, h, a] = a + 1
                bi[0, h, a, :a + 1] = np.arange(a + 1)
    idx.block_count.copy_(torch.from_numpy(bc))
    idx.block_idx.copy_(torch.from_numpy(bi))
    for pat in (W.BSPARSE, W.VSLASH):
        o, lse = mi.sparse_prefill(q, k, v, [pat] * hq, idx)
        torch.cuda.synchronize()
        of, lf = f64(o), f64(lse)
        for h in range(hq):
            for a in range(nb):
                rows = slice(64 * a, 64 * a + 64)
                if (h, a) in empty:
                    assert not of[0, h, rows].any() and np.all(np.isneginf(lf[0, h, rows])), (pat, h, a)
                else:
                    ref, rlse = O.attention_from_index(q64[0, h], k64[0, 0], v64[0, 0], d ** -0.5, a,
                                                       np.arange(a + 1), np.zeros(0, np.int64))
                    assert np.abs(of[0, h, rows] - ref).max() < BF16_ATOL, (pat, h, a)
                    assert np.abs(lf[0, h, rows] - rlse).max() < 1e-3
