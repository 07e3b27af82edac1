"""The allocation-free attention entry point (mi_sparse_prefill_noalloc),
called through the C ABI, against mi_sparse_prefill with a caller workspace:
the same kernels on the same schedule, so outputs must be bit-identical.
Two calls in a row, the second with a smaller layer, then a layer whose
schedule exceeds the built-in buffer (rejected, nothing enqueued)."""
import ctypes

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_amd as mi
import workloads as W
from tests.parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mi.lib()


def _layer(seed, hq, hkv, n, pat):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(1, hq, n, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(1, hkv, n, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(1, hkv, n, 128, generator=g).to(torch.bfloat16).cuda()
    vs_h = [h for h, p in enumerate(pat) if p == W.VSLASH]
    bs_h = [h for h, p in enumerate(pat) if p == W.BSPARSE]
    vidx = sidx = bidx = bcnt = None
    if vs_h:
        vidx, sidx, _, _ = mi.vs_estimate(q, k, vs_h, 64, 60, 90, return_scores=False)
    if bs_h:
        bidx, bcnt, _ = mi.block_estimate(q, k, bs_h, 7, return_scores=False)
    idx = mi.build_index(q, k, pat, vidx, sidx, bidx, bcnt, 7, sink=100, local=600)
    return q, k, v, idx


def _both(q, k, v, pat, idx):
    o1, l1 = mi.sparse_prefill(q, k, v, pat, idx, sink=100, local=600, schedule=True)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full(l1.shape, float("nan"), dtype=torch.float32, device="cuda")
    mi.sparse_prefill_noalloc(q, k, v, pat, idx, sink=100, local=600, out=o2, lse=l2)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def test_noalloc_equals_workspace_entry_twice_then_smaller():
    pat = [W.VSLASH, W.ASHAPE, W.BSPARSE, W.DENSE, W.VSLASH, W.BSPARSE, W.DENSE, W.ASHAPE]
    for n, hq, hkv in ((64 * 90, 8, 2), (64 * 90, 8, 2), (64 * 23, 4, 2)):
        say(f"noalloc n={n} hq={hq} hkv={hkv}")
        p = pat[:hq]
        q, k, v, idx = _layer(n + hq, hq, hkv, n, p)
        (o1, l1), (o2, l2) = _both(q, k, v, p, idx)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # dense comparator (no index) through the same entry
    q, k, v, _ = _layer(5, 4, 1, 64 * 40, [W.DENSE] * 4)
    (o1, l1), (o2, l2) = _both(q, k, v, None, None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # all heads Block-Sparse with lists short enough for the split schedule
    bs = [W.BSPARSE] * 4
    q, k, v, idx = _layer(9, 4, 2, 64 * 40, bs)
    assert 4 * idx.block_cap <= 40
    (o1, l1), (o2, l2) = _both(q, k, v, bs, idx)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_rejects_schedules_above_the_buffer():
    # batch * heads_q * ceil(nb / 4) > the buffer: rejected on the host
    hq, n = 256, 64 * 4 * 1025
    # zero-stride views of one row: the call must reject before any launch
    row = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    q = row.as_strided((1, hq, n, 64), (0, 0, 0, 1))
    k = row.as_strided((1, 1, n, 64), (0, 0, 0, 1))
    o = torch.zeros(64, dtype=torch.bfloat16, device="cuda").as_strided((1, hq, n, 64), (0, 0, 0, 1))
    assert hq * (n // 256) > mi.NOALLOC_SCHEDULE_ENTRIES
    with pytest.raises(mi.MiError) as e:
        mi.sparse_prefill_noalloc(q, k, k, None, None, out=o)
    assert e.value.status == 5 and "built-in buffer" in str(e.value)


def test_noalloc_under_graph_capture():
    """The allocation-free entry point captured in a HIP graph (the callers it
    is for) and replayed three times, the outputs overwritten between replays:
    every replay equals the eager call bit for bit."""
    pat = [W.VSLASH, W.ASHAPE, W.BSPARSE, W.DENSE]
    q, k, v, idx = _layer(13, 4, 2, 64 * 50, pat)
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 64 * 50), dtype=torch.float32, device="cuda")
    mi.sparse_prefill_noalloc(q, k, v, pat, idx, sink=100, local=600, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mi.sparse_prefill_noalloc(q, k, v, pat, idx, sink=100, local=600, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mi.sparse_prefill_noalloc(q, k, v, pat, idx, sink=100, local=600, out=o, lse=lse)
    for rep in range(3):
        say(f"noalloc graph replay {rep}")
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep
