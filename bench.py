"""Benchmark of one layer of dynamic sparse prefill attention on one MI355X.

A step is one pass of the whole hot path over a resident synthetic layer:
the Vertical-Slash / Block-Sparse estimates (with top-k), the index build and
the sparse attention, all enqueued on one stream.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config c3|c5|c2|c4|c1] [--no-cpu-baseline] [--no-1m]

Default workload: the LLaMA-3-8B-shaped Vertical-Slash layer at 128K tokens
(32 query / 8 kv heads, d=128, bf16, budgets 1000 verticals / 6096 slashes);
`value` is its ms/layer.  The same line also carries the 1M-token layer of the
same shape (two timed steps) and, for both, the dense causal attention kernel
of the library timed on the same inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/layer sparse prefill attention at 128K & 1M; achieved MFMA TFLOP/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
W_VS = 1  # Vertical-Slash pattern code


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense causal comparator")
    ap.add_argument("--no-1m", action="store_true", help="skip the 1M-token secondary measurement")
    ap.add_argument("--no-gather", action="store_true", help="skip the isolated column-gather rate")
    ap.add_argument("--no-antidiag", action="store_true", help="skip the antidiagonal block estimate")
    ap.add_argument("--library-context", action="store_true",
                    help="also time torch's bf16 GEMM and its flash SDPA (causal) at the layer's shape")
    ap.add_argument("--dense-sweep", action="store_true",
                    help="also time the dense causal comparator and torch's flash SDPA over sequence lengths")
    ap.add_argument("--no-exact", action="store_true",
                    help="skip the exact (element-masked) Vertical-Slash variant and the clustered-slash layer")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 4 times (counter calibration)")
    ap.add_argument("--gather-only", action="store_true",
                    help="only the isolated column-gather measurement on the workload's inputs "
                         "(eight attention launches: four with the column index, four without columns)")
    return ap.parse_args()


def calibrate_copy():
    """A copy of known size: 4 launches, each reading and writing 1 GiB, so
    that HBM byte counters can be scaled against known traffic."""
    import torch
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(4):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": {"launches": 4, "bytes_read_per_launch": 1 << 30,
                                         "bytes_written_per_launch": 1 << 30}}))


def profile_record(workload: str):
    """The committed rocprofv3 record of this workload's layer if it was taken
    on the current kernel sources, else None."""
    from dynamic_sparse_attention_amd import profile_tables
    return profile_tables.current_record(workload)


def measured_traffic(rec):
    """HBM bytes per attention launch (scaled FETCH_SIZE + WRITE_SIZE) from a
    current profile record, else None."""
    if rec is None:
        return None
    for r in rec["kernels"]:
        if r["kernel"].startswith("sparse_attn_kernel") and "measured_bytes" in r:
            return float(r["measured_bytes"])
    return None


def kernels_hbm(rec):
    """Per-kernel HBM rate and share of the 8 TB/s peak from a current profile
    record (measured bytes from the counters, algorithmic bytes from the
    shapes), or None when the record is missing or describes older kernels."""
    if rec is None:
        return None
    keys = ("avg_us", "measured_GBps", "measured_pct_hbm", "algorithmic_GBps", "algorithmic_pct_hbm",
            "clock_MHz", "mfma_busy")
    return {r["kernel"]: {k: r[k] for k in keys if k in r} for r in rec["kernels"]}


def index_work(plan, d):
    """Issued MFMA FLOP of the attention launch, from the index counts:
    4*d*64*64 per computed 64x64 tile, 4*d*64 per gathered column per query
    block (QK^T and PV, multiply-add = 2 FLOP)."""
    import torch
    import workloads as W
    B, Hq, N, _ = plan.q.shape
    nb = N // 64
    tiles = 0
    cols = 0
    bc = plan.index.block_count.to(torch.int64)
    cc = plan.index.col_count.to(torch.int64)
    for h, p in enumerate(plan.pat):
        if p == W.DENSE:
            tiles += B * nb * (nb + 1) // 2
        else:
            tiles += int(bc[:, h].sum())
            if p in (W.VSLASH, W.VSLASH_EXACT):
                cols += int(cc[:, h].sum())
    flop = 4.0 * d * 64 * 64 * tiles + 4.0 * d * 64 * cols
    dense_flop = 4.0 * d * B * Hq * (N * (N + 1) / 2)
    return tiles, cols, flop, dense_flop


def exact_pairs(plan, w):
    """Attended (i, j) pairs of the exact per-element patterns, from the
    selections the GPU made (host arithmetic, no attention):
    Vertical-Slash |{j in V} u {i - o : o in S}| per row, summed as
    sum(N - j) + sum(N - o) - #{(j, o) : j + o <= N - 1}; Block-Sparse the
    causal pairs of the kept blocks; A-shape |{j <= i : j < sink or
    i - j < local}|; dense N(N+1)/2."""
    import torch
    import workloads as W
    B, Hq, N, _ = plan.q.shape
    nb = N // 64
    total = 0
    vidx = plan.vidx.cpu().numpy() if plan.vidx is not None else None
    sidx = plan.sidx.cpu().numpy() if plan.sidx is not None else None
    bcnt = plan.bcnt.cpu().numpy() if plan.bcnt is not None else None
    i = np.arange(N, dtype=np.int64)
    # keys j < sink, plus the window [max(i - local + 1, sink), i]
    ashape = int(np.sum(np.minimum(i + 1, w.sink) +
                        np.maximum(0, i + 1 - np.maximum(i - w.local + 1, w.sink))))
    for b in range(B):
        for h, p in enumerate(plan.pat):
            if p in (W.VSLASH, W.VSLASH_EXACT):
                V = np.sort(vidx[b, h][vidx[b, h] >= 0]).astype(np.int64)
                S = np.sort(sidx[b, h][sidx[b, h] >= 0]).astype(np.int64)
                both = int(np.searchsorted(S, N - 1 - V, side="right").sum())
                total += int((N - V).sum() + (N - S).sum()) - both
            elif p == W.BSPARSE:
                # every kept block is whole except the diagonal one (64*65/2 causal pairs)
                total += int(bcnt[b, h].sum()) * 4096 - nb * (4096 - 2080)
            elif p == W.ASHAPE:
                total += ashape
            else:
                total += N * (N + 1) // 2
    return total


def cpu_baseline(w, data, plan, budget_s):
    """The oracle, untuned, on a bounded sample of the same layer, scaled to
    ms/layer: estimates + selection + index of a few heads, attention of a
    few (head, query block) items, extrapolated by head count and by the
    index's tile/column work."""
    import workloads as W
    from oracle import minference_oracle as O
    cores = len(os.sched_getaffinity(0))
    pats = list(plan.pat)
    nb = w.n_blocks
    g = w.group
    q64 = lambda h: W.to_f64(data["q"][0, h], w.dtype)
    k64 = lambda h: W.to_f64(data["k"][0, h // g], w.dtype)
    v64 = lambda h: W.to_f64(data["v"][0, h // g], w.dtype)
    rng = np.random.default_rng(0)
    t_est = {}
    n_est = {}
    idx_cache = {}
    start = time.perf_counter()
    # estimates: one head per pattern kind
    for kind in sorted(set(pats)):
        h = pats.index(kind)
        t0 = time.perf_counter()
        idx, _ = O.build_head_index(kind, q64(h), k64(h), w.scale, last_q=w.last_q,
                                    n_vertical=w.n_vertical, n_slash=w.n_slash,
                                    force_vertical=w.force_vertical, force_slash=w.force_slash,
                                    top_blocks=w.top_blocks, sink=w.sink, local=w.local)
        t_est[kind] = time.perf_counter() - t0
        n_est[kind] = sum(1 for p in pats if p == kind)
        idx_cache[kind] = (h, idx)
    # attention: sampled query blocks until about half the budget is used
    att_time, att_work, items = 0.0, 0.0, 0
    while time.perf_counter() - start < budget_s and items < 256:
        kind = pats[int(rng.integers(len(pats)))]
        h, idx = idx_cache[kind]
        a = int(rng.integers(nb))
        t0 = time.perf_counter()
        blocks = idx.blocks(a)
        cols = idx.cols(a)
        O.head_attention(q64(h), k64(h), v64(h), w.scale, idx, [a])
        att_time += time.perf_counter() - t0
        att_work += len(blocks) * 64 * 64 + len(cols) * 64
        items += 1
    elapsed = time.perf_counter() - start
    tiles, ncols, _, _ = index_work(plan, w.head_dim)
    layer_work = tiles * 64 * 64 + ncols * 64
    est_total = sum(t_est[k] * n_est[k] for k in t_est)
    att_total = att_time / max(att_work, 1) * layer_work
    ms = (est_total + att_total) * 1e3
    return {"value": ms, "unit": "ms/layer", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 numpy oracle: estimate+select+index of 1 head per pattern "
                       f"({', '.join(str(n_est[k]) + 'x' for k in sorted(n_est))} heads by count), "
                       f"attention of {items} random (head, query block) items; extrapolated to "
                       f"the layer by head count and by the index's tile+column work; "
                       f"{elapsed:.1f} s of CPU time")}


def measure(w, steps, warmup, dense, keep=False, exact=False, data=None):
    """Generates the workload, runs `warmup` untimed and `steps` timed passes
    of the hot path (events around each call, on the stream the library
    launches on), and optionally times the dense comparator (median of three
    launches).  exact=True runs the Vertical-Slash heads as exact
    (element-masked) heads."""
    import torch
    import dynamic_sparse_attention_amd as mi
    import workloads as W
    if data is None:
        log(f"[bench] generating {w.name} (N={w.seq_len}, Hq={w.heads_q}, Hkv={w.heads_kv})")
        t0 = time.time()
        data = W.generate(w)
        log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def up(x):
        if w.dtype == "f32":
            return torch.from_numpy(x).to(dev)
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(data["q"]), up(data["k"]), up(data["v"])
    pats = [int(p) for p in data["patterns"]]
    if exact:
        pats = [W.VSLASH_EXACT if p == W.VSLASH else p for p in pats]
    if not keep:
        data = {"patterns": data["patterns"]}
    plan = mi.LayerPlan(q, k, v, pats, last_q=w.last_q, n_vertical=w.n_vertical, n_slash=w.n_slash,
                        force_vertical=w.force_vertical, force_slash=w.force_slash,
                        top_blocks=w.top_blocks, sink=w.sink, local=w.local)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: warmup done ({warmup} steps)")

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(steps):
        e = ev[s]
        e[0].record(stream)
        plan.estimate()
        e[1].record(stream)
        plan.build_index()
        e[2].record(stream)
        plan.attention()
        e[3].record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    per_step = [e[0].elapsed_time(e[3]) for e in ev]
    res = {"ms_step": (t_end - t_start) * 1e3 / steps,
           "median_ms": float(np.median(per_step)),
           "est_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
           "idx_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])),
           "att_ms": float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))}
    log(f"[bench] {w.name}: {steps} steps: {res['ms_step']:.3f} ms/step (estimate {res['est_ms']:.3f}, "
        f"index {res['idx_ms']:.3f}, attention {res['att_ms']:.3f})")
    res["tiles"], res["cols"], res["flop"], res["dense_flop"] = index_work(plan, w.head_dim)
    res["exact_pairs"] = exact_pairs(plan, w)
    nb = w.n_blocks
    res["causal_tiles"] = w.batch * w.heads_q * nb * (nb + 1) // 2
    if dense:
        plan.attention(dense=True)
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            plan.attention(dense=True)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        dms = float(np.median(times))
        res["dense"] = {"ms": round(dms, 3),
                        "tflops": round(4.0 * w.head_dim * 64 * 64 * res["causal_tiles"] / (dms * 1e-3) / 1e12, 2)}
        log(f"[bench] {w.name}: dense causal attention {dms:.3f} ms")
    return res, plan, data


def gather_rate(q, k, v, w, n_vertical=1000):
    """The column gather on its own: the same Q/K/V with a column-only index
    (slash set {0}: each query block computes its diagonal tile only, plus
    up to n_vertical gathered key columns, seeded and spread over the
    sequence).  Bytes are the gathered K and V rows (2 * d * elem per column
    per query block); the diagonal tiles' share of the time is measured with
    no columns at all and taken out."""
    import torch
    import dynamic_sparse_attention_amd as mi
    B, Hq, N, d = q.shape
    es = q.element_size()
    dev = q.device
    g = np.random.default_rng(77)
    vidx = torch.empty((B, Hq, n_vertical), dtype=torch.int32)
    for b in range(B):
        for h in range(Hq):
            vidx[b, h] = torch.from_numpy(np.sort(np.concatenate(
                [[0], g.choice(np.arange(1, N), n_vertical - 1, replace=False)])).astype(np.int32))
    vidx = vidx.to(dev)
    sidx = torch.zeros((B, Hq, 1), dtype=torch.int32, device=dev)
    pats = [W_VS] * Hq
    idx = mi.build_index(q, k, pats, vidx, sidx)
    none = mi.build_index(q, k, pats, vidx[..., :1], sidx)  # key 0 only: in the diagonal tile of block 0
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def timed(ix):
        mi.sparse_prefill(q, k, v, pats, ix, out=out, return_lse=False)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mi.sparse_prefill(q, k, v, pats, ix, out=out, return_lse=False)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    ms = timed(idx)
    base = timed(none)
    cols = int(idx.col_count.to(torch.int64).sum())
    byts = cols * 2 * d * es
    rate = byts / max(ms - base, 1e-6) / 1e6
    return {"columns": cols, "bytes": byts, "attention_ms": round(ms, 3), "diagonal_only_ms": round(base, 3),
            "gather_GBps": round(rate, 1), "frac_of_hbm_peak": round(rate / PEAK_HBM_GBS, 4),
            "note": "gathered K/V rows per query block over the time the columns add; rows are served "
                    "from L2/MALL as much as from HBM"}


def antidiag_rate(q, k, w):
    """The antidiagonal block estimate (scores, softmax, top-k) of every head
    of the layer, weights not stored: median of three launches.  FLOP are the
    definition's: 2*64*d per (query block, earlier key block) pair and 2*32*d
    per diagonal pair."""
    import torch
    import dynamic_sparse_attention_amd as mi
    B, Hq, N, d = q.shape
    nb = N // 64
    heads = list(range(Hq))
    dev = q.device
    outs = (torch.zeros((B, Hq, nb, w.top_blocks), dtype=torch.int32, device=dev),
            torch.zeros((B, Hq, nb), dtype=torch.int32, device=dev), None)
    mi.antidiag_estimate(q, k, heads, w.top_blocks, return_scores=False, outputs=outs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        mi.antidiag_estimate(q, k, heads, w.top_blocks, return_scores=False, outputs=outs)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    flop = B * Hq * (2.0 * 64 * d * nb * (nb - 1) / 2 + 2.0 * 32 * d * nb)
    tf = flop / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 3), "flop": flop, "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "note": "scores as a dense contraction over 64*d per block pair (MFMA), then the block softmax and top-k"}


def plant_recall(plan, w):
    """Diagnostic of the synthetic plants' strength: the fraction of a kv
    head's planted keys found among each Vertical-Slash head's selected
    verticals (key 0 is always one of the plants), and the fraction of
    (query block, planted hot block at or before it) pairs that the
    Block-Sparse heads' lists select.  Not a parity check: the plants are
    weak beside the logit noise at these lengths and are left as specified."""
    import workloads as W
    g = w.heads_q // w.heads_kv
    out = {}
    vs = [h for h, pt in enumerate(plan.pat) if pt in (W.VSLASH, W.VSLASH_EXACT)]
    if vs and w.n_vertical_plants > 0 and plan.vidx is not None:
        vidx = plan.vidx[0].cpu().numpy()
        rec = [float(np.isin(W.vertical_plants(w, h // g), vidx[h]).mean()) for h in vs]
        out["vertical"] = {"heads": len(vs), "plants_per_kv_head": int(w.n_vertical_plants),
                           "mean_recall": round(float(np.mean(rec)), 4), "min_recall": round(min(rec), 4),
                           "max_recall": round(max(rec), 4)}
    bs = [h for h, pt in enumerate(plan.pat) if pt == W.BSPARSE]
    if bs and w.n_hot_blocks > 0 and plan.bidx is not None:
        bidx = plan.bidx[0].cpu().numpy()
        bcnt = plan.bcnt[0].cpu().numpy()
        nb = bidx.shape[1]
        hits = elig = 0
        for h in bs:
            hot = np.zeros(nb, bool)
            hot[W.hot_blocks(w, h // g)] = True
            valid = np.arange(bidx.shape[2])[None, :] < bcnt[h][:, None]
            hits += int((hot[np.clip(bidx[h], 0, nb - 1)] & valid).sum())
            elig += int(np.cumsum(hot).sum())
        out["hot_blocks"] = {"heads": len(bs), "hot_blocks_per_kv_head": int(w.n_hot_blocks),
                             "recall": round(hits / max(elig, 1), 4)}
    return out


def library_context(q, k, v, dense_ms):
    """Reference points from the libraries on the same GPU (not part of the
    path): hipBLASLt's bf16 GEMM through torch.matmul (8192^3, median of
    three bursts of 50), and torch's flash SDPA, causal, on the layer's Q/K/V
    with the kv heads repeated (median of three), against this library's
    dense causal comparator on the same inputs."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    out = {}
    stream = torch.cuda.current_stream()

    def med(f, n, reps=3):
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / n)
        return float(np.median(ts))

    g = torch.Generator(device=q.device).manual_seed(7)
    m = 8192
    a = torch.randn(m, m, device=q.device, dtype=torch.bfloat16, generator=g)
    b = torch.randn(m, m, device=q.device, dtype=torch.bfloat16, generator=g)
    ms = med(lambda: torch.matmul(a, b), 50)
    tf = 2.0 * m ** 3 / (ms * 1e-3) / 1e12
    out["gemm_bf16"] = {"shape": [m, m, m], "ms": round(ms, 4), "tflops": round(tf, 1),
                        "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del a, b
    B, Hq, N, d = q.shape
    g_ = Hq // k.shape[1]
    kk = k.repeat_interleave(g_, dim=1).contiguous()
    vv = v.repeat_interleave(g_, dim=1).contiguous()
    flop = 4.0 * d * B * Hq * N * (N + 1) / 2
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            ms = med(lambda: torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True), 1)
        out["sdpa_flash_causal"] = {"ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                                    "dense_comparator_ms": None if dense_ms is None else round(dense_ms, 3),
                                    "flop": "4*d*H*N(N+1)/2"}
    except RuntimeError as e:
        out["sdpa_flash_causal"] = {"error": str(e)[:200]}
    del kk, vv
    return out


def dense_sweep(lengths=(16384, 32768, 65536, 131072, 262144), hq=32, hkv=8, d=128):
    """The dense causal comparator (this library, no index) and torch's flash
    SDPA (kv heads repeated) on seeded N(0,1) bf16 inputs over sequence
    lengths: median of three launches each, TFLOP/s on 4*d*H*N(N+1)/2."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import dynamic_sparse_attention_amd as mi
    stream = torch.cuda.current_stream()

    def med(f, reps=3):
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    rows = []
    for n in lengths:
        g = torch.Generator(device="cuda").manual_seed(n)
        q = torch.randn(1, hq, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
        k = torch.randn(1, hkv, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
        v = torch.randn(1, hkv, n, d, device="cuda", dtype=torch.bfloat16, generator=g)
        o = torch.empty_like(q)
        flop = 4.0 * d * hq * n * (n + 1) / 2
        ours = med(lambda: mi.sparse_prefill(q, k, v, None, None, out=o, return_lse=False, schedule=True))
        row = {"seq_len": n, "ours_ms": round(ours, 3), "ours_tflops": round(flop / ours / 1e9, 1)}
        kk = k.repeat_interleave(hq // hkv, dim=1).contiguous()
        vv = v.repeat_interleave(hq // hkv, dim=1).contiguous()
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                lib = med(lambda: torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True))
            row.update({"sdpa_ms": round(lib, 3), "sdpa_tflops": round(flop / lib / 1e9, 1),
                        "ratio": round(lib / ours, 3)})
        except RuntimeError as e:
            row["sdpa_error"] = str(e)[:120]
        rows.append(row)
        log(f"[bench] dense sweep N={n}: {row}")
        del q, k, v, o, kk, vv
        torch.cuda.empty_cache()
    return rows


def sampled_parity(plan, w, data, n_items=8):
    """Attention rows of the plan (relaunched on its index, since the dense
    comparator shares the output buffer) against the oracle fed the GPU's
    own index, on seeded (head, query block) samples (the oracle at full size
    would take hours): the largest absolute difference."""
    import torch
    import workloads as W
    from oracle import minference_oracle as O
    plan.attention()
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    nb, g = w.n_blocks, w.group
    worst = 0.0
    items = []
    for _ in range(n_items):
        h = int(rng.integers(w.heads_q))
        a = int(rng.choice([0, nb - 1, int(rng.integers(nb))]))
        items.append((h, a))
    for h, a in items:
        bc = int(plan.index.block_count[0, h, a])
        blocks = plan.index.block_idx[0, h, a, :bc].cpu().numpy()
        cc = int(plan.index.col_count[0, h, a])
        cols = plan.index.col_idx[0, h, a, :cc].cpu().numpy() if plan.pat[h] == W.VSLASH else []
        q64, k64, v64 = (W.to_f64(data[x][0, hh], w.dtype) for x, hh in (("q", h), ("k", h // g), ("v", h // g)))
        if plan.pat[h] == W.ASHAPE:
            ref, _ = O.ashape_attention(q64, k64, v64, w.scale, np.arange(64 * a, 64 * a + 64), w.sink, w.local)
        else:
            ref, _ = O.attention_from_index(q64, k64, v64, w.scale, a, blocks, cols)
        got = plan.o[0, h, 64 * a: 64 * a + 64].double().cpu().numpy()
        worst = max(worst, float(np.abs(got - ref).max()))
    tol = 1e-4 if w.dtype == "f32" else 2e-2
    return {"attention_max_abs": worst, "tolerance": tol, "items": len(items), "ok": worst < tol,
            "reference": "fp64 oracle fed the GPU's index, seeded (head, query block) samples"}


def mi_layer_plan(q, k, v, pats, w):
    import dynamic_sparse_attention_amd as mi
    return mi.LayerPlan(q, k, v, pats, last_q=w.last_q, n_vertical=w.n_vertical, n_slash=w.n_slash,
                        force_vertical=w.force_vertical, force_slash=w.force_slash,
                        top_blocks=w.top_blocks, sink=w.sink, local=w.local)


def time_attention(plan, launches):
    """Median of `launches` timed attention launches of a plan whose index is built."""
    import torch
    stream = torch.cuda.current_stream()
    plan.attention()
    torch.cuda.synchronize()
    times = []
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plan.attention()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def exact_summary(r, d):
    """Exact-pattern work beside the issued tile work: how much the aligned
    64x64 tiles and 64-key column chunks add, and the effective TFLOP/s
    (4*d per attended pair over the attention time)."""
    issued = r["tiles"] * 4096 + r["cols"] * 64
    return {"attended_pairs": r["exact_pairs"], "issued_pairs": issued,
            "tiling_overhead": round(issued / max(r["exact_pairs"], 1), 3),
            "effective_tflops": round(4.0 * d * r["exact_pairs"] / (r["att_ms"] * 1e-3) / 1e12, 2)}


def gather_hbm(workload: str):
    """HBM bytes and rate of the column gather from a current rocprofv3
    record (FETCH_SIZE + WRITE_SIZE of the column launches minus those of
    the launches without columns), or None."""
    from dynamic_sparse_attention_amd import profile_tables
    rec = profile_tables.current_gather_record(workload)
    if rec is None:
        return None
    g = rec["gather"]
    return {k: g[k] for k in ("hbm_bytes", "time_us", "hbm_GBps", "hbm_pct", "staged_GBps", "staged_pct")}


def gather_only(w):
    """The isolated column gather alone on the workload's inputs (for the
    rocprofv3 passes that measure its HBM bytes): one JSON line."""
    import torch
    import workloads as W
    if w.dtype != "bf16":
        raise SystemExit("the gather measurement takes a bf16 workload")
    log(f"[bench] generating {w.name} (N={w.seq_len}) for the gather measurement")
    data = W.generate(w)
    dev = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = up(data["q"]), up(data["k"]), up(data["v"])
    del data
    log("[bench] column gather rate")
    print(json.dumps({"workload": w.name, "gather": gather_rate(q, k, v, w)}), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding by kv-head "
                          "group is designed but not built", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import workloads as W

    w = W.WORKLOADS[args.config]
    if args.gather_only:
        gather_only(w)
        return
    r, plan, data = measure(w, args.steps, args.warmup, not args.no_dense, keep=not args.no_cpu_baseline)
    d = w.head_dim
    achieved = r["flop"] / (r["att_ms"] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    prof = profile_record(w.name)
    out = {
        "metric": METRIC,
        "value": round(r["ms_step"], 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "median_ms_per_step": round(r["median_ms"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V with RoPE and planted keys; no weights or datasets)",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seq_len": w.seq_len, "head_dim": d, "patterns": w.patterns,
                   "last_q": w.last_q, "n_vertical": w.n_vertical, "n_slash": w.n_slash,
                   "top_blocks": w.top_blocks, "sink": w.sink, "local": w.local},
        "roofline": {"bound": "mfma", "kernel": "sparse_attn_kernel", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(prof),
                     "flop_per_launch": r["flop"]},
        "kernels_ms": {"estimate": round(r["est_ms"], 4), "build_index": round(r["idx_ms"], 4),
                       "attention": round(r["att_ms"], 4)},
        "mfma_tflops": round(achieved, 2),
        "effective_dense_equiv_tflops": round(r["dense_flop"] / (r["ms_step"] * 1e-3) / 1e12, 2),
        "index": {"tiles": r["tiles"], "columns": r["cols"],
                  "tile_density": round(r["tiles"] / r["causal_tiles"], 4)},
        "exact_pattern": exact_summary(r, d),
        "kernels_hbm": kernels_hbm(prof),
    }
    if "dense" in r:
        out["dense_comparator"] = r["dense"]
    out["plant_recall"] = plant_recall(plan, w)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w, data, plan, args.cpu_seconds)
    if not args.no_cpu_baseline:
        log("[bench] sampled parity against the oracle")
        out["parity"] = sampled_parity(plan, w, data)
    if not args.no_gather and w.seq_len >= 65536 and w.dtype == "bf16":
        log("[bench] column gather rate")
        out["gather"] = gather_rate(plan.q, plan.k, plan.v, w)
        out["gather"]["measured_hbm"] = gather_hbm(w.name)
    if not args.no_antidiag:
        log("[bench] antidiagonal block estimate")
        out["antidiag_estimate"] = antidiag_rate(plan.q, plan.k, w)
    if args.dense_sweep:
        log("[bench] dense causal attention over sequence lengths")
        out["dense_sweep"] = dense_sweep()
    if args.library_context and w.dtype == "bf16":
        log("[bench] library reference points")
        out["library_context"] = library_context(plan.q, plan.k, plan.v, r["dense"]["ms"] if "dense" in r else None)
    if not args.no_exact and any(p == W.VSLASH for p in plan.pat):
        # the same layer with the Vertical-Slash heads element-masked to their
        # exact key sets: attention time on the same estimate and index lists
        q, k, v = plan.q, plan.k, plan.v
        ex = mi_layer_plan(q, k, v, [W.VSLASH_EXACT if p == W.VSLASH else p for p in plan.pat], w)
        ex.run()
        torch.cuda.synchronize()
        ems = time_attention(ex, 3)
        out["exact_variant"] = {
            "attention_ms": round(ems, 3), "aligned_attention_ms": round(r["att_ms"], 3),
            "effective_tflops": round(4.0 * d * r["exact_pairs"] / (ems * 1e-3) / 1e12, 2),
            "aligned_effective_tflops": out["exact_pattern"]["effective_tflops"]}
        log(f"[bench] {w.name}: exact variant attention {ems:.3f} ms")
        del ex
    del plan, data
    if not args.no_exact and args.config == "c3":
        # the clustered-slash variant of the layer: aligned tiles vs exact
        torch.cuda.empty_cache()
        wl = W.WORKLOADS["c3local"]
        rl, pl, dl = measure(wl, 5, 2, False, keep=True)
        del pl
        re_, pe, _ = measure(wl, 5, 2, False, exact=True, data=dl)
        del pe, dl
        out["clustered_slash"] = {
            "workload": wl.name, "seq_len": wl.seq_len,
            "aligned": {"ms_per_layer": round(rl["ms_step"], 3), "attention_ms": round(rl["att_ms"], 3),
                        "index": {"tiles": rl["tiles"], "columns": rl["cols"],
                                  "tile_density": round(rl["tiles"] / rl["causal_tiles"], 4)},
                        "exact_pattern": exact_summary(rl, wl.head_dim)},
            "exact": {"ms_per_layer": round(re_["ms_step"], 3), "attention_ms": round(re_["att_ms"], 3),
                      "effective_tflops": round(4.0 * wl.head_dim * re_["exact_pairs"] /
                                                (re_["att_ms"] * 1e-3) / 1e12, 2)},
        }
    if not args.no_1m and args.config == "c3":
        torch.cuda.empty_cache()
        w5 = W.WORKLOADS["c5"]
        r5, plan5, _ = measure(w5, 2, 1, not args.no_dense)
        ach5 = r5["flop"] / (r5["att_ms"] * 1e-3) / 1e12
        out["secondary"] = {
            "workload": w5.name, "seq_len": w5.seq_len, "steps": 2, "warmup": 1,
            "ms_per_layer": round(r5["ms_step"], 3),
            "kernels_ms": {"estimate": round(r5["est_ms"], 3), "build_index": round(r5["idx_ms"], 3),
                           "attention": round(r5["att_ms"], 3)},
            "mfma_tflops": round(ach5, 2), "frac": round(ach5 / PEAK_BF16_TFLOPS, 4),
            "index": {"tiles": r5["tiles"], "columns": r5["cols"],
                      "tile_density": round(r5["tiles"] / r5["causal_tiles"], 4)},
            "exact_pattern": exact_summary(r5, w5.head_dim),
        }
        if "dense" in r5:
            out["secondary"]["dense_comparator"] = r5["dense"]
            out["secondary"]["speedup_vs_dense_attention"] = round(r5["dense"]["ms"] / r5["ms_step"], 3)
        out["secondary"]["plant_recall"] = plant_recall(plan5, w5)
        del plan5
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
