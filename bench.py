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
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 4 times (counter calibration)")
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


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on this workload with the current kernel source;
    otherwise None (the counters describe another kernel)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "sparse_attn_vs128k_hbm.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in ("sparse_attn.hip", "mi_device.h"))
    if rec.get("workload") != workload or rec.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return float(rec["traffic_bytes_per_launch"])


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
            if p == W.VSLASH:
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
            if p == W.VSLASH:
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


def measure(w, steps, warmup, dense, keep=False):
    """Generates the workload, runs `warmup` untimed and `steps` timed passes
    of the hot path (events around each call, on the stream the library
    launches on), and optionally times the dense comparator once."""
    import torch
    import dynamic_sparse_attention_amd as mi
    import workloads as W
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        plan.attention(dense=True)
        torch.cuda.synchronize()
        e0.record(stream)
        plan.attention(dense=True)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        res["dense"] = {"ms": round(dms, 3),
                        "tflops": round(4.0 * w.head_dim * 64 * 64 * res["causal_tiles"] / (dms * 1e-3) / 1e12, 2)}
        log(f"[bench] {w.name}: dense causal attention {dms:.3f} ms")
    return res, plan, data


def exact_summary(r, d):
    """Exact-pattern work beside the issued tile work: how much the aligned
    64x64 tiles and 64-key column chunks add, and the effective TFLOP/s
    (4*d per attended pair over the attention time)."""
    issued = r["tiles"] * 4096 + r["cols"] * 64
    return {"attended_pairs": r["exact_pairs"], "issued_pairs": issued,
            "tiling_overhead": round(issued / max(r["exact_pairs"], 1), 3),
            "effective_tflops": round(4.0 * d * r["exact_pairs"] / (r["att_ms"] * 1e-3) / 1e12, 2)}


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
    r, plan, data = measure(w, args.steps, args.warmup, not args.no_dense, keep=not args.no_cpu_baseline)
    d = w.head_dim
    achieved = r["flop"] / (r["att_ms"] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
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
                     "traffic": measured_traffic(w.name),
                     "flop_per_launch": r["flop"]},
        "kernels_ms": {"estimate": round(r["est_ms"], 4), "build_index": round(r["idx_ms"], 4),
                       "attention": round(r["att_ms"], 4)},
        "mfma_tflops": round(achieved, 2),
        "effective_dense_equiv_tflops": round(r["dense_flop"] / (r["ms_step"] * 1e-3) / 1e12, 2),
        "index": {"tiles": r["tiles"], "columns": r["cols"],
                  "tile_density": round(r["tiles"] / r["causal_tiles"], 4)},
        "exact_pattern": exact_summary(r, d),
    }
    if "dense" in r:
        out["dense_comparator"] = r["dense"]
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w, data, plan, args.cpu_seconds)
    del plan, data
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
        del plan5
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
