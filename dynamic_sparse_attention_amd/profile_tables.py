"""rocprofv3 summaries -> the per-kernel tables kept with the sources.

Reads the CSV files of up to five rocprofv3 runs of the same bench command
(a kernel trace with --stats, a FETCH_SIZE pass, a WRITE_SIZE pass, and the
same two counters over a device copy of known size) plus an optional pass of
SQ/GRBM counters, and writes a Markdown table and a JSON record:

  kernel, calls, average duration, HBM bytes per launch (counter values in
  KiB scaled by what the same counter reads for the copy), GB/s and share of
  the 8 TB/s HBM peak, and the algorithmic bytes per launch with their rate.

The record carries the SHA-256 of the kernel sources it was measured with;
``current_record`` returns it only while the sources still hash the same, so
that numbers taken on an older kernel are never reported as current.

Usage (from the repository root):
  python -m dynamic_sparse_attention_amd.profile_tables --workload c3 \
      --steps 3 --trace DIR --fetch DIR --write DIR --copy-fetch DIR \
      --copy-write DIR [--sq DIR] --command "..." --out profiles/NAME
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30  # bytes read and written by each launch of the calibration copy


def source_sha256(files=None) -> str:
    """SHA-256 over the kernel sources (all of csrc/ by default), in name order."""
    if files is None:
        files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without return type, namespaces and argument list; template
    arguments kept (``sparse_attn_kernel<bf16, 128, false>``).  A type
    template argument that names a namespace keeps it."""
    n = name.strip().replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    lt = n.find("<")
    head = n if lt < 0 else n[:lt]
    n = head.split("::")[-1] + ("" if lt < 0 else n[lt:])
    # the kernels carry bf16 as its 16-bit storage type
    return n.replace("unsigned short", "bf16").replace("__hip_bfloat16", "bf16")


def _one(pattern: str, run_dir: str) -> str:
    hits = sorted(glob.glob(os.path.join(run_dir, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {run_dir}")
    return hits[0]


def kernel_stats(run_dir: str) -> dict:
    """name -> {calls, avg_us} from a ``--stats`` kernel summary."""
    out = {}
    with open(_one("*kernel_stats.csv", run_dir)) as fh:
        for row in csv.DictReader(fh):
            out[short_name(row["Name"])] = {"calls": int(row["Calls"]),
                                            "avg_us": float(row["AverageNs"]) / 1e3}
    return out


def counter_means(run_dir: str) -> dict:
    """name -> {counter: mean value per dispatch} from a ``--pmc`` run."""
    per = defaultdict(lambda: defaultdict(list))
    with open(_one("*counter_collection.csv", run_dir)) as fh:
        for row in csv.DictReader(fh):
            per[short_name(row["Kernel_Name"])][row["Counter_Name"]].append(float(row["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in per.items()}


def copy_factor(run_dir: str, counter: str) -> tuple[float, float]:
    """(factor, raw KiB) for a counter: COPY_BYTES over what the counter reads
    (in bytes) for the calibration copy, the dispatch kind with the largest value."""
    means = counter_means(run_dir)
    raw = max(v.get(counter, 0.0) for v in means.values())
    return COPY_BYTES / (raw * 1024.0), raw


# ----------------------------------------------------------------------------
# Algorithmic bytes per layer, by kernel family
# ----------------------------------------------------------------------------

def algorithmic_bytes(w) -> dict:
    """Bytes that each kernel family must move per layer at the least: one read
    of every input it needs and one write of every output (padded lists as
    stored).  Keys are name prefixes; families not listed have no figure."""
    import numpy as np
    import workloads as W
    from . import index_caps
    es = 2 if w.dtype == "bf16" else 4
    B, Hq, Hkv, N, d, L = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.last_q
    g = w.group
    nb = N // 64
    pats = [int(p) for p in W.head_patterns(w)]
    vs = [h for h, p in enumerate(pats) if p in (W.VSLASH, W.VSLASH_EXACT)]
    bs = [h for h, p in enumerate(pats) if p == W.BSPARSE]
    kv_vs = len({h // g for h in vs})
    kv_bs = len({h // g for h in bs})
    hv, hb = len(vs) * B, len(bs) * B
    nv, ns = min(w.n_vertical, N), min(w.n_slash, N)
    bcap, ccap = index_caps(N, pats, w.n_vertical if vs else 0, w.n_slash if vs else 0,
                            w.top_blocks, w.sink, w.local)
    k_vs = B * kv_vs * N * d * es
    out = {}
    if hv:
        q_last = hv * L * d * es
        out["vs_rowstat_partial"] = k_vs + q_last
        out["vs_rowstat_combine"] = hv * L * 8
        out["vs_scores"] = k_vs + q_last + hv * 2 * N * 4
        # the L-1 spilled offsets of every 128-key chunk: read, and added into
        # the slash row (read and written)
        out["vs_slash_combine"] = hv * (N // 128) * (L - 1) * 12
        rows = 2 * hv
        # the first digit's histogram comes from the score kernels; each of
        # the three top-k launches reads the rows once
        out["topk_pass2"] = rows * N * 4
        out["topk_pass3"] = rows * N * 4
        out["topk_write"] = rows * N * 4 + hv * (nv + ns) * 4
        out["tile_set_kernel"] = hv * ns * 4 + hv * nb * 4
    if hb:
        k_bs = B * kv_bs * N * d * es
        out["bs_pool"] = hb * N * d * es + k_bs + (hb + B * kv_bs) * nb * d * 4
        tri = nb * (nb + 1) // 2
        out["bs_scores"] = (hb + B * kv_bs) * nb * d * 4 + hb * tri * 4
        sel = hb * tri * 4 + hb * nb * (4 * min(w.top_blocks, nb) + 4)
        out["bs_select_wave"] = sel
        out["bs_select"] = sel
        # fused scores + selection (rows of up to 512 blocks): the pooled rows
        # in, the lists out
        out["bs_fused"] = (hb + B * kv_bs) * nb * d * 4 + hb * nb * (4 * min(w.top_blocks, nb) + 4)
    out["build_index_kernel"] = B * Hq * nb * (4 * bcap + 4 * ccap + 8)
    out["sparse_attn_kernel"] = 2 * B * Hq * N * d * es + 2 * B * Hkv * N * d * es + B * Hq * N * 4
    return out


def _alg_for(name: str, alg: dict):
    base = name.split("<")[0]
    return alg.get(base)


# ----------------------------------------------------------------------------
# Table
# ----------------------------------------------------------------------------

def build_record(args) -> dict:
    import workloads as W
    w = W.WORKLOADS[args.workload]
    stats = kernel_stats(args.trace)
    fetch = counter_means(args.fetch) if args.fetch else {}
    write = counter_means(args.write) if args.write else {}
    ff, fraw = copy_factor(args.copy_fetch, "FETCH_SIZE") if args.copy_fetch else (None, None)
    wf, wraw = copy_factor(args.copy_write, "WRITE_SIZE") if args.copy_write else (None, None)
    sq = counter_means(args.sq) if args.sq else {}
    alg = algorithmic_bytes(w)
    ours = lambda n: n.split("<")[0] in alg or n.split("<")[0] in OWN_KERNELS
    rows = []
    for name, st in sorted(stats.items(), key=lambda kv: -kv[1]["calls"] * kv[1]["avg_us"]):
        if not ours(name):
            continue
        per_step = st["calls"] / args.steps
        r = {"kernel": name, "calls": st["calls"], "avg_us": round(st["avg_us"], 2)}
        if ff is not None and name in fetch and wf is not None and name in write:
            byts = fetch[name]["FETCH_SIZE"] * 1024 * ff + write[name]["WRITE_SIZE"] * 1024 * wf
            r["measured_bytes"] = round(byts)
            r["measured_GBps"] = round(byts / (st["avg_us"] * 1e3), 1)
            r["measured_pct_hbm"] = round(100 * r["measured_GBps"] / PEAK_HBM_GBS, 2)
        a = _alg_for(name, alg)
        if a is not None:
            a_launch = a / per_step
            r["algorithmic_bytes"] = round(a_launch)
            r["algorithmic_GBps"] = round(a_launch / (st["avg_us"] * 1e3), 1)
            r["algorithmic_pct_hbm"] = round(100 * r["algorithmic_GBps"] / PEAK_HBM_GBS, 2)
        if name in sq and st["avg_us"] >= 1000.0:
            # clock and MFMA busy from counters only where the kernel is long
            # against the dispatch overhead of a counter run
            c = sq[name]
            if "GRBM_GUI_ACTIVE" in c and st["avg_us"] > 0:
                r["clock_MHz"] = round(c["GRBM_GUI_ACTIVE"] / 8 / st["avg_us"], 0)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
                r["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * c["GRBM_GUI_ACTIVE"] / 8), 3)
            if "SQ_INSTS_LDS" in c and "SQ_LDS_BANK_CONFLICT" in c:
                r["lds_bank_conflict_cycles_per_inst"] = round(c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_INSTS_LDS"], 1), 3)
        rows.append(r)
    bench_att = None
    if args.bench_log:
        with open(args.bench_log) as fh:
            for line in fh:
                if line.startswith('{"metric"'):
                    bench_att = json.loads(line)["kernels_ms"]["attention"]
    return {"workload": w.name, "config": args.workload, "steps_in_trace": args.steps,
            "bench_attention_ms_events": bench_att,
            "kernel_source_sha256": source_sha256(), "command": args.command,
            "copy_calibration": {"bytes_per_launch": COPY_BYTES, "fetch_size_kib_raw": fraw,
                                 "write_size_kib_raw": wraw, "fetch_factor": ff, "write_factor": wf},
            "kernels": rows}


OWN_KERNELS = {"attn_schedule_kernel", "vs_bits_kernel"}


def _fmt(v, nd=1):
    return "—" if v is None else (f"{v:.{nd}f}" if isinstance(v, float) else str(v))


def markdown(rec: dict, title: str) -> str:
    lines = [f"# {title}", "",
             f"Kernel sources (csrc/, SHA-256): `{rec['kernel_source_sha256']}`", "",
             "Command (its rocprofv3 passes run from /tmp with TMPDIR=/tmp; OUT = an output folder):", "", "```",
             rec["command"], "```", ""]
    cc = rec["copy_calibration"]
    if cc["fetch_factor"]:
        lines += [f"FETCH_SIZE is scaled by {cc['fetch_factor']:.4f} and WRITE_SIZE by "
                  f"{cc['write_factor']:.4f}: a device copy that reads and writes 1 GiB "
                  f"(`bench.py --calibrate-copy`) reads FETCH_SIZE = {cc['fetch_size_kib_raw']:.1f} KiB "
                  f"and WRITE_SIZE = {cc['write_size_kib_raw']:.1f} KiB per launch. Algorithmic bytes: "
                  "one read of every input a kernel needs and one write of every output, lists as "
                  "stored (padded); attention: Q, K, V, O and the log-sum-exp once.", ""]
    if rec.get("bench_attention_ms_events") is not None:
        att = next((r for r in rec["kernels"] if r["kernel"].startswith("sparse_attn_kernel")), None)
        lines += [f"The traced bench run timed the attention launch with HIP events on its stream at "
                  f"{rec['bench_attention_ms_events']:.3f} ms (timed steps only); the trace average "
                  f"below, which also counts the warmup launch, is "
                  f"{att['avg_us'] / 1e3:.3f} ms." if att else "", ""]
    sqc = any("clock_MHz" in r for r in rec["kernels"])
    if sqc:
        lines += ["Clock and MFMA busy (kernels of 1 ms or more only): clock = GRBM_GUI_ACTIVE / 8 "
                  "(summed over the eight XCDs) over the traced average duration; MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x those cycles).", ""]
    hdr = ("| kernel | calls | average us | measured MB/launch | measured GB/s | % of 8 TB/s | "
           "algorithmic MB/launch | algorithmic GB/s | % of 8 TB/s |")
    sep = "|---|---|---|---|---|---|---|---|---|"
    if sqc:
        hdr += " clock MHz | MFMA busy |"
        sep += "---|---|"
    lines += [hdr, sep]
    for r in rec["kernels"]:
        mb = lambda x: None if x is None else x / 1e6
        line = (f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.1f} | {_fmt(mb(r.get('measured_bytes')))} | "
                f"{_fmt(r.get('measured_GBps'), 0)} | {_fmt(r.get('measured_pct_hbm'))} | "
                f"{_fmt(mb(r.get('algorithmic_bytes')))} | {_fmt(r.get('algorithmic_GBps'), 0)} | "
                f"{_fmt(r.get('algorithmic_pct_hbm'))} |")
        if sqc:
            line += f" {_fmt(r.get('clock_MHz'), 0)} | {_fmt(r.get('mfma_busy'), 3)} |"
        lines.append(line)
    lines += ["", "Kernels of torch (fills, copies, reductions) belong to the bench's set-up and "
              "statistics outside the timed region and are left out."]
    return "\n".join(lines) + "\n"


# ----------------------------------------------------------------------------
# The column gather: per-dispatch values of the isolated gather measurement
# ----------------------------------------------------------------------------

ATTN = "sparse_attn_kernel"


def attn_dispatch_times(run_dir: str) -> list:
    """Durations (us) of the attention dispatches of a kernel trace, in dispatch order."""
    rows = []
    with open(_one("*kernel_trace.csv", run_dir)) as fh:
        for row in csv.DictReader(fh):
            if short_name(row["Kernel_Name"]).startswith(ATTN):
                rows.append((int(row["Dispatch_Id"]),
                             (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3))
    return [t for _, t in sorted(rows)]


def attn_dispatch_counter(run_dir: str, counter: str) -> list:
    """A counter's value (KiB) per attention dispatch of a --pmc run, in dispatch order."""
    rows = defaultdict(float)
    with open(_one("*counter_collection.csv", run_dir)) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] == counter and short_name(row["Kernel_Name"]).startswith(ATTN):
                rows[int(row["Dispatch_Id"])] += float(row["Counter_Value"])
    return [rows[k] for k in sorted(rows)]


def _median(x):
    x = sorted(x)
    n = len(x)
    return x[n // 2] if n % 2 else 0.5 * (x[n // 2 - 1] + x[n // 2])


def build_gather_record(args) -> dict:
    """The gather launch sequence of ``bench.py --gather-only``: one warmup and
    three timed attention launches with the column index, then the same
    without columns.  The gather's time and HBM bytes are the differences of
    the two groups (median of the timed launches; counters scaled by the
    copy calibration)."""
    times = attn_dispatch_times(args.trace)
    fetch = attn_dispatch_counter(args.fetch, "FETCH_SIZE")
    write = attn_dispatch_counter(args.write, "WRITE_SIZE")
    for what, xs in (("trace", times), ("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        if len(xs) != 8:
            raise ValueError(f"{what}: expected 8 attention dispatches, found {len(xs)}")
    ff, fraw = copy_factor(args.copy_fetch, "FETCH_SIZE")
    wf, wraw = copy_factor(args.copy_write, "WRITE_SIZE")
    bench = {}
    if args.bench_log and os.path.exists(args.bench_log):
        with open(args.bench_log) as fh:
            for line in fh:
                if line.startswith("{"):
                    bench = json.loads(line)["gather"]
    groups = {}
    for name, sl in (("columns", slice(1, 4)), ("diagonal_only", slice(5, 8))):
        f = _median(fetch[sl]) * 1024.0 * ff
        wb = _median(write[sl]) * 1024.0 * wf
        groups[name] = {"avg_us": round(_median(times[sl]), 2), "fetch_bytes": round(f), "write_bytes": round(wb)}
    c, d0 = groups["columns"], groups["diagonal_only"]
    t_us = c["avg_us"] - d0["avg_us"]
    hbm = (c["fetch_bytes"] + c["write_bytes"]) - (d0["fetch_bytes"] + d0["write_bytes"])
    staged = float(bench.get("bytes", 0))
    g = {"time_us": round(t_us, 2), "hbm_bytes": round(hbm),
         "hbm_GBps": round(hbm / (t_us * 1e3), 1), "hbm_pct": round(100.0 * hbm / (t_us * 1e3) / PEAK_HBM_GBS, 1),
         "staged_bytes": round(staged), "columns": bench.get("columns"),
         "staged_GBps": round(staged / (t_us * 1e3), 1) if staged else None,
         "staged_pct": round(100.0 * staged / (t_us * 1e3) / PEAK_HBM_GBS, 1) if staged else None}
    return {"workload": bench_workload(args.workload), "kernel_source_sha256": source_sha256(),
            "command": args.command, "fetch_scale": ff, "write_scale": wf,
            "copy_fetch_kib": fraw, "copy_write_kib": wraw, "launches": groups, "gather": g}


def bench_workload(key: str) -> str:
    import workloads as W
    return W.WORKLOADS[key].name


def gather_markdown(rec: dict) -> str:
    g, L = rec["gather"], rec["launches"]
    lines = [f"# Column gather: HBM bytes and rate ({rec['workload']})", "",
             f"Kernel sources (csrc/, SHA-256): `{rec['kernel_source_sha256']}`", "",
             "Command (its rocprofv3 passes run from /tmp with TMPDIR=/tmp; OUT = an output folder):", "",
             "```", rec["command"], "```", "",
             "The isolated gather of `bench.py --gather-only`: the layer's Q/K/V with a column-only index (slash set "
             "{0}: each query block computes its diagonal tile only, plus up to 1000 gathered key columns per head), "
             "one warmup and three timed attention launches, then the same launches without columns. The gather's "
             "time and HBM bytes are the differences of the two groups (medians of the timed launches). "
             f"FETCH_SIZE is scaled by {rec['fetch_scale']:.4f} and WRITE_SIZE by {rec['write_scale']:.4f} "
             "(a device copy that reads and writes 1 GiB). The algorithmic bytes of the gather are the gathered "
             "K and V rows staged into LDS (2 d x 2 bytes per column per query block); a row that several query "
             "blocks gather, or that is still in L2/MALL, is staged each time but fetched from HBM once, so the "
             "measured HBM bytes can be far below them.", "",
             "| launches | average us | HBM read MB | HBM written MB |", "|---|---|---|---|"]
    for name in ("columns", "diagonal_only"):
        x = L[name]
        lines.append(f"| {name.replace('_', ' ')} | {x['avg_us']:.1f} | {x['fetch_bytes'] / 1e6:.1f} | "
                     f"{x['write_bytes'] / 1e6:.1f} |")
    lines += ["", "| gather | value |", "|---|---|",
              f"| time the columns add | {g['time_us']:.1f} us |",
              f"| columns gathered (per query block, summed) | {g['columns']} |",
              f"| HBM bytes the columns add | {g['hbm_bytes'] / 1e6:.1f} MB |",
              f"| HBM rate | {g['hbm_GBps']:.0f} GB/s, {g['hbm_pct']:.1f}% of 8 TB/s |",
              f"| algorithmic bytes (K and V rows staged into LDS) | {g['staged_bytes'] / 1e6:.1f} MB |",
              f"| algorithmic rate | {g['staged_GBps']:.0f} GB/s, {g['staged_pct']:.1f}% of 8 TB/s |",
              f"| share of the staged rows fetched from HBM | "
              f"{100.0 * g['hbm_bytes'] / max(g['staged_bytes'], 1):.1f}% |", ""]
    return "\n".join(lines)


def gather_record_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"gather_{workload_name}.json")


def current_gather_record(workload_name: str):
    """The committed gather record for a workload if it was taken on the
    current kernel sources, else None."""
    p = gather_record_path(workload_name)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != source_sha256():
        return None
    return rec


def record_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"layer_kernels_{workload_name}.json")


def current_record(workload_name: str):
    """The committed record for a workload if it was taken on the current
    kernel sources, else None."""
    p = record_path(workload_name)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != source_sha256():
        return None
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", required=True, help="workload key (c2, c3, ...)")
    ap.add_argument("--steps", type=int, required=True, help="passes of the layer in the trace (warmup + timed)")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--sq")
    ap.add_argument("--bench-log", help="output of the traced bench run (its JSON line)")
    ap.add_argument("--command", default="")
    ap.add_argument("--title", default=None)
    ap.add_argument("--out", default=None, help="output path without extension (default profiles/layer_kernels_<name>)")
    ap.add_argument("--gather", action="store_true",
                    help="the runs are of bench.py --gather-only: write profiles/gather_<name>")
    args = ap.parse_args(argv)
    if args.gather:
        rec = build_gather_record(args)
        out = args.out or os.path.splitext(gather_record_path(rec["workload"]))[0]
        with open(out + ".json", "w") as fh:
            json.dump(rec, fh, indent=1)
        with open(out + ".md", "w") as fh:
            fh.write(gather_markdown(rec))
        print(out + ".md")
        return
    rec = build_record(args)
    out = args.out or os.path.splitext(record_path(rec["workload"]))[0]
    import workloads as W
    w = W.WORKLOADS[args.workload]
    title = args.title or (f"Kernel trace and HBM bytes: {w.name} (B={w.batch}, {w.heads_q}/{w.heads_kv} heads, "
                           f"N={w.seq_len}, d={w.head_dim}, {w.dtype}, patterns {w.patterns})")
    with open(out + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(out + ".md", "w") as fh:
        fh.write(markdown(rec, title))
    print(out + ".md")


if __name__ == "__main__":
    main()
