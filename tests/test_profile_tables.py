"""The rocprofv3 table step: name parsing, counter scaling, algorithmic bytes
and the source-hash guard (CPU only, on small synthetic CSV files)."""
import json
import os

import pytest

from dynamic_sparse_attention_amd import profile_tables as P
import workloads as W


def test_short_names():
    assert P.short_name("void mi::(anonymous namespace)::sparse_attn_kernel<unsigned short, 128, false>"
                        "(mi::(anonymous namespace)::Params)") == "sparse_attn_kernel<bf16, 128, false>"
    assert P.short_name("mi::(anonymous namespace)::topk_hist(mi::TopkP, int)") == "topk_hist"
    assert P.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def _stats(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "t_kernel_stats.csv"), "w") as fh:
        fh.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        for name, calls, avg in rows:
            fh.write(f'"{name}",{calls},{calls * avg},{avg},1,{avg},{avg},0\n')


def _pmc(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w") as fh:
        fh.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for i, (name, ctr, val) in enumerate(rows):
            fh.write(f'{i},"{name}","{ctr}",{val}\n')


def test_record_scaling_and_rates(tmp_path):
    att = "void mi::(anonymous namespace)::sparse_attn_kernel<unsigned short, 128, false>(P)"
    _stats(tmp_path / "trace", [(att, 3, 100e6), ("void at::native::fill(int)", 5, 1e3)])
    _pmc(tmp_path / "fetch", [(att, "FETCH_SIZE", 1000.0), (att, "FETCH_SIZE", 3000.0)])
    _pmc(tmp_path / "write", [(att, "WRITE_SIZE", 500.0)])
    copy = "void at::native::copy_kernel(int)"
    _pmc(tmp_path / "cf", [(copy, "FETCH_SIZE", (1 << 20) / 2), ("small(int)", "FETCH_SIZE", 4.0)])
    _pmc(tmp_path / "cw", [(copy, "WRITE_SIZE", 1 << 20)])

    class A:
        workload, steps, command, bench_log, sq = "c3", 3, "cmd", None, None
        trace, fetch, write = str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write")
        copy_fetch, copy_write = str(tmp_path / "cf"), str(tmp_path / "cw")
    rec = P.build_record(A)
    assert rec["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    assert [r["kernel"] for r in rec["kernels"]] == ["sparse_attn_kernel<bf16, 128, false>"]
    r = rec["kernels"][0]
    # mean FETCH 2000 KiB x 2 + WRITE 500 KiB x 1, over 100 ms
    assert r["measured_bytes"] == (2000 * 2 + 500) * 1024
    assert r["measured_GBps"] == pytest.approx(r["measured_bytes"] / 1e8, abs=0.1)
    w = W.C3
    alg = 2 * 32 * w.seq_len * 128 * 2 + 2 * 8 * w.seq_len * 128 * 2 + 32 * w.seq_len * 4
    assert r["algorithmic_bytes"] == alg  # one launch per pass
    assert "sparse_attn_kernel" in P.markdown(rec, "t")


def test_current_record_needs_the_same_sources(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256": P.source_sha256(), "kernels": []}
    monkeypatch.setattr(P, "record_path", lambda name: str(tmp_path / f"{name}.json"))
    (tmp_path / "x.json").write_text(json.dumps(rec))
    assert P.current_record("x") == rec
    rec["kernel_source_sha256"] = "0" * 64
    (tmp_path / "x.json").write_text(json.dumps(rec))
    assert P.current_record("x") is None
    assert P.current_record("absent") is None


def test_committed_records_name_their_workload():
    d = os.path.join(P.ROOT, "profiles")
    names = {w.name for w in W.WORKLOADS.values()}
    for f in os.listdir(d):
        if f.endswith(".json"):
            rec = json.load(open(os.path.join(d, f)))
            assert rec["workload"] in names
            assert len(rec["kernel_source_sha256"]) == 64


def test_gather_record_takes_the_difference_of_the_two_launch_groups(tmp_path):
    """bench.py --gather-only launches the attention eight times: one warmup
    and three timed with the column index, then the same without columns;
    the gather's time and HBM bytes are the differences of the medians of
    the timed launches, with the counters scaled by the copy calibration."""
    att = "void mi::(anonymous namespace)::sparse_attn_kernel<unsigned short, 128, false, false>(P)"
    other = "mi::(anonymous namespace)::build_index_kernel(P)"
    (tmp_path / "trace").mkdir()
    with open(tmp_path / "trace" / "t_kernel_trace.csv", "w") as fh:
        fh.write('"Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        durs = [9e6, 5e6, 5.2e6, 4.8e6, 3e6, 2e6, 2.1e6, 1.9e6]  # ns: warmup, timed x3; twice
        t = 0
        for i, dn in enumerate(durs):
            fh.write(f'{2 * i},"{other}",{t},{t + 1000}\n')
            fh.write(f'{2 * i + 1},"{att}",{t + 2000},{t + 2000 + int(dn)}\n')
            t += 10 ** 8
    fetch = [50.0, 40.0, 41.0, 39.0, 20.0, 10.0, 10.0, 10.0]  # KiB
    write = [8.0, 6.0, 6.0, 6.0, 6.0, 5.0, 5.0, 5.0]
    _pmc(tmp_path / "fetch", [(n, "FETCH_SIZE", v) for i, v in enumerate(fetch) for n in (other, att)])
    _pmc(tmp_path / "write", [(n, "WRITE_SIZE", v) for i, v in enumerate(write) for n in (other, att)])
    copy = "void at::native::copy_kernel(int)"
    _pmc(tmp_path / "cf", [(copy, "FETCH_SIZE", (1 << 20) / 2)])
    _pmc(tmp_path / "cw", [(copy, "WRITE_SIZE", 1 << 20)])
    log = tmp_path / "bench.log"
    log.write_text('[bench] column gather rate\n{"workload": "x", "gather": {"columns": 7, "bytes": 9000000}}\n')

    class A:
        workload, steps, command = "c3", 8, "cmd"
        trace, fetch, write = str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write")
        copy_fetch, copy_write, bench_log = str(tmp_path / "cf"), str(tmp_path / "cw"), str(log)
    rec = P.build_gather_record(A)
    assert rec["launches"]["columns"]["avg_us"] == pytest.approx(5000.0)
    assert rec["launches"]["diagonal_only"]["avg_us"] == pytest.approx(2000.0)
    g = rec["gather"]
    assert g["time_us"] == pytest.approx(3000.0)
    # FETCH medians 40 and 10 KiB (x 2), WRITE 6 and 5 KiB (x 1)
    assert g["hbm_bytes"] == (40 - 10) * 2 * 1024 + (6 - 5) * 1024
    assert g["hbm_GBps"] == pytest.approx(g["hbm_bytes"] / 3e6, abs=0.1)
    assert g["staged_bytes"] == 9000000 and g["columns"] == 7
    assert g["staged_GBps"] == pytest.approx(3.0)  # 9 MB in 3 ms
    assert rec["workload"] == W.C3.name
    assert "Column gather" in P.gather_markdown(rec)
    # a run that lost a launch is refused
    _pmc(tmp_path / "write", [(att, "WRITE_SIZE", v) for v in write[:7]])
    with pytest.raises(ValueError):
        P.build_gather_record(A)
