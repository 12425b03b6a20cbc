"""bench.py on the host (no GPU): --summarize on synthetic rocprofv3 CSV
files (the library's dispatches are matched in order to the workloads of the
profile run, other kernels are ignored, and a dispatch out of plan is an
error); --gpus above 1 is refused; measured traffic is reported only from a
profile of the current kernel sources."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def plan_names():
    out = []
    for name, kernels in bench.PROFILE_PLAN:
        for _ in range(bench.PROFILE_LAUNCHES):
            out.extend((name, k) for k in kernels)
    return out


def write_trace(path, entries):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Correlation_Id", "Kernel_Name", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        for i, (name, dur) in enumerate(entries):
            w.writerow({"Correlation_Id": i + 1, "Kernel_Name": name, "Start_Timestamp": 1000 * i,
                        "End_Timestamp": 1000 * i + dur})


def run(directory):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize",
                           str(directory)], capture_output=True, text=True)


def test_durations_per_workload(tmp_path):
    entries = []
    for n, (w, k) in enumerate(plan_names()):
        entries.append(("void at::native::fill_kernel(int)", 5))  # torch's own kernels interleave
        entries.append((f"void rowstats::{k}(rowstats::RowStatsParams)",
                        100 + 10 * [x for x, _ in bench.PROFILE_PLAN].index(w)))
    write_trace(tmp_path / "t_kernel_trace.csv", entries)
    r = run(tmp_path)
    assert r.returncode == 0, r.stderr
    rows = [l.split(" | ") for l in r.stdout.splitlines() if not l.startswith("#")]
    got = {(w, k): (int(n), float(mean)) for w, k, _, n, mean, *_ in rows}
    for i, (w, kernels) in enumerate(bench.PROFILE_PLAN):
        for k in kernels:
            assert got[(w, k)] == (bench.PROFILE_LAUNCHES, 100.0 + 10 * i)


def test_a_dispatch_out_of_plan_is_an_error(tmp_path):
    names = plan_names()
    entries = [(f"void rowstats::{k}(x)", 100) for _, k in names]
    entries[3] = ("void rowstats::topk_kernel<true>(x)", 100)
    write_trace(tmp_path / "t_kernel_trace.csv", entries)
    r = run(tmp_path)
    assert r.returncode != 0 and "the plan has" in r.stderr


def test_a_missing_dispatch_is_an_error(tmp_path):
    entries = [(f"void rowstats::{k}(x)", 100) for _, k in plan_names()][:-1]
    write_trace(tmp_path / "t_kernel_trace.csv", entries)
    r = run(tmp_path)
    assert r.returncode != 0 and "dispatches of this library" in r.stderr


def test_the_one_time_table_packing_is_not_a_step(tmp_path):
    # the embedding table is packed once before the product's timed calls
    names = plan_names()
    entries = [(f"void rowstats::{k}(x)", 100) for _, k in names]
    at = next(i for i, (w, _) in enumerate(names) if w == "SP")
    entries.insert(at, ("void rowstats::(anonymous namespace)::pack_embed_kernel(x)", 7))
    write_trace(tmp_path / "t_kernel_trace.csv", entries)
    r = run(tmp_path)
    assert r.returncode == 0, r.stderr
    assert "pack_embed" not in r.stdout


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    # traffic is reported only from a profile taken of the current kernel sources
    f = tmp_path / "hbm_traffic.txt"
    line = "C2 kernel=k fetch_kib=1 write_kib=1 fetch_bytes=1000 write_bytes=24 ratio=1\n"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(f"# header\nsource_hash {bench.source_hash()}\n" + line)
    assert bench.recorded_traffic("C2") == 1024
    assert bench.recorded_traffic("C3") is None
    f.write_text("# header\nsource_hash 0123456789abcdef\n" + line)
    assert bench.recorded_traffic("C2") is None
