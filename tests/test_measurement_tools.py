"""CPU checks of the measurement tooling: the rocprofv3 summaries (trace
averages after warm-up launches, counter scaling by the calibration copy,
traffic lookup guarded by the source hash) and the bench's CPU-side contract
(one GPU only, the per-kernel byte model)."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from zero_sharded_mixed_tensor_amd import profiling as P  # noqa: E402

ADAM = "void zds::adam_wide_kernel<1, 1, true, 16>(zds::AdamArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_skips_warm_up_launches(tmp_path):
    d = str(tmp_path / "trace")
    _write(os.path.join(d, "x", "bench_kernel_stats.csv"),
           ["Name", "Calls", "AverageNs", "TotalDurationNs", "Percentage"],
           [[ADAM, 5, 3000.0, 15000.0, 100.0]])
    # two slow warm-up launches, then three of 2 us
    durs = [5000, 4000, 2000, 2000, 2000]
    rows, t = [], 0
    for d_ns in durs:
        rows.append([ADAM, t, t + d_ns])
        t += 10_000
    _write(os.path.join(d, "x", "bench_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           rows)
    out = P.trace_summary(d, "cmd --flag", skip=2)
    line = [ln for ln in out.splitlines() if ln.startswith("| adam_wide_kernel<1, 1, true, 16>")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "5" and cells[2] == "3.00" and cells[3] == "2.00" and cells[4] == "15.0"
    assert "    cmd --flag" in out


def test_counters_scale_by_the_calibration_copy(tmp_path, monkeypatch):
    # FETCH_SIZE reads half of the bytes of the 1 GiB copy (factor 2), WRITE_SIZE all of them
    gib_kib = (1 << 30) / 1024
    params = 1000
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(os.path.join(fd, "bench_counter_collection.csv"), hdr,
           [[COPY, "FETCH_SIZE", gib_kib / 2], [ADAM, "FETCH_SIZE", 7.0], [ADAM, "FETCH_SIZE", 7.0]])
    _write(os.path.join(wd, "bench_counter_collection.csv"), hdr,
           [[COPY, "WRITE_SIZE", gib_kib], [ADAM, "WRITE_SIZE", 14.0], [ADAM, "WRITE_SIZE", 14.0]])
    out = P.counters_summary(fd, wd, ["c1", "c2"], "wl", params)
    line = [ln for ln in out.splitlines() if ln.startswith("| adam_wide_kernel")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    # read 7 KiB x 2 = 14336 B, written 14 KiB = 14336 B per launch
    assert cells[1] == "2" and cells[4] == "14.336" and cells[5] == "14.336" and cells[6] == "28672"
    assert "scaled by 2.0000" in out and "by 1.0000" in out
    path = tmp_path / "summary.md"
    path.write_text(out)
    assert P.traffic_from_summary(str(path), "adam_wide_kernel") == 28672
    # a changed source invalidates the figure
    monkeypatch.setattr(P, "kernel_source_hash", lambda k: "0" * 16)
    assert P.traffic_from_summary(str(path), "adam_wide_kernel") is None
    assert P.traffic_from_summary(str(tmp_path / "missing.md"), "adam_wide_kernel") is None


def test_counters_need_the_calibration_copy(tmp_path):
    fd = str(tmp_path / "f")
    _write(os.path.join(fd, "bench_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           [[ADAM, "FETCH_SIZE", 7.0]])
    with pytest.raises(SystemExit):
        P.counters_summary(fd, fd, ["c"], "wl", 10)


def test_committed_summaries_name_their_commands():
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        text = open(os.path.join(ROOT, "profiles", f)).read()
        assert "rocprofv3 " in text and "bench.py --workload" in text, f


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_bench_byte_model():
    sys.path.insert(0, ROOT)
    import bench
    w = bench._workload("llama7b_s1")
    assert bench._bytes_per_param(w, True) == dict(accum_total=4, norm=0, adam=28)
    assert bench._bytes_per_param(w, False) == dict(accum_total=4, norm=2, adam=28)
    w = bench._workload("llama7b_s1_accum16")
    assert bench._bytes_per_param(w, True) == dict(accum_total=6 + 10 * 15, norm=0, adam=30)
    w = bench._workload("llama7b_s2_intake8")
    assert bench._bytes_per_param(w, False) == dict(accum_total=20, norm=4, adam=30)
    assert bench._bytes_per_param(w, True) == dict(accum_total=20, norm=0, adam=30)


@pytest.mark.parametrize("workload", ["llama7b_s1", "llama7b_s1_accum16", "llama7b_s2_intake8", "llama7b_s1_onebit8"])
def test_cpu_baselines_time_the_workloads_own_oracle_step(workload):
    sys.path.insert(0, ROOT)
    import bench
    w = bench._workload(workload)
    if w.get("onebit"):
        c = bench.run_cpu_baseline_onebit(w, 4096, 1, min_seconds=0.0)
    else:
        # several processes over pieces with a ragged last one
        c = bench.run_cpu_baseline(w, 4096 + 1000, 1, procs=3, chunk=1024)
        assert c["what"] == {"llama7b_s1": "copy", "llama7b_s1_accum16": "accumulation of 16 micro-batches",
                             "llama7b_s2_intake8": "intake of 8 peers' slices"}[workload]
        assert c["procs"] == 3 and c["n"] == 5096 and c["shard"] == 842301440
        c["n"] -= 1000
    assert c["repeats"] == 1 and c["n"] == 4096 and c["value"] > 0
