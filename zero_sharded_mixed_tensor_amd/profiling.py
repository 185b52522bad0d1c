"""Summaries of rocprofv3 runs of bench.py, kept as short text under profiles/.

    python -m zero_sharded_mixed_tensor_amd.profiling trace  --dir D --command CMD --out profiles/X.md
    python -m zero_sharded_mixed_tensor_amd.profiling counters --fetch D1 --write D2 --command CMD \
        --workload W --params N --out profiles/Y.md

`trace` turns a `--kernel-trace --stats` CSV directory into a per-kernel table
(calls, average and total duration). `counters` turns two `--pmc FETCH_SIZE`
and `--pmc WRITE_SIZE` runs into HBM bytes per launch for each kernel of the
library. Both counters are scaled by what they read for a device copy of
known size in the same run (bench.py --copy-calibration copies 1 GiB five
times): FETCH_SIZE's derived formula assumes 64-byte read requests, so on
this GPU it reads half of the bytes moved and the factor comes out near 2.
The counters summary records a hash of the kernel sources; bench.py reports
the traffic only while the sources still match it.
"""

import argparse
import collections
import csv
import glob
import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# kernel name prefix -> sources that define it
KERNEL_SOURCES = {
    "adam_wide_kernel": ["csrc/zds_adam.hip", "csrc/zds_device.h", "csrc/zds_internal.h", "build.py"],
    "norm_stage1": ["csrc/zds_norm.hip", "csrc/zds_device.h", "csrc/zds_internal.h", "build.py"],
    "accumulate_kernel": ["csrc/zds_accumulate.hip", "csrc/zds_device.h", "csrc/zds_internal.h", "build.py"],
    "reduce_peers_kernel": ["csrc/zds_reduce.hip", "csrc/zds_device.h", "csrc/zds_internal.h", "build.py"],
    "onebit_encode_kernel": ["csrc/zds_onebit.hip", "csrc/zds_onebit.h", "csrc/zds_device.h", "csrc/zds_internal.h",
                             "build.py"],
    "onebit_decode_kernel": ["csrc/zds_onebit.hip", "csrc/zds_onebit.h", "csrc/zds_device.h", "csrc/zds_internal.h",
                             "build.py"],
    "onebit_decode_quarter_kernel": ["csrc/zds_onebit.hip", "csrc/zds_onebit.h", "csrc/zds_device.h",
                                     "csrc/zds_internal.h", "build.py"],
}
CALIB_BYTES = 1 << 30


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name):
    m = re.search(r"zds::(\w+)", name)
    if m:
        t = re.search(r"<([^>]*)>", name)
        return m.group(1) + ("<%s>" % t.group(1) if t else "")
    return name[:60]


def _csv(d, suffix):
    fs = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not fs:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return fs[0]


def trace_summary(d, command, skip=0):
    """Per-kernel table from --stats, plus the average over each kernel's
    launches after the first `skip` (the bench's warm-up steps), taken from
    the per-dispatch trace."""
    rows = list(csv.DictReader(open(_csv(d, "kernel_stats.csv"))))
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(_csv(d, "kernel_trace.csv"))):
        per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = ["# rocprofv3 kernel trace", "", "Command:", "", "    " + command, "",
           "| kernel | calls | avg us | avg us after %d warm-up launches | total us | %% |" % skip,
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        d_ns = per.get(r["Name"], [])
        steady = d_ns[skip:] if len(d_ns) > skip else d_ns
        out.append("| %s | %s | %.2f | %s | %.1f | %s |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            ("%.2f" % (sum(steady) / len(steady) / 1e3)) if steady else "-",
            float(r["TotalDurationNs"]) / 1e3, r["Percentage"]))
    return "\n".join(out) + "\n"


def _counter_rows(d, counter):
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(_csv(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def _calibration(per):
    """KiB the counter reads per launch of the 1 GiB calibration copy: the
    non-library kernel whose value is closest to 1 GiB (or half of it)."""
    best = None
    for name, vals in per.items():
        if "zds::" in name or "copy" not in name.lower():
            continue
        for v in vals:
            for frac in (1.0, 0.5):
                err = abs(v - frac * CALIB_BYTES / 1024) / (CALIB_BYTES / 1024)
                if err < 0.01 and (best is None or err < best[0]):
                    best = (err, v, name)
    if best is None:
        raise SystemExit("calibration copy not found in the counter run")
    return best[1], best[2]


def counters_summary(fetch_dir, write_dir, command, workload, params):
    fr = _counter_rows(fetch_dir, "FETCH_SIZE")
    wr = _counter_rows(write_dir, "WRITE_SIZE")
    fc, fname = _calibration(fr)
    wc, wname = _calibration(wr)
    ffac = (CALIB_BYTES / 1024) / fc
    wfac = (CALIB_BYTES / 1024) / wc
    out = ["# rocprofv3 HBM byte counters", "", "Workload: %s (%d params per launch)" % (workload, params), "",
           "Commands (one counter per run):", ""]
    for c in command:
        out.append("    " + c)
    out += ["", "Calibration: a device copy of 1 GiB read + 1 GiB write (%s) reads FETCH_SIZE %.1f KiB "
            "and WRITE_SIZE %.1f KiB per launch, so FETCH_SIZE is scaled by %.4f and WRITE_SIZE by %.4f."
            % (_short(fname), fc, wc, ffac, wfac), "",
            "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read B/param | write B/param | "
            "traffic bytes/launch |", "|---|---:|---:|---:|---:|---:|---:|"]
    for name in sorted(set(fr) | set(wr)):
        if "zds::" not in name:
            continue
        f = sum(fr.get(name, [0])) / max(1, len(fr.get(name, [])))
        w = sum(wr.get(name, [0])) / max(1, len(wr.get(name, [])))
        rb = f * 1024 * ffac
        wb = w * 1024 * wfac
        out.append("| %s | %d | %.1f | %.1f | %.3f | %.3f | %d |" % (
            _short(name), len(fr.get(name, [])), f, w, rb / params, wb / params, int(rb + wb)))
    out += ["", "Source hashes at the time of the runs:", ""]
    for k in sorted(KERNEL_SOURCES):
        out.append("    source_hash %s %s" % (k, kernel_source_hash(k)))
    return "\n".join(out) + "\n"


def traffic_from_summary(path, kernel):
    """Bytes per launch of `kernel` from a counters summary, or None if the
    file is missing or the kernel's sources changed since it was written."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_hash %s (\w+)" % kernel, text)
    if not m or m.group(1) != kernel_source_hash(kernel):
        return None
    for line in text.splitlines():
        if line.startswith("| %s" % kernel):
            return int(line.rstrip("|").split("|")[-1])
    return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--skip", type=int, default=0, help="warm-up launches per kernel to leave out")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--params", type=int, required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "trace":
        text = trace_summary(a.dir, a.command, a.skip)
    else:
        text = counters_summary(a.fetch, a.write, a.command, a.workload, a.params)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
