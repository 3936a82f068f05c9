"""Summaries of rocprofv3 CSV output for the read's kernels (markdown).

    python -m hyper_connection_residual_amd.rocprof_summary stats <kernel_stats.csv> > out.md
    python -m hyper_connection_residual_amd.rocprof_summary trace <kernel_trace.csv> > out.md
    python -m hyper_connection_residual_amd.rocprof_summary bytes <fetch counter_collection.csv> \
        <write counter_collection.csv> <fetch run log> <write run log> > out.md

`stats` tabulates per-kernel durations; `trace` does the same per (kernel,
workgroup count), which separates launches of one kernel at different sizes.  `bytes` tabulates HBM bytes per
dispatch from one FETCH_SIZE run and one WRITE_SIZE run (KiB per dispatch).
Both counters are scaled by what they read for a plain device-to-device copy of
known size run in the same process (the runtime's copy kernel, which bench.py
--calib-copy launches: 5 copies of 256 MiB); the scale factors are printed.  The
short-window kernel's sweep average (T = 1..8) is printed on a line bench.py
reads, together with the hash of the kernel sources the profiled runs were
built from, taken from those runs' own output (bench.py prints it; both runs
must agree), so a later change to the kernels makes bench.py report the
traffic as unknown.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import os
import re
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_PKG, "csrc")
COPY_BYTES = 5 * (256 << 20)  # bench.py --calib-copy


def source_hash() -> str:
    """Hash of the library's kernel and host sources and its build flags."""
    from hyper_connection_residual_amd import build
    h = hashlib.sha256(" ".join(build.FLAGS).encode())
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def hash_in_log(path: str):
    """The kernel source hash a bench.py run printed, or None."""
    with open(path, errors="replace") as f:
        for line in f:
            m = re.search(r"kernel source hash: (\w+)", line)
            if m:
                return m.group(1)
    return None


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def stats(path: str) -> str:
    out = ["| kernel | calls | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    with open(path) as f:
        for row in csv.DictReader(f):
            out.append("| %s | %s | %.3f | %.3f | %.3f | %.3f |" % (
                short_name(row["Name"]), row["Calls"], float(row["AverageNs"]) / 1e3,
                float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3,
                float(row["TotalDurationNs"]) / 1e6))
    return "\n".join(out)


def trace(path: str) -> str:
    groups = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            wgs = int(row["Grid_Size_X"]) // max(1, int(row["Workgroup_Size_X"]))
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups[(short_name(row["Kernel_Name"]), wgs)].append(dur)
    out = ["| kernel | workgroups | calls | avg us | median us | min us | max us |", "|---|---|---|---|---|---|---|"]
    for (name, wgs), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d = sorted(d)
        out.append("| %s | %d | %d | %.3f | %.3f | %.3f | %.3f |" % (
            name, wgs, len(d), sum(d) / len(d), d[len(d) // 2], d[0], d[-1]))
    return "\n".join(out)


def _per_kernel(path):
    acc = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            acc[short_name(row["Kernel_Name"])].append(float(row["Counter_Value"]) * 1024.0)
    return acc


def traffic(fetch_path: str, write_path: str, fetch_log: str, write_log: str) -> str:
    hashes = {hash_in_log(fetch_log), hash_in_log(write_log)}
    if len(hashes) != 1 or None in hashes:
        raise SystemExit("the two profiled runs printed different (or no) kernel source hashes: %s" % hashes)
    run_hash = hashes.pop()
    fetch, write = _per_kernel(fetch_path), _per_kernel(write_path)
    copy = "__amd_rocclr_copyBuffer"
    f_scale = COPY_BYTES / sum(fetch[copy]) if fetch.get(copy) else float("nan")
    w_scale = COPY_BYTES / sum(write[copy]) if write.get(copy) else float("nan")
    out = ["copy-kernel calibration: FETCH_SIZE x %.3f, WRITE_SIZE x %.3f "
           "(%d MiB copied)" % (f_scale, w_scale, COPY_BYTES >> 20), "",
           "| kernel | dispatches | HBM read MB | HBM write MB |", "|---|---|---|---|"]
    sweep = []
    for k in sorted(set(fetch) | set(write)):
        fr = fetch.get(k, [0.0])
        wr = write.get(k, [0.0])
        rd = f_scale * sum(fr) / len(fr)
        wt = w_scale * sum(wr) / len(wr)
        out.append("| %s | %d | %.3f | %.3f |" % (k, len(fr), rd / 1e6, wt / 1e6))
        m = re.match(r"hc::decode_kernel<(\d+)>", k)
        if m and 1 <= int(m.group(1)) <= 8:  # the verify-window sweep's instances
            sweep.append(rd + wt)
    if sweep:
        out += ["", "short-window kernel HBM bytes per launch (sweep average): %d" % round(sum(sweep) / len(sweep)),
                "short-window kernel source hash: %s" % run_hash]
    return "\n".join(out)


def read_traffic(md_path: str):
    """(bytes per launch, source hash) from a `bytes` summary, or None."""
    if not os.path.exists(md_path):
        return None
    val = h = None
    with open(md_path) as f:
        for line in f:
            m = re.match(r"short-window kernel HBM bytes per launch \(sweep average\): (\d+)", line)
            if m:
                val = int(m.group(1))
            m = re.match(r"short-window kernel source hash: (\w+)", line)
            if m:
                h = m.group(1)
    return (val, h) if val is not None else None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "trace":
        print(trace(sys.argv[2]))
    elif sys.argv[1] == "bytes":
        print(traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5]))
    else:
        raise SystemExit(__doc__)
