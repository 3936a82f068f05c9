"""Summaries of rocprofv3 CSV output for the read's kernels (markdown).

    python -m hyper_connection_residual_amd.rocprof_summary stats <kernel_stats.csv> > out.md
    python -m hyper_connection_residual_amd.rocprof_summary trace <kernel_trace.csv> > out.md
    python -m hyper_connection_residual_amd.rocprof_summary counters <run log>... -- <counter_collection.csv>... > out.md

`stats` tabulates per-kernel durations; `trace` does the same per (kernel,
workgroup count), which separates launches of one kernel at different sizes.
`counters` averages every collected counter per dispatch and kernel size and
derives HBM bytes from the per-size request counters (no calibration factor),
the matrix cores' busy share and bf16 matrix flops.  It also writes the
short-window kernel's HBM bytes per launch, averaged over the verify-window
sweep, on a line bench.py reads, together with the hash of the kernel sources
the profiled runs were built from, taken from those runs' own output (bench.py
prints it; every run must agree), so a later change to the kernels makes
bench.py report the traffic as unknown.
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


def _clusters(d):
    """Sorted durations split where one is more than 1.6x the one before (a
    persistent kernel launched at several read sizes keeps its grid); a group
    of fewer than 3 durations is an outlier of the group below it, not a size
    of its own."""
    d = sorted(d)
    out, cur = [], [d[0]]
    for v in d[1:]:
        if v > 1.6 * cur[-1] and len(cur) >= 3:
            out.append(cur)
            cur = []
        cur.append(v)
    if out and len(cur) < 3:
        out[-1].extend(cur)
    else:
        out.append(cur)
    return out


def trace(path: str) -> str:
    """The library's kernels (hc::) per (kernel, workgroup count); a group
    whose durations fall into clusters more than 1.6x apart gets a row each."""
    groups = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if not row["Kernel_Name"].replace("void ", "").startswith("hc::"):
                continue
            wgs = int(row["Grid_Size_X"]) // max(1, int(row["Workgroup_Size_X"]))
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups[(short_name(row["Kernel_Name"]), wgs)].append(dur)
    rows = []
    for (name, wgs), d in groups.items():
        cl = _clusters(d)
        for i, c in enumerate(cl):
            tag = "" if len(cl) == 1 else " (size %d of %d)" % (i + 1, len(cl))
            p10, p90 = c[(len(c) - 1) // 10], c[(9 * (len(c) - 1)) // 10]  # (nearest rank, lower)
            rows.append((sum(c), "| %s%s | %d | %d | %.3f | %.3f | %.3f | %.3f | %.3f | %.3f |" % (
                name, tag, wgs, len(c), sum(c) / len(c), c[len(c) // 2], p10, p90, c[0], c[-1])))
    out = ["| kernel | workgroups | calls | avg us | median us | p10 us | p90 us | min us | max us |",
           "|---|---|---|---|---|---|---|---|---|"]
    out += [r for _, r in sorted(rows, key=lambda x: -x[0])]
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


def _counter_rows(paths, split=r"prefill_upmix3"):
    """{(kernel, workgroups, size): {counter: [value per dispatch]}} over
    counter runs.  A persistent kernel (`split`) keeps its grid at every read
    size, so its dispatches are split by size: within each run they are
    clustered by their summed counter values (clusters more than 1.6x apart),
    and size i is the i-th smallest cluster of every run.  Other kernels keep
    one row per grid (a grid run at several sizes is averaged over them)."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        disp = collections.defaultdict(dict)  # (kernel, wgs, dispatch id) -> {counter: value}
        with open(path) as f:
            for row in csv.DictReader(f):
                wgs = int(row["Grid_Size"]) // max(1, int(row["Workgroup_Size"]))
                disp[(short_name(row["Kernel_Name"]), wgs, row["Dispatch_Id"])][row["Counter_Name"]] = \
                    float(row["Counter_Value"])
        by_kernel = collections.defaultdict(list)
        for (k, wgs, _), cs in disp.items():
            by_kernel[(k, wgs)].append(cs)
        for (k, wgs), ds in by_kernel.items():
            ds.sort(key=lambda cs: sum(cs.values()))
            size = 0
            prev = None
            for cs in ds:
                tot = sum(cs.values())
                if re.search(split, k) and prev is not None and prev > 0 and tot > 1.6 * prev:
                    size += 1
                prev = tot
                for c, v in cs.items():
                    acc[(k, wgs, size)][c].append(v)
    return acc


def counters(log_paths, csv_paths, kernels=r"hc::|copyBuffer") -> str:
    """Per (kernel, workgroup count): every collected counter averaged per
    dispatch, and the figures derived from them: HBM bytes from the per-size
    request counters (32 / 64 / 128-byte reads, 32 / 64-byte writes: no
    calibration factor), MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES, summed over
    the 1024 SIMDs, over SQ_BUSY_CYCLES, summed over the 32 shader engines of
    32 SIMDs each) and bf16 matrix flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512).
    The short-window kernel's HBM bytes per launch, averaged over the
    verify-window sweep (T = 1..8), go on a line bench.py reads, with the
    kernel-source hash that every profiled run printed (they must agree)."""
    hashes = {hash_in_log(p) for p in log_paths}
    if len(hashes) != 1 or None in hashes:
        raise SystemExit("the profiled runs printed different (or no) kernel source hashes: %s" % hashes)
    run_hash = hashes.pop()
    acc = _counter_rows(csv_paths)
    names = sorted({c for v in acc.values() for c in v})
    sweep = []
    out = ["counters taken on kernel source hash %s" % run_hash, "",
           "| kernel | workgroups | dispatches | " + " | ".join(names) + " | derived |",
           "|---|---|---|" + "---|" * len(names) + "---|"]
    sizes = collections.Counter((k, wgs) for (k, wgs, _) in acc)
    for (k, wgs, size), cs in sorted(acc.items()):
        if not re.search(kernels, k):
            continue
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        der = []
        rd = None
        if all(c in mean for c in ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")):
            rd = 32 * mean["TCC_EA0_RDREQ_32B_sum"] + 64 * mean["TCC_EA0_RDREQ_64B_sum"] + \
                128 * mean["TCC_EA0_RDREQ_128B_sum"]
            der.append("read %.3f MB" % (rd / 1e6))
        if all(c in mean for c in ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")):
            wr = 64 * mean["TCC_EA0_WRREQ_64B_sum"] + 32 * (mean["TCC_EA0_WRREQ_sum"] - mean["TCC_EA0_WRREQ_64B_sum"])
            der.append("written %.3f MB" % (wr / 1e6))
            mm = re.match(r"hc::decode_kernel<(\d+)>", k)
            if mm and 1 <= int(mm.group(1)) <= 8 and rd is not None:
                sweep.append(rd + wr)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("SQ_BUSY_CYCLES", 0) > 0:
            der.append("MFMA busy %.1f %%" % (100 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (32 * mean["SQ_BUSY_CYCLES"])))
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean:
            der.append("bf16 MFMA %.2f GFLOP" % (512 * mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / 1e9))
        tag = "" if sizes[(k, wgs)] == 1 else " (size %d of %d)" % (size + 1, sizes[(k, wgs)])
        out.append("| %s%s | %d | %d | " % (k, tag, wgs, n) + " | ".join(
            ("%.4g" % mean[c]) if c in mean else "" for c in names) + " | " + "; ".join(der) + " |")
    if sweep:
        out += ["", "short-window kernel HBM bytes per launch (sweep average): %d" % round(sum(sweep) / len(sweep)),
                "short-window kernel source hash: %s" % run_hash]
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "trace":
        print(trace(sys.argv[2]))
    elif sys.argv[1] == "counters":  # counters <log>... -- <csv>...
        cut = sys.argv.index("--")
        print(counters(sys.argv[2:cut], sys.argv[cut + 1:]))
    else:
        raise SystemExit(__doc__)
