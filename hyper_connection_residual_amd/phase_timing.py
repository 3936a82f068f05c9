"""Where the time of a short-window read goes: per-phase clock stamps.

    python -m hyper_connection_residual_amd.build --probe
    python -m hyper_connection_residual_amd.phase_timing [--T 1,2,...] [--reads 64] > out.md

Loads the timing build (libhc_probe.so, whose short-window kernel records the
100 MHz wall clock per workgroup at numbered points) in place of libhc.so, runs
back-to-back reads of the verify-window sweep's shape (pending write, 48
rotated weight sets, as bench.py), and prints a markdown table per token count:
for each point, the median over reads of the median and the latest workgroup,
in microseconds after the read's first workgroup started.  Measurement only:
the product never loads the timing build.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(_PKG))

POINTS = [(0, "entry"), (1, "W_down tile + activations landed"), (2, "down products done"),
          (3, "partial dots stored"), (12, "hop 1: partials seen (reducers)"),
          (13, "hop 1: lo published (reducers)"), (14, "hop 2: lo seen"), (7, "lo staged"),
          (8, "W_up tile landed, lo complete"), (9, "outputs stored"), (15, "exit")]
N_SETS = 48


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--T", default="1,2,3,4,5,6,7,8")
    ap.add_argument("--reads", type=int, default=64)
    args = ap.parse_args()
    assert 1 <= args.reads <= 64, "the stamp ring holds 64 launches"
    import torch
    from hyper_connection_residual_amd import binding, build, workloads as wl
    if not os.path.exists(build.PROBE_LIB):
        raise SystemExit("build the timing library first: python -m hyper_connection_residual_amd.build --probe")
    binding.LIB_PATH = build.PROBE_LIB
    lib = binding.library()
    import ctypes
    lib.hc_probe_stamps.argtypes = [ctypes.c_void_p]
    lib.hc_probe_stamps.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    sets = []
    for m in range(N_SETS):
        w_norm, W_down, W_up = wl.draw_weights(np.random.default_rng((1, m)))
        sets.append((torch.from_numpy(w_norm).to(dev), torch.from_numpy(W_down.view(np.int16)).to(dev),
                     torch.from_numpy(W_up.view(np.int16)).to(dev)))
    print("# Short-window read: per-phase clock stamps (timing build)\n")
    print("MI355X (gfx950). %d back-to-back reads per token count, pending write, 48 rotated weight sets; "
          "microseconds after the read's first workgroup started (100 MHz wall clock): median over reads of the "
          "median workgroup / the latest workgroup.\n" % args.reads)
    for T in [int(t) for t in args.T.split(",")]:
        rng = np.random.default_rng((1, 1000 + T, 0))
        R = torch.from_numpy(wl._normal_residual(rng, T, 4, 2560)).to(dev)
        P = torch.from_numpy(wl._normal_residual(rng, T, 4, 2560, 0.1)).to(dev)
        o = (torch.empty((T, 2560), device=dev), torch.empty((T, 2560), dtype=torch.int16, device=dev),
             torch.empty((T, 2560), dtype=torch.int16, device=dev))

        def read(k):
            w, wd, wu = sets[k % N_SETS]
            st = binding.hc_read(T, R, P, w, wd, wu, o[0], o[1], o[2], None)
            if st != 0:
                raise binding.HCError(st, "hc_read")

        for k in range(16):
            read(k)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for k in range(args.reads):
            read(k)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.reads
        ring = np.zeros(64 * 256 * 16, dtype=np.uint64)
        assert lib.hc_probe_stamps(ring.ctypes.data) == 0
        ring = ring.reshape(64, 256, 16).astype(np.int64)
        launches = [g for g in range(64) if ring[g, :, 0].min() > 0][-args.reads:]
        med, late = {p: [] for p, _ in POINTS}, {p: [] for p, _ in POINTS}
        for g in launches:
            t0 = ring[g, :, 0].min()
            for p, _ in POINTS:
                v = ring[g, :, p]
                v = v[v > 0]
                if len(v):
                    med[p].append(np.median(v - t0) / 100.0)
                    late[p].append(np.max(v - t0) / 100.0)
        print("## T = %d (%.2f us per read back to back, event-timed)\n" % (T, us))
        print("| point | median workgroup, us | latest workgroup, us |")
        print("|---|---|---|")
        for p, name in POINTS:
            if med[p]:
                print("| %d %s | %.2f | %.2f |" % (p, name, np.median(med[p]), np.median(late[p])))
        print()
        if binding.hc_timeouts() != 0:
            print("(expired waits during these reads)\n")


if __name__ == "__main__":
    main()
