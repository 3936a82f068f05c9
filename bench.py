"""Benchmark of the hyper-connection read on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (the configuration the headline metric is quoted on): verify windows
of T = 1..8 tokens with a pending write, 48 independent weight sets (631 MB,
more than the 256 MB Infinity Cache) rotated per read so every read streams its
13,148,160 weight bytes from HBM.  One step = one sweep T = 1..8 (8 reads, each
on the next weight set).  Inputs are resident in HBM before timing starts.
Before the K timed steps run at least W untimed steps, and as many more as it
takes to keep the GPU busy for 60 ms: the engine clock of an idle GPU ramps up
over its first tens of milliseconds of work, and the timed steps measure the
steady state of back-to-back reads (`warmup_run` says what ran).

Prints ONE JSON line.  `value` = weight bytes streamed per second over the
timed sweeps (GB/s), one hc_read call per read; the same sweeps replayed from
captured HIP graphs (one graph per step) are reported under `graph`.  Per-T
microseconds per read, the times of reads of 9..512 tokens, the read with
the pending write committed (hc_read_commit) against the read plus a separate
R += pending, and the prefill read times are reported beside it.  The
roofline object describes the short-window kernel, next to `stream_floor_us`:
one launch of that kernel's shape that only streams 13,148,160 bytes (48
rotated buffers, cold), the floor for a single launch moving the weights, and
`launch_floor_us`: the same launch moving 16 bytes, back to back (eager, and
replayed from a HIP graph), the cost of any launch of that shape.  The
CPU baseline is the plain oracle on the host, on all its cores (one read per
core) and on one.  The run prints a hash of the kernel sources it was built
from, so a profiler run's summary can be tied to the kernels it measured.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WEIGHT_BYTES = 2 * 320 * 10240 * 2 + 4 * 2560 * 4   # W_down + W_up (bf16) + w_norm (fp32)
TOKEN_BYTES_P = 4 * 2560 * 4 * 2 + 2560 * (4 + 2 + 2)  # R and pending read, mixed + images written
HBM_PEAK_GBPS = 8000.0
N_SETS = 48
TS = list(range(1, 9))
WINDOWS = [9, 12, 16, 17, 24, 32, 33, 48, 64, 128, 256, 512]  # reads above 8 tokens, timed beside the sweep
WARM_WIDE_MS = 60.0  # GPU time of untimed wide reads before each prefill timing (engine clock ramp)
WARM_STEP_MS = 60.0  # GPU time of untimed sweep steps (at least --warmup of them) before the timed steps


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU time for the baseline")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run 5 plain device copies of 256 MiB (a known byte count that checks the "
                         "HBM byte counters of a profiler run)")
    ap.add_argument("--light", action="store_true",
                    help="fewer reads per timing loop (for profiler runs that serialize every dispatch)")
    ap.add_argument("--no-launch-floor", action="store_true",
                    help="skip the 16-byte launches of the launch floor (profiler runs: they share the "
                         "streaming reference's kernel and grid, so a summary could not tell them apart)")
    ap.add_argument("--cpu-cores", type=int, default=0,
                    help="host cores for the all-core oracle leg (0: all, at most 16)")
    ap.add_argument("--traffic-md", default=os.path.join(ROOT, "profiles", "decode_sweep_and_wide_reads_counters.md"),
                    help="summary of the profiler's counter runs (rocprof_summary counters); its HBM "
                         "bytes are reported only if they were measured on the current kernel sources")
    return ap.parse_args()


def make_sets(torch):
    """48 weight sets and, per (T, set), the activations of the sweep (config 2)."""
    from hyper_connection_residual_amd import workloads as wl
    sets = []
    for m in range(N_SETS):
        rng = np.random.default_rng((1, m))
        w_norm, W_down, W_up = wl.draw_weights(rng)
        sets.append(dict(w_norm=torch.from_numpy(w_norm).cuda(),
                         W_down=torch.from_numpy(W_down.view(np.int16)).cuda(),
                         W_up=torch.from_numpy(W_up.view(np.int16)).cuda()))
    acts = {}
    for T in TS:
        for m in range(N_SETS):
            rng = np.random.default_rng((1, 1000 + T, m))
            R = wl._normal_residual(rng, T, wl.N_STREAMS, wl.WIDTH)
            P = wl._normal_residual(rng, T, wl.N_STREAMS, wl.WIDTH, 0.1)
            acts[(T, m)] = (torch.from_numpy(R).cuda(), torch.from_numpy(P).cuda())
    return sets, acts


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args):
    """The oracle (fp64, as it stands) on the host over a bounded sample of the
    sweep: reads cycling T = 1..8 and the weight sets.  All-core leg: one read
    per core at a time (each read single-threaded; the oracle releases the
    interpreter while it runs); then a one-core leg.  Weight bytes per second."""
    import concurrent.futures as cf
    from oracle import oracle as orc
    from hyper_connection_residual_amd import workloads as wl
    nproc = os.cpu_count() or 1
    cores = args.cpu_cores or min(16, nproc)
    inputs = [wl.config_inputs(2, T=TS[i % len(TS)], weight_set=i % N_SETS) for i in range(2 * cores)]

    def one(inp):
        orc.oracle_read(inp.R, inp.w_norm, inp.W_down, inp.W_up, inp.pending, threads=1)

    legs = {}
    for n in (cores, 1):
        budget = args.cpu_seconds / 2
        reads, t0 = 0, time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=n) as pool:
            while time.perf_counter() - t0 < budget:
                list(pool.map(one, [inputs[(reads + j) % len(inputs)] for j in range(n)]))
                reads += n
        wall = time.perf_counter() - t0
        legs[n] = (reads, wall)
    reads, wall = legs[cores]
    r1, w1 = legs[1]
    return {"value": round(reads * WEIGHT_BYTES / wall / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d oracle reads (fp64, one read per core at a time, %d cores of %d, %s) of the T=1..8 "
                      "verify-window sweep with pending, cycling T and weight sets, %.1f s wall"
                      % (reads, cores, nproc, _cpu_model(), wall),
            "one_core": {"value": round(r1 * WEIGHT_BYTES / w1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "sample": "%d reads, %.1f s" % (r1, w1)}}


def main():
    args = parse()
    # reads per timing loop: per-T sweep, windows, commit, prefill
    n_per_T, n_win, n_commit = (24, 24, 8) if args.light else (300, 96, 96)
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the read has no cross-GPU "
              "exchange; see the sharding paragraph of the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from hyper_connection_residual_amd import binding
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    binding.library()
    from hyper_connection_residual_amd import rocprof_summary
    src_hash = rocprof_summary.source_hash()
    print("# kernel source hash: %s" % src_hash, file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    t_gen = time.time()
    sets, acts = make_sets(torch)
    outs = {T: (torch.empty((T, 2560), dtype=torch.float32, device=dev),
                torch.empty((T, 2560), dtype=torch.int16, device=dev),
                torch.empty((T, 2560), dtype=torch.int16, device=dev)) for T in TS}
    print("# inputs ready in %.1f s" % (time.time() - t_gen), file=sys.stderr, flush=True)

    def read_on(T, m, s):
        ws = sets[m]
        R, P = acts[(T, m)]
        o = outs[T]
        st = binding.hc_read(T, R, P, ws["w_norm"], ws["W_down"], ws["W_up"], o[0], o[1], o[2], s.cuda_stream)
        if st != 0:
            raise binding.HCError(st, "hc_read")

    # read number i of a run uses weight set i mod 48: step k covers sets
    # 8 k .. 8 k + 7 (mod 48), so 6 consecutive steps touch every set once
    n_pos = N_SETS // len(TS)

    def eager_step(k):
        for i, T in enumerate(TS):
            read_on(T, (len(TS) * k + i) % N_SETS, stream)

    def time_region(s, body, n):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        with torch.cuda.stream(s):
            for k in range(n):
                body(k)
        b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def warm_steps(s, body):
        # at least --warmup untimed steps, continued until WARM_STEP_MS of GPU
        # time has passed: the engine clock of an idle GPU ramps up over the
        # first tens of milliseconds of work, and the timed steps measure the
        # steady state of back-to-back reads
        done, ms = 0, 0.0
        while done < args.warmup or ms < (5.0 if args.light else WARM_STEP_MS):
            n = max(args.warmup - done, 20)
            ms += time_region(s, lambda k: body(done + k), n)
            done += n
        return {"steps": done, "gpu_ms": round(ms, 1)}

    # ---- eager: one hc_read call per read, back to back on one stream
    warm_eager = warm_steps(stream, eager_step)
    t0 = time.perf_counter()
    ms_eager = time_region(stream, eager_step, args.steps)
    print("# eager: %d steps, %.3f ms/step (event), wall %.3f s"
          % (args.steps, ms_eager / args.steps, time.perf_counter() - t0), file=sys.stderr, flush=True)
    us_eager = {}
    for T in TS:
        for m in range(10):
            read_on(T, m, stream)
        ms = time_region(stream, lambda k, T=T: read_on(T, k % N_SETS, stream), n_per_T)
        us_eager[str(T)] = round(ms * 1e3 / n_per_T, 3)
    print("# eager us per read by T: %s" % us_eager, file=sys.stderr, flush=True)

    # ---- the floor: one launch of the short-window kernel's shape that only
    # streams WEIGHT_BYTES from memory (48 rotated buffers, 631 MB, cold)
    floor_bufs = [torch.empty(WEIGHT_BYTES // 4, dtype=torch.float32, device=dev).fill_(float(m))
                  for m in range(N_SETS)]
    sink = torch.empty(256, dtype=torch.int32, device=dev)

    def stream_once(k):
        st = binding.hc_stream_read(floor_bufs[k % N_SETS], WEIGHT_BYTES, sink, stream.cuda_stream)
        if st != 0:
            raise binding.HCError(st, "hc_stream_read")

    for k in range(N_SETS):
        stream_once(k)
    ms_floor = time_region(stream, stream_once, n_per_T)
    floor_us = round(ms_floor * 1e3 / n_per_T, 3)
    print("# stream floor: %.3f us per launch (%.0f GB/s)" % (floor_us, WEIGHT_BYTES / (floor_us * 1e-6) / 1e9),
          file=sys.stderr, flush=True)
    del floor_bufs

    # ---- reads of 9..512 tokens (up to 25: one short-window launch; beyond:
    # the wide path), eager, weights rotated over the 48 sets.  Every input
    # is made first, and the reads run after WARM_STEP_MS of GPU time of
    # window reads, so that no host-side pause between two token counts
    # lets the engine clock drop before a timing.
    from hyper_connection_residual_amd import workloads as wl
    window_inputs = {}
    for T in WINDOWS:
        rng = np.random.default_rng((1, 2000 + T))
        R = torch.from_numpy(wl._normal_residual(rng, T, wl.N_STREAMS, wl.WIDTH)).cuda()
        P = torch.from_numpy(wl._normal_residual(rng, T, wl.N_STREAMS, wl.WIDTH, 0.1)).cuda()
        o = (torch.empty((T, 2560), dtype=torch.float32, device=dev),
             torch.empty((T, 2560), dtype=torch.int16, device=dev),
             torch.empty((T, 2560), dtype=torch.int16, device=dev))
        window_inputs[T] = (R, P, o)

    def window_read(k, T):
        R, P, o = window_inputs[T]
        ws = sets[k % N_SETS]
        st = binding.hc_read(T, R, P, ws["w_norm"], ws["W_down"], ws["W_up"], o[0], o[1], o[2],
                             stream.cuda_stream)
        if st != 0:
            raise binding.HCError(st, "hc_read")

    warm_windows = warm_steps(stream, lambda k: window_read(k, WINDOWS[k % len(WINDOWS)]))
    us_windows = {}
    for T in WINDOWS:
        for k in range(8):
            window_read(k, T)
        ms = time_region(stream, lambda k, T=T: window_read(k, T), n_win)
        us_windows[str(T)] = round(ms * 1e3 / n_win, 3)
    print("# windows above 8 tokens, us per read: %s" % us_windows, file=sys.stderr, flush=True)

    # ---- the pending write committed by the read (hc_read_commit) against
    # the read followed by a separate R += pending, at T = 8 and T = 8192
    commit = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for T in (8, 8192):
        R = torch.randn((T, 4, 2560), generator=gen, device=dev)
        P = 0.1 * torch.randn((T, 4, 2560), generator=gen, device=dev)
        o = (torch.empty((T, 2560), dtype=torch.float32, device=dev),
             torch.empty((T, 2560), dtype=torch.int16, device=dev),
             torch.empty((T, 2560), dtype=torch.int16, device=dev))

        def call(fn, k, T=T, R=R, P=P, o=o):
            ws = sets[k % N_SETS]
            st = fn(T, R, P, ws["w_norm"], ws["W_down"], ws["W_up"], o[0], o[1], o[2], stream.cuda_stream)
            if st != 0:
                raise binding.HCError(st, "read")

        def read_then_add(k, R=R, P=P):
            call(binding.hc_read, k)
            R.add_(P)

        n = n_commit if T <= 8 else (2 if args.light else 10)
        for k in range(4):
            call(binding.hc_read_commit, k)
            read_then_add(k)
        ms_c = time_region(stream, lambda k: call(binding.hc_read_commit, k), n)
        ms_a = time_region(stream, read_then_add, n)
        commit[str(T)] = {"read_commit_us": round(ms_c * 1e3 / n, 3), "read_then_add_us": round(ms_a * 1e3 / n, 3)}
        del R, P, o
    print("# pending write committed: %s" % commit, file=sys.stderr, flush=True)

    ms_per_step = ms_eager / args.steps
    n_reads = args.steps * len(TS)
    weight_gbps = n_reads * WEIGHT_BYTES / (ms_eager * 1e-3) / 1e9
    us_per_read = us_eager

    # the short-window kernel's roofline over the sweep: algorithmic bytes per
    # launch (weights + each token's R, pending and outputs) / event-timed
    # average launch duration (back-to-back launches on one stream)
    alg_bytes_per_step = sum(WEIGHT_BYTES + T * TOKEN_BYTES_P for T in TS)
    achieved = alg_bytes_per_step / (ms_per_step * 1e-3) / 1e9
    timeouts = binding.hc_timeouts(stream)

    if args.calib_copy:
        src = torch.empty(256 << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    traffic = None
    measured = rocprof_summary.read_traffic(args.traffic_md)
    if measured and measured[1] == src_hash:
        traffic = measured[0]  # HBM bytes per launch, sweep average

    prefill = None
    prefill_all = None
    if not args.no_prefill:
        from hyper_connection_residual_amd import workloads as wl

        def time_wide(T, R, P, w_norm, Wd, Wu, reps, fn=None):
            fn = fn or binding.hc_read
            o = (torch.empty((T, 2560), dtype=torch.float32, device=dev),
                 torch.empty((T, 2560), dtype=torch.int16, device=dev),
                 torch.empty((T, 2560), dtype=torch.int16, device=dev))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            # Warm-up by time, not by count: over the first tens of ms of
            # sustained matrix work the reads speed up by ~15 % (the engine
            # clock ramps: the s_memtime / s_memrealtime ratio inside the
            # kernels goes from ~19.4 to ~22), so reads are timed once
            # WARM_WIDE_MS of them have run.
            warm = 0.0
            while warm < (5.0 if args.light else WARM_WIDE_MS):
                a.record(stream)
                for _ in range(3):
                    fn(T, R, P, w_norm, Wd, Wu, o[0], o[1], o[2], stream.cuda_stream)
                b.record(stream)
                torch.cuda.synchronize()
                warm += a.elapsed_time(b)
            a.record(stream)
            for _ in range(reps):
                fn(T, R, P, w_norm, Wd, Wu, o[0], o[1], o[2], stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            return {"T": T, "pending": P is not None, "ms_per_read": round(ms, 4),
                    "tokens_per_s": round(T / (ms * 1e-3), 1), "warmup_ms": round(warm, 1)}

        prefill_all = {}
        # configs 3 and 4: the seeded generator (outlier channels, no pending)
        for c in (3, 4):
            inp = wl.config_inputs(c)
            R = torch.from_numpy(inp.R).cuda()
            w_norm = torch.from_numpy(inp.w_norm).cuda()
            Wd = torch.from_numpy(inp.W_down.view(np.int16)).cuda()
            Wu = torch.from_numpy(inp.W_up.view(np.int16)).cuda()
            r = time_wide(inp.T, R, None, w_norm, Wd, Wu, 2 if args.light else (40 if inp.T <= 2048 else 20))
            prefill_all["T%d" % inp.T] = r
            print("# prefill T=%d: %.4f ms per read" % (inp.T, r["ms_per_read"]), file=sys.stderr, flush=True)
            if inp.T == 8192:  # the bf16-lo mode (hc_read_bf16_lo), its own error-bound contract
                r = time_wide(inp.T, R, None, w_norm, Wd, Wu, 2 if args.light else 20, fn=binding.hc_read_bf16_lo)
                prefill_all["T8192_bf16_lo"] = r
                print("# prefill T=8192, bf16 lo: %.4f ms per read" % r["ms_per_read"], file=sys.stderr,
                      flush=True)
            del R
        # config 5 (T = 32768 with pending): the same distributions drawn on the
        # device (R ~ Student-t(4) / sqrt(2), pending ~ N(0, 0.05)); the read's
        # time does not depend on the values, and the seeded CPU draw of 2.7 GB
        # takes ~40 s
        g = torch.Generator(device=dev)
        g.manual_seed(4)
        T5 = 32768
        z = torch.randn((T5, 4, 2560), device=dev, generator=g)
        chi = torch.distributions.Chi2(torch.tensor(4.0, device=dev)).sample((T5, 4, 2560))
        R5 = (z / torch.sqrt(chi / 4.0) / np.sqrt(2.0)).contiguous()
        del z, chi
        P5 = (0.05 * torch.randn((T5, 4, 2560), device=dev, generator=g)).contiguous()
        r = time_wide(T5, R5, P5, w_norm, Wd, Wu, 1 if args.light else 5)
        prefill_all["T32768_pending"] = r
        print("# prefill T=32768 with pending: %.4f ms per read" % r["ms_per_read"], file=sys.stderr, flush=True)
        del R5, P5, Wd, Wu
        prefill = prefill_all["T8192"]

    # ---- HIP graphs (last: the first calls on the capture stream make the
    # library order short-window reads across streams for a while, which the
    # eager legs above must not pay): each step position of the rotation captured once (8
    # reads per graph) and replayed; the same reads, inputs and outputs as the
    # eager run.  Scratch of the capture stream is created eagerly first.
    gstream = torch.cuda.Stream()
    with torch.cuda.stream(gstream):
        for T in TS:
            read_on(T, 0, gstream)
    torch.cuda.synchronize()
    step_graphs = []
    for j in range(n_pos):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            for i, T in enumerate(TS):
                read_on(T, (len(TS) * j + i) % N_SETS, gstream)
        step_graphs.append(g)
    warm_graph = warm_steps(gstream, lambda k: step_graphs[k % n_pos].replay())
    t0 = time.perf_counter()
    ms_graph = time_region(gstream, lambda k: step_graphs[k % n_pos].replay(), args.steps)
    print("# graph: %d steps, %.3f ms/step (event), wall %.3f s"
          % (args.steps, ms_graph / args.steps, time.perf_counter() - t0), file=sys.stderr, flush=True)
    us_graph = {}
    for T in TS:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            for m in range(N_SETS):
                read_on(T, m, gstream)
        with torch.cuda.stream(gstream):
            g.replay()
        ms = time_region(gstream, lambda k, g=g: g.replay(), 6)
        us_graph[str(T)] = round(ms * 1e3 / (6 * N_SETS), 3)
        del g
    print("# graph us per read by T: %s" % us_graph, file=sys.stderr, flush=True)
    del step_graphs

    # ---- the launch floor: one launch of the same shape that moves 16 bytes,
    # back to back, eager (bounded by the host's launch rate) and replayed from
    # a graph of 100 launches (the device's own cost per launch)
    launch_floor = None
    if not args.no_launch_floor:
        tiny = torch.zeros(4, dtype=torch.float32, device=dev)

        def tiny_once(s):
            st = binding.hc_stream_read(tiny, 16, sink, s.cuda_stream)
            if st != 0:
                raise binding.HCError(st, "hc_stream_read")

        for _ in range(100):
            tiny_once(stream)
        n_tiny, n_tiny_g = (200, 2) if args.light else (2000, 20)
        ms_tiny = time_region(stream, lambda k: tiny_once(stream), n_tiny)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            for _ in range(100):
                tiny_once(gstream)
        with torch.cuda.stream(gstream):
            g.replay()
        ms_tiny_g = time_region(gstream, lambda k: g.replay(), n_tiny_g)
        del g
        launch_floor = {"eager": round(ms_tiny * 1e3 / n_tiny, 3),
                        "graph": round(ms_tiny_g * 1e3 / (100 * n_tiny_g), 3)}
        print("# launch floor (16 bytes per launch): %s us" % launch_floor, file=sys.stderr, flush=True)
    timeouts += binding.hc_timeouts(stream) + binding.hc_timeouts(gstream)
    if timeouts:
        print("# WARNING: %d bounded waits expired" % timeouts, file=sys.stderr)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args)
        print("# cpu baseline: %s" % cpu, file=sys.stderr, flush=True)

    line = {
        "metric": "hc read µs at T=1..8 (weight GB/s vs HBM peak); fused read ms at T=8192",
        "value": round(weight_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"eager": warm_eager, "windows": warm_windows, "graph": warm_graph},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "verify-window sweep T=1..8 with pending write, 48 rotated weight "
                               "sets (631 MB), one step = 8 reads",
                   "T": TS, "weight_sets": N_SETS, "reads_per_step": len(TS),
                   "streams": 4, "width": 2560, "rank": 320},
        "us_per_read": us_per_read,
        "graph": {"value": round(n_reads * WEIGHT_BYTES / (ms_graph * 1e-3) / 1e9, 2),
                  "ms_per_step": round(ms_graph / args.steps, 5), "us_per_read": us_graph},
        "windows_us_per_read": us_windows,
        "commit": commit,
        "prefill_T8192": prefill,
        "prefill": prefill_all,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "stream_floor_us": floor_us,
        "launch_floor_us": launch_floor,
        "timeouts": timeouts,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
