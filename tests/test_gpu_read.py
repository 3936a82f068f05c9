"""Parity of the HIP read (through the C ABI) with the CPU oracle on MI355X.

Every case prints what it runs before its GPU step.  Bars: the fp32 output
within max|diff| / max|oracle| <= 2e-6, and the bf16 / fp16 images within
1 ulp of the oracle's images on >= 99.9 % of the values (tests/hc_testlib.py).
"""
import dataclasses
import os

import numpy as np
import pytest

from hyper_connection_residual_amd import workloads as wl
from oracle import oracle as orc
from tests.hc_testlib import assert_parity, hip_read, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"
    from hyper_connection_residual_amd import binding
    binding.library()
    yield


@pytest.fixture(autouse=True)
def no_expired_waits():
    """Every test leaves the default stream's bounded-wait counter at zero."""
    from hyper_connection_residual_amd import binding
    binding.hc_timeouts()  # (reading clears it)
    yield
    n = binding.hc_timeouts()
    assert n == 0, "%d bounded waits expired (or workgroups ran off their XCD) during this test" % n


def _case(label):
    print("\n[case] " + label, flush=True)


# oracle threads: the host cores one GPU's share offers (at most 16)
THREADS = max(1, min(16, os.cpu_count() or 1))


def _oracle(inp, tokens=None, threads=THREADS):
    R = inp.R if tokens is None else inp.R[tokens]
    P = inp.pending if (tokens is None or inp.pending is None) else inp.pending[tokens]
    return orc.oracle_read(R, inp.w_norm, inp.W_down, inp.W_up, P, eps=inp.eps, threads=threads)


def test_config1_single_token():
    _case("config 1: T=1, no pending, seed 0")
    inp = wl.config_inputs(1)
    gpu = hip_read(to_device(inp))
    assert_parity(gpu, _oracle(inp), label="config1")


@pytest.mark.parametrize("weight_set", [0, 7, 47])
def test_config2_verify_windows_with_pending(weight_set):
    for T in range(1, 9):
        _case("config 2: T=%d, pending, weight set %d" % (T, weight_set))
        inp = wl.config_inputs(2, T=T, weight_set=weight_set)
        gpu = hip_read(to_device(inp))
        assert_parity(gpu, _oracle(inp), label="config2 T=%d set=%d" % (T, weight_set))


def test_windows_of_9_to_16_every_count():
    """Every token count of the single-launch range above 8 (three MFMA
    chains, 16 token slots), with pending.  Full oracle."""
    for T in range(9, 17):
        _case("window of %d tokens, pending, weight set 21" % T)
        inp = wl.config_inputs(2, T=T, weight_set=21)
        assert_parity(hip_read(to_device(inp)), _oracle(inp), label="T=%d" % T)


def test_windows_of_17_to_32_every_count():
    """Every token count from 17 to 32, with pending: 17..25 on the six-chain
    short-window kernel (32 token slots, LDS regions shared between phases),
    26..32 on the wide path (the faster one there).  Full oracle."""
    for T in range(17, 33):
        _case("window of %d tokens, pending, weight set 22" % T)
        inp = wl.config_inputs(2, T=T, weight_set=22)
        assert_parity(hip_read(to_device(inp)), _oracle(inp), label="T=%d" % T)


def test_verify_windows_without_pending():
    for T in range(1, 9):
        _case("config 2 inputs without pending: T=%d" % T)
        inp = wl.config_inputs(2, T=T, weight_set=3)
        inp.pending = None
        gpu = hip_read(to_device(inp))
        assert_parity(gpu, _oracle(inp), label="no pending T=%d" % T)


@pytest.mark.parametrize("T", [9, 13, 17, 64])
def test_ragged_token_counts(T):
    _case("config 2 distributions, T=%d" % T)
    inp = wl.config_inputs(2, T=T, weight_set=1)
    gpu = hip_read(to_device(inp))
    assert_parity(gpu, _oracle(inp), label="T=%d" % T)


@pytest.mark.parametrize("T, pending", [(9, True), (12, False), (16, True), (17, True), (24, False), (25, False),
                                        (26, False), (32, True), (33, True)])
def test_windows_above_eight(T, pending):
    """9..16 tokens run as one short-window launch with three MFMA chains and
    16 token slots per partial row, 17..25 with six chains and 32 slots; 26
    is the first count hc_read sends to the wide path.  Full oracle."""
    _case("window of %d tokens, pending=%s" % (T, pending))
    inp = wl.config_inputs(2, T=T, weight_set=5)
    if not pending:
        inp.pending = None
    gpu = hip_read(to_device(inp))
    assert_parity(gpu, _oracle(inp), label="T=%d pending=%s" % (T, pending))


@pytest.mark.parametrize("T, half", [(24, 12), (20, 10)])
def test_window_equals_its_halves(T, half):
    """Above 8 tokens a token's arithmetic does not depend on the window: the
    six-chain kernel (17..25 tokens from hc_read) gives every token the bits
    that the three-chain kernel gives it in a window of half the size (26..32
    tokens, which only hc_read_noalloc runs on this kernel: its own test)."""
    _case("T=%d against two T=%d reads of its halves" % (T, half))
    inp = wl.config_inputs(2, T=T, weight_set=9)
    whole = hip_read(to_device(inp))
    for lo in (0, half):
        part_in = dataclasses.replace(inp, R=inp.R[lo:lo + half].copy(), pending=inp.pending[lo:lo + half].copy())
        part = hip_read(to_device(part_in))
        for a, b in zip(part, whole):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  (b.view(np.uint32) if b.dtype == np.float32 else b)[lo:lo + half])


@pytest.mark.parametrize("T, pending", [(1, True), (5, True), (8, False), (16, True), (24, True), (300, True),
                                        (8193, True)])
def test_commit_writes_the_pending_update(T, pending):
    """hc_read_commit: the outputs are hc_read's, bit for bit, and R then holds
    the oracle's committed residual fl32(R + pending), bit for bit (untouched
    without a pending write).  Covers the short-window kernel at 1, 2, 3 and 6
    MFMA chains, and the wide path over two chunks (8192 + 1 tokens)."""
    _case("commit: T=%d, pending=%s" % (T, pending))
    inp = wl.config_inputs(2, T=T, weight_set=2) if T <= 24 else wl.config_inputs(5, T=T, seed=T)
    if not pending:
        inp.pending = None
    dev = to_device(inp)
    plain = hip_read(dev)
    committed = hip_read(dev, commit=True)
    for a, b in zip(committed, plain):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
    want = orc.oracle_commit(inp.R, inp.pending)
    got = dev["R"].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_short_window_check_passes():
    """The start-up check keeps the short-window kernel on an MI355X."""
    _case("start-up check of the short-window kernel")
    from hyper_connection_residual_amd import binding
    assert binding.hc_short_window_on()


_FALLBACK_CHILD = """
import sys
sys.path.insert(0, '.')
from hyper_connection_residual_amd import binding, workloads as wl
from oracle import oracle as orc
from tests.hc_testlib import assert_parity, hip_read, to_device
assert not binding.hc_short_window_on(), 'the forced check should fail'
for T in (1, 4, 8, 12, 16, 20):
    print('[child] T=%d on the wide path' % T, flush=True)
    inp = wl.config_inputs(2, T=T, weight_set=4)
    gpu = hip_read(to_device(inp))
    ref = orc.oracle_read(inp.R, inp.w_norm, inp.W_down, inp.W_up, inp.pending, threads=8)
    assert_parity(gpu, ref, label='fallback T=%d' % T)
print('[child] ok', flush=True)
"""


def test_forced_check_failure_falls_back_to_the_wide_path():
    """With the bounded waits' limit forced to 0 ticks for the start-up check
    (every wait of the check's read gives up at its first miss, and the
    kernel still ends normally), the check fails, the library logs it, and
    every read then runs the wide path, still at parity.  Run
    in a child process, since the check runs once per process."""
    import os
    import subprocess
    import sys
    _case("forced start-up check failure (child process, HC_SELFCHECK_WAIT_TICKS=0)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, HC_SELFCHECK_WAIT_TICKS="0", HC_LOG="1")
    r = subprocess.run([sys.executable, "-c", _FALLBACK_CHILD], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    assert "[child] ok" in r.stdout
    assert "the short-window read is OFF" in r.stderr


def _bf16_grid(v):
    """(RNE of each value to bf16, the distance to the nearest midpoint between
    two adjacent bf16 values, the bf16 spacing there), from the format's
    definition (8 significant bits, minimum normal exponent -126)."""
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.exp2(np.maximum(e, -126.0) - 7.0)
    f = a / q
    rne = np.sign(v) * np.rint(f) * q  # np.rint: half to even (f's integer part is the significand)
    return rne, np.abs(f - (np.floor(f) + 0.5)) * q, q


def _flip_effect(inp, toks, near, q):
    """Per token, the largest change of any mixed value if every lo value
    flagged `near` were rounded to its other bf16 neighbour (q apart):
    sum over those j of q_j * sum_s |R'[t,s,c]| * |W_up[s*C + c, j]|."""
    n, C = inp.w_norm.shape
    R = inp.R[toks].astype(np.float32)
    if inp.pending is not None:
        R = R + inp.pending[toks]
    Rp = np.abs(R.astype(np.float64))                                        # [t, n, C]
    Wu = np.abs((inp.W_up.astype(np.uint32) << 16).view(np.float32).astype(np.float64))  # [n C, r], exact
    out = np.zeros(len(toks))
    for i in range(len(toks)):
        js = np.nonzero(near[i])[0]
        if len(js):
            A = (Wu[:, js] @ q[i, js]).reshape(n, C)                            # [n, C]
            out[i] = np.max(np.sum(Rp[i] * A, axis=0))
    return out


# The GPU's lo is within this fraction of the token's largest |lo| of the
# exact lo (asserted by test_lo_is_at_fp32_level; measured 1.8e-7 median and
# 3.3e-7 worst per token with outlier channels).
LO_TOL = 1e-6


def _gpu_lo(inp):
    """The GPU's fp32 lo, read out through the C ABI: W_up one-hot puts lo[t, j]
    alone into output column 8 j of stream 0, so mixed[t, 8 j] = fl(lo[t, j] *
    R'[t, 0, 8 j]) (the three bf16 pieces of lo times 1.0 add back exactly; the
    other streams contribute 0).  Dividing by R' recovers lo to 2^-24."""
    n, C = inp.w_norm.shape
    r = inp.W_down.shape[0]
    Wu = np.zeros((n * C, r), np.float32)
    Wu[8 * np.arange(r), np.arange(r)] = 1.0
    sel = dataclasses.replace(inp, W_up=wl.bf16_bits_from_f32(Wu))
    m = hip_read(to_device(sel))[0].astype(np.float64)
    Rp = inp.R.astype(np.float32) if inp.pending is None else (inp.R + inp.pending).astype(np.float32)
    return m[:, 8 * np.arange(r)] / Rp[:, 0, 8 * np.arange(r)].astype(np.float64)


@pytest.mark.parametrize("T, pending", [(8, True), (100, False), (300, False), (2000, True)])
def test_lo_is_at_fp32_level(T, pending):
    """lo, stage-wise: the GPU's lo (read out through a one-hot W_up) against
    the oracle's exact lo, every token: within LO_TOL of each token's largest
    |lo| (the short-window kernel at 8 tokens; the wide path with 80, 80 and 16
    K splits)."""
    _case("lo at fp32 level: T=%d, pending=%s" % (T, pending))
    inp = wl.config_inputs(5 if pending else 3, T=T, seed=T + 7)
    if T <= 32:
        inp = wl.config_inputs(2, T=T, weight_set=14)
    lo_gpu = _gpu_lo(inp)
    _, lo = orc.oracle_read(inp.R, inp.w_norm, inp.W_down, inp.W_up, inp.pending, eps=inp.eps,
                            threads=THREADS, want_lo=True)
    rel = np.max(np.abs(lo_gpu - lo), axis=1) / np.max(np.abs(lo), axis=1)
    print("lo error / max|lo| per token: median %.2e, max %.2e (bound %.1e)"
          % (np.median(rel), np.max(rel), LO_TOL), flush=True)
    assert np.max(rel) <= LO_TOL


@pytest.mark.parametrize("T, pending", [(40, True), (60, False), (100, False), (120, True), (150, True),
                                        (180, False), (230, False), (240, True), (300, False), (2048, False),
                                        (4097, True)])
def test_bf16_lo_mode_against_the_oracle_fed_bf16_lo(T, pending):
    """hc_read_bf16_lo, stage-wise: the oracle's mode that rounds its exact lo
    to bf16 (nearest even) before the up projection is the reference, held to
    hc_read's 2e-6.  The GPU rounds its own fp32 lo, which differs from the
    exact lo by fp32 rounding (test_lo_is_at_fp32_level), so a lo value next to
    a bf16 rounding midpoint may legitimately round the other way.  The test
    reads the GPU's fp32 lo out through the C ABI (one-hot W_up) and flags the
    values whose bf16 rounding differs from the exact lo's, or that lie within
    the read-out's resolution of a midpoint; a token is compared unless
    rounding its flagged values the other way could move one of its mixed
    values by more than 1e-6 of max|mixed| (half the tolerance).  The expected
    values are the oracle's alone; the test prints how many tokens it leaves
    out.  T = 40, 60, 100, 120: 16-column up+mix tiles (one and two token
    tiles, with and without pending); T = 150, 180, 230, 240: 32-column tiles
    (three and four token tiles, with and without pending); T = 300 and 2048:
    the persistent up+mix; T = 4097 (two chunks, with pending): the
    per-tile up+mix, a sample of tokens.  The mode
    must also differ from the exact read (the fast path ran)."""
    _case("bf16-lo mode against the oracle fed bf16(lo): T=%d, pending=%s" % (T, pending))
    inp = wl.config_inputs(5 if pending else 3, T=T, seed=T + 1)
    gpu = hip_read(to_device(inp), bf16_lo=True)
    toks = np.arange(T) if T <= 300 else np.array(sorted(set(_sample_tokens(T, k=64, seed=T).tolist()) |
                                                        {0, T - 1} | ({4095, 4096} if T > 4096 else set())))
    R = inp.R[toks]
    P = None if inp.pending is None else inp.pending[toks]
    ref, lo = orc.oracle_read(R, inp.w_norm, inp.W_down, inp.W_up, P, eps=inp.eps, threads=THREADS,
                              mode="f64_bf16_lo", want_lo=True)
    exact = orc.oracle_read(R, inp.w_norm, inp.W_down, inp.W_up, P, eps=inp.eps, threads=THREADS)
    lo_gpu = _gpu_lo(inp)[toks]
    rne, _, q = _bf16_grid(lo)
    rne_g, dist_g, _ = _bf16_grid(lo_gpu)
    flagged = (rne != rne_g) | (dist_g <= 2.0 ** -22 * np.abs(lo_gpu))
    effect = _flip_effect(inp, toks, flagged, q)
    keep = effect <= 1e-6 * np.max(np.abs(ref))
    print("bf16-lo: %d of %d tokens compared (%d lo values round differently in fp32 or sit at a midpoint; "
          "%d tokens left out, where they could move mixed by more than 1e-6)"
          % (int(keep.sum()), len(toks), int(flagged.sum()), int((~keep).sum())), flush=True)
    assert keep.sum() >= 0.75 * len(toks)
    assert_parity(tuple(a[toks][keep] for a in gpu), ref[keep], label="bf16-lo T=%d" % T)
    e_exact = np.max(np.abs(gpu[0][toks].astype(np.float64) - exact)) / np.max(np.abs(exact))
    assert e_exact > 1e-5, "bf16(lo) should move the result (%.2e from the exact read)" % e_exact


_EXPIRY_CHILD = """
import sys
import numpy as np
sys.path.insert(0, '.')
import torch
from hyper_connection_residual_amd import binding, workloads as wl
from oracle import oracle as orc
from tests.hc_testlib import hip_read, to_device, REL_TOL
assert binding.hc_short_window_on(), 'the start-up check keeps its own limit and passes'
expired_total = 0
for T in (1, 5, 8, 16, 24, 32):
    for commit in (False, True):
        print('[child] T=%d commit=%s with every wait limited to 0 ticks' % (T, commit), flush=True)
        inp = wl.config_inputs(2, T=T, weight_set=12)
        dev = to_device(inp)
        binding.hc_timeouts()
        m, b, h = hip_read(dev, commit=commit)
        n = binding.hc_timeouts()
        expired_total += n
        bad = np.isnan(m)
        # a workgroup owns whole columns: NaN for every token of a column or none
        assert np.array_equal(bad, np.broadcast_to(bad.any(axis=0), bad.shape)), 'NaN not by whole columns'
        assert (n > 0) == bool(bad.any()), 'expired waits %d but NaN outputs %d' % (n, int(bad.sum()))
        # the images are NaN exactly where mixed is
        assert np.array_equal(bad, ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0))
        assert np.array_equal(bad, ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0))
        ref = orc.oracle_read(inp.R, inp.w_norm, inp.W_down, inp.W_up, inp.pending, threads=8)
        good = ~bad
        if good.any():
            err = np.max(np.abs(m[good].astype(np.float64) - ref[good])) / np.max(np.abs(ref))
            assert err <= REL_TOL, 'valid outputs off by %.2e' % err
        if commit:
            # R committed exactly in the columns whose outputs are valid
            Rn = dev['R'].cpu().numpy()
            want = orc.oracle_commit(inp.R, inp.pending)
            cols = bad[0]
            assert np.array_equal(Rn[:, :, ~cols].view(np.uint32), want[:, :, ~cols].view(np.uint32))
            assert np.array_equal(Rn[:, :, cols].view(np.uint32), inp.R[:, :, cols].view(np.uint32))
        print('[child] %d expired waits, %d of %d columns NaN' % (n, int(bad[0].sum()), bad.shape[1]), flush=True)
assert expired_total > 0, 'no wait expired: the forced case did not happen'
print('[child] ok', flush=True)
"""


def test_expired_waits_give_nan_outputs_never_silent_ones():
    """With every bounded wait of ordinary reads limited to 0 ticks
    (HC_WAIT_TICKS=0: a wait gives up at its first miss, and every kernel
    still ends normally), waits expire; the outputs of every workgroup
    concerned are NaN (whole columns, in mixed and in both images), every
    other output is at parity with the oracle, hc_read_commit leaves the NaN
    columns of R uncommitted and commits the others, and the counter is
    non-zero exactly when NaN appears.  In a child process (the limit is read
    once per process)."""
    import subprocess
    import sys
    _case("expired waits forced (child process, HC_WAIT_TICKS=0)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, HC_WAIT_TICKS="0", HC_LOG="1")
    r = subprocess.run([sys.executable, "-c", _EXPIRY_CHILD], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout[-3000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    assert "[child] ok" in r.stdout


def test_release_stream_then_read_again():
    """hc_release_stream frees a stream's workspace after synchronizing it;
    the next read on the stream allocates again and gives the same bits.  A
    stream without a workspace is released without error."""
    import torch
    from hyper_connection_residual_amd import binding
    _case("hc_release_stream between reads, T=5 and T=40")
    st = torch.cuda.Stream()
    binding.hc_release_stream(st)  # (no workspace yet)
    for T in (5, 40):
        dev = to_device(wl.config_inputs(2, T=T, weight_set=13))
        with torch.cuda.stream(st):
            a = hip_read(dev, stream=st)
        binding.hc_release_stream(st)
        with torch.cuda.stream(st):
            b = hip_read(dev, stream=st)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y)
    assert binding.hc_timeouts(st) == 0
    binding.hc_release_stream(st)


def test_bf16_lo_mode_short_windows_are_exact():
    """Up to 25 tokens hc_read_bf16_lo is the short-window read: hc_read's bits."""
    _case("bf16-lo mode at T=8 and T=24 against hc_read")
    for T in (8, 24):
        dev = to_device(wl.config_inputs(2, T=T, weight_set=6))
        for a, b in zip(hip_read(dev, bf16_lo=True), hip_read(dev)):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b)


def test_outlier_channels_full_oracle():
    _case("config 3 distributions at T=300 (several tiles, ragged tail), full oracle")
    inp = wl.config_inputs(3, T=300)
    gpu = hip_read(to_device(inp))
    assert_parity(gpu, _oracle(inp), label="config3 T=300")


def _sample_tokens(T, k=40, seed=0):
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(T, size=min(k, T), replace=False).tolist())
    picks |= {0, 1, T - 2, T - 1}
    return np.array(sorted(picks))


@pytest.mark.parametrize("config", [3, 4])
def test_full_size_configs_every_token(config):
    """Configurations 3 and 4 at full size (2048 and 8192 tokens, outlier
    channels), every token against the oracle (threaded over the host cores)."""
    T = {3: 2048, 4: 8192}[config]
    _case("config %d: T=%d full size, every token against the oracle (%d threads)" % (config, T, THREADS))
    inp = wl.config_inputs(config)
    gpu = hip_read(to_device(inp))
    assert_parity(gpu, _oracle(inp), label="config%d every token" % config)


def test_full_size_config5_every_tile():
    """Configuration 5 at full size (32768 tokens with pending, eight 4096-token
    chunks): one seeded token of every 64-token tile of every chunk, plus the
    first and last token of each chunk."""
    T = 32768
    _case("config 5: T=%d full size, one token per 64-token tile (%d threads)" % (T, THREADS))
    inp = wl.config_inputs(5)
    gpu = hip_read(to_device(inp))
    rng = np.random.default_rng(5)
    toks = set((np.arange(0, T, 64) + rng.integers(0, 64, size=T // 64)).tolist())
    toks |= {c + d for c in range(0, T, 4096) for d in (0, 4095)}
    toks = np.array(sorted(toks))
    assert_parity(gpu, _oracle(inp, toks), tokens=toks, label="config5 every tile")


@pytest.mark.parametrize("T, pending", [(128, False), (129, True), (256, True), (257, False), (384, False),
                                        (385, True), (700, False), (1024, True), (1025, False), (2000, True),
                                        (3968, False), (3969, True), (4097, False), (8064, False), (8065, False),
                                        (8192, True), (8193, False)])
def test_wide_path_boundaries(T, pending):
    """Token counts at the wide path's internal boundaries: one token past a
    128-token down tile; the up+mix tile changes from 16 to 32 columns after
    128 tokens and to 64 after 256 (4 token tiles); the down projection's K-split count changes
    from 80 (128-column splits) to 32 after 384 tokens, to 16 (stream
    quarters) after 1024, to 8 (stream halves) after 3968 and, without
    pending, to 4 (whole streams) after 8064; one token past an 8192-token
    chunk (the second chunk holds a single token).  700 and 2000 run the 32-
    and 16-split down projections with and without pending, 8192 the 8-split
    one with pending, so that every instance a valid call reaches runs.
    Oracle on the tokens around each boundary plus a random sample."""
    _case("wide path boundary: T=%d, pending=%s" % (T, pending))
    inp = wl.config_inputs(5 if pending else 3, T=T, seed=T)
    gpu = hip_read(to_device(inp))
    edges = {t for b in (64, 127, 128, 129, 256, 384, 1024, 3968, 4095, 4096, 8064, 8191, 8192)
             for t in (b - 1, b) if 0 <= t < T}
    toks = np.array(sorted(set(_sample_tokens(T, k=24, seed=T).tolist()) | edges))
    assert_parity(gpu, _oracle(inp, toks), tokens=toks, label="T=%d pending=%s" % (T, pending))


@pytest.mark.parametrize("T, pending", [(33, False), (64, False), (96, True), (97, False), (160, True),
                                        (192, False), (193, True), (250, False)])
def test_short_chunk_down_tiles(T, pending):
    """Chunks of at most 192 tokens run the down projection on 80 x NT
    workgroups of 32-token tiles (up to 96 tokens) or 64-token tiles (97..192),
    every load issued at entry; 193 is the first count on the 128-token down
    kernel.  Both tile sizes with and without pending, ragged last tiles.  The
    up+mix of these chunks: 16-column tiles for one and two token tiles,
    32-column tiles for three (160, 192) and four (193, 250).  Full oracle."""
    _case("short-chunk down tiles: T=%d, pending=%s" % (T, pending))
    inp = wl.config_inputs(2, T=T, weight_set=9)
    if not pending:
        inp.pending = None
    gpu = hip_read(to_device(inp))
    assert_parity(gpu, _oracle(inp), label="T=%d pending=%s" % (T, pending))


# ---------------------------------------------------------------------------
# Invariants that hold bitwise on the GPU.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def base():
    inp = wl.config_inputs(2, T=6, weight_set=11)
    return inp, hip_read(to_device(inp))


def test_deterministic_run_to_run(base):
    _case("run-to-run determinism, T=6")
    inp, ref = base
    for _ in range(3):
        again = hip_read(to_device(inp))
        for a, b in zip(again, ref):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b)


def test_pending_equals_preadded(base):
    _case("pending vs pre-added residual, T=6")
    inp, ref = base
    pre = wl.ReadInputs((inp.R + inp.pending).astype(np.float32), None, inp.w_norm,
                        inp.W_down, inp.W_up)
    got = hip_read(to_device(pre))
    assert np.array_equal(got[0], ref[0])
    zero = wl.ReadInputs(inp.R, np.zeros_like(inp.R), inp.w_norm, inp.W_down, inp.W_up)
    none = wl.ReadInputs(inp.R, None, inp.w_norm, inp.W_down, inp.W_up)
    assert np.array_equal(hip_read(to_device(zero))[0], hip_read(to_device(none))[0])


def _scaled_bf16(bits, factor):
    return wl.bf16_bits_from_f32(orc.bf16_bits_to_f64(bits).astype(np.float32) * np.float32(factor))


def test_power_of_two_scaling_and_sign_flip(base):
    # Power-of-two scaling of a weight leaves every alignment inside the matrix
    # cores unchanged, so the output scales exactly.  Negation is exact in the
    # definition but the matrix cores' fp32 accumulation does not round
    # symmetrically under a sign flip, so a flipped sign is checked to the
    # rounding level only.
    _case("2*W_up, 4*W_down (exact); -W_up, -2*w_norm (rounding level), T=6")
    inp, ref = base
    m = ref[0]
    for label, W_up, W_down, w, factor, exact in (
            ("2 W_up", _scaled_bf16(inp.W_up, 2), inp.W_down, inp.w_norm, 2.0, True),
            ("4 W_down", inp.W_up, _scaled_bf16(inp.W_down, 4), inp.w_norm, 4.0, True),
            ("0.5 w_norm", inp.W_up, inp.W_down, (0.5 * inp.w_norm).astype(np.float32), 0.5, True),
            ("-W_up", _scaled_bf16(inp.W_up, -1), inp.W_down, inp.w_norm, -1.0, False),
            ("-2 w_norm", inp.W_up, inp.W_down, (-2 * inp.w_norm).astype(np.float32), -2.0, False)):
        got = hip_read(to_device(wl.ReadInputs(inp.R, inp.pending, w, W_down, W_up)))[0]
        want = (factor * m).astype(np.float32)
        if exact:
            assert np.array_equal(got, want), label
        else:
            err = np.max(np.abs(got - want)) / np.max(np.abs(want))
            assert err <= 1e-6, "%s: %.3e" % (label, err)


def test_token_permutation(base):
    _case("token permutation, T=6")
    inp, ref = base
    perm = [3, 0, 5, 1, 4, 2]
    got = hip_read(to_device(wl.ReadInputs(inp.R[perm], inp.pending[perm], inp.w_norm,
                                           inp.W_down, inp.W_up)))
    assert np.array_equal(got[0], ref[0][perm])


def test_zero_weights_give_zero(base):
    _case("zero W_down / zero W_up, T=6")
    inp, _ = base
    for Wd, Wu in ((np.zeros_like(inp.W_down), inp.W_up), (inp.W_down, np.zeros_like(inp.W_up))):
        m, b, h = hip_read(to_device(wl.ReadInputs(inp.R, inp.pending, inp.w_norm, Wd, Wu)))
        assert not np.any(m) and not np.any(b & 0x7FFF) and not np.any(h & 0x7FFF)


def test_selection_matrices_closed_form():
    _case("one-hot W_down / W_up at full shape, closed form, T=3")
    rng = np.random.default_rng(21)
    n, C, r = wl.N_STREAMS, wl.WIDTH, wl.RANK
    T = 3
    a = rng.uniform(0.5, 3.0, size=(T, n)).astype(np.float32)
    signs = np.where(rng.random((T, n, C)) < 0.5, -1.0, 1.0)
    R = (signs * a[:, :, None]).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal((n, C))).astype(np.float32)
    ks = rng.choice(n * C, size=r, replace=False)
    Wd = np.zeros((r, n * C), np.float32)
    Wu = np.zeros((n * C, r), np.float32)
    for j, k in enumerate(ks):
        Wd[j, k] = 1.0
        Wu[k, j] = 1.0
    inp = wl.ReadInputs(R, None, w, wl.bf16_bits_from_f32(Wd), wl.bf16_bits_from_f32(Wu))
    got = hip_read(to_device(inp))[0]
    want = np.zeros((T, C))
    for t in range(T):
        for k in ks:
            s, c = divmod(int(k), C)
            aa = float(a[t, s])
            want[t, c] += float(w[s, c]) * aa * aa / np.sqrt(aa * aa + 1e-6)
    err = np.max(np.abs(got - want)) / np.max(np.abs(want))
    print("selection closed form rel err %.3e" % err, flush=True)
    assert err <= 2e-6


def test_two_streams_have_separate_scratch():
    import torch
    _case("two streams interleaved, T=4 and T=7")
    a = wl.config_inputs(2, T=4, weight_set=20)
    b = wl.config_inputs(2, T=7, weight_set=21)
    ref_a = hip_read(to_device(a))[0]
    ref_b = hip_read(to_device(b))[0]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    da, db = to_device(a), to_device(b)
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            ga = hip_read(da, stream=s1)[0]
        with torch.cuda.stream(s2):
            gb = hip_read(db, stream=s2)[0]
        assert np.array_equal(ga, ref_a) and np.array_equal(gb, ref_b)


def test_short_window_reads_on_three_streams():
    """Short-window reads issued back to back on three streams with no host
    synchronisation in between (each launch needs every CU; the library
    orders them across streams): every result equals the same read run alone,
    and no bounded wait expired."""
    import torch
    from hyper_connection_residual_amd import binding
    _case("short-window reads on three streams, T=8, 5 and 24, 12 rounds, no host sync")
    cases = [wl.config_inputs(2, T=T, weight_set=ws) for T, ws in ((8, 40), (5, 41), (24, 42))]
    devs = [to_device(c) for c in cases]
    refs = [hip_read(d) for d in devs]
    streams = [torch.cuda.Stream() for _ in devs]
    outs = [(torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.float32, device="cuda"),
             torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.int16, device="cuda"),
             torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.int16, device="cuda")) for d in devs]
    torch.cuda.synchronize()
    for st in streams:
        binding.hc_timeouts(st)  # (reset the counters)
    for _ in range(12):
        for d, o, st in zip(devs, outs, streams):
            assert binding.hc_read(d["R"].shape[0], d["R"], d["pending"], d["w_norm"], d["W_down"], d["W_up"],
                                   o[0], o[1], o[2], st) == 0
    torch.cuda.synchronize()
    assert [binding.hc_timeouts(st) for st in streams] == [0, 0, 0]
    for o, ref in zip(outs, refs):
        assert np.array_equal(o[0].cpu().numpy().view(np.uint32), ref[0].view(np.uint32))
        assert np.array_equal(o[1].cpu().numpy().view(np.uint16), ref[1].view(np.uint16))


def test_stream_switches_after_a_long_run_on_one_stream():
    """The cross-stream order through both of its mechanisms: reads that
    alternate between two streams (an event after each), then 70 reads in a
    row on one stream (recording stops after 64), then a read on the other
    stream again (no event covers the last read: the device is
    synchronized).  No host synchronisation between the calls; every result
    equals the read run alone, and no bounded wait expired."""
    import torch
    from hyper_connection_residual_amd import binding
    _case("stream switches: alternate, 70 reads on one stream, switch back (T=8 and 17)")
    cases = [wl.config_inputs(2, T=T, weight_set=ws) for T, ws in ((8, 43), (17, 44))]
    devs = [to_device(c) for c in cases]
    refs = [hip_read(d) for d in devs]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [(torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.float32, device="cuda"),
             torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.int16, device="cuda"),
             torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.int16, device="cuda")) for d in devs]
    torch.cuda.synchronize()
    for st in (sa, sb):
        binding.hc_timeouts(st)

    def call(k, st):
        d, o = devs[k], outs[k]
        assert binding.hc_read(d["R"].shape[0], d["R"], d["pending"], d["w_norm"], d["W_down"], d["W_up"],
                               o[0], o[1], o[2], st) == 0

    plan = [(0, sa), (1, sb)] * 4 + [(0, sa)] * 70 + [(1, sb), (0, sa), (1, sb)]
    for k, st in plan:
        call(k, st)
    torch.cuda.synchronize()
    assert [binding.hc_timeouts(st) for st in (sa, sb)] == [0, 0]
    for o, ref in zip(outs, refs):
        assert np.array_equal(o[0].cpu().numpy().view(np.uint32), ref[0].view(np.uint32))


def test_graph_replay_matches_eager():
    """Reads captured in a HIP graph (short windows with pending, and one wide
    read) replay to the same bits as eager reads, replay after replay, with
    eager reads on the same stream and synchronisations in between."""
    import torch
    from hyper_connection_residual_amd import binding
    _case("graph replay: T=1, 5, 8, 13, 16 and 20 with pending and T=40 without, 4 replays")
    inps = [wl.config_inputs(2, T=T, weight_set=30 + T % 18) for T in (1, 5, 8, 13, 16, 20)] + \
        [wl.config_inputs(1, T=40)]
    devs = [to_device(i) for i in inps]
    log = []

    def expired(label, s=None):
        torch.cuda.synchronize()
        log.append((label, binding.hc_timeouts(None), binding.hc_timeouts(s) if s is not None else 0))

    expired("before")
    refs = [hip_read(d) for d in devs]
    expired("eager references")
    gs = torch.cuda.Stream()
    outs = [(torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.float32, device="cuda"),
             torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.int16, device="cuda"),
             torch.empty((d["R"].shape[0], d["R"].shape[2]), dtype=torch.int16, device="cuda")) for d in devs]

    def issue():
        for d, o in zip(devs, outs):
            st = binding.hc_read(d["R"].shape[0], d["R"], d["pending"], d["w_norm"], d["W_down"], d["W_up"],
                                 o[0], o[1], o[2], gs)
            assert st == 0, binding.hc_status_string(st)

    torch.cuda.synchronize()
    with torch.cuda.stream(gs):
        issue()  # eager first calls on this stream allocate its scratch (not allowed under capture)
    expired("eager on the capture stream", gs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        issue()
    expired("capture", gs)
    other = to_device(wl.config_inputs(2, T=6, weight_set=44))
    for rep in range(4):
        for o in outs:
            for t in o:
                t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            g.replay()
        expired("replay %d" % rep, gs)
        hip_read(other, stream=gs)  # eager work on the same stream between replays
        expired("eager after replay %d" % rep, gs)
        for k, (o, ref) in enumerate(zip(outs, refs)):
            got = (o[0].cpu().numpy(), o[1].cpu().numpy().view(np.uint16), o[2].cpu().numpy().view(np.uint16))
            for a, b in zip(got, ref):
                assert np.array_equal(a, b), "replay %d, read %d differs from the eager read" % (rep, k)
    print("expired waits (default stream, capture stream) by phase: %s" % log, flush=True)
    assert all(a == 0 and b == 0 for _, a, b in log), "expired waits: %s" % log
