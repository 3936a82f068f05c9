"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to a closed form, an invariant, an exhaustively
checked number format, or a hand-built case whose every intermediate is exact.
Together they are chosen so that a dropped term, a wrong sign or index, a
transposed operand or a wrong normalisation group fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as orc
from hyper_connection_residual_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    """bf16 bits of values that are exactly representable (test helper)."""
    return wl.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def test_bf16_decode_every_pattern_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_hand_values():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133,
             0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126,
             0x3E80: 0.25, 0x4049: 3.140625}
    for b, v in cases.items():
        assert orc.bf16_bits_to_f64(np.array([b], np.uint16))[0] == v
    assert math.isinf(orc.bf16_bits_to_f64(np.array([0x7F80], np.uint16))[0])


def _format_probe_values(rng):
    """float32 values that stress rounding: ties, subnormals, overflow edges."""
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30,
            3.3895314e38, 3.3961776e38, 3.4028235e38, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -15 * 1.5, 1 + 2.0 ** -8,
            1 + 3 * 2.0 ** -8, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -126,
            2.0 ** -133, 2.0 ** -134, 1e-45, 6e-8, 1.1754942e-38]
    vals += [-v for v in vals]
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    rand = u.view(np.float32)
    rand = rand[np.isfinite(rand)]
    # values near every bf16 and fp16 rounding boundary
    mant = rng.integers(0, 2 ** 23, size=50_000).astype(np.uint32)
    expo = rng.integers(100, 160, size=50_000).astype(np.uint32)
    near = ((expo << 23) | (mant & ~np.uint32(0xFFF)) | np.uint32(0x1000)).view(np.float32)
    near16 = ((expo << 23) | (mant & ~np.uint32(0x1FFF)) | np.uint32(0x1000)).view(np.float32)
    return np.concatenate([np.array(vals, np.float32), rand, near, near16,
                           rng.standard_normal(50_000).astype(np.float32) * 1e-5])


def test_f32_to_f16_matches_numpy():
    x = _format_probe_values(np.random.default_rng(7))
    ours = orc.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = _format_probe_values(np.random.default_rng(8))
    ours = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # the input generator's weight rounding agrees too (finite inputs)
    assert np.array_equal(wl.bf16_bits_from_f32(x), ref)


def test_format_hand_values():
    assert orc.f32_to_bf16_bits(np.float32(1 + 2.0 ** -8)) == 0x3F80      # tie -> even
    assert orc.f32_to_bf16_bits(np.float32(1 + 3 * 2.0 ** -8)) == 0x3F82  # tie -> even
    assert orc.f32_to_bf16_bits(np.float32(3.4028235e38)) == 0x7F80       # overflow
    assert orc.f32_to_f16_bits(np.float32(65520.0)) == 0x7C00             # tie -> inf
    assert orc.f32_to_f16_bits(np.float32(65504.0)) == 0x7BFF
    assert orc.f32_to_f16_bits(np.float32(2.0 ** -25)) == 0x0000          # tie -> even (0)
    assert orc.f32_to_f16_bits(np.float32(3 * 2.0 ** -25)) == 0x0002      # tie -> even
    assert orc.f32_to_f16_bits(np.float32(-2.0 ** -24)) == 0x8001


def test_images_are_rne_of_fl32():
    rng = np.random.default_rng(3)
    m = rng.standard_normal(4096) * 10.0 ** rng.integers(-9, 5, size=4096)
    b, h = orc.oracle_images(m)
    f = m.astype(np.float32)
    assert np.array_equal(h, f.astype(np.float16).view(np.uint16))
    assert np.array_equal(b, orc.f32_to_bf16_bits(f))


# --------------------------------------------------------------------------
# The hand-built T = 1 case: n = 4, C = 8, D = 32, r = 2, w_norm = 1.
# sigma_c = +1 (even c) / -1 (odd c); R[s,c] = (s+1) sigma_c, so rs_s = 1/(s+1)
# and xn[s,c] = sigma_c.  W_down row 0 = sigma on stream 1; W_down[1, 24] = 0.5
# (stream 3, c = 0): lo = (8, 0.5).  W_up rows 0..7 (stream 0) = 0.125 in
# column 0; W_up rows 16..23 (stream 2) = c in column 1: up = 1 on stream 0 and
# 0.5 c on stream 2.  mixed[c] = sigma_c (1 + 3 * 0.5 c) = sigma_c (1 + 1.5 c).
# --------------------------------------------------------------------------

def _toy(pending=False, eps=0.0):
    n, C, r = 4, 8, 2
    sig = np.array([1 if c % 2 == 0 else -1 for c in range(C)], np.float32)
    R = np.stack([(s + 1) * sig for s in range(n)])[None].astype(np.float32)
    w = np.ones((n, C), np.float32)
    Wd = np.zeros((r, n * C), np.float32)
    Wd[0, 8:16] = sig
    Wd[1, 24] = 0.5
    Wu = np.zeros((n * C, r), np.float32)
    Wu[0:8, 0] = 0.125
    Wu[16:24, 1] = np.arange(C)
    P = R.copy() if pending else None
    return orc.oracle_read(R, w, _bf16(Wd), _bf16(Wu), P, eps=eps,
                           want_rs=True, want_lo=True)


def test_toy_case_exact():
    mixed, rs, lo = _toy()
    assert mixed[0].tolist() == [1.0, -2.5, 4.0, -5.5, 7.0, -8.5, 10.0, -11.5]
    assert rs[0].tolist() == [1.0, 0.5, 1 / 3, 0.25]
    assert lo[0].tolist() == [8.0, 0.5]


def test_toy_case_pending_is_applied_to_norm_and_mix():
    # P = R: R' = 2R, the norm cancels the factor (lo unchanged) and the mix
    # with R' doubles the output.
    mixed, rs, lo = _toy(pending=True)
    assert mixed[0].tolist() == [2.0, -5.0, 8.0, -11.0, 14.0, -17.0, 20.0, -23.0]
    assert lo[0].tolist() == [8.0, 0.5]


def test_toy_case_eps_is_added_to_the_mean_of_squares():
    eps = 1e-6
    mixed, rs, lo = _toy(eps=eps)
    for s in range(4):
        assert rs[0, s] == pytest.approx(1 / math.sqrt((s + 1) ** 2 + eps), rel=1e-15)
    # stream 1 carries lo[0], stream 3 carries lo[1]
    up0 = 0.125 * 8 * 2 / math.sqrt(4 + eps)
    lo1 = 0.5 * 4 / math.sqrt(16 + eps)
    want = [(1 if c % 2 == 0 else -1) * (up0 + 3 * c * lo1) for c in range(8)]
    np.testing.assert_allclose(mixed[0], want, rtol=1e-15, atol=0)
    assert mixed[0, 0] == pytest.approx(0.999999875, abs=1e-12)


# --------------------------------------------------------------------------
# Closed forms at the real shapes (n = 4, C = 2560, r = 320).
# --------------------------------------------------------------------------

def _signed_constant_residual(rng, T, a):
    """R[t,s,c] = +-a[t,s] with random signs: the mean square is a^2 exactly."""
    n, C = wl.N_STREAMS, wl.WIDTH
    signs = np.where(rng.random((T, n, C)) < 0.5, -1.0, 1.0)
    return (signs * a[:, :, None]).astype(np.float32)


def test_rs_closed_form_real_shape():
    rng = np.random.default_rng(11)
    T = 3
    a = np.array([[1.0, 2.0, 0.5, 4.0], [0.25, 8.0, 1.0, 2.0], [0, 1, 2, 3]], np.float32)
    R = _signed_constant_residual(rng, T, a)
    inp = wl.custom_inputs(T, seed=1)
    _, rs = orc.oracle_read(R, inp.w_norm, inp.W_down, inp.W_up, eps=1e-6, want_rs=True)
    want = 1.0 / np.sqrt(a.astype(np.float64) ** 2 + 1e-6)
    np.testing.assert_allclose(rs, want, rtol=1e-14)
    assert rs[2, 0] == pytest.approx(1000.0, rel=1e-14)  # zero stream -> 1/sqrt(eps)


def test_rs_brute_force_random_rows():
    inp = wl.config_inputs(2, T=2, weight_set=0)
    _, rs = orc.oracle_read(inp.R, inp.w_norm, inp.W_down, inp.W_up, inp.pending,
                            want_rs=True)
    Rp = (inp.R + inp.pending).astype(np.float64)
    for t in range(2):
        for s in range(4):
            ms = math.fsum(float(v) * float(v) for v in Rp[t, s]) / 2560
            assert rs[t, s] == pytest.approx(1 / math.sqrt(ms + 1e-6), rel=1e-13)


def _selection_weights(ks):
    """W_down row j = one-hot at k_j, W_up row k_j = one-hot at column j."""
    D, r = wl.N_STREAMS * wl.WIDTH, wl.RANK
    Wd = np.zeros((r, D), np.float32)
    Wu = np.zeros((D, r), np.float32)
    for j, k in enumerate(ks):
        Wd[j, k] = 1.0
        Wu[k, j] = 1.0
    return _bf16(Wd), _bf16(Wu)


def test_selection_matrices_closed_form():
    rng = np.random.default_rng(5)
    n, C, r = wl.N_STREAMS, wl.WIDTH, wl.RANK
    T = 2
    a = rng.uniform(0.5, 3.0, size=(T, n)).astype(np.float32)
    R = _signed_constant_residual(rng, T, a)
    w = (1 + 0.1 * rng.standard_normal((n, C))).astype(np.float32)
    # 320 distinct flat indices over every stream; some columns chosen twice
    ks = list(rng.choice(n * C, size=r - 8, replace=False))
    cols = [c for c in range(C) if all((s * C + c) not in ks for s in range(n))][:4]
    for c in cols:  # column c selected in streams 0 and 3
        ks += [c, 3 * C + c]
    Wd, Wu = _selection_weights(ks)
    mixed = orc.oracle_read(R, w, Wd, Wu, eps=1e-6)
    want = np.zeros((T, C))
    for t in range(T):
        for k in ks:
            s, c = divmod(int(k), C)
            aa = float(a[t, s])
            want[t, c] += float(w[s, c]) * aa * aa / math.sqrt(aa * aa + 1e-6)
    np.testing.assert_allclose(mixed, want, rtol=1e-13, atol=1e-300)


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small_case():
    return wl.config_inputs(2, T=3, weight_set=5)


def test_zero_weights_give_zero(small_case):
    i = small_case
    z = np.zeros_like(i.W_down)
    assert not np.any(orc.oracle_read(i.R, i.w_norm, z, i.W_up, i.pending))
    z = np.zeros_like(i.W_up)
    assert not np.any(orc.oracle_read(i.R, i.w_norm, i.W_down, z, i.pending))


def test_linearity_in_w_up(small_case):
    i = small_case
    rng = np.random.default_rng(1)
    mask = rng.random(i.W_up.shape) < 0.5
    Wa = np.where(mask, i.W_up, 0).astype(np.uint16)
    Wb = np.where(mask, 0, i.W_up).astype(np.uint16)
    m = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending)
    ma = orc.oracle_read(i.R, i.w_norm, i.W_down, Wa, i.pending)
    mb = orc.oracle_read(i.R, i.w_norm, i.W_down, Wb, i.pending)
    assert _rel(ma + mb, m) < 1e-13
    # power-of-two scaling and sign flip are exact
    wu = orc.bf16_bits_to_f64(i.W_up).astype(np.float32)
    m2 = orc.oracle_read(i.R, i.w_norm, i.W_down, _bf16(2 * wu), i.pending)
    mn = orc.oracle_read(i.R, i.w_norm, i.W_down, _bf16(-wu), i.pending)
    assert np.array_equal(m2, 2 * m)
    assert np.array_equal(mn, -m)


def test_linearity_in_w_down_and_w_norm_scaling(small_case):
    i = small_case
    m = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending)
    wd = orc.bf16_bits_to_f64(i.W_down).astype(np.float32)
    m4 = orc.oracle_read(i.R, i.w_norm, _bf16(4 * wd), i.W_up, i.pending)
    assert np.array_equal(m4, 4 * m)
    mw = orc.oracle_read(i.R, -2 * i.w_norm, i.W_down, i.W_up, i.pending)
    assert np.array_equal(mw, -2 * m)


def test_pending_equals_preadded_residual(small_case):
    i = small_case
    m = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending)
    Rp = (i.R + i.pending).astype(np.float32)
    assert np.array_equal(m, orc.oracle_read(Rp, i.w_norm, i.W_down, i.W_up, None))
    zero = np.zeros_like(i.R)
    assert np.array_equal(orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, zero),
                          orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, None))


def test_commit_hand_values():
    """The committed residual is the IEEE binary32 sum, rounded to nearest even:
    ties go to the even neighbour, x + (-x) is +0, -0 + -0 is -0, overflow
    goes to infinity, subnormals add exactly."""
    f = np.float32
    R = np.array([1, 1, 1, 3, -0.0, 3.4028235e38, 1e-45, 2.5], dtype=f)
    P = np.array([2.0 ** -24, 3 * 2.0 ** -24, -2.0 ** -25, -3, -0.0, 3.4028235e38, 1e-45, 0.0], dtype=f)
    out = orc.oracle_commit(R, P)
    want = np.array([1, 1 + 2.0 ** -22, 1, 0, -0.0, np.inf, 2.8e-45, 2.5], dtype=f)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(orc.oracle_commit(R, None), R)


def test_commit_matches_exact_sum_rounded_once():
    """For N(0,1) + N(0,0.1) operands the sum is exact in binary64 (exponents
    differ by far less than 29), so one binary64 -> binary32 rounding gives
    the correctly rounded float sum."""
    rng = np.random.default_rng(5)
    R = rng.standard_normal(100000).astype(np.float32)
    P = (0.1 * rng.standard_normal(100000)).astype(np.float32)
    want = (R.astype(np.float64) + P.astype(np.float64)).astype(np.float32)
    assert np.array_equal(orc.oracle_commit(R, P).view(np.uint32), want.view(np.uint32))


def test_commit_is_the_reads_own_residual(small_case):
    """Reading the committed residual without a pending write gives the read
    with the pending write, bit for bit."""
    i = small_case
    m = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending)
    Rc = orc.oracle_commit(i.R, i.pending)
    assert np.array_equal(m, orc.oracle_read(Rc, i.w_norm, i.W_down, i.W_up, None))


def test_tokens_are_independent(small_case):
    i = small_case
    m = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending)
    for t in range(i.T):
        mt = orc.oracle_read(i.R[t:t + 1], i.w_norm, i.W_down, i.W_up, i.pending[t:t + 1])
        assert np.array_equal(mt[0], m[t])
    perm = [2, 0, 1]
    mp = orc.oracle_read(i.R[perm], i.w_norm, i.W_down, i.W_up, i.pending[perm])
    assert np.array_equal(mp, m[perm])


def test_stream_relabelling(small_case):
    i = small_case
    n, C, r = wl.N_STREAMS, wl.WIDTH, wl.RANK
    perm = [2, 0, 3, 1]
    flat = np.concatenate([np.arange(s * C, (s + 1) * C) for s in perm])
    m = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending)
    mp = orc.oracle_read(i.R[:, perm], i.w_norm[perm], i.W_down[:, flat],
                         i.W_up[flat], i.pending[:, perm])
    assert _rel(mp, m) < 1e-14


def test_threads_do_not_change_bits():
    i = wl.config_inputs(2, T=5, weight_set=2)
    a = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending, threads=1)
    b = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, i.pending, threads=4)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# The fp32 mode (diagnostic): pinned by hand-derived cases in which the
# rounding of each step is forced, so that each of its stated rules (two
# roundings of xn, every sum one rounded addition at a time in ascending
# order, eps inside the square root next to the mean) changes the result
# if it is broken.  u = 2^-23 is the binary32 spacing just above 1.
# --------------------------------------------------------------------------

def _one_hot_bf16(shape, entries):
    W = np.zeros(shape, np.float32)
    for idx, v in entries.items():
        W[idx] = v
    return _bf16(W)


def _f32_read(R, w, Wd, Wu, eps, mode="f32"):
    return orc.oracle_read(np.asarray(R, np.float32), np.asarray(w, np.float32), Wd, Wu,
                           eps=eps, mode=mode)


def test_fp32_mode_toy_case_exact():
    """Every intermediate of the toy case is exact in binary32 too (rs of the
    streams the down projection reads are 1/2 and 1/4; stream 2's rs = fl(1/3)
    times 3 rounds back to 1), so the fp32 mode gives the exact output."""
    n, C, r = 4, 8, 2
    sig = np.array([1 if c % 2 == 0 else -1 for c in range(C)], np.float32)
    R = np.stack([(s + 1) * sig for s in range(n)])[None].astype(np.float32)
    Wd = np.zeros((r, n * C), np.float32)
    Wd[0, 8:16] = sig
    Wd[1, 24] = 0.5
    Wu = np.zeros((n * C, r), np.float32)
    Wu[0:8, 0] = 0.125
    Wu[16:24, 1] = np.arange(C)
    m = _f32_read(R, np.ones((n, C)), _bf16(Wd), _bf16(Wu), 0.0)
    assert m[0].tolist() == [1.0, -2.5, 4.0, -5.5, 7.0, -8.5, 10.0, -11.5]


def test_fp32_mode_rounds_xn_twice():
    """n = C = r = 1, R' = 3, w_norm = 1 + u, W = 1, eps = 0.  rs = fl(1/3) =
    11184811 * 2^-25.  First rounding: 3 (1 + u) = 3 + 1.5 * 2^-22 is a tie
    between 3 + 2^-22 (odd) and 3 + 2^-21 (even): 3 + 2^-21.  Second: (3 +
    2^-21) rs = 1 + 2^-25 + 11184811 * 2^-46 = 1 + 1.58 u -> 1 + 2u.  The mix
    then gives 3 (1 + 2u) = 3 + 3 * 2^-22, exact (binary32 values in [2, 4)
    are 2^-22 apart).  One rounding of R' w rs = 1 + 1.25 u would give 1 + u
    and the output fl(3 + 1.5 * 2^-22) = 3 + 2^-21 (tie to even); the exact
    read is 3 (1 + u)."""
    one = _bf16(np.ones((1, 1)))
    R = np.full((1, 1, 1), 3.0)
    w = np.full((1, 1), 1 + 2.0 ** -23)
    assert _f32_read(R, w, one, one, 0.0)[0, 0] == 3 + 3 * 2.0 ** -22
    assert _f32_read(R, w, one, one, 0.0, mode="f64")[0, 0] == 3 * (1 + 2.0 ** -23)


def test_fp32_mode_sums_in_ascending_order():
    """Each sum adds one term at a time, index ascending, rounding each
    addition: 1 + 2^-24 + 2^-24 + 2^-24 is then 1 (every step is a tie that
    goes to the even 1), where the exact sum is 1 + 3 * 2^-24, a descending
    order gives 1 + 2^-22, a pairwise order 1 + 2^-23 and a binary64
    accumulator rounded at the end 1 + 2^-22.  One case per sum."""
    e = 2.0 ** -24
    # (a) the down projection's dot: n = 1, C = 4, r = 1, xn = 1
    Wd = _one_hot_bf16((1, 4), {(0, 0): 1.0, (0, 1): e, (0, 2): e, (0, 3): e})
    Wu = _bf16(np.ones((4, 1)))
    m = _f32_read(np.ones((1, 1, 4)), np.ones((1, 4)), Wd, Wu, 0.0)
    assert m[0].tolist() == [1.0, 1.0, 1.0, 1.0]
    # (b) the up projection's dot: n = C = 1, r = 4, lo = (1, e, e, e)
    Wd = _one_hot_bf16((4, 1), {(0, 0): 1.0, (1, 0): e, (2, 0): e, (3, 0): e})
    Wu = _bf16(np.ones((1, 4)))
    assert _f32_read(np.ones((1, 1, 1)), np.ones((1, 1)), Wd, Wu, 0.0)[0, 0] == 1.0
    # (c) the mix over the streams: n = 4, C = r = 1, up = (1, e, e, e), R' = 1
    Wd = _one_hot_bf16((1, 4), {(0, 0): 1.0})
    Wu = _one_hot_bf16((4, 1), {(0, 0): 1.0, (1, 0): e, (2, 0): e, (3, 0): e})
    assert _f32_read(np.ones((1, 4, 1)), np.ones((4, 1)), Wd, Wu, 0.0)[0, 0] == 1.0
    # (d) the sum of squares: n = 1, C = 4, R' = (1, 2^-12, 2^-12, 2^-12): the
    #     squares sum to 1, mean 1/4, rs = 2 exactly, and the read selects
    #     xn[0] = 2 and mixes it with R'[0] = 1.  Summed exactly (1 + 3 e) the
    #     mean is 1/4 + 0.75 e and rs is below 2.
    R = np.array([[[1.0, 2.0 ** -12, 2.0 ** -12, 2.0 ** -12]]])
    Wd = _one_hot_bf16((1, 4), {(0, 0): 1.0})
    Wu = _one_hot_bf16((4, 1), {(0, 0): 1.0})
    m = _f32_read(R, np.ones((1, 4)), Wd, Wu, 0.0)
    assert m[0].tolist() == [2.0, 0.0, 0.0, 0.0]
    assert _f32_read(R, np.ones((1, 4)), Wd, Wu, 0.0, mode="f64")[0, 0] < 2.0


def test_fp32_mode_eps_goes_under_the_root_with_the_mean():
    """n = 1, C = 2, R' = (1, 1), eps = 3: mean 1, rs = 1/sqrt(1 + 3) = 1/2.
    (eps added to the sum of squares before the mean: 1/sqrt(2.5); added
    after the root: 1/4.)  xn = 1/2, lo = xn[0], up = (lo, lo), mixed = up."""
    Wd = _one_hot_bf16((1, 2), {(0, 0): 1.0})
    Wu = _bf16(np.ones((2, 1)))
    m = _f32_read(np.ones((1, 1, 2)), np.ones((1, 2)), Wd, Wu, 3.0)
    assert m[0].tolist() == [0.5, 0.5]


# --------------------------------------------------------------------------
# The bf16-lo mode: the fp64 read with lo rounded to bf16 (nearest, ties to
# even) before the up projection.  The toy case with lo[1] = 0.5 + d, where
# bf16 values next to 0.5 are 2^-8 apart: mixed[c] = sigma_c (1 + 3 c lo[1]).
# --------------------------------------------------------------------------

def _toy_lo1(extra, mode):
    n, C, r = 4, 8, 2
    sig = np.array([1 if c % 2 == 0 else -1 for c in range(C)], np.float32)
    R = np.stack([(s + 1) * sig for s in range(n)])[None].astype(np.float32)
    Wd = np.zeros((r, n * C), np.float32)
    Wd[0, 8:16] = sig
    Wd[1, 24] = 0.5
    for c, v in extra.items():  # stream 3, even columns: xn = +1
        Wd[1, 24 + c] = v
    Wu = np.zeros((n * C, r), np.float32)
    Wu[0:8, 0] = 0.125
    Wu[16:24, 1] = np.arange(C)
    return orc.oracle_read(R, np.ones((n, C), np.float32), _bf16(Wd), _bf16(Wu), None,
                           eps=0.0, mode=mode, want_lo=True)


def _toy_mixed(lo1):
    return [(1 if c % 2 == 0 else -1) * (1 + 3 * c * lo1) for c in range(8)]


def test_bf16_lo_mode_toy_case_exact():
    """lo = (8, 0.5) is exact in bf16: the mode gives the exact read."""
    m, lo = _toy_lo1({}, "f64_bf16_lo")
    assert lo[0].tolist() == [8.0, 0.5]
    assert m[0].tolist() == [1.0, -2.5, 4.0, -5.5, 7.0, -8.5, 10.0, -11.5]


def test_bf16_lo_mode_rounds_to_nearest_even():
    """lo[1] = 0.5 + 2^-9 is a tie between 0.5 (even) and 0.5 + 2^-8: it
    rounds to 0.5.  lo[1] = 0.5 + 2^-9 + 2^-10 lies above the tie: 0.5 +
    2^-8.  lo[1] = 0.5 + 2^-10 lies below it: 0.5.  (Truncation would give
    0.5 for all three, rounding ties up 0.5 + 2^-8 for the first.)  lo is
    reported unrounded, and the fp64 mode keeps the exact value."""
    for extra, rounded in (({2: 2.0 ** -9}, 0.5),
                           ({2: 2.0 ** -9, 4: 2.0 ** -10}, 0.5 + 2.0 ** -8),
                           ({4: 2.0 ** -10}, 0.5)):
        exact = 0.5 + sum(extra.values())
        m, lo = _toy_lo1(extra, "f64_bf16_lo")
        assert lo[0, 1] == exact
        assert m[0].tolist() == _toy_mixed(rounded)
        m64, _ = _toy_lo1(extra, "f64")
        np.testing.assert_allclose(m64[0], _toy_mixed(exact), rtol=1e-15)


def test_fp32_mode_is_at_fp32_level():
    # Two fp32 implementations agree to about 1e-7 relative on the pages (the
    # fused read against the pair); a plain sequential fp32 dot over 10240
    # terms sits a little further from the exact value.
    i = wl.config_inputs(1)
    m64 = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up)
    m32 = orc.oracle_read(i.R, i.w_norm, i.W_down, i.W_up, mode="f32")
    e = _rel(m32, m64)
    assert 1e-9 < e < 1e-5


def test_generic_dimensions_match_matrix_form():
    # A cross-check through numpy matrix products (not a pin on its own: the
    # pins above are what fix the oracle; this guards the generic-size loops).
    inp = wl.custom_inputs(4, n=3, C=40, r=7, seed=9, pending_sigma=0.2, w_sigma=0.1)
    mixed, rs, lo = orc.oracle_read(inp.R, inp.w_norm, inp.W_down, inp.W_up,
                                    inp.pending, eps=1e-3, want_rs=True, want_lo=True)
    Rp = (inp.R + inp.pending).astype(np.float32).astype(np.float64)
    Wd = orc.bf16_bits_to_f64(inp.W_down)
    Wu = orc.bf16_bits_to_f64(inp.W_up)
    rs_ref = 1 / np.sqrt(np.mean(Rp ** 2, axis=2) + 1e-3)
    xn = (Rp * inp.w_norm.astype(np.float64)[None] * rs_ref[:, :, None]).reshape(4, -1)
    lo_ref = xn @ Wd.T
    up = (lo_ref @ Wu.T).reshape(4, 3, 40)
    np.testing.assert_allclose(rs, rs_ref, rtol=1e-14)
    np.testing.assert_allclose(lo, lo_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(mixed, np.sum(up * Rp, axis=1), rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# The dimension readings and the byte model, against the figures the pages
# print (tests/golden/page_dimensions.json).
# --------------------------------------------------------------------------

def test_dimensions_and_byte_model_match_the_pages():
    with open(os.path.join(GOLDEN, "page_dimensions.json")) as f:
        facts = {e["name"]: e["printed"] for e in json.load(f)["facts"]}
    n, C, r = wl.N_STREAMS, wl.WIDTH, wl.RANK
    D = n * C
    assert D == facts["gated_row_width"]
    assert C // 2 == facts["half_stream_tile_floats"]
    assert facts["half_stream_tile_floats"] == 160 * 8
    assert r == facts["up_k"] and r % facts["up_k_slice"] == 0
    assert n == facts["streams_per_tile"]
    blocks, cols = facts["up_blocks_times_columns"]
    assert blocks * cols == C  # the output has C columns, not D
    weight_bytes = 2 * r * D * 2 + n * C * 4
    assert round(weight_bytes / 1e6) == facts["weight_megabytes_per_read"]
    assert round(8192 * D * 4 / 1e6) == facts["gated_megabytes_at_8192_tokens"]
    # gr_mix_r per token: gated and R read (fp32, D each), mixed fp32 plus
    # bf16 and fp16 images written (C columns each)
    mix_bytes = D * 4 + D * 4 + C * (4 + 2 + 2)
    assert round(mix_bytes / 1e3) == facts["mix_kilobytes_per_token"]
    tbps = 8192 * mix_bytes / (facts["mix_ms_at_8192_tokens_rtx5090"] * 1e-3) / 1e12
    assert 1.65 < tbps < 1.80  # "about 96 %" of a 1.79 TB/s card
