"""hc_read_noalloc, the allocation-free entry point, through the C ABI against
hc_read on the same inputs: up to 25 tokens the same kernel, so the same bits
(and hc_read is held to the oracle elsewhere); from 26 to 32 tokens, where
hc_read takes the wide path, against two hc_read reads of the window's parts
(above 8 tokens a token's bits do not depend on the window).  Two calls in a
row, the second smaller; a capture on a stream that never allocated; and the
size limit."""
import numpy as np
import pytest

from hyper_connection_residual_amd import workloads as wl
from tests.hc_testlib import hip_read, to_device

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] " + label, flush=True)


@pytest.fixture(scope="module", autouse=True)
def setup():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"
    from hyper_connection_residual_amd import binding
    # set-up of the allocation-free reads on this device (the start-up check)
    assert binding.hc_short_window_on()
    binding.hc_timeouts()
    yield
    assert binding.hc_timeouts() == 0


def _outputs(T):
    import torch
    return (torch.empty((T, 2560), dtype=torch.float32, device="cuda"),
            torch.empty((T, 2560), dtype=torch.int16, device="cuda"),
            torch.empty((T, 2560), dtype=torch.int16, device="cuda"))


def _noalloc(dev, o, stream=None):
    from hyper_connection_residual_amd import binding
    T = dev["R"].shape[0]
    return binding.hc_read_noalloc(T, dev["R"], dev["pending"], dev["w_norm"], dev["W_down"], dev["W_up"],
                                   o[0], o[1], o[2], stream)


def _same(got, ref, label):
    g = (got[0].cpu().numpy(), got[1].cpu().numpy().view(np.uint16), got[2].cpu().numpy().view(np.uint16))
    for a, b in zip(g, ref):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), label


@pytest.mark.parametrize("sizes, pending", [((24, 5), True), ((25, 1), False), ((9, 8), True)])
def test_noalloc_matches_hc_read_on_two_calls(sizes, pending):
    import torch
    devs, refs = [], []
    for k, T in enumerate(sizes):
        inp = wl.config_inputs(2, T=T, weight_set=15 + k)
        if not pending:
            inp.pending = None
        devs.append(to_device(inp))
        refs.append(hip_read(devs[-1]))
    outs = [_outputs(T) for T in sizes]
    _case("hc_read_noalloc: T=%d then T=%d, pending=%s, against hc_read" % (sizes + (pending,)))
    for d, o in zip(devs, outs):  # two calls in a row, no synchronisation between them
        assert _noalloc(d, o) == 0
    torch.cuda.synchronize()
    for k, (o, ref) in enumerate(zip(outs, refs)):
        _same(o, ref, "call %d (T=%d)" % (k, sizes[k]))


def test_noalloc_windows_of_26_to_32_equal_their_parts():
    """26..32 tokens, which hc_read sends to the wide path: hc_read_noalloc (the
    six-chain short-window kernel) gives every token the bits of hc_read reads
    of the window's two parts (13..16 tokens each, the three-chain kernel)."""
    import dataclasses
    import torch
    for T in range(26, 33):
        _case("hc_read_noalloc T=%d against hc_read of its parts" % T)
        inp = wl.config_inputs(2, T=T, weight_set=30 + T)
        o = _outputs(T)
        assert _noalloc(to_device(inp), o) == 0
        torch.cuda.synchronize()
        got = (o[0].cpu().numpy(), o[1].cpu().numpy().view(np.uint16), o[2].cpu().numpy().view(np.uint16))
        a = T // 2
        for lo, hi in ((0, a), (a, T)):
            part = dataclasses.replace(inp, R=inp.R[lo:hi].copy(), pending=inp.pending[lo:hi].copy())
            ref = hip_read(to_device(part))
            for x, y in zip(ref, got):
                assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                      (y.view(np.uint32) if y.dtype == np.float32 else y)[lo:hi]), \
                    "T=%d tokens %d..%d" % (T, lo, hi - 1)


def test_noalloc_under_capture_on_a_stream_that_never_allocated():
    """A stream with no workspace cannot take hc_read's first call under
    capture (it would allocate); hc_read_noalloc is captured and replayed,
    every replay equal to hc_read, with eager work in between."""
    import torch
    from hyper_connection_residual_amd import binding
    _case("hc_read_noalloc captured on a fresh stream, T=16 and T=3, 3 replays")
    cases = [to_device(wl.config_inputs(2, T=T, weight_set=17 + T)) for T in (16, 3)]
    refs = [hip_read(d) for d in cases]
    outs = [_outputs(d["R"].shape[0]) for d in cases]
    gs = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for d, o in zip(cases, outs):
            assert _noalloc(d, o, gs) == 0
    other = to_device(wl.config_inputs(2, T=6, weight_set=44))
    for rep in range(3):
        for o in outs:
            for t in o:
                t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(gs):
            g.replay()
        torch.cuda.synchronize()
        hip_read(other)
        for k, (o, ref) in enumerate(zip(outs, refs)):
            _same(o, ref, "replay %d, read %d" % (rep, k))


def test_noalloc_refuses_windows_above_32():
    _case("hc_read_noalloc with T=33: HC_ERR_SIZE, nothing written")
    from hyper_connection_residual_amd import binding
    import torch
    d = to_device(wl.config_inputs(2, T=33, weight_set=1))
    o = _outputs(33)
    o[0].fill_(7.0)
    assert _noalloc(d, o) == binding.HC_ERR_SIZE
    torch.cuda.synchronize()
    assert bool(torch.all(o[0] == 7.0))
