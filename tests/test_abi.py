"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")


@pytest.fixture(scope="module")
def lib():
    from hyper_connection_residual_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from hyper_connection_residual_amd import build
        build.build()
    return binding.library()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"HC_API\s+[\w\s\*]+?\b(hc_\w+)\s*\(", text)


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == ["hc_read", "hc_read_commit", "hc_read_bf16_lo", "hc_read_noalloc", "hc_short_window_on",
                     "hc_status_string",
                     "hc_last_hip_error", "hc_dims", "hc_timeouts", "hc_stream_read", "hc_release_stream", "hc_release"]


def test_library_exports_every_declared_function(lib):
    from hyper_connection_residual_amd import binding
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_library_targets_gfx950_only():
    from hyper_connection_residual_amd import binding
    out = subprocess.run(["strings", binding.LIB_PATH], capture_output=True, text=True).stdout
    assert "amdgcn-amd-amdhsa--gfx950" in out
    assert not re.search(r"amdgcn-amd-amdhsa--gfx(?!950)\d+", out)


def test_dims(lib):
    from hyper_connection_residual_amd import binding
    n, C, r, eps = binding.hc_dims()
    assert (n, C, r) == (4, 2560, 320)
    assert eps == pytest.approx(1e-6, rel=1e-7)


def test_status_strings(lib):
    from hyper_connection_residual_amd import binding
    texts = {binding.hc_status_string(s) for s in range(8)}
    assert len(texts) == 8 and all(texts) and "unknown status" not in texts
    assert binding.hc_status_string(99) == "unknown status"


@pytest.mark.parametrize("entry", ["hc_read", "hc_read_commit", "hc_read_bf16_lo", "hc_read_noalloc"])
def test_argument_checks_happen_before_any_hip_call(lib, entry):
    from hyper_connection_residual_amd import binding
    fn = getattr(binding, entry)
    good = 0x10000  # never dereferenced: the checks below reject first
    args = [good] * 8
    # T < 1
    assert fn(0, *args, 0) == binding.HC_ERR_ARG
    assert fn(-5, *args, 0) == binding.HC_ERR_ARG
    # a required pointer is NULL (pending may be NULL)
    for i in (0, 2, 3, 4, 5, 6, 7):
        a = list(args)
        a[i] = None
        assert fn(1, *a, 0) == binding.HC_ERR_ARG, i
    # misalignment of any pointer, pending included
    for i in range(8):
        a = list(args)
        a[i] = good + 4
        assert fn(1, *a, 0) == binding.HC_ERR_ALIGN, i


def test_stream_read_checks_arguments_first(lib):
    from hyper_connection_residual_amd import binding
    good = 0x10000
    assert binding.hc_stream_read(None, 1024, good, 0) == binding.HC_ERR_ARG
    assert binding.hc_stream_read(good, 1024, None, 0) == binding.HC_ERR_ARG
    assert binding.hc_stream_read(good, 8, good, 0) == binding.HC_ERR_ARG
    assert binding.hc_stream_read(good, 1000, good, 0) == binding.HC_ERR_ARG
    assert binding.hc_stream_read(good + 4, 1024, good, 0) == binding.HC_ERR_ALIGN
    assert binding.hc_stream_read(good, 1024, good + 4, 0) == binding.HC_ERR_ALIGN


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK),
                    reason="a GPU is present; this checks the no-device error path")
def test_no_device_is_an_error_not_a_fallback(lib):
    from hyper_connection_residual_amd import binding
    good = 0x10000
    for fn in (binding.hc_read, binding.hc_read_commit, binding.hc_read_bf16_lo, binding.hc_read_noalloc):
        st = fn(1, good, good, good, good, good, good, good, good, 0)
        assert st == binding.HC_ERR_DEVICE
    with pytest.raises(binding.HCError):
        binding.hc_short_window_on()
    assert binding.library().hc_short_window_on(None) == binding.HC_ERR_ARG


def test_python_read_refuses_cpu_tensors(lib):
    import torch
    from hyper_connection_residual_amd import binding
    R = torch.zeros((1, 4, 2560))
    w = torch.ones((4, 2560))
    Wd = torch.zeros((320, 10240), dtype=torch.int16)
    Wu = torch.zeros((10240, 320), dtype=torch.int16)
    with pytest.raises(ValueError):
        binding.read(R, w, Wd, Wu)
    with pytest.raises(TypeError):
        binding.read(R.double(), w, Wd, Wu)


def test_python_read_refuses_image_buffers_of_the_wrong_width(lib):
    """The image outputs hold 16-bit patterns: a caller-supplied buffer of
    1-byte (or 4-byte) elements is refused before any launch, since the
    kernels store 2 bytes per element."""
    import torch
    from hyper_connection_residual_amd import binding
    T = 2
    R = torch.zeros((T, 4, 2560))
    w = torch.ones((4, 2560))
    Wd = torch.zeros((320, 10240), dtype=torch.int16)
    Wu = torch.zeros((10240, 320), dtype=torch.int16)
    mixed = torch.empty((T, 2560))
    good = torch.empty((T, 2560), dtype=torch.int16)
    for bad in (torch.uint8, torch.int8, torch.float32, torch.int32):
        img = torch.empty((T, 2560), dtype=bad)
        with pytest.raises(TypeError, match="out_bf16"):
            binding.read(R, w, Wd, Wu, out=(mixed, img, good))
        with pytest.raises(TypeError, match="out_fp16"):
            binding.read(R, w, Wd, Wu, out=(mixed, good, img))
    with pytest.raises(TypeError, match="out_bf16"):  # an fp16 tensor is not a bf16 image
        binding.read(R, w, Wd, Wu, out=(mixed, torch.empty((T, 2560), dtype=torch.float16), good))


def test_noalloc_rejects_windows_above_32_before_any_hip_call(lib):
    from hyper_connection_residual_amd import binding
    good = 0x10000
    for T in (33, 64, 4096):
        assert binding.hc_read_noalloc(T, *([good] * 8), 0) == binding.HC_ERR_SIZE
