"""Thin Python binding of the C ABI in include/hc.h (libhc.so).

Argument marshalling only: every step of the read runs in the HIP kernels of
libhc.so.  PyTorch provides device memory and the current stream.  There is no
CPU fallback: if the library is missing or the device is not a gfx950 GPU the
calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libhc.so then binds to the HIP runtime torch uses

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhc.so")

HC_OK = 0
HC_ERR_ARG = 1
HC_ERR_ALIGN = 2
HC_ERR_DEVICE = 3
HC_ERR_NOMEM = 4
HC_ERR_LAUNCH = 5
HC_ERR_SIZE = 6
HC_ERR_STATE = 7

# Every function the header exports, with its ctypes signature.
_P = ctypes.c_void_p
SIGNATURES = {
    "hc_read": (ctypes.c_int, [ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hc_read_commit": (ctypes.c_int, [ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hc_read_bf16_lo": (ctypes.c_int, [ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hc_read_noalloc": (ctypes.c_int, [ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hc_short_window_on": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int)]),
    "hc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hc_last_hip_error": (ctypes.c_int, []),
    "hc_dims": (None, [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                       ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)]),
    "hc_timeouts": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_uint32)]),
    "hc_stream_read": (ctypes.c_int, [_P, ctypes.c_int64, _P, _P]),
    "hc_release_stream": (ctypes.c_int, [_P]),
    "hc_release": (None, []),
}

_lib = None


class HCError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d, hip error %d)" % (
            what, hc_status_string(status), status, hc_last_hip_error()))
        self.status = status


def library():
    """Load libhc.so (it must have been built: python -m hyper_connection_residual_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libhc.so is not built; run `python -m hyper_connection_residual_amd.build` "
                "(the read has no CPU implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def hc_read(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, stream=None):
    """hc_read of the C ABI: device tensors (or raw device pointers as ints).

    Returns the status code (0 = HC_OK)."""
    return library().hc_read(int(T), _ptr(R), _ptr(pending), _ptr(w_norm), _ptr(W_down),
                             _ptr(W_up), _ptr(out_mixed), _ptr(out_bf16), _ptr(out_fp16),
                             _stream(stream))


def hc_read_commit(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, stream=None):
    """hc_read_commit of the C ABI: hc_read, then R <- R + pending in place.

    Returns the status code (0 = HC_OK)."""
    return library().hc_read_commit(int(T), _ptr(R), _ptr(pending), _ptr(w_norm), _ptr(W_down),
                                    _ptr(W_up), _ptr(out_mixed), _ptr(out_bf16), _ptr(out_fp16),
                                    _stream(stream))


def hc_read_bf16_lo(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, stream=None):
    """hc_read_bf16_lo of the C ABI: the wide path's up projection on bf16(lo).

    Returns the status code (0 = HC_OK)."""
    return library().hc_read_bf16_lo(int(T), _ptr(R), _ptr(pending), _ptr(w_norm), _ptr(W_down),
                                     _ptr(W_up), _ptr(out_mixed), _ptr(out_bf16), _ptr(out_fp16),
                                     _stream(stream))


def hc_read_noalloc(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, stream=None):
    """hc_read_noalloc of the C ABI: the short-window read for T <= 32 without any device
    allocation (after hc_short_window_on() on the device).

    Returns the status code (0 = HC_OK)."""
    return library().hc_read_noalloc(int(T), _ptr(R), _ptr(pending), _ptr(w_norm), _ptr(W_down),
                                     _ptr(W_up), _ptr(out_mixed), _ptr(out_bf16), _ptr(out_fp16),
                                     _stream(stream))


def hc_short_window_on() -> bool:
    """Whether the current device reads short windows (up to 25 tokens; 32 without allocation) with the
    short-window kernel (the library's start-up check decides; it runs now if
    it has not yet)."""
    on = ctypes.c_int()
    st = library().hc_short_window_on(ctypes.byref(on))
    if st != HC_OK:
        raise HCError(st, "hc_short_window_on")
    return bool(on.value)


def hc_status_string(status: int) -> str:
    return library().hc_status_string(int(status)).decode()


def hc_last_hip_error() -> int:
    return library().hc_last_hip_error()


def hc_dims():
    n, C, r, eps = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_float()
    library().hc_dims(ctypes.byref(n), ctypes.byref(C), ctypes.byref(r), ctypes.byref(eps))
    return n.value, C.value, r.value, eps.value


def hc_timeouts(stream=None) -> int:
    cnt = ctypes.c_uint32()
    st = library().hc_timeouts(_stream(stream), ctypes.byref(cnt))
    if st != HC_OK:
        raise HCError(st, "hc_timeouts")
    return cnt.value


def hc_stream_read(src, nbytes, sink, stream=None):
    """hc_stream_read of the C ABI (a measurement reference): one launch that
    streams `nbytes` of the device buffer `src` and writes sink[256].
    Returns the status code."""
    return library().hc_stream_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream))


def hc_release_stream(stream=None) -> None:
    st = library().hc_release_stream(_stream(stream))
    if st != HC_OK:
        raise HCError(st, "hc_release_stream")


def hc_release() -> None:
    library().hc_release()


def _check_kind(t, name, dtype, shape):
    """dtype and shape (checked for every argument before any device check)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if isinstance(dtype, tuple):
        if t.dtype not in dtype:
            raise TypeError("%s must be one of %s, got %s" % (name, dtype, t.dtype))
    elif t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_place(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_BITS16 = (torch.bfloat16, torch.int16, torch.uint16)


def read(R, w_norm, W_down, W_up, pending=None, out=None, stream=None, commit=False):
    """The hyper-connection read on the current stream.

    R, pending: float32 [T, 4, 2560]; w_norm: float32 [4, 2560];
    commit=True also writes R + pending back into R (hc_read_commit);
    W_down: bf16 bits as int16/uint16 [320, 10240] (or a torch.bfloat16 tensor);
    W_up: [10240, 320] likewise.  out: optional (mixed float32 [T, 2560],
    bf16 image as bfloat16 / int16 / uint16, fp16 image as float16 / int16 /
    uint16).  Returns (mixed float32 [T, 2560], bf16 image as torch.bfloat16
    [T, 2560], fp16 image as torch.float16 [T, 2560]) unless `out` is given.
    """
    n, C, r, _ = hc_dims()
    if not isinstance(R, torch.Tensor) or R.dim() != 3:
        raise ValueError("R must be a [T, %d, %d] tensor" % (n, C))
    T = int(R.shape[0])
    args = [(R, "R", torch.float32, (T, n, C)), (w_norm, "w_norm", torch.float32, (n, C)),
            (W_down, "W_down", _BITS16, (r, n * C)), (W_up, "W_up", _BITS16, (n * C, r))]
    if pending is not None:
        args.append((pending, "pending", torch.float32, (T, n, C)))
    if out is not None:
        mixed, img_bf16, img_fp16 = out
        # the images are 16-bit patterns: bf16 bits (bfloat16, or int16 /
        # uint16 holding them) and fp16 bits (float16, int16 or uint16)
        args += [(mixed, "out_mixed", torch.float32, (T, C)), (img_bf16, "out_bf16", _BITS16, (T, C)),
                 (img_fp16, "out_fp16", (torch.float16, torch.int16, torch.uint16), (T, C))]
    for a in args:
        _check_kind(*a)
    for a in args:
        _check_place(a[0], a[1])
    if out is None:
        out = (torch.empty((T, C), dtype=torch.float32, device=R.device),
               torch.empty((T, C), dtype=torch.bfloat16, device=R.device),
               torch.empty((T, C), dtype=torch.float16, device=R.device))
    if T == 0:  # nothing to read: no launch
        return out
    mixed, img_bf16, img_fp16 = out
    fn = hc_read_commit if commit else hc_read
    st = fn(T, R, pending, w_norm, W_down, W_up, mixed, img_bf16, img_fp16, stream)
    if st != HC_OK:
        raise HCError(st, fn.__name__)
    return mixed, img_bf16, img_fp16
