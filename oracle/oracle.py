"""ctypes binding of the plain-C oracle (hc_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the package's smoke check and the
benchmark's CPU-baseline leg, never by the library path.  The arithmetic lives
in hc_oracle.c; this file only compiles it, loads it and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hc_oracle.c")
_LIB = os.path.join(_HERE, "libhc_oracle.so")
# -ffp-contract=off: no fused multiply-adds the source does not write;
# no fast-math: IEEE arithmetic exactly as written.
_CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", "-Wall", "-Wextra"]

_lib = None


def build() -> str:
    """Compile the oracle into oracle/libhc_oracle.so (always recompiles)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def load():
    """Load the compiled oracle, compiling it first if it is missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_LIB)
            or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    lib.hc_oracle_read.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_double, p, p, p, p, p,
                                   ctypes.c_int, ctypes.c_int, p, p, p]
    lib.hc_oracle_read.restype = ctypes.c_int
    lib.hc_oracle_images.argtypes = [p, ctypes.c_int64, p, p]
    lib.hc_oracle_images.restype = None
    lib.hc_oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.hc_oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.hc_oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.hc_oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.hc_oracle_commit.argtypes = [ctypes.c_int64, p, p, p]
    lib.hc_oracle_commit.restype = ctypes.c_int
    lib.hc_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.hc_oracle_bf16_to_double.restype = ctypes.c_double
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


def oracle_read(R, w_norm, W_down, W_up, pending=None, *, eps=1e-6,
                mode="f64", threads=1, want_rs=False, want_lo=False):
    """Run the oracle.

    R, pending: float32 [T, n, C]; w_norm float32 [n, C];
    W_down: uint16 (bf16 bits) [r, n*C]; W_up: uint16 [n*C, r].
    mode: "f64" (the parity reference), "f32" (diagnostic) or "f64_bf16_lo"
    (the fp64 read with lo rounded to bf16 before the up projection: the
    reference of the library's bf16-lo mode; lo is returned unrounded).
    Returns mixed as float64 [T, C] (plus rs [T, n] and lo [T, r] on request).
    """
    lib = load()
    R = _c(R, np.float32)
    if R.ndim != 3:
        raise ValueError("R must be [T, n, C]")
    T, n, C = R.shape
    w_norm = _c(w_norm, np.float32)
    W_down = _c(W_down, np.uint16)
    W_up = _c(W_up, np.uint16)
    r = W_down.shape[0]
    if w_norm.shape != (n, C) or W_down.shape != (r, n * C) or W_up.shape != (n * C, r):
        raise ValueError("shape mismatch")
    if pending is not None:
        pending = _c(pending, np.float32)
        if pending.shape != R.shape:
            raise ValueError("pending must match R")
    mixed = np.empty((T, C), dtype=np.float64)
    rs = np.empty((T, n), dtype=np.float64) if want_rs else None
    lo = np.empty((T, r), dtype=np.float64) if want_lo else None
    m = {"f64": 0, "f32": 1, "f64_bf16_lo": 2}[mode]
    st = lib.hc_oracle_read(T, n, C, r, float(eps), _ptr(R), _ptr(pending),
                            _ptr(w_norm), _ptr(W_down), _ptr(W_up), m,
                            int(threads), _ptr(mixed), _ptr(rs), _ptr(lo))
    if st != 0:
        raise RuntimeError("hc_oracle_read failed with status %d" % st)
    out = [mixed]
    if want_rs:
        out.append(rs)
    if want_lo:
        out.append(lo)
    return out[0] if len(out) == 1 else tuple(out)


def oracle_commit(R, pending):
    """R' = fl32(R + pending) elementwise (R unchanged when pending is None):
    what hc_read_commit leaves in R.  float32 in, float32 out."""
    lib = load()
    R = _c(R, np.float32)
    if pending is not None:
        pending = _c(pending, np.float32)
        if pending.shape != R.shape:
            raise ValueError("pending must match R")
    out = np.empty_like(R)
    st = lib.hc_oracle_commit(R.size, _ptr(R), _ptr(pending), _ptr(out))
    if st != 0:
        raise RuntimeError("hc_oracle_commit failed with status %d" % st)
    return out


def oracle_images(mixed):
    """bf16 and fp16 images (uint16 bits) of a float64 output: RNE of fl32."""
    lib = load()
    mixed = _c(mixed, np.float64)
    b = np.empty(mixed.shape, dtype=np.uint16)
    h = np.empty(mixed.shape, dtype=np.uint16)
    lib.hc_oracle_images(_ptr(mixed), mixed.size, _ptr(b), _ptr(h))
    return b, h


def f32_to_bf16_bits(x):
    lib = load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.hc_oracle_f32_to_bf16(float(v)) for v in x.ravel()],
                    dtype=np.uint16).reshape(x.shape)


def f32_to_f16_bits(x):
    lib = load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.hc_oracle_f32_to_f16(float(v)) for v in x.ravel()],
                    dtype=np.uint16).reshape(x.shape)


def bf16_bits_to_f64(b):
    lib = load()
    b = np.asarray(b, dtype=np.uint16)
    return np.array([lib.hc_oracle_bf16_to_double(int(v)) for v in b.ravel()],
                    dtype=np.float64).reshape(b.shape)
