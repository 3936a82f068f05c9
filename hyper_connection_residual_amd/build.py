"""Build the HIP library libhc.so (gfx950) in the package directory.

    python -m hyper_connection_residual_amd.build

compiles every source under csrc/ with hipcc for gfx950 only.  Packed fp32
arithmetic is turned off for device code (its forms are avoided on this part);
the host pass warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhc.so")

SOURCES = ["hc_api.hip", "hc_decode.hip", "hc_prefill.hip", "hc_stream.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments arrive preloaded in SGPRs (the code keeps a prologue
    # that loads them for firmware without the feature)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


PROBE_LIB = os.path.join(PKG, "libhc_probe.so")


def build(verbose: bool = False, probe: bool = False) -> str:
    """Compile libhc.so (always recompiles); returns its path.  probe=True
    builds the timing variant libhc_probe.so instead: the short-window kernel
    records clock stamps per workgroup (hc_probe_stamps); the library never
    loads it."""
    out = PROBE_LIB if probe else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, *(["-DHC_PROBE_STAMPS"] if probe else []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, probe="--probe" in sys.argv[1:]))
