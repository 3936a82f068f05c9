"""Helpers shared by the GPU tests: device transfer, the HIP read through the C
ABI, and the parity comparators.  The oracle and the HIP path only meet here,
on the same input bytes."""
from __future__ import annotations

import numpy as np

# max_t,c |gpu - oracle| / max_t,c |oracle| on the fp32 output
REL_TOL = 2e-6
# images: at most 1 ulp apart on at least this fraction of the values
IMG_FRACTION = 0.999


def ordered16(bits: np.ndarray) -> np.ndarray:
    """Monotone integer key of 16-bit float patterns; +0 and -0 map together."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, 0x8000 - mag, 0x8000 + mag)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(ordered16(a_bits) - ordered16(b_bits))


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(gpu.astype(np.float64) - ref))) / (scale if scale > 0 else 1.0)


def to_device(inp, device="cuda"):
    import torch
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(R=t(inp.R), pending=t(inp.pending), w_norm=t(inp.w_norm),
                W_down=t(inp.W_down.view(np.int16)), W_up=t(inp.W_up.view(np.int16)))


def hip_read(dev, stream=None, commit=False, bf16_lo=False):
    """The read through the C ABI (hc_read; hc_read_commit, which also updates
    dev["R"] in place; or hc_read_bf16_lo); returns numpy (mixed f32, bf16
    bits, fp16 bits)."""
    import torch
    from hyper_connection_residual_amd import binding
    R = dev["R"]
    T, C = R.shape[0], R.shape[2]
    mixed = torch.empty((T, C), dtype=torch.float32, device=R.device)
    b16 = torch.empty((T, C), dtype=torch.int16, device=R.device)
    f16 = torch.empty((T, C), dtype=torch.int16, device=R.device)
    fn = binding.hc_read_commit if commit else binding.hc_read_bf16_lo if bf16_lo else binding.hc_read
    st = fn(T, R, dev["pending"], dev["w_norm"], dev["W_down"], dev["W_up"], mixed, b16, f16, stream)
    assert st == 0, "hc_read failed: %s" % binding.hc_status_string(st)
    torch.cuda.synchronize()
    return (mixed.cpu().numpy(), b16.cpu().numpy().view(np.uint16),
            f16.cpu().numpy().view(np.uint16))


def assert_parity(gpu, ref64, tokens=None, label=""):
    """gpu = (mixed, bf16 bits, fp16 bits); ref64 = oracle float64 mixed.

    `tokens` selects the GPU rows that ref64's rows correspond to."""
    from oracle import oracle as orc
    mixed, b16, f16 = gpu
    if tokens is not None:
        mixed, b16, f16 = mixed[tokens], b16[tokens], f16[tokens]
    assert np.all(np.isfinite(mixed)), label + ": non-finite output"
    e = rel_err(mixed, ref64)
    rb, rh = orc.oracle_images(ref64)
    db = ulp_distance(b16, rb)
    dh = ulp_distance(f16, rh)
    fb = float(np.mean(db <= 1))
    fh = float(np.mean(dh <= 1))
    print("%s: rel err %.3e, bf16 within 1 ulp %.5f (max %d), fp16 within 1 ulp %.5f (max %d)"
          % (label, e, fb, int(db.max()), fh, int(dh.max())), flush=True)
    assert e <= REL_TOL, "%s: rel err %.3e > %.1e" % (label, e, REL_TOL)
    assert fb >= IMG_FRACTION, "%s: bf16 images within 1 ulp on only %.5f" % (label, fb)
    assert fh >= IMG_FRACTION, "%s: fp16 images within 1 ulp on only %.5f" % (label, fh)
    return e
