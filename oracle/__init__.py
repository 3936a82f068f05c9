"""CPU oracle for the hyper-connection read (test infrastructure only).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
import this package.  The library path never does.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    oracle_read,
    oracle_images,
    f32_to_bf16_bits,
    f32_to_f16_bits,
    bf16_bits_to_f64,
)
