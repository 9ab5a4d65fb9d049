"""bf16 <-> float helpers for the oracle (test infrastructure only).

bf16 keeps the top 16 bits of an IEEE float32.  Upcasting is exact; the
float32 -> bf16 direction rounds to nearest, ties to even, on the 16 dropped
bits (the usual definition of the format's rounding).
"""

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 patterns, round to nearest even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == np.uint64(1)))
    out = (upper + round_up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out[nan] = (upper[nan] | np.uint64(0x40)).astype(np.uint16)
    return out
