"""bfloat16 storage emulation for the oracle (test infrastructure only).

bf16 keeps the sign, the 8 exponent bits and the top 7 mantissa bits of an
IEEE float32.  Rounding is round-to-nearest, ties to even, applied directly to
the input's own bits (float64 inputs are rounded from float64, never through
float32, so there is no double rounding).  Inputs are finite and within the
normal float32 range.
"""
from __future__ import annotations

import numpy as np


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 values."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rne_drop(u, drop: int, utype):
    one = utype(1)
    lsb = (u >> utype(drop)) & one
    half_minus_one = (one << utype(drop - 1)) - one
    mask = ~((one << utype(drop)) - one)
    return (u + half_minus_one + lsb) & mask


def round_bf16(x) -> np.ndarray:
    """Rounds to the nearest bf16 value (ties to even); returns float32."""
    a = np.asarray(x)
    if a.dtype == np.float64:
        u = np.ascontiguousarray(a).view(np.uint64)
        # float64 has 52 mantissa bits, bf16 keeps 7: drop 45.
        return _rne_drop(u, 45, np.uint64).view(np.float64).astype(np.float32)
    f = np.ascontiguousarray(a.astype(np.float32, copy=False))
    u = f.view(np.uint32)
    # float32 has 23 mantissa bits, bf16 keeps 7: drop 16.
    return _rne_drop(u, 16, np.uint32).view(np.float32)
