"""bfloat16 bit handling for the oracle (float64 <-> bfloat16, nearest-even).

A bfloat16 value has 8 significant bits, an 8-bit exponent and subnormals
below 2**-126 spaced by 2**-133.  ``round_rne`` rounds a float64 directly to
the nearest bfloat16 (ties to the even significand) -- never through float32,
which could round twice.  Test infrastructure only (see ``oracle/__init__``).
"""

from __future__ import annotations

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def widen(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    The quantum of the result is ``2**(max(e, -126) - 7)`` where ``e`` is the
    binary exponent of ``|x|``; ``np.rint`` rounds half to even.  Magnitudes
    that round above the largest finite bfloat16 become infinity.  NaN is not
    expected on the path and maps to a quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e2 = np.frexp(a)                 # a = f * 2**e2 with f in [0.5, 1)
    e = np.maximum(e2 - 1, -126)        # exponent of the leading bit
    quantum = np.ldexp(1.0, e - 7)
    r = np.rint(a / quantum) * quantum  # exact scaling by a power of two
    r = np.where(a == 0, 0.0, r)
    r = np.where(r > _BF16_MAX, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    r = np.copysign(r, x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def round_value(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value, returned as float64."""
    return widen(round_rne(x))
