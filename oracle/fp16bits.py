"""fp16 helpers for the oracle: exact values and bit patterns.

Every finite fp16 number is exactly representable in fp64, and the product
of an fp16 number and an integer below 2^12 is exact in fp64 too, so all the
comparisons made here are exact.
"""

from __future__ import annotations

import numpy as np

# All positive finite fp16 values, ascending (bit patterns 0x0001 .. 0x7BFF are
# monotone in value for positive numbers).
POSITIVE_F16 = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)


def smallest_f16_at_least(d: np.ndarray, levels: int) -> np.ndarray:
    """For each d > 0: the smallest positive fp16 h with h * levels >= d.

    A binary search over the sorted table of positive fp16 values; h * levels
    is exact in fp64, so this is the exact definition, with no division.
    """
    d = np.asarray(d, dtype=np.float64)
    idx = np.searchsorted(POSITIVE_F16 * levels, d, side="left")
    if np.any(idx >= POSITIVE_F16.size):
        raise ValueError("range too large for an fp16 scale")
    return POSITIVE_F16[idx]


def f16_bits(x) -> np.ndarray:
    """fp16 bit patterns (uint16) of values that are exactly fp16."""
    a = np.asarray(x, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), a), "value is not an fp16 number"
    return h.view(np.uint16)


def f16_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
