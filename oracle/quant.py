"""Asymmetric uniform min-max quantisation (oracle).

PackKV's first step quantises the cache to low-bit integers (TL;DR; Fig. 2
caption), with the two granularities of Fig. 5 ("token-wise and
channel-wise").  Readings adopted where the pages are silent:

* K is quantised per channel over the tokens of one block, V per token over
  its D channels;
* asymmetric min-max: zero-point = the group minimum, kept as an fp16 number
  (a float offset, not an integer zero-point), with -0 stored as +0;
* the step ("scale") is the smallest positive fp16 number h with
  h * L >= max - min, L = 2^b - 1, so that every value lies within L steps of
  the minimum; a group whose values are all equal gets scale +0 and q = 0;
* q = round-half-to-even of (x - min) / scale, computed with an exact fp64
  subtraction and a correctly rounded fp64 division.

Why that q is the exact nearest level: x - min is a multiple of 2^-24 and
(k + 1/2) * scale a multiple of 2^-25, so a quotient that is not exactly a
tie lies at least 2^-25 / scale >= 2^-41 away from every half-integer, while
the fp64 division errs by at most 16 * 2^-53 = 2^-49.  Hence
|x - (min + q * scale)| <= scale / 2 holds exactly.
"""

from __future__ import annotations

import numpy as np

from .fp16bits import smallest_f16_at_least


def quantize_groups(x16: np.ndarray, bits: int, axis: int):
    """Quantise fp16 ``x16`` in groups that run along ``axis``.

    Returns (q, scale, zero): q is int64 with x16's shape; scale and zero are
    fp64 arrays holding exact fp16 values, one per group (``axis`` removed).
    """
    L = (1 << bits) - 1
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    assert np.all(np.isfinite(x)), "non-finite input is not supported"
    mn = x.min(axis=axis)
    mx = x.max(axis=axis)
    d = mx - mn                         # exact in fp64
    scale = np.zeros_like(d)
    nz = d > 0
    if np.any(nz):
        scale[nz] = smallest_f16_at_least(d[nz], L)
    zero = mn + 0.0                     # canonical +0 for a zero minimum
    mn_b = np.expand_dims(mn, axis)
    sc_b = np.expand_dims(scale, axis)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((x - mn_b) / sc_b)  # round half to even
    r = np.where(sc_b > 0, r, 0.0)
    q = np.clip(r, 0, L).astype(np.int64)
    return q, scale, zero


def quantize_k_block(k16: np.ndarray, bits: int):
    """K of one block [n, D]: one (scale, zero) per channel over the n tokens."""
    return quantize_groups(k16, bits, axis=0)


def quantize_v_tokens(v16: np.ndarray, bits: int):
    """V [n, D]: one (scale, zero) per token over its D channels."""
    return quantize_groups(v16, bits, axis=1)


def dequantize(q, scale, zero, axis: int) -> np.ndarray:
    """x_hat = zero + scale * q, exact in fp64 (fp16 * int <= 255 plus fp16)."""
    return np.expand_dims(zero, axis) + np.expand_dims(scale, axis) * np.asarray(q, np.float64)
