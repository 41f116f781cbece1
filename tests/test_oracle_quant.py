"""Pins of the oracle's quantiser against exact rational arithmetic.

The brute force here works in Python Fractions: it scans every positive fp16
number for the step and every level for the nearest one, so it relies on no
fp64 exactness argument and shares no code with ``oracle.quant``.
"""

from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import quant, fp16bits

ALL_POS_F16 = [Fraction(float(v)) for v in
               np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)]


def brute_quant(x16, bits):
    """Exact min-max quantisation of one group by exhaustive search."""
    L = (1 << bits) - 1
    xs = [Fraction(float(v)) for v in np.asarray(x16, np.float16)]
    mn, mx = min(xs), max(xs)
    if mx == mn:
        return [0] * len(xs), Fraction(0), mn
    d = mx - mn
    h = next(v for v in ALL_POS_F16 if v * L >= d)       # smallest fp16 step
    q = []
    for x in xs:
        dist = [abs(x - (mn + k * h)) for k in range(L + 1)]
        best = min(dist)
        cands = [k for k in range(L + 1) if dist[k] == best]
        q.append(cands[0] if len(cands) == 1 else next(k for k in cands if k % 2 == 0))
    return q, h, mn


def check_group(x16, bits):
    q, sc, ze = quant.quantize_groups(np.asarray(x16, np.float16)[None, :], bits, axis=1)
    bq, bh, bmn = brute_quant(x16, bits)
    assert list(q[0]) == bq
    assert Fraction(float(sc[0])) == bh
    assert Fraction(float(ze[0])) == bmn


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_random_groups_match_brute_force(bits):
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 12))
        mag = 10.0 ** rng.uniform(-6, 4)
        x = (rng.standard_normal(n) * mag).astype(np.float16)
        check_group(x, bits)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_exact_ties_round_to_even(bits):
    """Values exactly halfway between two levels go to the even level."""
    L = (1 << bits) - 1
    h = 0.125
    mn = -1.0
    ties = [mn + (k + 0.5) * h for k in range(L)]
    x = np.array([mn, mn + L * h] + ties, dtype=np.float16)
    q, sc, _ = quant.quantize_groups(x[None, :], bits, axis=1)
    assert sc[0] == h
    expect = [0, L] + [k if k % 2 == 0 else k + 1 for k in range(L)]
    assert list(q[0]) == expect
    check_group(x, bits)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=0x7BFF), min_size=1, max_size=9),
       st.lists(st.booleans(), min_size=9, max_size=9),
       st.sampled_from([2, 3, 4, 5, 6, 7, 8]))
def test_hypothesis_groups(mags, signs, bits):
    bits_arr = np.array(mags, np.uint16) | (np.array(signs[:len(mags)], np.uint16) << 15)
    x = bits_arr.view(np.float16)
    check_group(x, bits)


def test_constant_group_has_zero_scale():
    x = np.full(7, 1.5, np.float16)
    q, sc, ze = quant.quantize_groups(x[None, :], 4, axis=1)
    assert sc[0] == 0 and ze[0] == 1.5 and not q.any()


def test_negative_zero_minimum_is_stored_as_plus_zero():
    x = np.array([-0.0, 0.5, 1.0], np.float16)
    _, _, ze = quant.quantize_groups(x[None, :], 4, axis=1)
    assert fp16bits.f16_bits(ze)[0] == 0


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_error_bound_and_scale_minimality(bits):
    """|x - x_hat| <= scale/2 exactly; the scale is the smallest fp16 that covers the range."""
    L = (1 << bits) - 1
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 128)) * np.where(rng.random(128) < 0.06, 10, 1)).astype(np.float16)
    for axis in (0, 1):
        q, sc, ze = quant.quantize_groups(x, bits, axis=axis)
        xh = quant.dequantize(q, sc, ze, axis)
        err = np.abs(x.astype(np.float64) - xh)
        assert np.all(err <= np.expand_dims(sc, axis) / 2)
        d = x.astype(np.float64).max(axis) - x.astype(np.float64).min(axis)
        assert np.all(sc * L >= d)
        prev = (sc.astype(np.float16).view(np.uint16) - 1).view(np.float16).astype(np.float64)
        assert np.all(prev * L < d)


def test_k_is_per_channel_and_v_per_token():
    """Each channel of a K block (and each V token) gets the step of its own range."""
    n, D = 64, 128
    t = np.arange(n)[:, None]
    c = np.arange(D)[None, :]
    x = ((t - 32) * (c + 1) / 256.0).astype(np.float16)   # range grows with c
    _, sk, zk = quant.quantize_k_block(x, 4)
    rng_c = x.astype(np.float64).max(0) - x.astype(np.float64).min(0)
    assert np.all(sk * 15 >= rng_c) and np.all(np.diff(sk) >= 0) and sk[-1] > 50 * sk[0]
    assert np.array_equal(zk, x.astype(np.float64).min(0))
    _, sv, zv = quant.quantize_v_tokens(x, 4)
    rng_t = x.astype(np.float64).max(1) - x.astype(np.float64).min(1)
    assert np.all(sv * 15 >= rng_t)
    assert sv.shape == (n,) and np.array_equal(zv, x.astype(np.float64).min(1) + 0.0)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_k_block_channel_hits_both_extremes(bits):
    """With a normal-range step, each K (block, channel) has min q = 0 and max q = L."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float16)
    q, sc, _ = quant.quantize_k_block(x, bits)
    normal = sc >= 2.0 ** -14
    assert normal.all()
    assert np.all(q.min(0) == 0) and np.all(q.max(0) == (1 << bits) - 1)
