"""Pins of the oracle's packing: widths, record layout, lossless round trip.

``bitstring_decode`` below reads a record through a string of '0'/'1'
characters, a third way of reading the layout, independent of both the
oracle's encoder (big integers) and its decoder (64-bit windows).
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import kvsynth
from oracle import Config, record, unpack, stream, quant


def bitstring_decode(kind, buf, n, D, B, R, hb=1):
    nr = -(-n // R)
    npar = D if kind == "K" else B
    raw = list(buf[4 * npar:4 * npar + hb * nr * D])
    # entries: one byte (w in the high nibble) or two little-endian bytes
    # (w in the high byte), read here byte by byte
    hdr = raw if hb == 1 else [raw[2 * i] + 256 * raw[2 * i + 1] for i in range(nr * D)]
    wsh, mmask = (4, 15) if hb == 1 else (8, 255)
    p0 = -(-(4 * npar + hb * nr * D) // 16) * 16
    q = np.zeros((nr * R, D), np.int64)
    pos = p0
    for r in range(nr):
        for c in range(D):
            w, m = hdr[r * D + c] >> wsh, hdr[r * D + c] & mmask
            words = buf[pos:pos + 4 * w]
            pos += 4 * w
            # bit k of the run = bit (k % 32) of word k // 32
            s = "".join(format(words[4 * j + (k // 8) % 4], "08b")[::-1][k % 8]
                        for j in range(w) for k in range(32))
            for i in range(R):
                u = int(s[i * w:(i + 1) * w][::-1], 2) if w else 0
                q[r * R + i, c] = m + u
    return q[:n], pos


def test_width_is_minimal():
    for span in range(0, 256):
        w = int(span).bit_length()
        assert (1 << w) > span and (w == 0 or (1 << (w - 1)) <= span)
        qs = np.array([[3], [3 + span]])
        ww, mm = record.run_widths(qs, 32)
        assert ww[0, 0] == w and mm[0, 0] == 3


@pytest.mark.parametrize("bits,block", [(2, 64), (3, 64), (4, 64), (4, 128), (3, 128), (5, 64), (6, 128),
                                        (7, 64), (8, 64), (8, 128)])
@pytest.mark.parametrize("n", [1, 5, 31, 32, 33, 63, 64, 100, 128])
def test_record_roundtrip_and_layout(bits, block, n):
    if n > block:
        pytest.skip("n > B")
    cfg = Config(bits=bits, block=block)
    rng = np.random.default_rng(n * 7 + bits)
    if n % 2:
        k, v = kvsynth.structured_kv(n, 128, block, 32, seed=n)
    else:
        k = rng.standard_normal((n, 128)).astype(np.float16)
        v = rng.standard_normal((n, 128)).astype(np.float16)
    code = stream.encode_block(k, v, cfg)
    for kind, rec, qs in (("K", code.k_record, code.qk_slots), ("V", code.v_record, code.qv_slots)):
        hb = cfg.header_bytes
        assert hb == (1 if bits <= 4 else 2)
        d = unpack.decode_record(kind, rec, n, 128, block, 32, hb)
        assert np.array_equal(d.q, qs)
        assert qs.max() <= (1 << bits) - 1
        bq, end = bitstring_decode(kind, rec, n, 128, block, 32, hb)
        assert np.array_equal(bq, qs)
        assert len(rec) == d.size == record.record_size(kind, d.w, 128, block, hb)
        assert len(rec) % 16 == 0
        assert not any(rec[end:])                         # tail padding is zero
        npar = 128 if kind == "K" else block
        hdr_end = 4 * npar + hb * d.w.size
        p0 = -(-hdr_end // 16) * 16
        assert not any(rec[hdr_end:p0])                   # header padding is zero
        assert np.all(d.w <= bits)
        # padding slots of a partial last run are zero bits: re-pack check
        assert record.pack_payload(qs, d.w, d.m, 32) == rec[p0:p0 + 4 * int(d.w.sum())]


@pytest.mark.parametrize("D,bits,block", [(64, 4, 64), (64, 7, 128), (256, 3, 64), (256, 8, 128)])
@pytest.mark.parametrize("n", [1, 33, 64])
def test_other_head_dims_roundtrip_and_layout(D, bits, block, n):
    """The record layout with D channels in place of 128: the oracle's decoder
    and the bit-string reader agree with the quantised ints, and the size is
    the closed form."""
    cfg = Config(head_dim=D, bits=bits, block=block)
    rng = np.random.default_rng([D, bits, n])
    k = (rng.standard_normal((n, D)) * np.where(rng.random(D) < 0.3, 0.01, 1.0)).astype(np.float16)
    v = rng.standard_normal((n, D)).astype(np.float16)
    code = stream.encode_block(k, v, cfg)
    hb = cfg.header_bytes
    for kind, rec, qs in (("K", code.k_record, code.qk_slots), ("V", code.v_record, code.qv_slots)):
        assert qs.shape == (n, D)
        d = unpack.decode_record(kind, rec, n, D, block, 32, hb)
        assert np.array_equal(d.q, qs) and d.w.shape == (-(-n // 32), D)
        assert np.array_equal(bitstring_decode(kind, rec, n, D, block, 32, hb)[0], qs)
        assert len(rec) == record.record_size(kind, d.w, D, block, hb)
        assert len(d.scale) == (D if kind == "K" else n)


def test_v_params_are_slot_ordered_and_zero_padded():
    cfg = Config(bits=4, block=64)
    k, v = kvsynth.structured_kv(40, 128, 64, 32, seed=2)
    code = stream.encode_block(k, v, cfg)
    _, sv, zv = quant.quantize_v_tokens(v, 4)
    d = unpack.decode_record("V", code.v_record, 40, 128, 64, 32)
    assert np.array_equal(d.scale, sv[code.perm]) and np.array_equal(d.zero, zv[code.perm])
    raw = np.frombuffer(code.v_record[:256], "<u2")
    assert not raw[40:64].any() and not raw[64 + 40:128].any()


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 64), st.sampled_from([2, 3, 4, 5, 6, 7, 8]), st.integers(0, 2**31 - 1))
def test_hypothesis_roundtrip(n, bits, seed):
    rng = np.random.default_rng(seed)
    cfg = Config(bits=bits, block=64)
    # mixture: some channels nearly constant so narrow widths appear
    base = rng.standard_normal((1, 128)) * 3
    spread = np.where(rng.random(128) < 0.5, 0.01, 1.0)
    k = (base + spread * rng.standard_normal((n, 128))).astype(np.float16)
    v = rng.standard_normal((n, 128)).astype(np.float16)
    code = stream.encode_block(k, v, cfg)
    for kind, rec, qs in (("K", code.k_record, code.qk_slots), ("V", code.v_record, code.qv_slots)):
        d = unpack.decode_record(kind, rec, n, 128, 64, 32, cfg.header_bytes)
        assert np.array_equal(d.q, qs)


@pytest.mark.parametrize("bits", [5, 8])
def test_wide_header_entries_by_hand(bits):
    """Two-byte entries: a run with every value equal has w = 0 and its
    minimum in the low byte; a run spanning 0..L has w = b and m = 0; a
    minimum above 15 (beyond a nibble) survives the round trip."""
    L = (1 << bits) - 1
    q = np.zeros((64, 128), np.int64)
    q[:, 0] = 0
    q[:32, 1] = np.arange(32) % (L + 1)
    q[32:, 1] = L
    q[:32, 2] = 200 if bits == 8 else 20
    q[32:, 2] = (200 if bits == 8 else 20) + 3
    q[:, 3] = np.arange(64) % 2 + 17
    rec = record.build_record("K", q, np.ones(128), np.zeros(128), 64, 32, hb=2)
    h = np.frombuffer(rec[512:512 + 2 * 2 * 128], "<u2").reshape(2, 128)
    assert h[0, 0] == 0 and h[1, 0] == 0
    assert h[0, 1] == (5 << 8) | 0 and h[1, 1] == (0 << 8) | L
    m2 = 200 if bits == 8 else 20
    assert h[0, 2] == m2 and h[1, 2] == m2 + 3
    assert h[0, 3] == (1 << 8) | 17 and h[1, 3] == (1 << 8) | 17
    d = unpack.decode_record("K", rec, 64, 128, 64, 32, 2)
    assert np.array_equal(d.q, q)
    assert np.array_equal(bitstring_decode("K", rec, 64, 128, 64, 32, 2)[0], q)


def test_lossless_grid_values_are_reproduced_exactly():
    """If every group is zero + k*h with k spanning 0..L, decoding returns the input."""
    rng = np.random.default_rng(9)
    cfg = Config(bits=4, block=64)
    T, D, L = 200, 128, 15
    # K: per channel and per block, an fp16 grid
    k = np.empty((T, D))
    for j in range(0, T, 64):
        n = min(64, T - j)
        kk = rng.integers(0, L + 1, (n, D))
        kk[0], kk[-1] = 0, L
        h = 2.0 ** rng.integers(-6, 2, D)
        z = rng.integers(-40, 40, D) * h
        k[j:j + n] = z + kk * h
    kint = rng.integers(0, L + 1, (T, D))
    kint[:, 0], kint[:, 1] = 0, L
    hv = 2.0 ** rng.integers(-6, 2, (T, 1))
    v = rng.integers(-40, 40, (T, 1)) * hv + kint * hv
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    assert np.array_equal(k16.astype(np.float64), k) and np.array_equal(v16.astype(np.float64), v)
    c = stream.compress(k16, v16, cfg)
    kh, vh, _, _ = stream.decode_stream(c)
    assert np.array_equal(stream.token_order(c, kh), k)
    assert np.array_equal(stream.token_order(c, vh), v)
