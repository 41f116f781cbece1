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


def bitstring_decode(kind, buf, n, D, B, R, hb=1, order=0):
    """order 1: each run row's payload holds the widest entries first, equal
    widths by channel; walked here width by width from the largest."""
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
    cb = 4 * hb                    # container field bits: 4 (b <= 4) or 8
    for r in range(nr):
        row_w = [hdr[r * D + c] >> wsh for c in range(D)]
        seq = list(range(D)) if order == 0 else [c for wv in range(8, -1, -1) for c in range(D) if row_w[c] == wv]
        assert sorted(seq) == list(range(D))
        for c in seq:
            w, m = hdr[r * D + c] >> wsh, hdr[r * D + c] & mmask
            words = buf[pos:pos + 4 * w]
            pos += 4 * w
            # bit k of the run = bit (k % 32) of word k // 32
            s = "".join(format(words[4 * j + (k // 8) % 4], "08b")[::-1][k % 8]
                        for j in range(w) for k in range(32))
            for i in range(R):
                # slot i sits in field f of container t; its bit p is in word
                # (t*w) // cb at cb*f + (t*w) % cb + p when w divides cb, else
                # in word t at cb*f + p (t < w) or in word p at cb*f + t
                t, f = i // (32 // cb), i % (32 // cb)
                u = 0
                for p in range(w):
                    if cb % w == 0:
                        word, bit = (t * w) // cb, cb * f + (t * w) % cb + p
                    elif t < w:
                        word, bit = t, cb * f + p
                    else:
                        word, bit = p, cb * f + t
                    u |= int(s[32 * word + bit]) << p
                q[r * R + i, c] = m + u
    return q[:n], pos


# Run words worked out by hand from the layout rule: (container bits, u of
# slots 0..31, expected run words).
HAND_RUNS = [
    # w = 4, nibbles: slot 8k + j in nibble j of word k (the plain order)
    (4, [i % 16 for i in range(32)], [0x76543210, 0xFEDCBA98, 0x76543210, 0xFEDCBA98]),
    # w = 3, nibbles: containers 0..2 in the low 3 bits of words 0..2; bit p
    # of container 3 (slots 24..31, u = j) in bit 3 of nibble j of word p
    (4, [i % 8 for i in range(32)], [0xF6D4B290, 0xFE54BA10, 0xFEDC3210]),
    # w = 2: word 0 = container 0 | container 1 << 2, word 1 = 2 | 3 << 2
    (4, [i % 4 for i in range(32)], [0xFA50FA50, 0xFA50FA50]),
    # w = 1: word 0 = sum of container k << k; slots 8..15 and 24..31 are 1
    (4, [(i >> 3) & 1 for i in range(32)], [0xAAAAAAAA]),
    # w = 5, bytes: containers 0..4 (slots 0..19) in the low 5 bits of words
    # 0..4; bit p of containers 5, 6, 7 (slots 20..31) in bits 5, 6, 7 of
    # byte j of word p
    (8, list(range(32)), [0xE302E100, 0xE7E60504, 0xABAAA9A8, 0xCFCECDCC, 0xF3F2F1F0]),
    # w = 4, bytes: word i = container 2i | container 2i+1 << 4
    (8, [i % 16 for i in range(32)], [0x73625140, 0xFBEAD9C8, 0x73625140, 0xFBEAD9C8]),
]


@pytest.mark.parametrize("cb,u,words", HAND_RUNS)
def test_run_layout_by_hand(cb, u, words):
    """The payload words of one run, built by hand from the layout rule, are
    what the encoder writes, and both readers recover the values."""
    w = max(u).bit_length()
    assert w == len(words)
    q = np.zeros((32, 128), np.int64)
    q[:, 5] = u
    q[0, :] = np.maximum(q[0, :], 0)
    wr, mr = record.run_widths(q, 32)
    assert wr[0, 5] == w and mr[0, 5] == 0
    pay = record.pack_payload(q, wr, mr, 32, cb)
    got = np.frombuffer(pay, "<u4")                       # only channel 5 has w > 0
    assert [int(x) for x in got] == words
    hb = cb // 4
    rec = record.build_record("K", q, np.ones(128), np.zeros(128), 64, 32, hb=hb)
    assert np.array_equal(unpack.decode_record("K", rec, 32, 128, 64, 32, hb).q, q)
    assert np.array_equal(bitstring_decode("K", rec, 32, 128, 64, 32, hb)[0], q)


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
        assert record.pack_payload(qs, d.w, d.m, 32, 4 * hb) == rec[p0:p0 + 4 * int(d.w.sum())]


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


# ---- payload order 1: K rows stored by decreasing width -------------------

def _single_channel_words(u, cb=4):
    """Run words of one channel's 32 values, from the channel-order layout
    (pinned by hand above)."""
    q = np.zeros((32, 128), np.int64)
    q[:, 0] = u
    w, m = record.run_widths(q, 32)
    return np.frombuffer(record.pack_payload(q, w, m, 32, cb), "<u4").tolist()


def test_width_sorted_payload_by_hand():
    """Two rows of a K block with chosen widths: the payload holds, row by
    row, the widest entries first and equal widths by channel; each entry's
    words are its channel-order words."""
    q = np.zeros((64, 128), np.int64)
    ua = [i % 8 for i in range(32)]                 # w = 3
    ub = [7 - (i % 8) for i in range(32)]           # w = 3
    uc = [i % 4 for i in range(32)]                 # w = 2
    ud = [(i >> 3) & 1 for i in range(32)]          # w = 1
    q[:32, 9], q[:32, 2], q[:32, 7], q[:32, 5] = ua, ub, uc, ud
    q[32:, 5], q[32:, 100], q[32:, 3] = ua, uc, uc  # row 1: 5 (w 3), then 3 and 100 (w 2)
    w, m = record.run_widths(q, 32)
    assert w[0, 9] == w[0, 2] == 3 and w[0, 7] == 2 and w[0, 5] == 1
    got = np.frombuffer(record.pack_payload(q, w, m, 32, 4, order=1), "<u4").tolist()
    want = (_single_channel_words(ub) + _single_channel_words(ua) + _single_channel_words(uc)
            + _single_channel_words(ud)
            + _single_channel_words(ua) + _single_channel_words(uc) + _single_channel_words(uc))
    assert got == want
    assert _single_channel_words(ua) == [0xF6D4B290, 0xFE54BA10, 0xFEDC3210]
    rec1 = record.build_record("K", q, np.ones(128), np.zeros(128), 64, 32, order=1)
    rec0 = record.build_record("K", q, np.ones(128), np.zeros(128), 64, 32)
    assert len(rec1) == len(rec0) and rec1[:512 + 256] == rec0[:512 + 256]   # params and header
    assert rec1 != rec0
    assert np.array_equal(unpack.decode_record("K", rec1, 64, 128, 64, 32, 1, order=1).q, q)
    assert np.array_equal(bitstring_decode("K", rec1, 64, 128, 64, 32, 1, order=1)[0], q)


@pytest.mark.parametrize("bits,block", [(2, 64), (3, 64), (4, 64), (4, 128), (3, 128), (6, 64), (8, 128)])
@pytest.mark.parametrize("n", [1, 31, 33, 64, 100, 128])
def test_width_sorted_roundtrip(bits, block, n):
    """Payload order 1 on data with mixed widths: both readers recover the
    ints, the size and header match order 0, the payload holds the same run
    words rearranged, and a row whose widths are all equal is unchanged."""
    if n > block:
        pytest.skip("n > B")
    cfg0 = Config(bits=bits, block=block)
    cfg1 = Config(bits=bits, block=block, payload_order=1)
    k, v = kvsynth.structured_kv(n, 128, block, 32, seed=n + bits)
    c0, c1 = stream.encode_block(k, v, cfg0), stream.encode_block(k, v, cfg1)
    assert c1.v_record == c0.v_record and np.array_equal(c1.perm, c0.perm)
    hb = cfg1.header_bytes
    d1 = unpack.decode_record("K", c1.k_record, n, 128, block, 32, hb, order=1)
    assert np.array_equal(d1.q, c1.qk_slots)
    assert np.array_equal(bitstring_decode("K", c1.k_record, n, 128, block, 32, hb, order=1)[0], c1.qk_slots)
    assert len(c1.k_record) == len(c0.k_record) == d1.size
    p0 = -(-(4 * 128 + hb * d1.w.size) // 16) * 16
    assert c1.k_record[:p0] == c0.k_record[:p0]
    w0 = np.frombuffer(c0.k_record[p0:], "<u4")
    w1 = np.frombuffer(c1.k_record[p0:], "<u4")
    assert sorted(w0.tolist()) == sorted(w1.tolist())
    # the orders coincide exactly where, in every row, the entries that hold
    # words (w > 0) already fall (weakly) in width from channel 0 to D-1
    already_sorted = all(np.all(np.diff(row[row > 0]) <= 0) for row in d1.w)
    assert (c1.k_record == c0.k_record) == already_sorted


def test_width_sorted_uniform_rows_equal_channel_order():
    """When every entry of a row has the same width the two orders coincide."""
    rng = np.random.default_rng(4)
    k = rng.standard_normal((64, 128)).astype(np.float16)
    k[0], k[1], k[32], k[33] = -4, 4, -4, 4          # every run of every channel spans 0..15
    v = rng.standard_normal((64, 128)).astype(np.float16)
    c0 = stream.encode_block(k, v, Config(bits=4, block=64, permute=0))
    c1 = stream.encode_block(k, v, Config(bits=4, block=64, permute=0, payload_order=1))
    d = unpack.decode_record("K", c0.k_record, 64, 128, 64, 32)
    assert np.all(d.w == 4)
    assert c1.k_record == c0.k_record


def test_width_sorted_stream_decodes_to_the_same_cache():
    k, v = kvsynth.structured_kv(300, 128, 64, 32, seed=8)
    a = stream.compress(k, v, Config(bits=3, block=64))
    b = stream.compress(k, v, Config(bits=3, block=64, payload_order=1))
    for x, y in zip(stream.decode_stream(a), stream.decode_stream(b)):
        assert np.array_equal(x, y)
    assert a.arena("K") != b.arena("K") and a.arena("V") == b.arena("V")
