"""Channel-direction bit-packing and the block record layout (oracle encoder).

PackKV's second step packs the quantised integers losslessly "in channel
direction" (Fig. 2 caption, step (2)); Fig. 4's caption calls the context
(token) axis the channel direction, i.e. a packed unit is the values of one
channel over consecutive tokens.  Readings adopted:

* a run is R = 32 consecutive slots of one channel inside a block; run r of
  a block holding n tokens covers slots r*R .. min(r*R + R, n) - 1;
* each (run, channel) is stored at its own minimal width
  w = bit_length(max - min) (0 <= w <= b) relative to its minimum m, as
  u = q - m; the header entry of the run is the byte (w << 4) | m for
  b <= 4 and the little-endian u16 (w << 8) | m for b = 5..8 (hb = 1 or 2
  bytes per entry);
* the R slots of a run fill exactly w little-endian 32-bit words; slots
  past n hold u = 0.  The bits are laid out for a decoder that works on
  "container" words: with c-bit containers (c = 4 for b <= 4, c = 8 for
  b = 5..8), slot i belongs to container word k = i // (32/c), field
  j = i % (32/c), and bit p (p < w) of its u is stored in run word W at
  bit c*j + Q, where
    - if w divides c (g = c/w containers share a word): W = k // g,
      Q = w*(k % g) + p;
    - otherwise, if k < w: W = k, Q = p (the container's low w bits);
    - otherwise: W = p, Q = k (the spare high bits of every word).
  The pages fix no bit order; they only ask that the packed layout suit
  the GPU that consumes it (explainer page, "PackKV as a staged dataflow").
  With this order a decoder rebuilds each container word (every slot's u in
  its own c-bit field) from the run words with a few shifts and masks.

Record of one block (all integers little-endian, every section contiguous):

    K:  scale[D] fp16 | zero[D] fp16 | hdr[nr][D] (hb B each) | 0-pad to 16 B |
        payload | 0-pad to 16 B
    V:  scale[B] fp16 | zero[B] fp16 (slot order; slots >= n hold 0) |
        hdr[nr][D] (hb B each) | 0-pad to 16 B | payload | 0-pad to 16 B

payload = for r in 0..nr-1, for c in row_order(r): the w words of run (r, c),
where row_order is 0, 1, ..., D-1 (payload order 0) or, for a K record in
payload order 1, the channels sorted by decreasing width w[r, c], equal
widths by increasing channel.  The header stays in channel order either way,
so the record's size does not depend on the order.
"""

from __future__ import annotations

import numpy as np

from .fp16bits import f16_bits


def _pad16(n: int) -> int:
    return (n + 15) & ~15


def run_widths(q_slots: np.ndarray, run: int):
    """Per-(run, channel) minimum m and width w of slot-ordered ints [n, D].

    w = bit_length(max - min): the fewest bits that hold every q - min.
    Returns (w, m), each int64 [nr, D].
    """
    q = np.asarray(q_slots, dtype=np.int64)
    n, D = q.shape
    nr = -(-n // run)
    w = np.zeros((nr, D), np.int64)
    m = np.zeros((nr, D), np.int64)
    for r in range(nr):
        seg = q[r * run:min(n, (r + 1) * run)]
        lo = seg.min(axis=0)
        hi = seg.max(axis=0)
        m[r] = lo
        w[r] = [int(x).bit_length() for x in (hi - lo)]
    return w, m


def bit_place(i: int, p: int, w: int, cont: int):
    """(word, bit) of bit p of slot i's u in a run stored at width w, for
    cont-bit containers (the layout rule in the module docstring)."""
    k, j = divmod(i, 32 // cont)
    if cont % w == 0:
        g = cont // w
        word, q = k // g, w * (k % g) + p
    elif k < w:
        word, q = k, p
    else:
        word, q = p, k
    return word, cont * j + q


def row_order(w_row, order: int = 0) -> list:
    """Channels of one run row in payload order: 0 by channel; 1 by
    decreasing width, equal widths by increasing channel."""
    D = len(w_row)
    if order == 0:
        return list(range(D))
    assert order == 1
    return sorted(range(D), key=lambda c: (-int(w_row[c]), c))


def pack_payload(q_slots: np.ndarray, w: np.ndarray, m: np.ndarray, run: int, cont: int = 4,
                 order: int = 0) -> bytes:
    """The payload words of all (run, channel) pairs, run-major, each row in
    row_order; cont = container bits (4 for b <= 4, 8 for b = 5..8)."""
    assert run == 32 and cont in (4, 8)
    q = np.asarray(q_slots, dtype=np.int64)
    n, D = q.shape
    out = bytearray()
    for r in range(w.shape[0]):
        for c in row_order(w[r], order):
            wr = int(w[r, c])
            if wr == 0:
                continue
            assert wr <= cont
            bits = 0
            for i in range(run):
                t = r * run + i
                u = int(q[t, c] - m[r, c]) if t < n else 0
                assert 0 <= u < (1 << wr)
                for p in range(wr):
                    word, pos = bit_place(i, p, wr, cont)
                    bits |= ((u >> p) & 1) << (32 * word + pos)
            out += bits.to_bytes(4 * wr, "little")
    return bytes(out)


def header_bytes(w: np.ndarray, m: np.ndarray, hb: int = 1) -> bytes:
    """The header entries [nr][D], hb bytes each (1: w << 4 | m, 2: w << 8 | m)."""
    w, m = np.asarray(w, np.int64), np.asarray(m, np.int64)
    if hb == 1:
        assert np.all(w <= 4) and np.all(m <= 15) and np.all(m >= 0)
        return ((w << 4) | m).astype(np.uint8).tobytes()
    assert hb == 2 and np.all(w <= 8) and np.all(m <= 255) and np.all(m >= 0)
    return ((w << 8) | m).astype("<u2").tobytes()


def build_record(kind: str, q_slots, scale, zero, block: int, run: int, hb: int = 1,
                 order: int = 0) -> bytes:
    """Assemble the record bytes of one block.

    kind 'K': scale/zero have D entries (per channel).
    kind 'V': scale/zero have n entries in slot order, padded to B with 0.
    order: payload order (1 is defined for K records only).
    """
    assert order == 0 or kind == "K"
    q = np.asarray(q_slots, dtype=np.int64)
    n, D = q.shape
    if kind == "K":
        assert len(scale) == D and len(zero) == D
        sc, ze = np.asarray(scale), np.asarray(zero)
    elif kind == "V":
        assert len(scale) == n and len(zero) == n
        sc = np.zeros(block)
        ze = np.zeros(block)
        sc[:n] = scale
        ze[:n] = zero
    else:
        raise ValueError(kind)
    w, m = run_widths(q, run)
    head = f16_bits(sc).astype("<u2").tobytes() + f16_bits(ze).astype("<u2").tobytes()
    head += header_bytes(w, m, hb)
    head += bytes(_pad16(len(head)) - len(head))
    body = pack_payload(q, w, m, run, 4 * hb, order)
    body += bytes(_pad16(len(body)) - len(body))
    return head + body


def record_size(kind: str, w: np.ndarray, D: int, block: int, hb: int = 1) -> int:
    """Closed-form record size in bytes from the run widths."""
    nr = w.shape[0]
    params = 4 * (D if kind == "K" else block)
    return _pad16(params + hb * nr * D) + _pad16(4 * int(w.sum()))
