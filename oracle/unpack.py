"""Record bytes -> quantised integers (oracle decoder).

A second implementation of the record layout described in ``record``: the
encoder there places every bit of every slot; here each run's container
words (one c-bit field per slot) are rebuilt from its w words with shifts
and masks, so a shared misreading of the bit order would have to be made
twice:

* w divides c (g = c/w containers per word): container k is word k // g
  shifted right by w*(k % g), masked to w bits per field;
* otherwise container k < w is word k masked to its low w bits per field,
  and container k >= w collects bit k of every field of word p as its bit p.

In payload order 1 (K records) a row's entries are stored by decreasing
width, equal widths by channel; the offsets below walk the rows in that
order, worked out here from the header without the encoder's helper.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .fp16bits import f16_from_bits


@dataclasses.dataclass
class Decoded:
    scale: np.ndarray     # fp64: [D] for K, [n] (slot order) for V
    zero: np.ndarray      # same shape as scale
    w: np.ndarray         # [nr, D] run widths
    m: np.ndarray         # [nr, D] run minima
    q: np.ndarray         # [n, D] int64 quantised values, slot order
    size: int             # bytes consumed (the record length)


def _entry_starts(w: np.ndarray, order: int) -> np.ndarray:
    """Word offset of every (run, channel) entry in the payload [nr, D]."""
    nr, D = w.shape
    start = np.zeros((nr, D), np.int64)
    pos = 0
    for r in range(nr):
        if order == 0:
            seq = range(D)
        else:
            # widest first; a stable sort on the negated width keeps equal
            # widths in channel order
            seq = np.argsort(-w[r], kind="stable")
        for c in seq:
            start[r, c] = pos
            pos += int(w[r, c])
    return start


def decode_record(kind: str, buf: bytes, n: int, D: int, block: int, run: int, hb: int = 1,
                  order: int = 0) -> Decoded:
    """Decode one record; hb is the header entry size (1 byte up to b = 4, 2
    above); order is the payload order (1 only for K records)."""
    assert order == 0 or kind == "K"
    nr = -(-n // run)
    b = np.frombuffer(buf, dtype=np.uint8)
    n_par = D if kind == "K" else block
    sc = f16_from_bits(b[0:2 * n_par].view("<u2"))
    ze = f16_from_bits(b[2 * n_par:4 * n_par].view("<u2"))
    if hb == 1:
        hdr = b[4 * n_par:4 * n_par + nr * D].astype(np.int64).reshape(nr, D)
        w, m = hdr >> 4, hdr & 15
    else:
        hdr = b[4 * n_par:4 * n_par + 2 * nr * D].view("<u2").astype(np.int64).reshape(nr, D)
        w, m = hdr >> 8, hdr & 255
    p0 = (4 * n_par + hb * nr * D + 15) // 16 * 16
    nwords = int(w.sum())
    words = np.frombuffer(buf[p0:p0 + 4 * nwords], dtype="<u4").astype(np.int64)
    start = _entry_starts(w, order)
    cb = 4 * hb                                   # container bits
    per = 32 // cb                                # slots per container word
    rep1 = sum(1 << (cb * j) for j in range(per))  # bit 0 of every field
    assert run == 32
    u = np.zeros((nr * D, run), np.int64)
    wf, sf = w.ravel(), start.ravel()
    for wr in range(1, cb + 1):                   # all runs of one width at once
        idx = np.nonzero(wf == wr)[0]
        if idx.size == 0:
            continue
        P = words[sf[idx][:, None] + np.arange(wr)[None, :]]           # [runs, wr]
        low = ((1 << wr) - 1) * rep1
        C = np.zeros((idx.size, cb), np.int64)                          # container words
        for k in range(cb):
            if cb % wr == 0:
                g = cb // wr
                C[:, k] = (P[:, k // g] >> (wr * (k % g))) & low
            elif k < wr:
                C[:, k] = P[:, k] & low
            else:
                for pb in range(wr):
                    C[:, k] |= ((P[:, pb] >> k) & rep1) << pb
        fields = (C[:, :, None] >> (cb * np.arange(per))[None, None, :]) & ((1 << cb) - 1)
        u[idx] = fields.reshape(idx.size, run)                         # slot k*per + j
    q_runs = u.reshape(nr, D, run) + m[:, :, None]                      # [nr, D, R]
    q = q_runs.transpose(0, 2, 1).reshape(nr * run, D)[:n]
    size = p0 + (4 * nwords + 15) // 16 * 16
    if kind == "V":
        sc, ze = sc[:n], ze[:n]
    return Decoded(sc, ze, w, m, q, size)
