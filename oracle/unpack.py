"""Record bytes -> quantised integers (oracle decoder).

A second implementation of the record layout described in ``record``:
vectorised 64-bit window reads here, against per-run big-integer assembly
there, so a shared misreading of the bit order would have to be made twice.
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


def decode_record(kind: str, buf: bytes, n: int, D: int, block: int, run: int, hb: int = 1) -> Decoded:
    """Decode one record; hb is the header entry size (1 byte up to b = 4, 2 above)."""
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
    words = np.frombuffer(buf[p0:p0 + 4 * nwords], dtype="<u4").astype(np.uint64)
    words = np.concatenate([words, np.zeros(1, np.uint64)])       # window guard
    start = np.concatenate([[0], np.cumsum(w.ravel())[:-1]]).reshape(nr, D)
    i = np.arange(run)
    bitpos = i[None, None, :] * w[:, :, None]                          # [nr, D, R]
    widx = start[:, :, None] + (bitpos >> 5)
    window = words[widx] | (words[np.minimum(widx + 1, nwords)] << np.uint64(32))
    mask = (np.uint64(1) << w[:, :, None].astype(np.uint64)) - np.uint64(1)
    u = ((window >> (bitpos & 31).astype(np.uint64)) & mask).astype(np.int64)
    q_runs = u + m[:, :, None]                                          # [nr, D, R]
    q = q_runs.transpose(0, 2, 1).reshape(nr * run, D)[:n]
    size = p0 + (4 * nwords + 15) // 16 * 16
    if kind == "V":
        sc, ze = sc[:n], ze[:n]
    return Decoded(sc, ze, w, m, q, size)
