"""Exact compression-ratio accounting (oracle).

The pages report PackKV's "memory reduction rate" relative to quantisation
baselines (abstract; TL;DR) without defining it.  Reading adopted: report
the compression ratio CR = fp16 bytes / compressed bytes, three ways, plus
the same ratio for plain b-bit quantisation with the same fp16 parameters:

* ideal    - payload bits (each run at R * w) + 8 header bits per run
             (16 for b > 4, where an entry takes two bytes)
             + parameter bits (K: 32 per channel per block; V: 32 per token);
* physical - the record bytes as stored, 16-byte padding included;
* full     - physical plus the one-byte-per-token permutation table.

plain quantisation = T * D * b bits + the same parameter bits.
"""

from __future__ import annotations

import numpy as np

from .perm import block_permutation
from .quant import quantize_k_block, quantize_v_tokens
from .record import run_widths
from .stream import StreamCache
from .unpack import decode_record


def ratios(cache: StreamCache, which: str) -> dict:
    cfg = cache.cfg
    D, R, b = cfg.head_dim, cfg.run, cfg.bits
    raw_bits = 16 * cache.n_tokens * D
    ideal = 0
    params = 0
    arena = cache.arena(which)
    off = cache.offsets(which)
    for j in range(len(cache.blocks)):
        n = cache.block_tokens(j)
        d = decode_record(which, arena[off[j]:off[j + 1]], n, D, cfg.block, R, cfg.header_bytes,
                          cfg.payload_order if which == "K" else 0)
        par = 32 * D if which == "K" else 32 * n
        ideal += R * int(d.w.sum()) + 8 * cfg.header_bytes * d.w.size + par
        params += par
    phys = 8 * len(arena)
    full = phys + 8 * cache.n_tokens
    plain = cache.n_tokens * D * b + params
    return {
        "cr_ideal": raw_bits / ideal,
        "cr_phys": raw_bits / phys,
        "cr_full": raw_bits / full,
        "cr_plain_quant": raw_bits / plain,
        "ideal_bits": ideal,
        "phys_bytes": len(arena),
    }


def closed_form_full_width(which: str, bits: int, block: int, run: int, D: int) -> float:
    """CR when every run needs the full b bits: 16 / (b + 8h/R + 32/B) for K,
    16 / (b + 8h/R + 32/D) for V (per-value bit cost of payload, header,
    params; h = 1 header byte per run up to b = 4, 2 above)."""
    per = block if which == "K" else D
    h = 1 if bits <= 4 else 2
    return 16.0 / (bits + 8.0 * h / run + 32.0 / per)


def run_length_bits(k16: np.ndarray, v16: np.ndarray, bits: int, block: int, permute: int, run: int):
    """Ideal bits of the K and of the V records of one stream if the packing
    run were ``run`` slots instead of the format's 32 (a study of the pages'
    open choice of run length; nothing is stored in this form).

    Every block is quantised as the format does, ordered by the permutation
    rule with groups of ``run`` tokens (and its identity fallback judged at
    that run length), and counted like ``ratios``' ideal figure: ``run * w``
    payload bits and 8 (b > 4: 16) header bits per (run, channel), plus the parameters
    (K: 32 bits per channel per block, V: 32 per token).
    """
    n_tok, D = k16.shape
    kb = vb = 0
    for j0 in range(0, n_tok, block):
        k, v = k16[j0:j0 + block], v16[j0:j0 + block]
        n = k.shape[0]
        qk = quantize_k_block(k, bits)[0]
        qv = quantize_v_tokens(v, bits)[0]
        perm = block_permutation(qk, qv, run, permute)
        wk, _ = run_widths(qk[perm], run)
        wv, _ = run_widths(qv[perm], run)
        hbits = 8 if bits <= 4 else 16
        kb += run * int(wk.sum()) + hbits * wk.size + 32 * D
        vb += run * int(wv.sum()) + hbits * wv.size + 32 * n
    return kb, vb


def run_length_study(streams, bits: int, block: int, permute: int, runs=(16, 32, 64)) -> dict:
    """CR (ideal) of K and V over ``streams`` [(k16, v16), ...] for each run length."""
    out = {}
    for r in runs:
        kb = vb = raw = 0
        for k16, v16 in streams:
            a, b = run_length_bits(k16, v16, bits, block, permute, r)
            kb, vb, raw = kb + a, vb + b, raw + 16 * k16.size
        out[r] = (raw / kb, raw / vb)
    return out

