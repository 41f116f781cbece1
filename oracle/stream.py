"""One stream's packed cache: bulk compress, append, arena layout (oracle).

The abstract says PackKV works with a KV cache that keeps growing during
decoding.  Reading adopted: the cache is cut into blocks of B tokens; every
closed block is encoded once and never changes; the newest, possibly partial
block (the "open tail") is kept as raw fp16 and re-encoded in full after
every append, so appending tokens one at a time gives exactly the bytes that
compressing them all at once gives.

Per block the encoder runs the pages' three steps in order: quantise
(``quant``), reorder tokens (``perm``), pack (``record``).  A stream's
records sit back to back in its arena; ``offsets[j]`` is the byte offset of
block j's record and ``offsets[nb]`` the arena's used length.  ``perm[j][i]``
is the in-block token index held by slot i (0xFF for slots past n).
"""

from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

from .config import Config
from .quant import quantize_k_block, quantize_v_tokens, dequantize
from .perm import block_permutation
from .record import build_record
from .unpack import decode_record


@dataclasses.dataclass
class BlockCode:
    k_record: bytes
    v_record: bytes
    perm: np.ndarray          # [n] slot -> in-block token index
    qk_slots: np.ndarray      # [n, D] quantised K in slot order
    qv_slots: np.ndarray      # [n, D] quantised V in slot order


def encode_block(k16: np.ndarray, v16: np.ndarray, cfg: Config) -> BlockCode:
    """Quantise -> permute -> pack one block of n <= B tokens (token order in)."""
    n, D = k16.shape
    assert 1 <= n <= cfg.block and D == cfg.head_dim and v16.shape == k16.shape
    qk, sk, zk = quantize_k_block(k16, cfg.bits)
    qv, sv, zv = quantize_v_tokens(v16, cfg.bits)
    perm = block_permutation(qk, qv, cfg.run, cfg.permute)
    k_rec = build_record("K", qk[perm], sk, zk, cfg.block, cfg.run, cfg.header_bytes, cfg.payload_order)
    v_rec = build_record("V", qv[perm], sv[perm], zv[perm], cfg.block, cfg.run, cfg.header_bytes)
    return BlockCode(k_rec, v_rec, perm, qk[perm], qv[perm])


@dataclasses.dataclass
class StreamCache:
    cfg: Config
    blocks: List[BlockCode]
    n_tokens: int
    tail_k: np.ndarray        # [n_tail, D] fp16 raw tokens of the open block
    tail_v: np.ndarray

    # ---- arena view -------------------------------------------------------
    def arena(self, which: str) -> bytes:
        return b"".join(b.k_record if which == "K" else b.v_record for b in self.blocks)

    def offsets(self, which: str) -> np.ndarray:
        sizes = [len(b.k_record if which == "K" else b.v_record) for b in self.blocks]
        return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)

    def perm_table(self) -> np.ndarray:
        t = np.full((len(self.blocks), self.cfg.block), 0xFF, np.uint8)
        for j, b in enumerate(self.blocks):
            t[j, :len(b.perm)] = b.perm
        return t

    def block_tokens(self, j: int) -> int:
        return min(self.cfg.block, self.n_tokens - j * self.cfg.block)


def compress(k16: np.ndarray, v16: np.ndarray, cfg: Config) -> StreamCache:
    """Encode T tokens [T, D] at once: every block, the last one possibly partial."""
    T = k16.shape[0]
    B = cfg.block
    blocks = [encode_block(k16[j:j + B], v16[j:j + B], cfg) for j in range(0, T, B)]
    nfull = T // B
    return StreamCache(cfg, blocks, T, k16[nfull * B:].copy(), v16[nfull * B:].copy())


def append(cache: StreamCache, k_new: np.ndarray, v_new: np.ndarray) -> StreamCache:
    """Append tokens one at a time, re-encoding the open tail block each time."""
    cfg = cache.cfg
    for t in range(k_new.shape[0]):
        tk = np.concatenate([cache.tail_k, k_new[t:t + 1]])
        tv = np.concatenate([cache.tail_v, v_new[t:t + 1]])
        code = encode_block(tk, tv, cfg)
        if cache.tail_k.shape[0] == 0:
            cache.blocks.append(code)          # a new block opens
        else:
            cache.blocks[-1] = code            # the open block is rewritten
        cache.n_tokens += 1
        if tk.shape[0] == cfg.block:           # the block is full: close it
            tk = tk[:0]
            tv = tv[:0]
        cache.tail_k, cache.tail_v = tk, tv
    return cache


def decode_stream(cache: StreamCache):
    """K_hat, V_hat [T, D] (fp64, exact) in slot order, plus ints, from the arena."""
    cfg = cache.cfg
    D = cfg.head_dim
    k_hat, v_hat, qk, qv = [], [], [], []
    ka, va = cache.arena("K"), cache.arena("V")
    ko, vo = cache.offsets("K"), cache.offsets("V")
    for j in range(len(cache.blocks)):
        n = cache.block_tokens(j)
        dk = decode_record("K", ka[ko[j]:ko[j + 1]], n, D, cfg.block, cfg.run, cfg.header_bytes,
                           cfg.payload_order)
        dv = decode_record("V", va[vo[j]:vo[j + 1]], n, D, cfg.block, cfg.run, cfg.header_bytes)
        assert dk.size == ko[j + 1] - ko[j] and dv.size == vo[j + 1] - vo[j]
        k_hat.append(dequantize(dk.q, dk.scale, dk.zero, axis=0))
        v_hat.append(dequantize(dv.q, dv.scale, dv.zero, axis=1))
        qk.append(dk.q)
        qv.append(dv.q)
    return (np.concatenate(k_hat), np.concatenate(v_hat),
            np.concatenate(qk), np.concatenate(qv))


def token_order(cache: StreamCache, slot_values: np.ndarray) -> np.ndarray:
    """Reorder per-slot rows [T, ...] back to token order using the perms."""
    out = np.empty_like(slot_values)
    B = cache.cfg.block
    for j, b in enumerate(cache.blocks):
        out[j * B + b.perm] = slot_values[j * B: j * B + len(b.perm)]
    return out
