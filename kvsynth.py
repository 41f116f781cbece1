"""Seeded synthetic KV-cache workloads.

This module only draws random numbers.  It holds none of the method's
arithmetic (no quantisation, permutation, packing or attention), so that both
the CPU oracle (``oracle/``) and the HIP path (``decode_gemv_amd``) can take
their inputs from it without sharing any code with each other.

The PackKV pages measure on six real models and six benchmarks, neither of
which is available here; these seeded tensors stand in for them, with the
shapes and value laws of the workloads the method is evaluated on:

* K ~ N(0, 1) per element, with 8 "outlier" channels per KV head scaled by 10
  (the same channels for every token and every batch entry of that head);
* V ~ N(0, 1), or for the 2-bit workload a bimodal mixture sign + 0.3 N(0, 1)
  with sign uniform in {-1, +1};
* q ~ N(0, 1);
* everything is rounded to fp16 (round to nearest even).

Streams are indexed s = batch_index * kv_heads + kv_head.  Every stream has
its own generator, seeded from (seed, 2, s), so any subset of streams can be
regenerated on its own, bit for bit, without drawing the others.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "outlier_channels",
    "stream_kv",
    "stream_q",
    "append_kv",
    "structured_kv",
]

N_OUTLIERS = 8
OUTLIER_GAIN = 10.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value laws of one synthetic decode workload."""

    key: str
    batch: int
    kv_heads: int
    group: int          # query heads per KV head (G)
    tokens: int         # cached tokens per stream (T) before any append
    head_dim: int       # D
    bits: int           # quantisation bits (b)
    block: int          # token block (B)
    v_law: str          # "gauss", "bimodal" or "struct" (clustered K and V)
    append_steps: int = 0

    @property
    def streams(self) -> int:
        return self.batch * self.kv_heads

    def describe(self) -> str:
        return (f"{self.key}: batch {self.batch} x {self.kv_heads} kv-heads "
                f"(S={self.streams}), G={self.group}, T={self.tokens}, "
                f"D={self.head_dim}, {self.bits}-bit, block={self.block}, "
                f"V {self.v_law}"
                + (f", +{self.append_steps} appends" if self.append_steps else ""))


WORKLOADS: Dict[str, Workload] = {
    # one head, end-to-end K GEMV -> softmax -> V GEMV
    "single-head-4k": Workload("single-head-4k", 1, 1, 1, 4096, 128, 4, 64, "gauss"),
    # Llama-7B-like decode: 8 x 32 heads, 32K context
    "llama7b-32k": Workload("llama7b-32k", 8, 32, 1, 32768, 128, 4, 64, "gauss"),
    # GQA decode: 4 queries share each packed stream
    "gqa-128k": Workload("gqa-128k", 4, 8, 4, 131072, 128, 4, 128, "gauss"),
    # aggressive 2-bit with bimodal V
    "2bit-16k": Workload("2bit-16k", 16, 32, 1, 16384, 128, 2, 64, "bimodal"),
    # prefill 64K then 256 single-token appends
    "append-64k": Workload("append-64k", 32, 8, 1, 65536, 128, 3, 64, "gauss",
                           append_steps=256),
    # the llama7b-32k shape on clustered data (structured_kv), where the
    # token order inside a block decides the run widths
    "struct-32k": Workload("struct-32k", 8, 32, 1, 32768, 128, 4, 64, "struct"),
    # the llama7b shape at 8 bits (two-byte run headers, byte containers)
    "8bit-16k": Workload("8bit-16k", 8, 32, 1, 16384, 128, 8, 64, "gauss"),
}


def outlier_channels(head: int, head_dim: int = 128, seed: int = 0) -> np.ndarray:
    """The 8 distinct outlier channels of KV head ``head`` (sorted)."""
    rng = np.random.default_rng([seed, 1, head])
    return np.sort(rng.choice(head_dim, N_OUTLIERS, replace=False))


def _draw_v(rng: np.random.Generator, shape, law: str) -> np.ndarray:
    if law == "gauss":
        return rng.standard_normal(shape, dtype=np.float32)
    if law == "struct":                 # appended tokens of the clustered workload
        return rng.standard_normal(shape, dtype=np.float32)
    if law == "bimodal":
        sign = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=shape)
        return sign + np.float32(0.3) * rng.standard_normal(shape, dtype=np.float32)
    raise ValueError(f"unknown V law {law!r}")


def stream_kv(w: Workload, s: int, seed: int = 0,
              tokens: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 K and V of stream ``s``, each [tokens, D] (token order)."""
    T = w.tokens if tokens is None else tokens
    D = w.head_dim
    if w.v_law == "struct":
        return structured_kv(T, D, w.block, 32, seed=(seed << 20) + s)
    rng = np.random.default_rng([seed, 2, s])
    k = rng.standard_normal((T, D), dtype=np.float32)
    k[:, outlier_channels(s % w.kv_heads, D, seed)] *= np.float32(OUTLIER_GAIN)
    v = _draw_v(rng, (T, D), w.v_law)
    return k.astype(np.float16), v.astype(np.float16)


def stream_q(w: Workload, s: int, seed: int = 0, step: int = -1) -> np.ndarray:
    """fp16 queries of stream ``s``, [G, D]; ``step`` >= 0 gives a decode step's."""
    rng = np.random.default_rng([seed, 3, s, step + 1])
    return rng.standard_normal((w.group, w.head_dim), dtype=np.float32).astype(np.float16)


def append_kv(w: Workload, s: int, step: int, n_new: int = 1,
              seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 K and V of the tokens appended to stream ``s`` at decode ``step``."""
    D = w.head_dim
    rng = np.random.default_rng([seed, 4, s, step])
    k = rng.standard_normal((n_new, D), dtype=np.float32)
    k[:, outlier_channels(s % w.kv_heads, D, seed)] *= np.float32(OUTLIER_GAIN)
    v = _draw_v(rng, (n_new, D), w.v_law)
    return k.astype(np.float16), v.astype(np.float16)


def structured_kv(tokens: int, head_dim: int, block: int, run: int,
                  seed: int = 0, noise: float = 0.02,
                  shuffle: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """A clustered workload (not one of the measured ones).

    Inside each block of ``block`` tokens there are ``block // run`` centroid
    vectors; every token is one centroid plus small noise, and the tokens of a
    block are shuffled.  Grouping similar tokens (the permutation step) then
    gives runs whose values span only a few quantisation levels, so this
    workload exercises narrow per-run widths that the Gaussian ones almost
    never produce.
    """
    rng = np.random.default_rng([seed, 5, tokens, head_dim, block, run])
    n_cent = max(1, block // run)
    k = np.empty((tokens, head_dim), np.float32)
    v = np.empty((tokens, head_dim), np.float32)
    for j0 in range(0, tokens, block):
        n = min(block, tokens - j0)
        ck = rng.standard_normal((n_cent, head_dim), dtype=np.float32) * 2
        cv = rng.standard_normal((n_cent, head_dim), dtype=np.float32)
        lab = np.arange(n) % n_cent
        if shuffle:
            lab = rng.permutation(lab)
        k[j0:j0 + n] = ck[lab] + noise * rng.standard_normal((n, head_dim), dtype=np.float32)
        v[j0:j0 + n] = cv[lab] + noise * rng.standard_normal((n, head_dim), dtype=np.float32)
    return k.astype(np.float16), v.astype(np.float16)
