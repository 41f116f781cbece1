"""Decode-time attention products over the decompressed cache (oracle).

Fig. 1's caption states the decode computation: each query is dotted with
every cached K vector, softmax turns the dots into weights, and the output is
the weight-scaled sum of the V vectors.  PackKV fuses decompression into the
two matrix-vector products (TL;DR; Fig. 2 caption); the fused kernel must
give the same numbers as decompress-then-multiply, which is what these plain
fp64 definitions compute.  Outputs are in slot order (the order of the packed
cache): attention does not depend on the order of the (K, V) pairs.

Reading adopted: the GEMVs return raw dot products; the softmax helper scales
them by 1/sqrt(D).
"""

from __future__ import annotations

import numpy as np


def qk(q: np.ndarray, k_hat: np.ndarray) -> np.ndarray:
    """scores[g, t] = sum_c q[g, c] * K_hat[t, c] (fp64).  q [G, D], K_hat [T, D]."""
    return np.asarray(q, np.float64) @ np.asarray(k_hat, np.float64).T


def softmax(scores: np.ndarray, head_dim: int) -> np.ndarray:
    """p[g, t] = exp(s/sqrt(D) - max) / sum over t (fp64)."""
    z = np.asarray(scores, np.float64) / np.sqrt(head_dim)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def pv(p: np.ndarray, v_hat: np.ndarray) -> np.ndarray:
    """out[g, c] = sum_t p[g, t] * V_hat[t, c] (fp64).  p [G, T], V_hat [T, D]."""
    return np.asarray(p, np.float64) @ np.asarray(v_hat, np.float64)


def rel_l2(y, ref) -> float:
    """||y - ref||_2 / ||ref||_2 in fp64."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / (den if den > 0 else 1.0))
