"""Token permutation inside a block (oracle).

PackKV reorders the quantised KV vectors so that the following bit-packing
step sees narrower value ranges (Fig. 2 caption, step (1)); this is allowed
because attention does not depend on the order of the (K, V) pairs as long
as each K stays bound to its V (TL;DR; the explainer page's "Permutation
invariance, visually").  The pages do not give the grouping rule.  Reading
adopted, a greedy seeded L1 grouping over the concatenated K and V ints:

    remaining = tokens 0 .. n-1, ascending
    while remaining is not empty:
        seed = the smallest index in remaining
        d[t] = sum_c |qK[t,c] - qK[seed,c]| + sum_c |qV[t,c] - qV[seed,c]|
               for every t in remaining
        take the min(R, |remaining|) tokens with the smallest key (d[t], t)
        (the seed has d = 0 and comes first), append them in key order,
        and drop them from remaining

Slot i of the block then holds token perm[i].  If this order does not make
the block's packed payload strictly smaller than the identity order (summed
over K and V, every run counted at its full R slots), the identity is used.
Everything here is integer and deterministic.

A second, cheaper rule (this build's, offered as a variant of the same
rearrangement step) sorts the tokens by one integer key:

    s[t] = sum_c qK[t,c] + sum_c qV[t,c]
    order = tokens ascending by (s[t], t)

with the same identity fallback.  It costs one pass over the ints and one
sort instead of a distance pass per run, and it groups tokens whose
quantised vectors have clearly different totals (a clustered block whose
centroids differ) but not tokens that merely share a total.

Modes: 0 identity, 1 greedy grouping, 2 sort key.
"""

from __future__ import annotations

from typing import List

import numpy as np


def greedy_order(qk: np.ndarray, qv: np.ndarray, run: int) -> List[int]:
    """The greedy grouping order (before the identity fallback)."""
    n = qk.shape[0]
    feats = np.concatenate([np.asarray(qk, np.int64), np.asarray(qv, np.int64)], axis=1)
    remaining = list(range(n))
    order: List[int] = []
    while remaining:
        seed = remaining[0]
        rem = np.array(remaining)
        d = np.abs(feats[rem] - feats[seed]).sum(axis=1)
        keyed = sorted(zip(d.tolist(), remaining))
        take = [t for _, t in keyed[:run]]
        order.extend(take)
        taken = set(take)
        remaining = [t for t in remaining if t not in taken]
    return order


def sort_key_order(qk: np.ndarray, qv: np.ndarray) -> List[int]:
    """The sort-key order (before the identity fallback)."""
    total = np.asarray(qk, np.int64).sum(axis=1) + np.asarray(qv, np.int64).sum(axis=1)
    return sorted(range(qk.shape[0]), key=lambda t: (int(total[t]), t))


def payload_words(qk: np.ndarray, qv: np.ndarray, order, run: int) -> int:
    """Packed payload size in 32-bit words of K plus V under slot order ``order``.

    A run of R slots of one channel at width w takes exactly w words.
    """
    from .record import run_widths  # width rule lives with the record format
    wk, _ = run_widths(np.asarray(qk)[list(order)], run)
    wv, _ = run_widths(np.asarray(qv)[list(order)], run)
    return int(wk.sum() + wv.sum())


def block_permutation(qk: np.ndarray, qv: np.ndarray, run: int, permute: int = 1) -> np.ndarray:
    """Slot -> token index for one block: the mode's order if it makes the
    payload strictly smaller, else the identity (mode 0: always identity)."""
    n = qk.shape[0]
    ident = list(range(n))
    mode = int(permute)
    if mode == 0 or n <= 1:
        return np.array(ident, dtype=np.int64)
    order = greedy_order(qk, qv, run) if mode == 1 else sort_key_order(qk, qv)
    if payload_words(qk, qv, order, run) < payload_words(qk, qv, ident, run):
        return np.array(order, dtype=np.int64)
    return np.array(ident, dtype=np.int64)
