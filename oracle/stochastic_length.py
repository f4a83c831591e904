"""Stochastic Length (SL) rule, host reference (test infrastructure only).

Source: ltzyclt.github.io, section 5.1 -- a user's sequence is kept or cut with
probability N^alpha / n^2; chenhuiyu.github.io, section "另外三块拼图", item 2 -- with
alpha = 1.6 a length-4096 history is mostly reduced to 776, the full context is kept
only sometimes, and the kept part is not simply the most recent tokens.

Reading used here (the pages do not spell out every step):
  * L = floor(N^(alpha/2)) is the subsample length (4096^0.8 = 776.05 -> 776).
  * A user of length n is kept whole when n <= L, or when u < N^alpha / n^2 for its
    uniform draw u (the probability reaches 1 exactly when n <= N^(alpha/2)).
  * Otherwise L distinct positions are kept, chosen uniformly: the L positions with the
    smallest random 32-bit priorities (ties to the lower position), in time order.
  * Kept tokens keep their timestamps and are re-indexed 0..L-1 inside the sequence.
The random numbers (u per user, one priority per raw token) are inputs, so any
implementation fed the same draws must select exactly the same tokens.
"""

from __future__ import annotations

import math

import numpy as np


def subsample_length(n_target: int, alpha: float) -> int:
    """L = floor(N^(alpha/2)) in float64."""
    return int(math.floor(math.pow(float(n_target), alpha / 2.0)))


def keep_threshold(n: int, n_target: int, alpha: float) -> float:
    """N^alpha / n^2 in float64 (may exceed 1)."""
    return math.pow(float(n_target), alpha) / (float(n) * float(n))


def keep_probability(n: int, n_target: int, alpha: float) -> float:
    return min(1.0, keep_threshold(n, n_target, alpha))


def select(offsets, u_keep, keys, n_target: int = 4096, alpha: float = 1.6):
    """Apply SL to a raw jagged batch.

    Returns (kept_tokens int64 [T_new] -- raw global token indices in order,
             new_offsets int32 [B+1]).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.uint32)
    L = subsample_length(n_target, alpha)
    kept = []
    lens = []
    for b in range(offsets.shape[0] - 1):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        n = s1 - s0
        if n <= L or float(u_keep[b]) < keep_threshold(n, n_target, alpha):
            idx = np.arange(s0, s1, dtype=np.int64)
        else:
            # smallest L (priority, position) pairs; lexsort sorts by the last key first
            pos = np.arange(n, dtype=np.int64)
            order = np.lexsort((pos, keys[s0:s1].astype(np.int64)))
            idx = s0 + np.sort(order[:L])
        kept.append(idx)
        lens.append(idx.size)
    kept = np.concatenate(kept) if kept else np.zeros(0, dtype=np.int64)
    new_off = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=new_off[1:])
    return kept, new_off.astype(np.int32)
