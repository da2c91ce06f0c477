"""Stochastic-length sampling and jagged re-packing, plain NumPy — the oracle.
TEST INFRASTRUCTURE ONLY.

Source: page "HSTU: The First Exploration of the Scaling Law", 7.1.5
Engineering Optimizations, "Stochastic Length".  A sequence of n tokens longer
than a threshold N^(alpha/2) is, with probability 1 - N^alpha / n^2, replaced
by a subsequence of floor(N^(alpha/2)) of its tokens; otherwise it is kept
whole.  N is the longest sequence length; alpha = 2 never truncates (every
n <= N then sits at or below the threshold).  The page's exponents are garbled
(N_{alpha/2}, N_alpha); they are read as powers of N.

Readings (where the page is silent):
  * the random draws are inputs: u[b], one uniform in [0, 1) per sequence
    (truncate when u[b] < 1 - N^alpha / n^2, compared in float64), and one
    uint32 key per token;
  * the subsequence is uniform over subsets (the page weights it by features
    that no input here has) and keeps the original order: the k tokens with
    the smallest (key, position) pairs, in position order;
  * the thresholds N^(alpha/2) and N^alpha are float64 powers (C pow).
"""

from __future__ import annotations

import math

import numpy as np


def sl_thresholds(n_max: int, alpha: float):
    """(threshold N^(alpha/2), kept length floor of it, N^alpha), float64."""
    thr = float(n_max) ** (alpha / 2.0)
    return thr, int(math.floor(thr)), float(n_max) ** alpha


def truncates(n: int, u: float, n_max: int, alpha: float) -> bool:
    thr, _, na = sl_thresholds(n_max, alpha)
    return n > thr and u < 1.0 - na / (float(n) * float(n))


def sl_sample(offsets, u, keys, n_max: int, alpha: float):
    """Returns (new offsets [B+1] int64, kept flat rows [T_out] int64)."""
    off = np.asarray(offsets, np.int64)
    keys = np.asarray(keys, np.uint32)
    B = len(off) - 1
    _, k, _ = sl_thresholds(n_max, alpha)
    new_off = [0]
    rows = []
    for b in range(B):
        s0, s1 = int(off[b]), int(off[b + 1])
        n = s1 - s0
        if truncates(n, float(u[b]), n_max, alpha):
            order = np.lexsort((np.arange(n), keys[s0:s1]))   # by key, then position
            keep = np.sort(order[:k])
            rows.append(s0 + keep)
            new_off.append(new_off[-1] + k)
        else:
            rows.append(np.arange(s0, s1))
            new_off.append(new_off[-1] + n)
    flat = np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)
    return np.asarray(new_off, np.int64), flat
