"""Pins of the stochastic-length oracle (oracle/sl.py; page "HSTU: The First
Exploration of the Scaling Law", 7.1.5 Stochastic Length), CPU only."""

import math

import numpy as np
import pytest

from oracle import sl


def test_alpha2_never_truncates():
    # every sequence is at most N long, and the threshold N^(2/2) = N
    rng = np.random.default_rng(0)
    lens = rng.integers(0, 4097, 50)
    off = np.concatenate([[0], np.cumsum(lens)])
    u = np.zeros(50)                       # the most eager draw
    keys = rng.integers(0, 1 << 32, off[-1], dtype=np.uint64).astype(np.uint32)
    new_off, rows = sl.sl_sample(off, u, keys, 4096, 2.0)
    np.testing.assert_array_equal(new_off, off)
    np.testing.assert_array_equal(rows, np.arange(off[-1]))


def test_thresholds_closed_form():
    thr, k, na = sl.sl_thresholds(4096, 1.6)
    assert k == 776 and abs(thr - 2 ** 9.6) < 1e-9 and abs(na - 2 ** 19.2) < 1e-6
    # keep-whole probability of a full-length sequence: N^alpha / N^2 = N^-0.4
    assert abs(na / 4096.0 ** 2 - 4096 ** -0.4) < 1e-15
    assert sl.truncates(4096, 0.0, 4096, 1.6)
    assert not sl.truncates(4096, 1.0 - 4096 ** -0.4 + 1e-9, 4096, 1.6)
    assert not sl.truncates(776, 0.0, 4096, 1.6)          # at or below the threshold
    assert sl.truncates(777, 0.0, 4096, 1.6)


def test_truncation_rate_matches_probability():
    n, N, a = 3000, 4096, 1.6
    p = 1.0 - N ** a / n ** 2
    u = np.random.default_rng(1).random(200000)
    rate = np.mean([sl.truncates(n, x, N, a) for x in u[:20000]])
    assert abs(rate - p) < 0.015


def test_subset_is_the_k_smallest_keys_in_order():
    rng = np.random.default_rng(2)
    lens = [5000, 10, 0, 900]
    off = np.concatenate([[0], np.cumsum(lens)])
    keys = rng.integers(0, 50, off[-1]).astype(np.uint32)      # many ties
    u = np.array([0.0, 0.0, 0.0, 0.999])
    new_off, rows = sl.sl_sample(off, u, keys, 4096, 1.6)
    assert new_off.tolist() == [0, 776, 786, 786, 1686]
    got = rows[:776]
    assert np.all(np.diff(got) > 0)                            # order kept
    # second formulation: a threshold key and a tie count, by brute counting
    kk = keys[:5000].astype(np.int64)
    kth = np.sort(kk)[775]
    below = int(np.sum(kk < kth))
    eq = np.nonzero(kk == kth)[0][:776 - below]
    want = np.sort(np.concatenate([np.nonzero(kk < kth)[0], eq]))
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(rows[776:786], np.arange(5000, 5010))
    np.testing.assert_array_equal(rows[786:], np.arange(5010, 5910))


def test_each_token_equally_likely():
    rng = np.random.default_rng(3)
    n, trials = 1000, 400
    counts = np.zeros(n)
    off = np.array([0, n])
    for _ in range(trials):
        keys = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        _, rows = sl.sl_sample(off, np.array([0.0]), keys, 4096, 1.6)
        counts[rows] += 1
    # each position kept with probability 776/1000; binomial sd ~ 8.3 over 400 trials
    assert abs(counts.mean() - 0.776 * trials) < 1e-9
    assert np.abs(counts - 0.776 * trials).max() < 6 * math.sqrt(trials * 0.776 * 0.224)
