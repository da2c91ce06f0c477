"""Integer indexing of the oracle: time buckets, position buckets, row -> (b, i),
mask.  Checked against hand-derived fixtures and second formulations."""

import os

import numpy as np
import pytest

from oracle import brute
from oracle import hstu_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _loop_log2(v: int) -> int:
    k = 0
    while (1 << (k + 1)) <= v:
        k += 1
    return k


def _loop_bucket(dt: int, nb: int, s: int) -> int:
    # third formulation: k by a counting loop, sub-bits by repeated halving
    if dt <= 0:
        return 0
    k = _loop_log2(dt)
    rem = dt - (1 << k)              # bits below the leading one
    sub = 0
    for bit in range(s):
        pos = k - 1 - bit
        sub = 2 * sub + (((rem >> pos) & 1) if pos >= 0 else 0)
    return min(nb - 1, 1 + k * (1 << s) + sub)


def test_golden_time_buckets():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "time_buckets.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 20
    for dt, s, nb, want in rows:
        dt, s, nb, want = int(dt), int(s), int(nb), int(want)
        got = int(O.time_bucket(np.array([dt], np.int64), nb, s)[0])
        assert got == want, (dt, s, nb, got, want)
        assert brute.time_bucket(dt, nb, s) == want
        assert _loop_bucket(dt, nb, s) == want


@pytest.mark.parametrize("s,nb", [(0, 64), (1, 128), (2, 256), (0, 16), (1, 40)])
def test_time_bucket_exhaustive_small(s, nb):
    dt = np.arange(-16, 1 << 16, dtype=np.int64)
    got = O.time_bucket(dt, nb, s)
    want = np.array([_loop_bucket(int(v), nb, s) for v in dt[::7]])
    np.testing.assert_array_equal(got[::7], want)
    # every value, against the bit_length formulation
    want_all = np.array([brute.time_bucket(int(v), nb, s) for v in dt])
    np.testing.assert_array_equal(got, want_all)


@pytest.mark.parametrize("s,nb", [(0, 64), (1, 128)])
def test_time_bucket_random_int64(s, nb):
    rng = np.random.default_rng(7)
    v = rng.integers(-(1 << 63), (1 << 63) - 1, size=20000, dtype=np.int64, endpoint=True)
    e = rng.integers(0, 63, size=20000)
    w = (rng.integers(1, 1 << 62, size=20000, dtype=np.int64) >> e)  # all magnitudes
    vals = np.concatenate([v, w, -w, np.array([1 << 62, (1 << 63) - 1, -(1 << 63)], np.int64)])
    got = O.time_bucket(vals, nb, s)
    want = np.array([brute.time_bucket(int(x), nb, s) for x in vals])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("s", [0, 1, 2])
def test_time_bucket_closed_forms(s):
    nb = 64 << s
    k = np.arange(0, 63, dtype=np.int64)
    np.testing.assert_array_equal(O.time_bucket(np.int64(1) << k, nb, s), 1 + (k << s))
    assert O.time_bucket(np.array([0, -1, -(1 << 63)], np.int64), nb, s).tolist() == [0, 0, 0]
    # monotone non-decreasing in dt, max over all int64 = 1 + 62*2^s + (2^s - 1)
    dt = np.sort(np.random.default_rng(s).integers(-1000, (1 << 63) - 1, 50000, dtype=np.int64))
    b = O.time_bucket(dt, nb, s)
    assert np.all(np.diff(b) >= 0)
    top = int(O.time_bucket(np.array([(1 << 63) - 1], np.int64), nb, s)[0])
    assert top == min(nb - 1, 1 + (62 << s) + (1 << s) - 1)


def test_pos_bucket_exhaustive():
    for P in (1, 3, 129, 257):
        R = (P - 1) // 2
        dp = np.arange(-3000, 3001, dtype=np.int64)
        got = O.pos_bucket(dp, P)
        want = np.array([brute.pos_bucket(int(v), P) for v in dp])
        np.testing.assert_array_equal(got, want)
        assert got.min() == 0 and got.max() == P - 1
        assert int(O.pos_bucket(np.array([0]), P)[0]) == R


def test_token_index_with_empty_sequences():
    rng = np.random.default_rng(3)
    for _ in range(50):
        B = int(rng.integers(1, 12))
        lens = rng.integers(0, 6, size=B)
        lens[rng.random(B) < 0.3] = 0
        off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(off[-1])
        b, i = O.token_index(off, T)
        # linear scan
        for t in range(T):
            bb = [q for q in range(B) if off[q] <= t < off[q + 1]]
            assert len(bb) == 1
            assert b[t] == bb[0] and i[t] == t - off[bb[0]]


def test_mask_truth_table():
    # history of 3, 2 candidates (local 3, 4): candidates see 0..2 and themselves
    n_hist, L = 3, 5
    M = O.attend_mask(np.arange(L)[:, None], np.arange(L)[None, :], n_hist).astype(int)
    want = np.array([[1, 0, 0, 0, 0],
                     [1, 1, 0, 0, 0],
                     [1, 1, 1, 0, 0],
                     [1, 1, 1, 1, 0],
                     [1, 1, 1, 0, 1]])
    np.testing.assert_array_equal(M, want)


def test_index_dump_matches_scalar():
    from hstu_sequential_transducer_layer_amd import synth
    w = synth.make_workload("small_fp32", lengths=[5, 0, 7, 1], candidates=[2, 0, 3, 0])
    cfg = w.dims
    T = w.T
    pairs = np.array([(a, c) for a in range(T) for c in range(T)], np.int64)
    got = O.index_dump(w.offsets, w.timestamps, w.num_candidates, pairs, cfg)
    for n, (qr, kr) in enumerate(pairs):
        bq = [b for b in range(w.B) if w.offsets[b] <= qr < w.offsets[b + 1]][0]
        bk = [b for b in range(w.B) if w.offsets[b] <= kr < w.offsets[b + 1]][0]
        if bq != bk:
            assert got["b"][n] == -1
            continue
        i, j = qr - w.offsets[bq], kr - w.offsets[bq]
        L = w.offsets[bq + 1] - w.offsets[bq]
        nh = L - w.num_candidates[bq]
        assert got["i"][n] == i and got["j"][n] == j
        assert got["bp"][n] == brute.pos_bucket(min(i, nh) - min(j, nh), cfg.pos_buckets)
        assert got["bt"][n] == brute.time_bucket(int(w.timestamps[qr]) - int(w.timestamps[kr]),
                                                 cfg.time_buckets, cfg.time_sub_bits)
        assert got["mask"][n] == int(j <= i and (j < nh or j == i))
