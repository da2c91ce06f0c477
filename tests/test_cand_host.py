"""Host index arithmetic of the cached candidate pass (no GPU): splitting a
packed batch into history and candidate rows, and candidate micro-batches."""

import numpy as np

from hstu_sequential_transducer_layer_amd import layer


def test_split_history_partitions_rows():
    off = np.array([0, 3, 3, 10, 12, 13], np.int64)
    nc = np.array([1, 0, 5, 2, 9], np.int32)          # last count exceeds L: clamped to 1
    hrows, hoff, crows, coff, m = layer.split_history(off, nc)
    np.testing.assert_array_equal(m, [1, 0, 5, 2, 1])
    np.testing.assert_array_equal(hoff, [0, 2, 2, 4, 4, 4])
    np.testing.assert_array_equal(coff, [0, 1, 1, 6, 8, 9])
    np.testing.assert_array_equal(np.sort(np.r_[hrows, crows]), np.arange(13))
    np.testing.assert_array_equal(hrows, [0, 1, 3, 4])
    np.testing.assert_array_equal(crows, [2, 5, 6, 7, 8, 9, 10, 11, 12])
    h2, hoff2, c2, coff2, m2 = layer.split_history(off, None)
    np.testing.assert_array_equal(h2, np.arange(13))
    assert len(c2) == 0 and m2.sum() == 0


def test_microbatches_cover_each_candidate_once_in_order():
    rng = np.random.default_rng(1)
    m = rng.integers(0, 40, 12)
    m[3] = 0
    coff = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    seen = []
    per_seq = [[] for _ in m]
    for rows, o in layer.candidate_microbatches(coff, 7):
        assert len(o) == len(m) + 1 and o[0] == 0 and o[-1] == len(rows)
        assert np.all(np.diff(o) <= 7)
        for b in range(len(m)):
            r = rows[o[b]:o[b + 1]]
            assert np.all((r >= coff[b]) & (r < coff[b + 1]))
            per_seq[b].extend(r.tolist())
        seen.extend(rows.tolist())
    assert sorted(seen) == list(range(int(coff[-1])))
    for b in range(len(m)):
        assert per_seq[b] == list(range(coff[b], coff[b + 1]))
    assert list(layer.candidate_microbatches(np.zeros(4, np.int64), 5)) == []
