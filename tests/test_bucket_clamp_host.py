"""Host check of the attention kernel's small-range time bucket (dt in
(-2^24, 2^24)): the bucket read from the float bits of dt, clamped to
[0, nb - 1] by one float median between two bounds built from bits, must equal
the oracle's log-bucket of dt (page "HSTU: The First Exploration of the Scaling
Law", 7.1.4 Innovation 2: log-bucketed time differences; page "4.4 Scaling
Recommendation Models", "Generative Recommenders and HSTU", the time bias).

The formula below restates the kernel's arithmetic in float32 / int32 on the
host; the bounds are the smallest floats whose bits give bucket 0 and bucket
nb - 1 (the upper one capped at 2^24).  Not a GPU test: it checks the
construction of the bounds for every sub-bucket count the library accepts."""

import numpy as np
import pytest

from oracle import hstu_oracle as O


def _first_bits(b: int, s: int) -> int:
    """int32 bits of the smallest float whose bucket (by the float-bits rule) is b."""
    return (b - 1 + (127 << s)) << (23 - s)


def _bucket_med3(dt: np.ndarray, nb: int, s: int) -> np.ndarray:
    lo = np.array([_first_bits(0, s)], dtype=np.int32).view(np.float32)[0]
    cap = int(np.array([16777216.0], dtype=np.float32).view(np.int32)[0])
    hi = np.array([min(_first_bits(nb - 1, s), cap)], dtype=np.int32).view(np.float32)[0]
    f = dt.astype(np.float32)
    fc = np.minimum(np.maximum(f, lo), hi)          # median of (f, lo, hi) with lo < hi
    bits = fc.view(np.int32).astype(np.int64)
    return (bits >> (23 - s)) + 1 - (127 << s)


@pytest.mark.parametrize("s", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("nb", [1, 2, 3, 5, 17, 64, 128, 129, 1000])
def test_med3_bucket_equals_oracle(s, nb):
    rng = np.random.default_rng(1000 * s + nb)
    dt = np.concatenate([np.arange(-300, 70000), rng.integers(-(1 << 24) + 1, 1 << 24, 200000),
                         np.array([(1 << 24) - 1, -(1 << 24) + 1, 0, 1, -1])]).astype(np.int64)
    want = O.time_bucket(dt, nb, s)
    got = _bucket_med3(dt, nb, s)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (dt[bad[:5]], got[bad[:5]], want[bad[:5]])
