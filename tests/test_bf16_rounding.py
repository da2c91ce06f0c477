"""Where the bf16 attention tap's tolerance comes from (CPU only).

The attention kernel rounds every pointwise weight SiLU(S_ij) (times a
constant) to bf16 before the A.V product on the matrix cores.  On the edge
workloads of the GPU parity tests, that rounding alone, applied inside the
float64 oracle to its own weights with everything else exact, already moves
av by up to 2.7e-2 of max(|av|, rms(av)) per element: the attention sums
terms of both signs, so a small relative error per weight can be a larger one
on a small sum.  The GPU tolerance on that tap (gpu_helpers.BF16_AV_TOL)
is 1.5x the largest of these."""

import numpy as np

from oracle import hstu_oracle as O

from edge_workloads import edge_workload
from gpu_helpers import BF16_AV_TOL, err_fp32


def _weight_rounding_error(kind, flags, scale):
    w = edge_workload(kind, **flags)
    prm = w.layers[0]
    _, v, q, k = O.project(w.x, prm, w.dims)
    r = O.round_to_bf16
    q, k, v = r(q), r(k), r(v)
    exact = O.attention(q, k, v, w.offsets, w.timestamps, w.num_candidates, prm, w.dims)
    real = O.silu
    try:
        O.silu = lambda z, *a: r(real(z) * scale) / scale
        rounded = O.attention(q, k, v, w.offsets, w.timestamps, w.num_candidates, prm, w.dims)
    finally:
        O.silu = real
    return err_fp32(rounded, exact)


def test_weight_rounding_alone_bounds_the_av_tolerance():
    errs = []
    for kind in ("bf16", "bf16_s1"):
        for flags in ({}, {"norm_len": 77}, {"cand_shared_pos": False}, {"input_norm": False, "residual": False}):
            for scale in (1.0, -1.4426950408889634):   # plain weights, and weights times -log2(e)
                errs.append(_weight_rounding_error(kind, flags, scale))
    worst = max(errs)
    assert 2e-2 < worst <= BF16_AV_TOL / 1.5 + 1e-9, worst
