"""Pins of the backward-pass oracle (oracle/hstu_grad.py), CPU only: its
forward is the NumPy oracle's forward, and central finite differences in
float64 match its gradients with respect to x and every parameter."""

import dataclasses

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import synth
from oracle import hstu_grad as G
from oracle import hstu_oracle as O


def _case(seed, lens, cands, **kw):
    dims = synth.LayerDims(8, 2, 4, 4, pos_buckets=5, time_buckets=16, dtype="fp32", **kw)
    w = synth.make_workload("small_fp32", seed=seed, lengths=[L - m for L, m in zip(lens, cands)],
                            candidates=cands, dims=dims, random_ln=True)
    prm = {k: v.astype(np.float64) * (4.0 if k in ("w1", "w2", "pos_table", "time_table") else 1.0)
           for k, v in w.layers[0].items()}
    return w, prm, dims


CASES = [
    (1, [6, 3], [2, 0], {}),
    (2, [5, 1, 4], [0, 1, 4], {"cand_shared_pos": False}),
    (3, [7], [3], {"norm_len": 5, "residual": False}),
    (4, [4, 5], [1, 1], {"input_norm": False}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"case{c[0]}")
def test_torch_forward_is_the_oracle_forward(case):
    seed, lens, cands, kw = case
    w, prm, dims = _case(seed, lens, cands, **kw)
    ref = O.layer_forward(w.x, w.offsets, w.timestamps, w.num_candidates, prm, dims)["y"]
    got = G.forward(torch.from_numpy(w.x.astype(np.float64)), w.offsets, w.timestamps, w.num_candidates,
                    {k: torch.from_numpy(v) for k, v in prm.items()}, dims).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"case{c[0]}")
def test_gradients_match_finite_differences(case):
    seed, lens, cands, kw = case
    w, prm, dims = _case(seed, lens, cands, **kw)
    rng = np.random.default_rng(seed)
    dy = rng.normal(0, 1, (w.T, dims.d_model))
    g = G.layer_grads(w.x, w.offsets, w.timestamps, w.num_candidates, prm, dims, dy)

    def loss(xv, pv):
        y = O.layer_forward(xv, w.offsets, w.timestamps, w.num_candidates, pv, dims)["y"]
        return float(np.sum(y * dy))

    eps = 1e-6
    for name in ["x"] + list(G.PARAMS):
        base = w.x.astype(np.float64) if name == "x" else prm[name]
        flat_idx = rng.choice(base.size, size=min(6, base.size), replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, base.shape)
            hi, lo = base.copy(), base.copy()
            hi[idx] += eps
            lo[idx] -= eps
            if name == "x":
                fd = (loss(hi, prm) - loss(lo, prm)) / (2 * eps)
            else:
                fd = (loss(w.x, {**prm, name: hi}) - loss(w.x, {**prm, name: lo})) / (2 * eps)
            assert abs(g[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, g[name][idx], fd)


def test_unused_table_entries_get_zero_gradient():
    # a 1-token sequence only ever uses position bucket R and time bucket 0
    w, prm, dims = _case(5, [1], [0])
    g = G.layer_grads(w.x, w.offsets, w.timestamps, w.num_candidates, prm, dims,
                      np.ones((1, dims.d_model)))
    R = (dims.pos_buckets - 1) // 2
    assert np.count_nonzero(g["pos_table"][:, np.arange(dims.pos_buckets) != R]) == 0
    assert np.count_nonzero(g["time_table"][:, 1:]) == 0
    assert np.count_nonzero(g["pos_table"][:, R]) == dims.num_heads


def test_attention_stage_gradients_match_the_layer_chain():
    # the attention stage's gradients are the layer's, seen through dL/dAV:
    # pin by finite differences of sum(AV * dav) on a tiny case
    w, prm, dims = _case(7, [6, 4], [2, 1])
    rng = np.random.default_rng(7)
    _, v, q, k = O.project(w.x, prm, dims)
    dav = rng.normal(0, 1, (w.T, dims.num_heads * dims.dv))
    g = G.attention_grads(q, k, v, dav, w.offsets, w.timestamps, w.num_candidates, prm, dims)

    def loss(qq, kk, vv, pp):
        av = O.attention(qq, kk, vv, w.offsets, w.timestamps, w.num_candidates, pp, dims)
        return float(np.sum(av * dav))

    eps = 1e-6
    for name, base in (("q", q), ("k", k), ("v", v), ("pos_table", prm["pos_table"]),
                       ("time_table", prm["time_table"])):
        for fi in rng.choice(base.size, size=min(5, base.size), replace=False):
            idx = np.unravel_index(fi, base.shape)
            hi, lo = base.copy(), base.copy()
            hi[idx] += eps
            lo[idx] -= eps
            args = {"q": q, "k": k, "v": v, "pp": prm}
            if name in ("pos_table", "time_table"):
                fd = (loss(q, k, v, {**prm, name: hi}) - loss(q, k, v, {**prm, name: lo})) / (2 * eps)
            else:
                a_hi, a_lo = dict(args), dict(args)
                a_hi[name], a_lo[name] = hi, lo
                fd = (loss(a_hi["q"], a_hi["k"], a_hi["v"], prm) - loss(a_lo["q"], a_lo["k"], a_lo["v"], prm)) / (2 * eps)
            assert abs(g[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx)
