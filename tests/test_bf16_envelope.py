"""The committed bf16 envelope of the end-to-end taps (CPU only).

tests/golden/bf16_envelope.json holds, per bf16 case of the GPU parity tests,
how far the float64 oracle moves when the values a bf16 layer must hold in
bf16 are rounded inside it (tests/bf16_envelope.py).  The GPU tests allow
that plus 2e-2 on LayerNorm(AV), z and the f2 branch.  Here:

* the file is what its generator computes, recomputed on the cases that run
  in seconds (the edge workloads and the whole zipf_bf16 batch), and it
  covers every case the GPU tests look up;
* the envelope is made of rounding only: with no rounding the same
  comparison gives zero, and rounding a single interface gives less;
* the check bites: plausible mistakes planted in the oracle move at least one
  end-to-end tap beyond envelope + 2e-2 on the zipf_bf16 workload at its
  real init.  (Mistakes in the bias indices barely move the layer at the
  workloads' N(0, 0.02) tables; the fp32 bucket-edge workload with
  unit-scale tables catches those: test_oracle_pins.py,
  test_bucket_edge_workload_detects_a_wrong_bucket.)
"""

import numpy as np
import pytest

from hstu_sequential_transducer_layer_amd import synth
from oracle import hstu_oracle as O

import bf16_envelope as E
from edge_workloads import edge_workload


def _edge_cases():
    return [(kind, fname, flags) for kind in ("bf16", "bf16_s1") for fname, flags in E.EDGE_FLAGS]


@pytest.mark.parametrize("kind,fname,flags", _edge_cases(), ids=lambda v: str(v))
def test_edge_envelopes_match_the_file(kind, fname, flags):
    env = E.envelope(edge_workload(kind, **flags))
    stored = E.load_envelopes()[E.edge_key(kind, fname)]
    for t in E.TAPS:
        np.testing.assert_allclose(env[t], stored[t], rtol=1e-6)


def test_zipf_envelope_matches_the_file():
    w, seqs = E.load_full_size_case("zipf_bf16")
    env = E.envelope(w.sub_batch(seqs))
    stored = E.load_envelopes()["zipf_bf16"]
    for t in E.TAPS:
        np.testing.assert_allclose(env[t], stored[t], rtol=1e-6)


def test_file_covers_every_case_the_gpu_tests_use():
    cases = E.load_envelopes()
    for key, name, n_layers, seqs in E.full_size_cases():
        assert key in cases, key
        assert cases[key]["sequences"] == seqs, key
        for t in E.TAPS:
            assert 0.0 < cases[key][t] < 0.5, (key, t)
    for kind, fname, _ in _edge_cases():
        assert E.edge_key(kind, fname) in cases


def test_envelope_is_rounding_only():
    w = edge_workload("bf16_s1")
    ex = E.exact_taps(w)
    # no rounding at all: the interface oracle is the oracle
    ident = lambda a: np.asarray(a, np.float64)
    real = O.round_to_bf16
    try:
        O.round_to_bf16 = ident
        none = E.bf16_interface_taps(w)
    finally:
        O.round_to_bf16 = real
    for t in E.TAPS:
        assert E.unit_err(none[t], ex[t]) < 1e-12, t
    # the full envelope exceeds what rounding the output alone gives
    full = E.envelope(w, exact=ex)
    out_only = E.unit_err(O.round_to_bf16(ex["branch"]), ex["branch"])
    assert full["branch"] > out_only
    assert full["ln_av"] > 1e-3


def _plant(monkeypatch, name):
    if name == "no_diagonal":
        monkeypatch.setattr(O, "attend_mask", lambda i, j, n: (np.asarray(j) < np.asarray(i)))
    elif name == "sigmoid_for_silu":
        real = O.silu
        monkeypatch.setattr(O, "silu", lambda z, *a: real(z) / np.where(np.asarray(z) == 0, 1.0, np.asarray(z)))
    elif name == "ln_without_centring":
        def ln(a, g, b, eps, *_):
            a = np.asarray(a, np.float64)
            var = (a ** 2).mean(axis=-1, keepdims=True)
            return a / np.sqrt(var + eps) * np.asarray(g, np.float64) + np.asarray(b, np.float64)
        monkeypatch.setattr(O, "layer_norm", ln)
    elif name == "split_u_v_swapped":
        real = O.project
        def proj(x, prm, cfg, **kw):
            u, v, q, k = real(x, prm, cfg, **kw)
            T, H, dv = v.shape
            return v.reshape(T, H * dv), u.reshape(T, H, dv), q, k
        monkeypatch.setattr(O, "project", proj)
    elif name == "keys_past_the_query":
        monkeypatch.setattr(O, "attend_mask", lambda i, j, n: np.ones(np.broadcast(i, j).shape, bool)
                            & (np.asarray(j) <= np.asarray(i) + 1))
    elif name == "candidates_see_each_other":
        monkeypatch.setattr(O, "attend_mask", lambda i, j, n: np.asarray(j) <= np.asarray(i))
    else:
        raise KeyError(name)


@pytest.mark.parametrize("name", ["no_diagonal", "sigmoid_for_silu", "ln_without_centring",
                                  "split_u_v_swapped", "keys_past_the_query"])
def test_planted_mistake_exceeds_the_envelope(name, monkeypatch):
    w, seqs = E.load_full_size_case("zipf_bf16")
    sub = w.sub_batch(seqs[:8])
    ex = E.exact_taps(sub)
    env = E.load_envelopes()["zipf_bf16"]
    _plant(monkeypatch, name)
    bad = E.exact_taps(sub)
    errs = {t: E.unit_err(bad[t], ex[t]) for t in E.TAPS}
    assert any(errs[t] > env[t] + E.MARGIN for t in E.TAPS), errs


def test_planted_candidate_mistake_exceeds_the_envelope(monkeypatch):
    w, seqs = E.load_full_size_case("ranking_cand")
    sub = w.sub_batch(seqs[:1])
    ex = E.exact_taps(sub)
    env = E.load_envelopes()["ranking_cand"]
    _plant(monkeypatch, "candidates_see_each_other")
    bad = E.exact_taps(sub)
    errs = {t: E.unit_err(bad[t], ex[t]) for t in E.TAPS}
    assert any(errs[t] > env[t] + E.MARGIN for t in E.TAPS), errs
