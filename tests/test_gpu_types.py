"""GPU parity of the token-type bias term ("HSTU: The First Exploration of the
Scaling Law", 7.1.4 Innovation 2: the bias depends on position difference,
time difference and the two tokens' types).  The oracle adds
type_table[h, type_i, type_j]; the kernel adds it through one extra MFMA step
per key half.  Tolerances: fp32 1e-4 element-relative on av (stage) and y;
bf16 2e-2 of the output's rms on y.  The tables are drawn at 10x the init
scale so that a wrong type pair moves y well past the tolerance; at that scale
bf16 rounding of the pointwise weights alone moves individual av elements by
up to ~5% of max(|av|, rms(av)) (checked on the CPU by rounding the oracle's
weights), so for bf16 the av stage error is printed, not asserted."""

import dataclasses

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import _lib, layer, synth
from oracle import hstu_oracle as O

from edge_workloads import edge_workload
from gpu_helpers import check, say

pytestmark = pytest.mark.gpu


def _typed(w, nt, seed=0, scale=1.0):
    """w with an nt-type table per layer and random token types."""
    rng = np.random.default_rng(100 + seed)
    w = synth.with_dims(w, num_types=nt)
    H = w.dims.num_heads
    cast = (lambda a: synth.round_bf16(a).astype(np.float32)) if w.dims.dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    w.layers = [dict(p, type_table=cast(rng.normal(0.0, 0.02 * scale, (H, nt, nt)))) for p in w.layers]
    w.token_types = rng.integers(0, nt, w.T).astype(np.uint8)
    return w


def _gpu_layer(w, token_types=None):
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    ty = dev["token_types"] if token_types is None else token_types
    prm = dev["layers"][0]
    acts = _lib.proj_fwd(desc, dev["x"], prm)
    _lib.attn_fwd(desc, dev["offsets"], dev["timestamps"], dev["num_candidates"], prm, acts, token_types=ty)
    y = _lib.layer_fwd(desc, dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"], prm,
                       token_types=ty)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    T, H, dv = w.T, w.dims.num_heads, w.dims.dv
    st = f(acts["av_stats"])
    av = (f(acts["av"]).reshape(T, H, dv) + st[:, :, :1]).reshape(T, H * dv)
    return {"y": f(y), "av": av, "q": f(acts["q"]).transpose(1, 0, 2), "k": f(acts["k"]).transpose(1, 0, 2),
            "v": f(acts["v"]).transpose(1, 0, 2)}


def _compare(w, seqs=None):
    g = _gpu_layer(w)
    sub = w if seqs is None else w.sub_batch(seqs)
    rows = np.arange(w.T) if seqs is None else \
        np.concatenate([np.arange(w.offsets[s], w.offsets[s + 1]) for s in seqs])
    prm = sub.layers[0]
    dt = w.dims.dtype
    av_iso = O.attention(g["q"][rows], g["k"][rows], g["v"][rows], sub.offsets, sub.timestamps,
                         sub.num_candidates, prm, w.dims, token_types=sub.token_types)
    if dt == "fp32":
        check("av (stage, typed)", g["av"][rows], av_iso, dt)
    else:
        from gpu_helpers import err_fp32
        say(f"  av (stage, typed; info): {err_fp32(g['av'][rows], av_iso):.3e}")
    ref = O.layer_forward(sub.x, sub.offsets, sub.timestamps, sub.num_candidates, prm, w.dims,
                          token_types=sub.token_types)
    check("y (end to end, typed)", g["y"][rows], ref["y"], dt, unit=True)
    return g


@pytest.mark.parametrize("kind", ["fp32", "bf16", "bf16_s1"])
@pytest.mark.parametrize("nt", [2, 3, 16])
def test_typed_edge_workload(kind, nt):
    # table 10x the init scale so a wrong type pair moves y well past the tolerance
    w = _typed(edge_workload(kind), nt, seed=nt, scale=10.0)
    say(f"typed edge {kind}, {nt} types: lengths {w.lengths().tolist()}")
    _compare(w)


def test_typed_ranking_full_size():
    w = synth.make_workload("ranking_cand", n_layers=1,
                            dims=dataclasses.replace(synth.WORKLOADS["ranking_cand"].dims, num_types=2))
    L = w.lengths()
    seqs = [int(np.argmin(L)), int(np.argmax(L))]
    say(f"typed ranking_cand (interleaved content/action, candidates content), oracle on {seqs}")
    _compare(w, seqs)


def test_zero_type_table_is_bitwise_untyped():
    w = _typed(edge_workload("bf16", seed=3), 3)
    w.layers[0]["type_table"] = np.zeros_like(w.layers[0]["type_table"])
    say("zero type table vs untyped layer")
    typed = _gpu_layer(w)["y"]
    plain = synth.with_dims(w, num_types=0)
    dev = layer.to_device(plain)
    prm = {k: v for k, v in dev["layers"][0].items() if k != "type_table"}
    y = _lib.layer_fwd(_lib.make_desc(plain.dims), dev["x"], dev["offsets"], dev["timestamps"],
                       dev["num_candidates"], prm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(typed, y.float().cpu().numpy().astype(np.float64))


def test_typed_cached_candidates():
    """The cached candidate pass with types: candidates' own types for the
    queries and the self term, the history's for the cached keys."""
    base = edge_workload("fp32", seed=8)
    w = _typed(base, 3, seed=8, scale=10.0)
    dev = layer.to_device(w)
    hrows, hoff, crows, coff, m = layer.split_history(w.offsets, w.num_candidates)
    D = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ty = dev["token_types"]
    ranker = layer.CachedRanker(w.dims, dev["layers"])
    ranker.encode_history(dev["x"][D(hrows)].contiguous(), D(hoff), dev["timestamps"][D(hrows)].contiguous(),
                          hist_types=ty[D(hrows)].contiguous())
    out = np.zeros((len(crows), w.dims.d_model))
    m_d = D(m.astype(np.int32))
    for rows, off in layer.candidate_microbatches(coff, 30):
        r = D(crows[rows])
        y = ranker.score(dev["x"][r].contiguous(), D(off), dev["timestamps"][r].contiguous(), m_d,
                         cand_types=ty[r].contiguous())
        out[rows] = y.float().cpu().numpy()
    ref = O.layer_forward(w.x, w.offsets, w.timestamps, w.num_candidates, w.layers[0], w.dims,
                          token_types=w.token_types)["y"][crows]
    say("typed cached candidates (fp32, 3 types)")
    check("cached typed candidates vs oracle", out, ref, "fp32")


def test_missing_token_types_rejected():
    w = _typed(edge_workload("bf16"), 2)
    dev = layer.to_device(w)
    with pytest.raises(_lib.HstuError) as e:
        _lib.layer_fwd(_lib.make_desc(w.dims), dev["x"], dev["offsets"], dev["timestamps"],
                       dev["num_candidates"], dev["layers"][0])
    assert e.value.status == _lib.HSTU_ERR_INVALID_ARG
