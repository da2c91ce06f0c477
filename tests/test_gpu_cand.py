"""GPU parity of the cached candidate pass (hstu_cand_fwd, M-FALCON).

A candidate's output row depends only on its own row and the history of its
sequence ("HSTU: The First Exploration of the Scaling Law", 7.1.5 M-FALCON;
"4.4 Scaling Recommendation Models", Efficiency tricks), so scoring the
candidates in micro-batches against a K/V cache of the history must give the
candidate rows of the full forward over history + all candidates.  The
reference is the float64 oracle's full forward (tolerances as in
test_gpu_parity: fp32 1e-4 element-relative, bf16 2e-2 of the output's rms);
the GPU full forward's candidate rows are compared at the same bar.
"""

import dataclasses

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import _lib, layer, synth
from oracle import hstu_oracle as O

from edge_workloads import edge_workload
from gpu_helpers import check, say

pytestmark = pytest.mark.gpu


def _dev(a, dt=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dt is None else t.to(dt)


def _cached_scores(w, per_seq, n_layers=1):
    """Candidate rows (full batch order) scored in micro-batches of `per_seq`
    candidates per sequence against the history cache."""
    dev = layer.to_device(w)
    hrows, hoff, crows, coff, m = layer.split_history(w.offsets, w.num_candidates)
    x = dev["x"]
    ts = dev["timestamps"]
    ranker = layer.CachedRanker(w.dims, dev["layers"][:n_layers])
    ranker.encode_history(x[_dev(hrows)].contiguous(), _dev(hoff), ts[_dev(hrows)].contiguous())
    m_dev = _dev(m.astype(np.int32))
    out = torch.zeros(len(crows), w.dims.d_model, dtype=x.dtype, device="cuda")
    nmb = 0
    for rows, off in layer.candidate_microbatches(coff, per_seq):
        r = _dev(crows[rows])
        y = ranker.score(x[r].contiguous(), _dev(off), ts[r].contiguous(), m_dev)
        out[_dev(rows)] = y
        nmb += 1
    torch.cuda.synchronize()
    say(f"  {nmb} micro-batch(es) of <= {per_seq} candidates per sequence, "
        f"{len(hrows)} history rows cached")
    return out.float().cpu().numpy().astype(np.float64), crows


def _full_gpu(w, n_layers=1):
    dev = layer.to_device(w)
    stack = layer.HSTUStack(w.dims, dev["layers"][:n_layers])
    y = stack.forward(dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"])
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check_against_full(w, per_seq, n_layers=1, seqs=None):
    got, crows = _cached_scores(w, per_seq, n_layers)
    full = _full_gpu(w, n_layers)[crows]
    dt = w.dims.dtype
    if seqs is None:
        ref = O.stack_forward(w.x, w.offsets, w.timestamps, w.num_candidates, w.layers[:n_layers],
                              w.dims)[crows]
        keep = np.arange(len(crows))
    else:
        sub = w.sub_batch(seqs)
        _, _, sub_crows, _, _ = layer.split_history(sub.offsets, sub.num_candidates)
        ref = O.stack_forward(sub.x, sub.offsets, sub.timestamps, sub.num_candidates,
                              sub.layers[:n_layers], w.dims)[sub_crows]
        # the same candidates' positions in the full batch's candidate order
        _, _, _, coff, _ = layer.split_history(w.offsets, w.num_candidates)
        keep = np.concatenate([np.arange(coff[s], coff[s + 1]) for s in seqs])
    check("cached candidates vs oracle", got[keep], ref, dt, unit=True)
    check("full forward candidates vs oracle", full[keep], ref, dt, unit=True)
    return got


@pytest.mark.parametrize("kind", ["fp32", "bf16", "bf16_s1"])
@pytest.mark.parametrize("flags", [{}, {"norm_len": 77}, {"input_norm": False, "residual": False}])
def test_cached_edge_workload(kind, flags):
    w = edge_workload(kind, **flags)
    say(f"cached candidates, edge {kind} {flags}: lengths {w.lengths().tolist()}, "
        f"candidates {w.num_candidates.tolist()}")
    _check_against_full(w, per_seq=50)


def test_cached_microbatch_size_is_bitwise_irrelevant():
    """Each row's arithmetic is the same whatever micro-batch it sits in: one
    candidate at a time, 7 at a time and all at once give the same bits."""
    w = edge_workload("bf16", seed=2)
    say("cached candidates, micro-batch sizes 1 / 7 / all")
    a, _ = _cached_scores(w, 1)
    b, _ = _cached_scores(w, 7)
    c, _ = _cached_scores(w, 1000)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_cached_ranking_full_size():
    w = synth.make_workload("ranking_cand", n_layers=1)
    L = w.lengths()
    seqs = [int(np.argmin(L)), int(np.argmax(L))]
    say(f"cached candidates, ranking_cand (bf16, B=16, T={w.T}, 512 candidates each) in "
        f"micro-batches of 128, oracle on sequences {seqs}")
    _check_against_full(w, per_seq=128, seqs=seqs)


def test_cached_two_layer_stack_fp32():
    dims = dataclasses.replace(synth.WORKLOADS["small_fp32"].dims, pos_buckets=9, time_buckets=16)
    lens, cands = [40, 1, 100, 0, 77], [10, 1, 33, 0, 0]
    w = synth.make_workload("small_fp32", seed=9, n_layers=2, lengths=[a - b for a, b in zip(lens, cands)],
                            candidates=cands, dims=dims, random_ln=True)
    say(f"cached candidates through 2 layers (fp32), lengths {w.lengths().tolist()}")
    _check_against_full(w, per_seq=8, n_layers=2)


def test_cached_long_history_fp32():
    """Histories split into several chunks (2100 keys: 33 key blocks, the
    8-chunk cap; 300 keys: 2 chunks; 5 keys: 1), summed by the reduction."""
    dims = dataclasses.replace(synth.WORKLOADS["small_fp32"].dims, pos_buckets=129, time_buckets=64)
    w = synth.make_workload("small_fp32", seed=12, lengths=[2100, 300, 5, 0], candidates=[3, 130, 2, 4],
                            dims=dims, random_ln=True)
    say(f"cached candidates, long histories (fp32), lengths {w.lengths().tolist()}")
    _check_against_full(w, per_seq=64)


def test_cached_without_history():
    """Sequences made only of candidates (an empty cache, Th = 0): each
    candidate sees itself alone."""
    dims = dataclasses.replace(synth.WORKLOADS["small_fp32"].dims, pos_buckets=9, time_buckets=16)
    w = synth.make_workload("small_fp32", seed=4, lengths=[0, 0, 0], candidates=[5, 0, 3], dims=dims)
    say("cached candidates with no history rows at all")
    _check_against_full(w, per_seq=2)


def test_graph_replay_matches_eager():
    """The layer pass, the history projection and cached micro-batches captured
    into one HIP graph: every replay (with eager work and synchronisations in
    between) gives the eager bits."""
    w = edge_workload("bf16", seed=6)
    dev = layer.to_device(w)
    prm = dev["layers"][0]
    desc = _lib.make_desc(w.dims)
    wts, tab = _lib.make_weights(prm), _lib.make_tables(prm)
    hrows, hoff, crows, coff, m = layer.split_history(w.offsets, w.num_candidates)
    x, ts = dev["x"], dev["timestamps"]
    xh, hts, hoff_d = x[_dev(hrows)].contiguous(), ts[_dev(hrows)].contiguous(), _dev(hoff)
    acts = _lib.alloc_activations(desc, len(hrows), "cuda")
    ws_p = _lib.alloc_workspace(_lib.proj_workspace_size(desc, len(hrows)), "cuda")
    ws_l = _lib.alloc_workspace(_lib.workspace_size(desc, w.T, w.B), "cuda")
    mbs = list(layer.candidate_microbatches(coff, 40))
    cin = [(x[_dev(crows[r])].contiguous(), _dev(o), ts[_dev(crows[r])].contiguous()) for r, o in mbs]
    ws_c = _lib.alloc_workspace(max(_lib.cand_workspace_size(desc, len(r), len(hrows), w.B)
                                    for r, _ in mbs), "cuda")
    m_d = _dev(m.astype(np.int32))
    y_l = torch.empty_like(x)
    y_c = [torch.empty_like(c[0]) for c in cin]

    def work():
        _lib.layer_fwd(desc, x, dev["offsets"], ts, dev["num_candidates"], prm, out=y_l,
                       workspace=ws_l, weights=wts, tables=tab)
        _lib.proj_fwd(desc, xh, prm, acts, workspace=ws_p, weights=wts)
        for (xc, oc, tc), yo in zip(cin, y_c):
            _lib.cand_fwd(desc, xc, oc, tc, m_d, hoff_d, hts, acts["k"], acts["v"], prm, out=yo,
                          workspace=ws_c, weights=wts, tables=tab)

    def snap():
        return [t.float().cpu().numpy() for t in [y_l] + y_c]

    work()
    torch.cuda.synchronize()
    ref = snap()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    say(f"graph of 1 layer pass + history projection + {len(mbs)} cached micro-batches")
    for rep in range(3):
        for t in [y_l] + y_c:
            t.fill_(float("nan"))
        _lib.layer_fwd(desc, x, dev["offsets"], ts, None, prm)     # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(snap(), ref):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}")


def test_cached_pass_requires_shared_positions():
    w = edge_workload("bf16", cand_shared_pos=False)
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    d = w.dims.d_model
    x = torch.zeros(4, d, dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 4], dtype=torch.int64, device="cuda")
    hk = torch.zeros(w.dims.num_heads, 8, w.dims.dqk, dtype=torch.bfloat16, device="cuda")
    hv = torch.zeros(w.dims.num_heads, 8, w.dims.dv, dtype=torch.bfloat16, device="cuda")
    ts = torch.zeros(4, dtype=torch.int64, device="cuda")
    hts = torch.zeros(8, dtype=torch.int64, device="cuda")
    hoff = torch.tensor([0, 8], dtype=torch.int64, device="cuda")
    m = torch.tensor([4], dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.HstuError) as e:
        _lib.cand_fwd(desc, x, off, ts, m, hoff, hts, hk, hv, dev["layers"][0])
    assert e.value.status == _lib.HSTU_ERR_UNSUPPORTED
