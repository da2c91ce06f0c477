"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances: fp32 layers max |y - ref| / max(|ref|, rms(ref)) <= 1e-4 at every
tap; bf16 layers max |y - ref| / rms(ref) <= 2e-2 on the unit-scale output y,
and max |y - ref| / max(|ref|, rms(ref)) <= 2e-2 on the intermediate taps
(u, v, q, k, z = LayerNorm(av) * u), which are stored in bf16, and <= 4e-2 on
av (gpu_helpers.BF16_AV_TOL: the bf16 rounding of the pointwise weights
alone reaches 2.7e-2 there).  Integer indexing is compared bitwise.  Full-size
workloads run on the GPU in full; the oracle recomputes a stated subset of
their sequences (sequences are independent, so those rows are exact
references), and the invariants below hold at any size.
"""

import dataclasses

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import _lib, layer, synth
from oracle import hstu_oracle as O

from edge_workloads import EDGE_DIMS, bucket_edge_workload, edge_workload as _edge_workload
from gpu_helpers import BF16_AV_TOL, check, gpu_taps, say
import bf16_envelope as E

pytestmark = pytest.mark.gpu


def _rows_of(w, seqs):
    return np.concatenate([np.arange(w.offsets[s], w.offsets[s + 1]) for s in seqs]) \
        if len(seqs) else np.zeros(0, np.int64)


def _compare_layer(w, seqs=None, layer_idx=0, env_key=None):
    """GPU layer on the whole batch vs oracle on sequences `seqs` (all if None).

    Stage by stage: u, v, q, k end to end; av against the oracle attention fed
    the GPU's own q, k, v; z and y against the oracle gate/projection fed the
    GPU's own av and u (each stage judged on its own arithmetic).

    End to end against the float64 oracle: y (unit scale), and the taps where
    an error cannot hide: LayerNorm(AV) (unit variance by construction), z,
    and the f2 branch (the layer run with the residual flag off, so that
    neither x nor the output's rounding at x's scale masks it).  fp32 layers
    hold these to the fp32 tolerance; bf16 layers to the committed bf16
    envelope of the case (tests/golden/bf16_envelope.json: how far the
    oracle itself moves when u, v, q, k, the pointwise weights, z and the
    output are rounded to bf16 inside it) plus 2e-2."""
    g = gpu_taps(w, layer_idx)
    np.testing.assert_array_equal(g["y"], g["y_layer"])   # same kernels, same bits
    sub = w if seqs is None else w.sub_batch(seqs)
    rows = np.arange(w.T) if seqs is None else _rows_of(w, seqs)
    prm = sub.layers[layer_idx]
    say(f"oracle on {sub.B} sequence(s), {sub.T} rows")
    ref = O.layer_forward(sub.x, sub.offsets, sub.timestamps, sub.num_candidates, prm, w.dims)
    dt = w.dims.dtype
    errs = {}
    for t in ("u", "v", "q", "k"):
        errs[t] = check(t, g[t][rows], ref[t], dt)
    av_iso = O.attention(g["q"][rows], g["k"][rows], g["v"][rows], sub.offsets, sub.timestamps,
                         sub.num_candidates, prm, w.dims)
    errs["av"] = check("av (stage)", g["av"][rows], av_iso, dt, tol=BF16_AV_TOL if dt == "bf16" else None)
    out_iso = O.gate_and_project(g["av"][rows], g["u"][rows], sub.x, prm, w.dims)
    errs["z"] = check("z (stage)", g["z"][rows], out_iso["z"], dt)
    errs["y_stage"] = check("y (stage)", g["y"][rows], out_iso["y"], dt, unit=True)
    errs["y"] = check("y (end to end)", g["y"][rows], ref["y"], dt, unit=True)
    # end to end on the taps that bite
    ln_gpu = O.layer_norm(g["av"][rows], prm["ln_av_g"], prm["ln_av_b"], w.dims.ln_eps)
    branch_ref = ref["y"] - np.asarray(sub.x, np.float64) if w.dims.residual else ref["y"]
    got = {"ln_av": ln_gpu, "z": g["z"][rows], "branch": g["branch"][rows]}
    want = {"ln_av": ref["ln_av"], "z": ref["z"], "branch": branch_ref}
    for t in E.TAPS:
        if dt == "bf16":
            assert env_key is not None, "a bf16 case needs its committed envelope"
            env = E.load_envelopes()[env_key][t]
            e = E.unit_err(got[t], want[t])
            say(f"  {t} end to end: err {e:.3e} (envelope {env:.3e} + {E.MARGIN:.0e})")
            assert np.all(np.isfinite(got[t])), t
            assert e <= env + E.MARGIN, f"{t}: end-to-end error {e:.3e} > envelope {env:.3e} + {E.MARGIN}"
            errs[t + "_e2e"] = e
        else:
            errs[t + "_e2e"] = check(f"{t} (end to end)", got[t], want[t], dt)
    return errs


# ---------------------------------------------------------------- workloads
def test_small_fp32_full():
    say("small_fp32 (fp32, B=4, L in [8,64], d=64, 2x32/32)")
    _compare_layer(synth.make_workload("small_fp32"))


def test_small_fp32_random_layernorm():
    say("small_fp32 with random LayerNorm affine")
    _compare_layer(synth.make_workload("small_fp32", random_ln=True, seed=3))


def test_zipf_bf16_full():
    w = synth.make_workload("zipf_bf16")
    say(f"zipf_bf16 (bf16, B=32, T={w.T}, d=256, 4x64/64), oracle on all rows")
    _compare_layer(w, env_key="zipf_bf16")


def test_ranking_candidates_full_size():
    w, seqs = E.load_full_size_case("ranking_cand")     # shortest and longest
    say(f"ranking_cand (bf16, B=16, T={w.T}, 512 candidates each), oracle on sequences {seqs}")
    _compare_layer(w, seqs, env_key="ranking_cand")


def test_stochastic_length_full_size():
    w, seqs = E.load_full_size_case("sl_train")         # one longest, two shortest
    say(f"sl_train (bf16, B=64, T={w.T}, 8x128/128), oracle on sequences {seqs}")
    _compare_layer(w, seqs, env_key="sl_train")


def test_len4k_full_size():
    w, seqs = E.load_full_size_case("len4k")
    say(f"len4k (bf16, B=16 x 4096, 8x128/128), oracle on sequence {seqs}")
    _compare_layer(w, seqs, env_key="len4k")


def test_stack8_first_layer_full_size():
    w, seqs = E.load_full_size_case("stack8_long_layer1")   # shortest and longest
    say(f"stack8_long layer 1 (bf16, B=8, T={w.T}, d=1024, 128 time buckets), oracle on {seqs} "
        f"({w.lengths()[seqs].tolist()} rows)")
    _compare_layer(w, seqs, env_key="stack8_long_layer1")


def test_stack8_full_stack():
    """8 layers on the GPU (full batch).

    Shortest sequence: every layer against the oracle layer applied to the
    GPU's own bf16 input of that layer (2e-2, unit scale), and the final
    output against the float64 oracle stack within the conditioning envelope
    (see below).  Longest sequence: every layer against the oracle layer on
    the GPU's own input of that layer, on 384 of its rows (its first 64, its
    last 128 and 192 drawn at random; the oracle projects every row, since
    each sampled row's attention needs all earlier keys)."""
    w = synth.make_workload("stack8_long")
    L = w.lengths()
    s, sl = int(np.argmin(L)), int(np.argmax(L))
    rows, rows_l = _rows_of(w, [s]), _rows_of(w, [sl])
    say(f"stack8_long, 8 layers (bf16, B=8, T={w.T}), oracle on sequence {s} "
        f"({L[s]} rows) and on sampled rows of sequence {sl} ({L[sl]} rows)")
    dev = layer.to_device(w)
    stack = layer.HSTUStack(w.dims, dev["layers"])
    y = stack.forward(dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"])
    # layer by layer through the same entry point
    desc = _lib.make_desc(w.dims)
    h = dev["x"]
    outs, outs_l = [], []
    for prm in dev["layers"]:
        h = _lib.layer_fwd(desc, h, dev["offsets"], dev["timestamps"], None, prm)
        hn = h.float().cpu().numpy().astype(np.float64)
        outs.append(hn[rows])
        outs_l.append(hn[rows_l])
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)[rows]
    np.testing.assert_array_equal(got, outs[-1])
    sub = w.sub_batch([s])
    prev = sub.x.astype(np.float64)
    for n, prm in enumerate(sub.layers):
        ref_n = O.layer_forward(prev, sub.offsets, sub.timestamps, None, prm, w.dims)["y"]
        check(f"layer {n + 1} (own input)", outs[n], ref_n, "bf16", unit=True)
        prev = outs[n]
    # the longest sequence, sampled rows of every layer
    sub_l = w.sub_batch([sl])
    n_l = int(L[sl])
    rng = np.random.default_rng(1)
    pick = np.unique(np.concatenate([np.arange(64), np.arange(n_l - 128, n_l),
                                     rng.choice(np.arange(64, n_l - 128), 192, replace=False)]))
    prev = sub_l.x.astype(np.float64)
    for n, prm in enumerate(sub_l.layers):
        ref_n = O.layer_forward(prev, sub_l.offsets, sub_l.timestamps, None, prm, w.dims, rows=pick)["y"]
        check(f"longest sequence, layer {n + 1} (own input, {len(pick)} rows)", outs_l[n][pick], ref_n,
              "bf16", unit=True)
        prev = outs_l[n]
    # End to end.  The 8-layer map is ill-conditioned at this init: rounding the
    # exact layers' outputs to bf16 (the stack's interface dtype) already moves
    # the float64 result by several percent.  The GPU must be no further from
    # the float64 stack than that exact bf16-interface stack is, plus the
    # single-layer tolerance.
    from gpu_helpers import BF16_TOL, err_bf16
    ref64 = O.stack_forward(sub.x, sub.offsets, sub.timestamps, None, sub.layers, w.dims)
    ref16 = O.stack_forward(sub.x, sub.offsets, sub.timestamps, None, sub.layers, w.dims,
                            io_dtype="bf16")
    envelope = err_bf16(ref16, ref64)
    e = err_bf16(got, ref64)
    say(f"  y after 8 layers vs float64 stack: {e:.3e}; exact bf16-interface stack vs "
        f"float64 stack: {envelope:.3e}; vs bf16-interface stack: {err_bf16(got, ref16):.3e}")
    assert np.all(np.isfinite(got))
    assert e <= envelope + BF16_TOL


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("kind", sorted(EDGE_DIMS))
@pytest.mark.parametrize("flags", [
    {},
    {"norm_len": 77},
    {"cand_shared_pos": False},
    {"input_norm": False, "residual": False},
])
def test_edge_cases(kind, flags):
    w = _edge_workload(kind, **flags)
    say(f"edge {kind} {flags}: lengths {w.lengths().tolist()}")
    key = E.edge_key(kind, E.flag_name_of(flags)) if w.dims.dtype == "bf16" else None
    _compare_layer(w, env_key=key)


@pytest.mark.parametrize("sub_bits,pos_buckets", [(0, 9), (1, 9), (2, 129)])
def test_time_bucket_edges_fp32(sub_bits, pos_buckets):
    """Every time-bucket edge (edge_workloads.bucket_edge_workload): fp32
    parity (1e-4) pins the bucket of every pair, since a pair moved to a
    neighbouring bucket changes y by far more (tests/test_oracle_pins.py,
    test_bucket_edge_workload_detects_a_wrong_bucket)."""
    w = bucket_edge_workload(sub_bits, pos_buckets)
    say(f"bucket edges s={sub_bits} P={pos_buckets}: {w.T} tokens")
    _compare_layer(w)


def test_shared_tables_stride0():
    w = _edge_workload("bf16", seed=4)
    dev = layer.to_device(w)
    prm = dict(dev["layers"][0])
    prm["pos_table"] = prm["pos_table"][0].contiguous()   # [P]  -> head stride 0
    prm["time_table"] = prm["time_table"][1].contiguous()
    desc = _lib.make_desc(w.dims)
    y = _lib.layer_fwd(desc, dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"], prm)
    torch.cuda.synchronize()
    p = dict(w.layers[0])
    p["pos_table"] = np.broadcast_to(w.layers[0]["pos_table"][0], w.layers[0]["pos_table"].shape)
    p["time_table"] = np.broadcast_to(w.layers[0]["time_table"][1], w.layers[0]["time_table"].shape)
    ref = O.layer_forward(w.x, w.offsets, w.timestamps, w.num_candidates, p, w.dims)["y"]
    check("y (shared tables)", y.float().cpu().numpy(), ref, "bf16", unit=True)


# ------------------------------------------------------------------ indices
@pytest.mark.parametrize("name", ["edge", "small_fp32", "ranking_cand", "stack8_long"])
def test_debug_indices_bitwise(name):
    if name == "edge":
        w = _edge_workload("bf16_s1")
        w.timestamps = w.timestamps.copy()
        w.timestamps[3] = -(1 << 62)        # wrapping differences
        w.timestamps[4] = (1 << 62) + 5
    else:
        w = synth.make_workload(name, n_layers=1)
    rng = np.random.default_rng(0)
    n = 200000
    qr = rng.integers(0, w.T, n)
    # mostly same-sequence keys near and far from the query
    b, _ = O.token_index(w.offsets, w.T)
    s0 = w.offsets[b[qr]]
    L = w.offsets[b[qr] + 1] - s0
    kr = np.where(rng.random(n) < 0.9, s0 + rng.integers(0, 1 << 30, n) % np.maximum(L, 1),
                  rng.integers(0, w.T, n))
    pairs = np.stack([qr, kr], 1).astype(np.int64)
    if w.T <= 400:
        g = np.stack(np.meshgrid(np.arange(w.T), np.arange(w.T), indexing="ij"), -1).reshape(-1, 2)
        pairs = np.concatenate([pairs, g]).astype(np.int64)
    say(f"debug indices {name}: {len(pairs)} pairs")
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    out = _lib.debug_indices(desc, dev["offsets"], dev["timestamps"], dev["num_candidates"],
                             torch.from_numpy(pairs).cuda()).cpu().numpy()
    ref = O.index_dump(w.offsets, w.timestamps, w.num_candidates, pairs, w.dims)
    for c, key in enumerate(["b", "i", "j", "bp", "bt", "mask"]):
        np.testing.assert_array_equal(out[:, c], ref[key], err_msg=key)


# --------------------------------------------------------------- invariants
def _layer_y(w, x=None, ts=None, nc="same"):
    dev = layer.to_device(w)
    if x is not None:
        dev["x"] = torch.from_numpy(x).to(dev["x"].dtype).cuda()
    if ts is not None:
        dev["timestamps"] = torch.from_numpy(ts).cuda()
    desc = _lib.make_desc(w.dims)
    y = _lib.layer_fwd(desc, dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"],
                       dev["layers"][0])
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def test_batch_equals_sequences_one_at_a_time_bitwise():
    w = synth.make_workload("ranking_cand", batch=5, lengths=[300, 0, 700, 1, 129],
                            candidates=[40, 0, 512, 1, 0])
    say(f"batch vs one-at-a-time, lengths {w.lengths().tolist()}")
    full = _layer_y(w)
    for b in range(w.B):
        sub = w.sub_batch([b])
        if sub.T == 0:
            continue
        np.testing.assert_array_equal(_layer_y(sub), full[w.offsets[b]:w.offsets[b + 1]])


def test_causality_bitwise():
    w = synth.make_workload("len4k", batch=2, n_layers=1)
    say("causality: perturb tokens after row 1000 of sequence 0")
    base = _layer_y(w)
    x2 = w.x.copy()
    x2[1001:4096] += 1.0
    ts2 = w.timestamps.copy()
    ts2[1001:4096] += 12345
    y2 = _layer_y(w, x=x2, ts=ts2)
    np.testing.assert_array_equal(y2[:1001], base[:1001])
    np.testing.assert_array_equal(y2[4096:], base[4096:])
    assert np.abs(y2[1001:4096] - base[1001:4096]).max() > 0


def test_candidates_independent_bitwise():
    w = synth.make_workload("ranking_cand", batch=2, n_layers=1)
    say("candidate independence: perturb one candidate")
    base = _layer_y(w)
    c = int(w.offsets[1]) - 100
    x2 = w.x.copy()
    x2[c] += 2.0
    y2 = _layer_y(w, x=x2)
    others = np.setdiff1d(np.arange(w.T), [c])
    np.testing.assert_array_equal(y2[others], base[others])


def test_zero_tables_remove_bias():
    w = synth.make_workload("zipf_bf16", batch=4)
    for key in ("pos_table", "time_table"):
        w.layers[0][key] = np.zeros_like(w.layers[0][key])
    say("zero tables: timestamps must not matter")
    a = _layer_y(w)
    b = _layer_y(w, ts=np.random.default_rng(0).permutation(w.timestamps))
    np.testing.assert_array_equal(a, b)


def test_deterministic_bitwise():
    w = synth.make_workload("sl_train", batch=8, n_layers=1)
    say("determinism: two runs")
    np.testing.assert_array_equal(_layer_y(w), _layer_y(w))


def test_reused_plan_is_bitwise_identical():
    """HSTU_REUSE_PLAN: a call that skips the attention plan gives the bits of a
    call that builds it, when an earlier call on the same workspace built the
    plan for the same metadata (here after an unrelated batch's plan was
    overwritten by this batch's)."""
    w = synth.make_workload("ranking_cand", batch=5, n_layers=2)
    other = synth.make_workload("ranking_cand", seed=3, batch=7, n_layers=1)
    dev, dev_o = layer.to_device(w), layer.to_device(other)
    desc = _lib.make_desc(w.dims)
    reuse = _lib.make_desc(w.dims, _lib.HSTU_REUSE_PLAN)
    T, B = w.T, w.B
    ws = _lib.alloc_workspace(max(_lib.workspace_size(desc, T, B),
                                  _lib.workspace_size(desc, other.T, other.B)), "cuda")
    args = (dev["offsets"], dev["timestamps"], dev["num_candidates"])
    _lib.layer_fwd(desc, dev_o["x"], dev_o["offsets"], dev_o["timestamps"], dev_o["num_candidates"],
                   dev_o["layers"][0], workspace=ws)
    fresh = [_lib.layer_fwd(desc, dev["x"], *args, dev["layers"][n], workspace=ws).clone() for n in (0, 1)]
    reused = _lib.layer_fwd(reuse, dev["x"], *args, dev["layers"][1], workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(reused.float().cpu().numpy(), fresh[1].float().cpu().numpy())
    acts = _lib.proj_fwd(desc, dev["x"], dev["layers"][0])
    a1 = {k: v.clone() for k, v in _lib.attn_fwd(desc, *args, dev["layers"][0], acts).items()}
    ws_a = _lib.alloc_workspace(_lib.attn_workspace_size(desc, T, B), "cuda")
    _lib.attn_fwd(desc, *args, dev["layers"][0], acts, workspace=ws_a)
    _lib.attn_fwd(reuse, *args, dev["layers"][0], acts, workspace=ws_a)
    torch.cuda.synchronize()
    for k in ("av", "av_stats"):
        np.testing.assert_array_equal(acts[k].float().cpu().numpy(), a1[k].float().cpu().numpy())


def test_out_aliases_x():
    w = synth.make_workload("zipf_bf16", batch=6)
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    ref = _lib.layer_fwd(desc, dev["x"], dev["offsets"], dev["timestamps"], None, dev["layers"][0])
    x = dev["x"].clone()
    _lib.layer_fwd(desc, x, dev["offsets"], dev["timestamps"], None, dev["layers"][0], out=x)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)


def test_validate_flag_rejects_bad_metadata():
    w = synth.make_workload("zipf_bf16", batch=3)
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims, _lib.HSTU_VALIDATE)
    bad = dev["offsets"].clone()
    bad[1] = bad[2] + 1
    with pytest.raises(_lib.HstuError) as e:
        _lib.layer_fwd(desc, dev["x"], bad, dev["timestamps"], None, dev["layers"][0])
    assert e.value.status == _lib.HSTU_ERR_INVALID_ARG
    nc = torch.tensor([0, 5000, 0], dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.HstuError):
        _lib.layer_fwd(desc, dev["x"], dev["offsets"], dev["timestamps"], nc, dev["layers"][0])
    # valid metadata passes
    _lib.layer_fwd(desc, dev["x"], dev["offsets"], dev["timestamps"], None, dev["layers"][0])
    torch.cuda.synchronize()
