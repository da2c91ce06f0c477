"""GPU parity of the layer backward (hstu_layer_bwd) against the float64
autograd oracle (oracle/hstu_grad.py, pinned by finite differences).

Tolerances.  fp32 layers: max |g - ref| / max(|ref|, rms(ref)) <= 1e-3 for
every gradient (the forward's 1e-4, widened tenfold: each weight gradient is
a sum over all T rows accumulated in fp32, and the backward chains four
GEMMs and two LayerNorm backwards).  bf16 layers: max |g - ref| / rms(ref)
<= 5e-2 (unit scale): the backward's GEMM operands (dY, Z, dpre, x~) are
rounded to bf16 as in the forward, so each gradient carries a few bf16 ulps
of every operand, on top of the forward activations' own rounding.  The bias
tables' gradients are sums over every attended pair of terms of both signs,
so they cancel heavily: rounding only dL/dAV to bf16 inside the float64
oracle already moves the position table's gradient by 3.5e-2 of its rms on
the 8 x 128/128 case (shown on the CPU), hence 1e-1 for those two in bf16."""

import dataclasses

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import _lib, layer, synth
from oracle import hstu_grad as G

from edge_workloads import edge_workload
from gpu_helpers import err_bf16, err_fp32, say

pytestmark = pytest.mark.gpu

NAMES = {"x": "x", "w1": "w1", "b1": "b1", "w2": "w2", "b2": "b2", "ln_in_g": "ln_in_g", "ln_in_b": "ln_in_b",
         "ln_av_g": "ln_av_g", "ln_av_b": "ln_av_b", "pos": "pos_table", "time": "time_table"}


def _gpu_bwd(w, dy):
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    dt = dev["x"].dtype
    dyt = torch.from_numpy(np.ascontiguousarray(dy, np.float32)).to(dt).cuda()
    dx, grads = _lib.layer_bwd(desc, dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"],
                               dev["layers"][0], dyt)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    out["x"] = dx.float().cpu().numpy().astype(np.float64)
    return out, dyt.float().cpu().numpy().astype(np.float64)


def _check_grads(w, seed=0):
    rng = np.random.default_rng(seed)
    dy = rng.normal(0, 1, (w.T, w.dims.d_model))
    got, dy_used = _gpu_bwd(w, dy)
    ref = G.layer_grads(w.x, w.offsets, w.timestamps, w.num_candidates, w.layers[0], w.dims, dy_used)
    fp32 = w.dims.dtype == "fp32"
    worst = 0.0
    for k, rk in NAMES.items():
        tol = 1e-3 if fp32 else (1e-1 if k in ("pos", "time") else 5e-2)
        r = ref[rk]
        if not w.dims.input_norm and k in ("ln_in_g", "ln_in_b"):
            assert np.all(got[k] == 0), k
            continue
        e = err_fp32(got[k], r) if fp32 else err_bf16(got[k], r)
        say(f"  d{k}: err {e:.3e} (tol {tol:.0e})")
        assert np.all(np.isfinite(got[k])), k
        worst = max(worst, e)
        assert e <= tol, f"d{k}: {e:.3e} > {tol:.0e}"
    return worst


BF16_64 = synth.LayerDims(64, 2, 64, 64, pos_buckets=9, time_buckets=16, dtype="bf16")


@pytest.mark.parametrize("flags", [{}, {"norm_len": 77}, {"cand_shared_pos": False},
                                   {"input_norm": False, "residual": False}])
def test_bwd_edge_fp32(flags):
    w = edge_workload("fp32", seed=1, **flags)
    say(f"backward, edge fp32 {flags}: lengths {w.lengths().tolist()}")
    _check_grads(w, seed=1)


def test_bwd_edge_bf16():
    w = synth.make_workload("small_fp32", seed=2, lengths=[0, 1, 127, 123, 0, 0, 130, 0, 1],
                            candidates=[0, 1, 0, 5, 129, 0, 70, 64, 2], dims=BF16_64, random_ln=True)
    say(f"backward, edge bf16 64/64: lengths {w.lengths().tolist()}")
    _check_grads(w, seed=2)


def test_bwd_zipf_bf16_subset():
    w = synth.make_workload("zipf_bf16", batch=6)
    say(f"backward, zipf_bf16 (bf16, d=256, 4x64/64), B=6, T={w.T}")
    _check_grads(w, seed=3)


# The widest layers the backward accepts: H * dv = 2048 (the gate's LayerNorm
# backward at its widest row) and d_model = 2048 (the input LayerNorm's).
# fp32 (head widths up to 64) checks the same paths at 1e-3.
WIDE = {"heads_2048_bf16": synth.LayerDims(64, 16, 128, 128, pos_buckets=33, time_buckets=32, dtype="bf16"),
        "model_2048_bf16": synth.LayerDims(2048, 2, 32, 32, pos_buckets=33, time_buckets=32, dtype="bf16"),
        "heads_2048_fp32": synth.LayerDims(64, 32, 64, 64, pos_buckets=33, time_buckets=32, dtype="fp32"),
        "model_2048_fp32": synth.LayerDims(2048, 2, 32, 32, pos_buckets=33, time_buckets=32, dtype="fp32")}


@pytest.mark.parametrize("name", sorted(WIDE))
def test_bwd_widest_rows(name):
    w = synth.make_workload("small_fp32", seed=11, lengths=[150, 0, 97], candidates=[0, 0, 5], dims=WIDE[name],
                            random_ln=True)
    say(f"backward, {name}: lengths {w.lengths().tolist()}")
    _check_grads(w, seed=12)


def test_bwd_long_128_bf16():
    dims = synth.WORKLOADS["sl_train"].dims
    w = synth.make_workload("sl_train", batch=2, lengths=[700, 300], dims=dims)
    say(f"backward, 8x128/128 bf16, d=512, lengths {w.lengths().tolist()}")
    _check_grads(w, seed=4)


FAR_FP32 = synth.LayerDims(64, 2, 32, 32, time_buckets=128, time_sub_bits=1, dtype="fp32")
# the same in bf16: the bf16 kernels (the merged dK/dV pass on 16 x 16 tiles)
# at head width 32
FAR_BF16 = dataclasses.replace(FAR_FP32, dtype="bf16")


def _far_block_kinds(w):
    """Count the backward kernels' far (32-row wave, 64-key block) pairs —
    every key a history key at least R positions before the wave's first
    row — by how many time buckets the wave's rows see over the block
    (host-side count with the oracle's bucket function; the wave's rows are
    positions r0 .. r0 + 31 of a sequence without candidates)."""
    from oracle import hstu_oracle as O
    d = w.dims
    R = (d.pos_buckets - 1) // 2
    kinds = {"one": 0, "two": 0, "more": 0}
    for b in range(len(w.offsets) - 1):
        s0, e = int(w.offsets[b]), int(w.offsets[b + 1])
        t, L = w.timestamps[s0:e], e - s0
        for r0 in range(0, L, 32):
            tq = t[r0:min(r0 + 32, L)]
            for j0 in range(0, L, 64):
                if not (j0 + 63 < r0 and r0 - (j0 + 63) >= R):
                    break
                kb = t[j0:j0 + 64]
                lo = O.time_bucket(tq - kb.max(), d.time_buckets, d.time_sub_bits)
                hi = O.time_bucket(tq - kb.min(), d.time_buckets, d.time_sub_bits)
                kinds["one" if np.all(lo == hi) else "two" if np.all(hi <= lo + 1) else "more"] += 1
    return kinds


def _far_modes_workload(dims):
    # long histories and two sub-buckets per octave: far blocks with one time
    # bucket per row, with two adjacent ones (per-key split), and with more
    return synth.make_workload("small_fp32", seed=7, lengths=[640, 450], candidates=[0, 0], dims=dims)


def _time_overflow_workload(dims):
    # a far block whose time span overflows int64 differences: key 0 at the
    # earliest representable time, the queries one second past the epoch, so
    # the span's endpoints both give bucket 0 while the keys in between are
    # 100+ seconds back; the per-pair path must take it (pairwise differences
    # wrap as in the oracle)
    w = synth.make_workload("small_fp32", seed=9, lengths=[300], candidates=[0], dims=dims)
    ts = np.zeros(w.T, np.int64)
    ts[0] = np.iinfo(np.int64).min + 1
    ts[1] = 5
    ts[2:64] = -100 - np.arange(62)
    ts[128:] = 1
    w.timestamps = ts
    return w


@pytest.mark.parametrize("dims", [FAR_FP32, FAR_BF16], ids=["fp32", "bf16"])
def test_bwd_far_block_modes(dims):
    w = _far_modes_workload(dims)
    kinds = _far_block_kinds(w)
    say(f"backward, far-block modes {dims.dtype}: lengths {w.lengths().tolist()}, far blocks {kinds}")
    assert kinds["one"] > 0 and kinds["two"] > 0
    _check_grads(w, seed=8)


@pytest.mark.parametrize("dims", [FAR_FP32, FAR_BF16], ids=["fp32", "bf16"])
def test_bwd_far_block_time_overflow(dims):
    w = _time_overflow_workload(dims)
    say(f"backward, int64-overflowing far block {dims.dtype}: lengths {w.lengths().tolist()}")
    _check_grads(w, seed=10)


def test_bwd_shared_tables_sum_heads():
    w = edge_workload("fp32", seed=5)
    dev = layer.to_device(w)
    prm = dict(dev["layers"][0])
    prm["pos_table"] = prm["pos_table"][0].contiguous()
    prm["time_table"] = prm["time_table"][0].contiguous()
    dy = torch.randn(w.T, w.dims.d_model, device="cuda", generator=torch.Generator(device="cuda").manual_seed(0))
    _, g = _lib.layer_bwd(_lib.make_desc(w.dims), dev["x"], dev["offsets"], dev["timestamps"],
                          dev["num_candidates"], prm, dy)
    p = dict(w.layers[0])
    p["pos_table"] = np.broadcast_to(w.layers[0]["pos_table"][0], w.layers[0]["pos_table"].shape).copy()
    p["time_table"] = np.broadcast_to(w.layers[0]["time_table"][0], w.layers[0]["time_table"].shape).copy()
    torch.cuda.synchronize()
    ref = G.layer_grads(w.x, w.offsets, w.timestamps, w.num_candidates, p, w.dims, dy.cpu().numpy())
    say("backward with head-shared tables: gradients summed over heads")
    assert err_fp32(g["pos"].cpu().numpy(), ref["pos_table"].sum(0)) <= 1e-3
    assert err_fp32(g["time"].cpu().numpy(), ref["time_table"].sum(0)) <= 1e-3


@pytest.mark.parametrize("name,batch", [("zipf_bf16", 4), ("zipf_bf16", None), ("sl_train", 16)])
def test_bwd_deterministic_bitwise(name, batch):
    """Two runs give the same bits.  The full zipf_bf16 batch (32 sequences,
    over 100 work items of equal cost across sequences, which the work-list
    builder may place in any order) and 16 stochastic-length sequences (many
    items of equal cost) check that the bias-table gradients do not depend
    on the work list's order."""
    w = synth.make_workload(name, batch=batch, n_layers=1)
    dy = np.random.default_rng(6).normal(0, 1, (w.T, w.dims.d_model))
    a, _ = _gpu_bwd(w, dy)
    b, _ = _gpu_bwd(w, dy)
    say(f"determinism {name} batch={w.B}: T={w.T}")
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_bwd_ranking_full_size():
    """The ranking workload (bf16, B=16, history U[512, 2048] + 512 candidates,
    d=512, 8 x 64/64) at full size: dx rows of the shortest sequence depend on
    that sequence alone, so they are compared with the oracle run on it; the
    parameter gradients of the same sequence run alone on the GPU (the kernels
    at the full-size shape, one sequence) against the oracle's."""
    w = synth.make_workload("ranking_cand", n_layers=1)
    s = int(np.argmin(w.lengths()))
    rng = np.random.default_rng(11)
    dy = rng.normal(0, 1, (w.T, w.dims.d_model))
    got, dy_used = _gpu_bwd(w, dy)
    sub = w.sub_batch([s])
    rows = np.arange(w.offsets[s], w.offsets[s + 1])
    ref = G.layer_grads(sub.x, sub.offsets, sub.timestamps, sub.num_candidates, sub.layers[0], w.dims,
                        dy_used[rows])
    say(f"backward, ranking_cand full batch (T={w.T}); oracle on sequence {s} ({len(rows)} rows)")
    e = err_bf16(got["x"][rows], ref["x"])
    say(f"  dx (full batch, sequence {s}): err {e:.3e} (tol 5e-02)")
    assert e <= 5e-2
    got1, _ = _gpu_bwd(sub, dy_used[rows])
    for k, rk in NAMES.items():
        tol = 1e-1 if k in ("pos", "time") else 5e-2
        e = err_bf16(got1[k], ref[rk])
        say(f"  d{k} (sequence {s} alone): err {e:.3e} (tol {tol:.0e})")
        assert e <= tol, k


def test_bwd_stack8_full_size():
    """The 8-layer workload's first layer (bf16, B=8, L in [4096, 8192], d=1024,
    8 x 128/128) at full size, where the fp32-output GEMMs and the
    pre-activation GEMM run on the 256 x 256 kernels (dZ and dx~ over 43,864
    rows; dW1 split over K): dx rows of the shortest sequence from the full
    batch, and every gradient of that sequence run alone (dW1 again split over
    K on the 256 x 256 kernel), against the oracle run on that sequence."""
    w = synth.make_workload("stack8_long", n_layers=1)
    s = int(np.argmin(w.lengths()))
    rng = np.random.default_rng(12)
    dy = rng.normal(0, 1, (w.T, w.dims.d_model))
    got, dy_used = _gpu_bwd(w, dy)
    sub = w.sub_batch([s])
    rows = np.arange(w.offsets[s], w.offsets[s + 1])
    say(f"backward, stack8_long layer 1 full batch (T={w.T}); oracle on sequence {s} ({len(rows)} rows)")
    ref = G.layer_grads(sub.x, sub.offsets, sub.timestamps, sub.num_candidates, sub.layers[0], w.dims,
                        dy_used[rows])
    e = err_bf16(got["x"][rows], ref["x"])
    say(f"  dx (full batch, sequence {s}): err {e:.3e} (tol 5e-02)")
    assert e <= 5e-2
    got1, _ = _gpu_bwd(sub, dy_used[rows])
    for k, rk in NAMES.items():
        tol = 1e-1 if k in ("pos", "time") else 5e-2
        e = err_bf16(got1[k], ref[rk])
        say(f"  d{k} (sequence {s} alone): err {e:.3e} (tol {tol:.0e})")
        assert e <= tol, k


@pytest.mark.parametrize("case", ["edge_fp32", "edge_bf16_64", "zipf_bf16", "sl_128_bf16", "far_modes_bf16_32",
                                  "time_overflow_bf16_32"])
def test_attention_stage_backward(case):
    """hstu_attn_bwd fed the GPU's own q, k, v and a bf16 dL/dAV, against the
    float64 autograd of the attention alone fed the same values: the stage's
    own arithmetic, element-relative (max |g - ref| / max(|ref|, rms(ref))).
    fp32: 1e-3.  bf16: 5e-2 — the kernels round the pointwise weights (for dV)
    and dS (for dQ, dK) to bf16 as MFMA operands, like the forward's weights;
    rounding only the weights to bf16 inside the float64 oracle already moves
    dV by 3.4e-2 on the bf16 edge case (a single-token sequence's key carries
    a weight of order 1 while most gradients are small), and the forward's
    attention tap has the same 4e-2-class bound."""
    if case == "edge_fp32":
        w = edge_workload("fp32", seed=3)
    elif case == "edge_bf16_64":
        w = synth.make_workload("small_fp32", seed=3, lengths=[0, 1, 127, 123, 0, 0, 130, 0, 1],
                                candidates=[0, 1, 0, 5, 129, 0, 70, 64, 2], dims=BF16_64, random_ln=True)
    elif case == "zipf_bf16":
        w = synth.make_workload("zipf_bf16", batch=6)
    elif case == "far_modes_bf16_32":
        w = _far_modes_workload(FAR_BF16)
    elif case == "time_overflow_bf16_32":
        w = _time_overflow_workload(FAR_BF16)
    else:
        w = synth.make_workload("sl_train", batch=2, lengths=[700, 300], dims=synth.WORKLOADS["sl_train"].dims)
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    prm = dev["layers"][0]
    acts = _lib.proj_fwd(desc, dev["x"], prm)
    H, dqk, dv = w.dims.num_heads, w.dims.dqk, w.dims.dv
    g = torch.Generator(device="cuda").manual_seed(9)
    dav = torch.randn(w.T, H * dv, generator=g, device="cuda").to(dev["x"].dtype)
    dqkv, dpos, dtime = _lib.attn_bwd(desc, dev["offsets"], dev["timestamps"], dev["num_candidates"], prm, acts, dav)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    q, k, v = (f(acts[n]).transpose(1, 0, 2) for n in ("q", "k", "v"))
    ref = G.attention_grads(q, k, v, f(dav), w.offsets, w.timestamps, w.num_candidates, w.layers[0], w.dims)
    K2 = H * dv
    D = f(dqkv)
    got = {"v": D[:, K2:2 * K2].reshape(w.T, H, dv), "q": D[:, 2 * K2:2 * K2 + H * dqk].reshape(w.T, H, dqk),
           "k": D[:, 2 * K2 + H * dqk:].reshape(w.T, H, dqk), "pos_table": f(dpos), "time_table": f(dtime)}
    fp32 = w.dims.dtype == "fp32"
    say(f"attention backward stage, {case}: T={w.T}")
    for n in got:
        e = err_fp32(got[n], ref[n])
        tol = 1e-3 if fp32 else 5e-2
        say(f"  d{n}: err {e:.3e} (tol {tol:.0e})")
        assert e <= tol, n
    assert np.all(D[:, :K2] == 0)   # the u block is not written


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_saved_forward_matches_recompute(dtype):
    """hstu_layer_fwd_train gives hstu_layer_fwd's output bit for bit, and
    hstu_layer_bwd with HSTU_SAVED_FWD on its workspace gives the recomputing
    backward's dx and gradients bit for bit (the same kernels on the same
    inputs; only the recompute is skipped)."""
    if dtype == "fp32":
        w = edge_workload("fp32", seed=4)
    else:
        w = synth.make_workload("small_fp32", seed=5, lengths=[3, 127, 0, 200, 64],
                                candidates=[0, 2, 0, 9, 64], dims=BF16_64, random_ln=True)
    say(f"saved forward, {dtype}: lengths {w.lengths().tolist()}")
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    saved = _lib.make_desc(w.dims, _lib.HSTU_SAVED_FWD)
    prm = dev["layers"][0]
    args = (dev["offsets"], dev["timestamps"], dev["num_candidates"], prm)
    rng = np.random.default_rng(4)
    dy = torch.from_numpy(rng.normal(0, 1, (w.T, w.dims.d_model)).astype(np.float32)).to(dev["x"].dtype).cuda()
    y_ref = _lib.layer_fwd(desc, dev["x"], *args)
    dx_ref, g_ref = _lib.layer_bwd(desc, dev["x"], *args, dy)
    ws = _lib.alloc_workspace(_lib.bwd_workspace_size(desc, w.T, w.B), "cuda")
    y = _lib.layer_fwd_train(desc, dev["x"], *args, workspace=ws)
    dx, g = _lib.layer_bwd(saved, dev["x"], *args, dy, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(dx, dx_ref)
    for k in g_ref:
        assert torch.equal(g[k], g_ref[k]), k
