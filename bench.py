"""HSTU layer forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stack8_long]

A step is one pass of the whole hot path over one batch of the workload: for
the default `stack8_long` (8 HSTU layers, 8 jagged sequences of 4096..8192
tokens, d=1024, 8 heads x 128/128, bf16) that is 8 hstu_layer_fwd calls
(input LayerNorm, projection GEMM + SiLU, work list, fused pointwise
attention, LayerNorm/gate kernel, output GEMM + residual per layer).  Inputs are
resident in HBM before timing starts.  Prints one JSON line.

Besides the step time, the attention kernel — the dominant kernel — is timed
on its own through hstu_attn_fwd (the work list and key-block summary built
once, as in the stack, and reused) with HIP events recorded on the stream it is
launched on, and its algorithmic FLOPs per launch (2 (dqk + dv) H per
attended (query, key) pair) give the roofline fraction against the dense bf16
MFMA peak.  The LayerNorm/gate kernel is timed the same way through
hstu_gate_fwd against the HBM peak (its algorithmic bytes: AV and U read and
Z written once, plus the per-head statistics).  The CPU oracle is timed on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6       # dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

METRIC = "HSTU layer fwd tokens/sec (jagged bf16); attention TFLOP/s vs MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_{workload}.json")
ATTN_SOURCES = ["attn.hip", "common.h", "kernels.h"]


def attn_source_hash() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "hstu_sequential_transducer_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def attended_pairs(lengths, ncand) -> int:
    """Unmasked (query, key) pairs: causal history plus candidates that see the
    history and themselves."""
    tot = 0
    for b, L in enumerate(lengths):
        m = 0 if ncand is None else int(ncand[b])
        n = int(L) - m
        tot += n * (n + 1) // 2 + m * n + m
    return tot


def load_traffic(workload: str):
    p = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("attn_source_hash") != attn_source_hash():
        return None          # counters were taken on a different kernel
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------ CPU baseline
# The float64 oracle is the parity reference; for timing, the same oracle
# functions run in float32 and are spread over worker processes (spawned:
# fresh interpreters that load NumPy and the oracle only, one BLAS thread
# each).  Inputs, parameters and results live in shared memory.  The work
# units: 1024-row blocks for the two GEMM stages, (sequence, 1024-row query
# block) for the attention, all heads of a unit together so that its bias
# indices are formed once.
_CPU = {}


def _shm_put(arr, registry, name):
    from multiprocessing import shared_memory
    arr = np.ascontiguousarray(arr)
    shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
    view = np.ndarray(arr.shape, arr.dtype, buffer=shm.buf)
    view[...] = arr
    registry[name] = (shm.name, arr.shape, arr.dtype.str)
    return shm, view


def _shm_get(spec):
    from multiprocessing import shared_memory
    shm = shared_memory.SharedMemory(name=spec[0])
    _CPU.setdefault("_keep", []).append(shm)
    return np.ndarray(spec[1], np.dtype(spec[2]), buffer=shm.buf)


def _cpu_init(registry, cfg):
    from threadpoolctl import threadpool_limits
    _CPU["_limits"] = threadpool_limits(1)
    _CPU["cfg"] = cfg
    _CPU["arr"] = {k: _shm_get(v) for k, v in registry.items()}


def _cpu_ready(_):
    return os.getpid()


def _cpu_task(task):
    from oracle import hstu_oracle as O
    kind, layer_i, a, b = task[:4]
    A, cfg = _CPU["arr"], _CPU["cfg"]
    prm = {k[len(f"p{layer_i}_"):]: v for k, v in A.items() if k.startswith(f"p{layer_i}_")}
    f32 = np.float32
    H, dqk, dv = cfg.num_heads, cfg.dqk, cfg.dv
    if kind == "proj":            # rows [a, b)
        u, v, q, k = O.project(A["h"][a:b], prm, cfg, dtype=f32)
        A["u"][a:b] = u
        A["v"][a:b] = v
        A["q"][a:b] = q
        A["k"][a:b] = k
    elif kind == "attn":          # sequence rows [a, b), local query rows task[4]
        r0, r1 = task[4]
        off = np.array([0, b - a], np.int64)
        nc = A["nc"][task[5]:task[5] + 1] if "nc" in A else None
        av = O.attention(A["q"][a:b], A["k"][a:b], A["v"][a:b], off, A["ts"][a:b], nc, prm, cfg,
                         rows=np.arange(r0, r1), dtype=f32)
        A["av"][a + r0:a + r1] = av
    else:                         # "out": rows [a, b)
        out = O.gate_and_project(A["av"][a:b], A["u"][a:b], A["h"][a:b], prm, cfg, dtype=f32)
        A["y"][a:b] = out["y"]
    return b - a


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 30.0, max_workers: int = 16):
    """The oracle's functions in float32 over the whole batch, layer after
    layer of the stack until every layer has run or the budget is spent; the
    value is tokens through the stack per second (measured, or, if the
    budget stopped the stack early, the measured per-layer time times the
    number of layers, which the sample text then says)."""
    import multiprocessing as mp
    workers = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    cfg = w.dims
    T, H, dqk, dv = w.T, cfg.num_heads, cfg.dqk, cfg.dv
    reg, keep = {}, []
    f32 = np.float32
    try:
        def put(name, arr):
            shm, view = _shm_put(arr, reg, name)
            keep.append(shm)
            return view
        h = put("h", w.x.astype(f32))
        put("u", np.zeros((T, H * dv), f32))
        put("v", np.zeros((T, H, dv), f32))
        put("q", np.zeros((T, H, dqk), f32))
        put("k", np.zeros((T, H, dqk), f32))
        put("av", np.zeros((T, H * dv), f32))
        y = put("y", np.zeros((T, cfg.d_model), f32))
        put("ts", w.timestamps)
        if w.num_candidates is not None:
            put("nc", np.asarray(w.num_candidates, np.int32))
        for li, prm in enumerate(w.layers):
            for k, v in prm.items():
                put(f"p{li}_{k}", np.asarray(v, f32))
        blocks = [(r, min(r + 1024, T)) for r in range(0, T, 1024)]
        attn_units = []
        for b in range(w.B):
            s0, s1 = int(w.offsets[b]), int(w.offsets[b + 1])
            for r in range(0, s1 - s0, 1024):
                attn_units.append((s0, s1, (r, min(r + 1024, s1 - s0)), b))
        # longest units first, so the pool's tail is short
        attn_units.sort(key=lambda u: -(u[2][1] ** 2 - u[2][0] ** 2))
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_cpu_init, initargs=(reg, cfg)) as pool:
            pool.map(_cpu_ready, range(workers * 4))      # every worker up and attached
            t_layers = []
            for li in range(len(w.layers)):
                t0 = time.perf_counter()
                pool.map(_cpu_task, [("proj", li, a, b) for a, b in blocks])
                pool.map(_cpu_task, [("attn", li, s0, s1, rr, bi) for s0, s1, rr, bi in attn_units],
                         chunksize=1)
                pool.map(_cpu_task, [("out", li, a, b) for a, b in blocks])
                t_layers.append(time.perf_counter() - t0)
                h[...] = y                                 # the next layer's input
                if sum(t_layers) > budget_s and li + 1 < len(w.layers):
                    break
        done = len(t_layers)
        n_layers = len(w.layers)
        t_used = sum(t_layers)
        value = T / (t_used / done * n_layers)
        ran = (f"all {n_layers} layers" if done == n_layers else
               f"layers 1-{done} of {n_layers} (the budget of {budget_s:.0f} s was spent; value = "
               f"tokens / (mean layer time x {n_layers}))")
        return {"value": value, "unit": "tokens/s", "cores": workers, "kind": "oracle",
                "precision": "float32 (the float64 mode is the parity reference)",
                "cpu_model": cpu_model(),
                "affinity_cores": len(os.sched_getaffinity(0)),
                "sample": f"the oracle's project / attention / gate_and_project in float32 over the whole "
                          f"batch ({w.B} sequences, {T} tokens, lengths {int(w.lengths().min())}.."
                          f"{int(w.lengths().max())}), {ran}, in {t_used:.1f} s on {workers} worker "
                          f"processes with one BLAS thread each (1024-row blocks for the GEMMs, "
                          f"(sequence, 1024-row query block) units for the attention)",
                "layer_seconds": t_layers}
    finally:
        for shm in keep:
            shm.close()
            shm.unlink()


def cand_inference(torch, _lib, layer, synth, per_seq: int = 128, reps: int = 20):
    """Scoring every candidate of the ranking workload (B=16, history
    U[512, 2048] + 512 candidates, d=512, 8 heads x 64/64, bf16) three ways:
    one batched pass over history + all candidates; micro-batches of
    `per_seq` candidates per sequence, each a full pass over history + those
    candidates; and the same micro-batches against a history K/V cache
    (history projected once, then hstu_cand_fwd per micro-batch).  Each way is
    captured once into a HIP graph and replayed (the small per-micro-batch
    kernels would otherwise time the host's launch rate); the eager times are
    reported too."""
    w = synth.make_workload("ranking_cand")
    dev = layer.to_device(w)
    D = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    hrows, hoff, crows, coff, m = layer.split_history(w.offsets, w.num_candidates)
    x, ts = dev["x"], dev["timestamps"]
    prm = dev["layers"][0]
    desc = _lib.make_desc(w.dims)
    wts, tab = _lib.make_weights(prm), _lib.make_tables(prm)
    B = w.B
    mbs = list(layer.candidate_microbatches(coff, per_seq))
    # full passes: batched, and per micro-batch over history + its candidates
    full_in = []
    for rows, moff in mbs:
        cnt = np.diff(moff)
        sel = np.concatenate([np.r_[hrows[hoff[b]:hoff[b + 1]], crows[rows[moff[b]:moff[b + 1]]]]
                              for b in range(B)])
        off = np.concatenate([[0], np.cumsum(np.diff(hoff) + cnt)]).astype(np.int64)
        full_in.append((x[D(sel)].contiguous(), D(off), ts[D(sel)].contiguous(), D(cnt.astype(np.int32))))
    ws_full = _lib.alloc_workspace(_lib.workspace_size(desc, w.T, B), "cuda")
    out_full = torch.empty_like(x)
    outs_mb = [torch.empty_like(a[0]) for a in full_in]
    # cached: history rows, then candidate micro-batches
    xh, hoff_d, hts = x[D(hrows)].contiguous(), D(hoff), ts[D(hrows)].contiguous()
    cand_in = [(x[D(crows[r])].contiguous(), D(o), ts[D(crows[r])].contiguous()) for r, o in mbs]
    m_d = D(m.astype(np.int32))
    acts_h = _lib.alloc_activations(desc, len(hrows), "cuda")
    ws_proj = _lib.alloc_workspace(_lib.proj_workspace_size(desc, len(hrows)), "cuda")
    Tc_max = max(len(r) for r, _ in mbs)
    ws_c = _lib.alloc_workspace(_lib.cand_workspace_size(desc, Tc_max, len(hrows), B), "cuda")
    outs_c = [torch.empty_like(a[0]) for a in cand_in]

    def batched():
        _lib.layer_fwd(desc, x, dev["offsets"], ts, dev["num_candidates"], prm, out=out_full,
                       workspace=ws_full, weights=wts, tables=tab)

    def microbatched():
        for (xi, oi, ti, ni), yo in zip(full_in, outs_mb):
            _lib.layer_fwd(desc, xi, oi, ti, ni, prm, out=yo, workspace=ws_full, weights=wts, tables=tab)

    def encode():
        _lib.proj_fwd(desc, xh, prm, acts_h, workspace=ws_proj, weights=wts)

    def cached_mbs():
        for (xc, oc, tc), yo in zip(cand_in, outs_c):
            _lib.cand_fwd(desc, xc, oc, tc, m_d, hoff_d, hts, acts_h["k"], acts_h["v"], prm, out=yo,
                          workspace=ws_c, weights=wts, tables=tab)

    def cached():
        encode()
        cached_mbs()

    def ev_time(fn):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        s.record(st)
        for _ in range(reps):
            fn()
        e.record(st)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def graph_time(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return ev_time(g.replay)

    res = {}
    for name, fn in (("batched", batched), ("microbatched", microbatched), ("cached", cached),
                     ("cache_encode", encode), ("cached_microbatches", cached_mbs)):
        res[name] = {"graph_ms": graph_time(fn), "eager_ms": ev_time(fn)}
    nmb = len(mbs)
    ncand = int(m.sum())
    per_unc = res["microbatched"]["graph_ms"] / nmb
    per_c = res["cached_microbatches"]["graph_ms"] / nmb
    return {
        "workload": f"ranking_cand: {synth.WORKLOADS['ranking_cand'].description}; 1 layer",
        "history_tokens": int(len(hrows)),
        "candidates": ncand,
        "micro_batch_per_seq": per_seq,
        "micro_batches": nmb,
        "ms": res,
        "per_microbatch_ms": {"full_pass": per_unc, "cached": per_c},
        "cache_speedup_per_microbatch": per_unc / per_c,
        "candidates_per_s": {k: ncand / (res[k]["graph_ms"] * 1e-3)
                             for k in ("batched", "microbatched", "cached")},
    }


def sl_repack(torch, _lib, reps: int = 20):
    """Stochastic length on the training shape (B = 64 sequences of 4096
    tokens, N = 4096, alpha = 1.6), then the re-pack of x (bf16, d = 512),
    timestamps and token types: events around sample + gathers."""
    B, L, d = 64, 4096, 512
    g = torch.Generator(device="cuda").manual_seed(11)
    off = torch.arange(0, (B + 1) * L, L, dtype=torch.int64, device="cuda")
    u = torch.rand(B, generator=g, device="cuda")
    keys = torch.randint(-(1 << 31), 1 << 31, (B * L,), generator=g, device="cuda", dtype=torch.int32)
    x = torch.randn(B * L, d, generator=g, device="cuda").to(torch.bfloat16)
    ts = torch.randint(0, 1 << 40, (B * L,), generator=g, device="cuda")
    ty = torch.randint(0, 2, (B * L,), generator=g, device="cuda").to(torch.uint8)
    new_off = torch.empty(B + 1, dtype=torch.int64, device="cuda")
    rows = torch.empty(B * L, dtype=torch.int64, device="cuda")
    xo, tso, tyo = torch.empty_like(x), torch.empty_like(ts), torch.empty_like(ty)
    ws = _lib.alloc_workspace(int(_lib.load().hstu_sl_workspace_size(B)), "cuda")

    def step():
        _lib.sl_sample(off, u, keys, L, 1.6, out_offsets=new_off, out_rows=rows, workspace=ws)
        cnt = new_off[-1:]
        _lib.gather_rows(x, rows, cnt, out=xo)
        _lib.gather_rows(ts, rows, cnt, out=tso)
        _lib.gather_rows(ty, rows, cnt, out=tyo)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    total_ms = timed(step)
    sample_ms = timed(lambda: _lib.sl_sample(off, u, keys, L, 1.6, out_offsets=new_off, out_rows=rows,
                                             workspace=ws))
    kept = int(new_off[-1].item())
    moved = kept * (2 * d * 2 + 2 * 8 + 2 * 1 + 3 * 8)   # rows read + written, and their index read thrice
    return {
        "workload": "64 x 4096 tokens, N = 4096, alpha = 1.6; re-pack x (bf16 x 512), timestamps, types",
        "kept_tokens": kept,
        "tokens": B * L,
        "sample_ms": sample_ms,
        "sample_and_repack_ms": total_ms,
        "repack_gbs": moved / ((total_ms - sample_ms) * 1e-3) / 1e9,
        "repack_hbm_frac": moved / ((total_ms - sample_ms) * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }


def config_measure(torch, _lib, layer, synth, name: str, reps: int = 20):
    """One workload's layer forward and its stages: tokens/s of the whole
    layer (hstu_layer_fwd, every kernel of the step), the attention kernel
    alone (plan built once and reused; events on its launch stream) against
    the MFMA peak of the layer's dtype, and the LayerNorm/gate kernel against
    the HBM peak.  For the 8-layer workload the layer is its first."""
    w = synth.make_workload(name, n_layers=1)
    dev = layer.to_device(w)
    x, off, ts, nc = dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"]
    prm = dev["layers"][0]
    desc = _lib.make_desc(w.dims)
    reuse = _lib.make_desc(w.dims, _lib.HSTU_REUSE_PLAN)
    T, B = w.T, w.B
    stream = torch.cuda.current_stream()
    ws = _lib.alloc_workspace(_lib.workspace_size(desc, T, B), x.device)
    out = torch.empty_like(x)
    wts, tab = _lib.make_weights(prm), _lib.make_tables(prm)

    def timed(fn, n=reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    layer_ms = timed(lambda: _lib.layer_fwd(desc, x, off, ts, nc, prm, out=out, workspace=ws, weights=wts,
                                            tables=tab))
    acts = _lib.proj_fwd(desc, x, prm)
    aws = _lib.alloc_workspace(_lib.attn_workspace_size(desc, T, B), x.device)
    _lib.attn_fwd(desc, off, ts, nc, prm, acts, workspace=aws)
    attn_ms = timed(lambda: _lib.attn_fwd(reuse, off, ts, nc, prm, acts, workspace=aws))
    zbuf = torch.empty_like(acts["u"])
    gate_ms = timed(lambda: _lib.gate_fwd(desc, prm, acts, z=zbuf))
    proj_ms = timed(lambda: _lib.proj_fwd(desc, x, prm, acts))
    out_ms = timed(lambda: _lib.out_fwd(desc, x, prm, acts, out=out, z=zbuf))
    dm, H, dqk, dv = w.dims.d_model, w.dims.num_heads, w.dims.dqk, w.dims.dv
    pairs = attended_pairs(w.lengths(), w.num_candidates)
    attn_flop = 2.0 * (dqk + dv) * H * pairs
    bf16 = w.dims.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_MFMA_TFLOPS
    e = 2 if bf16 else 4
    gate_bytes = T * (3 * H * dv * e + 8 * H) + 2 * H * dv * e
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    return {
        "workload": f"{name}: {synth.WORKLOADS[name].description}" + (" (layer 1 of 8)" if name == "stack8_long" else ""),
        "tokens": T,
        "sequences": B,
        "seq_len": f"{int(w.lengths().min())}..{int(w.lengths().max())}",
        "layer_ms": layer_ms,
        "tokens_per_s": T / (layer_ms * 1e-3),
        "stages_ms": {"proj": proj_ms, "attn": attn_ms, "out (gate + f2)": out_ms},
        "attention": {"kernel": "attn_kernel", "bound": "mfma", "achieved": attn_tflops, "peak": peak,
                      "unit": "TFLOP/s", "frac": attn_tflops / peak, "launch_ms": attn_ms,
                      "flop_per_launch": attn_flop, "pairs_per_launch": pairs,
                      "mfma_dtype": "bf16" if bf16 else "fp32"},
        "gate": {"kernel": "gate_kernel", "bound": "hbm", "achieved": gate_bytes / (gate_ms * 1e-3) / 1e9,
                 "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": gate_bytes / (gate_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "launch_ms": gate_ms,
                 "bytes_per_launch": gate_bytes},
    }


CONFIGS = ["small_fp32", "zipf_bf16", "ranking_cand", "sl_train", "len4k", "stack8_long"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="stack8_long")
    ap.add_argument("--attn-reps", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-cand", action="store_true", help="skip the cached-candidate measurement")
    ap.add_argument("--cand-only", action="store_true",
                    help="run only the cached-candidate measurement and print its JSON object")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--minimal", action="store_true",
                    help="only the step and its attention / gate timings (for profiler runs)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload measurements")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 4 times (a plain copy kernel of "
                         "known size, to scale profiler byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the HSTU layer "
              "forward here is a single-GPU path; sequences are independent, so a multi-GPU "
              "deployment shards the jagged batch by sequence with no collectives.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hstu_sequential_transducer_layer_amd import _lib, layer, synth

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)
        return

    _lib.load()   # fails loudly if the HIP library is missing
    if args.cand_only:
        print(json.dumps({"cand_inference": cand_inference(torch, _lib, layer, synth)}), flush=True)
        return
    w = synth.make_workload(args.workload)
    dev = layer.to_device(w)
    stack = layer.HSTUStack(w.dims, dev["layers"])
    x, off, ts, nc = dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"]
    T, B = w.T, w.B
    out = torch.empty_like(x)

    for _ in range(args.warmup):
        stack.forward(x, off, ts, nc, out=out)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        stack.forward(x, off, ts, nc, out=out)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # Attention kernel alone, one layer's launch, events on the launch stream.
    # The work list and key-block summary are built once, as the stack does on
    # its first layer; the timed launches reuse them (HSTU_REUSE_PLAN, as
    # layers 2-8 do), so the events cover the attention kernel only.
    desc = stack.desc
    acts = _lib.proj_fwd(desc, x, dev["layers"][0])
    stream = torch.cuda.current_stream()
    aws = _lib.alloc_workspace(_lib.attn_workspace_size(desc, T, B), x.device)
    _lib.attn_fwd(desc, off, ts, nc, dev["layers"][0], acts, workspace=aws)
    for _ in range(3):
        _lib.attn_fwd(stack.desc_reuse, off, ts, nc, dev["layers"][0], acts, workspace=aws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.attn_reps)]
    for a, b in ev:
        a.record(stream)
        _lib.attn_fwd(stack.desc_reuse, off, ts, nc, dev["layers"][0], acts, workspace=aws)
        b.record(stream)
    torch.cuda.synchronize()
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # the other two stages of one layer, for context
    def timed(fn, reps=10):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps
    typed_ms = bwd_ms = train_fwd_ms = train_ms = None
    if not args.minimal:
        # The same launch with the token-type term: two types, the history
        # interleaving content (0) and action (1) tokens, a random [H, 2, 2] table.
        rng = np.random.default_rng(7)
        types = np.concatenate([np.arange(L) % 2 for L in w.lengths()]).astype(np.uint8)
        tdims = dataclasses.replace(w.dims, num_types=2)
        tdesc = _lib.make_desc(tdims)
        tdesc_reuse = _lib.make_desc(tdims, _lib.HSTU_REUSE_PLAN)
        tprm = dict(dev["layers"][0])
        tprm["type_table"] = torch.from_numpy(synth.round_bf16(
            rng.normal(0.0, 0.02, (w.dims.num_heads, 2, 2)))).to(x.dtype).cuda()
        ttypes = torch.from_numpy(types).cuda()
        tws = _lib.alloc_workspace(_lib.attn_workspace_size(tdesc, T, B), x.device)
        _lib.attn_fwd(tdesc, off, ts, nc, tprm, acts, workspace=tws, token_types=ttypes)  # plan with the key types
        typed_ms = timed(lambda: _lib.attn_fwd(tdesc_reuse, off, ts, nc, tprm, acts, workspace=tws, token_types=ttypes),
                         reps=args.attn_reps)
        # The layer backward (forward recompute + all gradients) of layer 1.
        gdy = torch.randn(x.shape, generator=torch.Generator(device="cuda").manual_seed(5), device="cuda").to(x.dtype)
        gdx = torch.empty_like(x)
        gws = _lib.alloc_workspace(_lib.bwd_workspace_size(desc, T, B), "cuda")
        gout = {}

        def bwd():
            nonlocal gout
            _, gout = _lib.layer_bwd(desc, x, off, ts, nc, dev["layers"][0], gdy, dx=gdx,
                                     grads=gout or None, workspace=gws)
        bwd_ms = timed(bwd, reps=5)
        # A training step with saved activations: hstu_layer_fwd_train, then
        # hstu_layer_bwd with HSTU_SAVED_FWD on the same workspace.
        sdesc = _lib.make_desc(w.dims, _lib.HSTU_SAVED_FWD)
        ty = torch.empty_like(x)

        def train_step():
            nonlocal gout
            _lib.layer_fwd_train(desc, x, off, ts, nc, dev["layers"][0], workspace=gws, out=ty)
            _, gout = _lib.layer_bwd(sdesc, x, off, ts, nc, dev["layers"][0], gdy, dx=gdx,
                                     grads=gout or None, workspace=gws)
        train_fwd_ms = timed(lambda: _lib.layer_fwd_train(desc, x, off, ts, nc, dev["layers"][0], workspace=gws,
                                                          out=ty), reps=5)
        train_ms = timed(train_step, reps=5)
    proj_ms = timed(lambda: _lib.proj_fwd(desc, x, dev["layers"][0], acts))
    zbuf = torch.empty_like(acts["u"])
    gate_ms = timed(lambda: _lib.gate_fwd(desc, dev["layers"][0], acts, z=zbuf), reps=20)
    out_ms = timed(lambda: _lib.out_fwd(desc, x, dev["layers"][0], acts, out=out, z=zbuf))

    pairs = attended_pairs(w.lengths(), w.num_candidates)
    dm, H, dqk, dv = w.dims.d_model, w.dims.num_heads, w.dims.dqk, w.dims.dv
    attn_flop = 2.0 * (dqk + dv) * H * pairs
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dims.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    tokens_per_s = T / (ms_step * 1e-3)
    e = 2 if w.dims.dtype == "bf16" else 4
    proj_flop = 2.0 * T * dm * w.dims.n1
    # gate kernel, algorithmic bytes: per row AV and U read, Z written (H*dv
    # elements each) and the H (mean, M2) fp32 partials read; plus gamma, beta.
    gate_bytes = T * (3 * H * dv * e + 8 * H) + 2 * H * dv * e
    gate_gbs = gate_bytes / (gate_ms * 1e-3) / 1e9
    f2_flop = 2.0 * T * H * dv * dm

    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dims.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {synth.WORKLOADS[args.workload].description}",
            "global_batch": B,
            "tokens": T,
            "layers": len(w.layers),
            "seq_len": f"{int(w.lengths().min())}..{int(w.lengths().max())}",
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "attn_kernel (fused pointwise attention, one layer)",
            "bound": "mfma",
            "achieved": attn_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": attn_tflops / peak,
            "traffic": load_traffic(args.workload),
            "launch_ms": attn_ms,
            "flop_per_launch": attn_flop,
            "pairs_per_launch": pairs,
        },
        "gate_roofline": {
            "kernel": "gate_kernel (LayerNorm over H*dv, times U; one layer)",
            "bound": "hbm",
            "achieved": gate_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gate_gbs / PEAK_HBM_GBS,
            "launch_ms": gate_ms,
            "bytes_per_launch": gate_bytes,
        },
        "stages_ms_per_layer": {
            "proj (ln_in + f1 GEMM + SiLU)": proj_ms,
            "attn (attention kernel; plan built once per step)": attn_ms,
            "out (gate + f2 GEMM + residual)": out_ms,
            "proj_tflops": proj_flop / (proj_ms * 1e-3) / 1e12,
            "f2_tflops_excl_gate": f2_flop / (max(out_ms - gate_ms, 1e-6) * 1e-3) / 1e12,
        },
        "layer_tokens_per_s": T * len(w.layers) / (ms_step * 1e-3),
    }
    if not args.minimal:
        rec.update({
            "backward": {
                "what": "hstu_layer_bwd of layer 1: forward recompute, then dx and every parameter gradient",
                "ms": bwd_ms,
                "tokens_per_s": T / (bwd_ms * 1e-3),
                "ratio_to_forward_layer": bwd_ms / (ms_step / len(w.layers)),
                "saved_activations": {
                    "what": "hstu_layer_fwd_train then hstu_layer_bwd with HSTU_SAVED_FWD (no recompute)",
                    "fwd_train_ms": train_fwd_ms,
                    "bwd_ms": train_ms - train_fwd_ms,
                    "step_ms": train_ms,
                    "step_tokens_per_s": T / (train_ms * 1e-3),
                },
            },
            "type_bias": {
                "what": "hstu_attn_fwd of layer 1 with a 2-type token-type term (interleaved content/action)",
                "launch_ms": typed_ms,
                "untyped_launch_ms": attn_ms,
                "overhead": typed_ms / attn_ms - 1.0,
                "tflops": attn_flop / (typed_ms * 1e-3) / 1e12,
            },
        })
    if not args.no_cand and not args.minimal:
        rec["cand_inference"] = cand_inference(torch, _lib, layer, synth)
        rec["stochastic_length"] = sl_repack(torch, _lib)
    if not args.no_configs and not args.minimal:
        rec["configs"] = {n: config_measure(torch, _lib, layer, synth, n) for n in CONFIGS}
    if not args.no_cpu and not args.minimal:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        # same workload and unit: the GPU's tokens/s over the oracle's
        rec["cpu_baseline"]["gpu_over_cpu"] = rec["value"] / rec["cpu_baseline"]["value"]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
