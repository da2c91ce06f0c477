"""Seeded synthetic workloads for the HSTU layer forward.

This module only draws inputs: sequence lengths, timestamps, activations and
layer parameters, with the shapes and distributions of the workloads the HSTU
pages describe.  It holds none of the layer's arithmetic; both the HIP path and
the CPU oracle receive exactly the arrays drawn here.

Workloads (all use seed 0 by default, one ``numpy.random.default_rng(seed)``
per workload, drawn in a fixed order: lengths, stochastic-length subsample
choices, timestamp gaps, candidate request gaps, x, then per layer
W1, b1, W2, b2, position table, time table):

* ``small_fp32``   fp32, 4 sequences, lengths uniform in [8, 64], d=64,
                   2 heads x 32/32, 64 octave time buckets.
* ``zipf_bf16``    bf16, 32 sequences, lengths from a truncated power law
                   p(L) ~ L^-1.25 on [64, 1024] (mean ~299), d=256, 4 x 64/64.
* ``ranking_cand`` bf16, 16 sequences, history uniform in [512, 2048] plus
                   512 appended candidates each, d=512, 8 x 64/64.
* ``sl_train``     bf16, 64 sequences of 4096 thinned by stochastic length
                   (alpha=1.6, N=4096), d=512, 8 x 128/128.
* ``stack8_long``  bf16, 8 sequences, lengths uniform in [4096, 8192], d=1024,
                   8 x 128/128, 128 half-octave time buckets, 8 layers.
* ``len4k``        bf16, 16 sequences of exactly 4096, d=512, 8 x 128/128.

Timestamps are int64 seconds: a fixed epoch plus the floor of the cumulative
sum of Exp(mean 60 s) gaps, so they exceed 2^32 and are non-decreasing.  All
candidates of one sequence share one request time: the last history
timestamp plus floor(Exp(mean 60 s)).

Parameters are N(0, 0.02) (drawn in float64, cast to float32, and for bf16
workloads rounded to nearest-even bf16); LayerNorm gains are 1 and offsets 0
unless ``random_ln`` is set, in which case gains are 1 + N(0, 0.1) and
offsets N(0, 0.1).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

EPOCH = 5_000_000_000  # int64 seconds; keeps every timestamp above 2^32
GAP_MEAN_S = 60.0


@dataclass(frozen=True)
class LayerDims:
    """Static description of one HSTU layer (shared by every layer of a stack)."""

    d_model: int
    num_heads: int
    dqk: int
    dv: int
    pos_buckets: int = 129          # odd; relative distance clamped to +-(P-1)/2
    time_buckets: int = 64          # log-bucketed time-difference table size
    time_sub_bits: int = 0          # sub-octave resolution bits
    dtype: str = "bf16"             # "bf16" or "fp32"
    input_norm: bool = True         # LayerNorm on x before f1
    residual: bool = True           # y = x + f2(...)
    cand_shared_pos: bool = True    # candidates all sit at position n_b
    ln_eps: float = 1e-5
    norm_len: int = 0               # 0 => divide by the sequence length L_b
    num_types: int = 0              # > 0: token-type bias table [H, types, types]

    @property
    def n1(self) -> int:
        return 2 * self.num_heads * (self.dqk + self.dv)


@dataclass
class Workload:
    name: str
    dims: LayerDims
    x: np.ndarray                   # [T, d] float32 (bf16-exact for bf16)
    offsets: np.ndarray             # [B+1] int64
    timestamps: np.ndarray          # [T] int64
    num_candidates: Optional[np.ndarray]  # [B] int32 or None
    layers: List[Dict[str, np.ndarray]] = field(default_factory=list)
    token_types: Optional[np.ndarray] = None  # [T] uint8 when dims.num_types > 0

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def B(self) -> int:
        return len(self.offsets) - 1

    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)

    def sub_batch(self, seqs) -> "Workload":
        """The workload restricted to sequences ``seqs`` (re-packed, same params)."""
        seqs = [int(s) for s in seqs]
        xs, ts, lens = [], [], []
        for s in seqs:
            a, b = int(self.offsets[s]), int(self.offsets[s + 1])
            xs.append(self.x[a:b])
            ts.append(self.timestamps[a:b])
            lens.append(b - a)
        off = np.zeros(len(seqs) + 1, np.int64)
        off[1:] = np.cumsum(lens)
        nc = None
        if self.num_candidates is not None:
            nc = self.num_candidates[seqs].copy()
        ty = None
        if self.token_types is not None:
            ty = np.concatenate([self.token_types[int(self.offsets[s]):int(self.offsets[s + 1])]
                                 for s in seqs] + [np.zeros(0, np.uint8)])
        d = self.dims.d_model
        return Workload(self.name + "[sub]", self.dims,
                        np.concatenate(xs) if xs else np.zeros((0, d), np.float32),
                        off,
                        np.concatenate(ts) if ts else np.zeros((0,), np.int64),
                        nc, self.layers, ty)


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dims: LayerDims
    batch: int
    lengths: str                    # "uniform", "powerlaw", "fixed", "sl"
    lo: int = 0
    hi: int = 0
    candidates: int = 0
    n_layers: int = 1
    sl_alpha: float = 2.0
    sl_max: int = 0
    description: str = ""


WORKLOADS: Dict[str, WorkloadSpec] = {
    "small_fp32": WorkloadSpec(
        "small_fp32", LayerDims(64, 2, 32, 32, dtype="fp32"), 4, "uniform", 8, 64,
        description="fp32, B=4, L~U[8,64], d=64, 2x32/32, causal"),
    "zipf_bf16": WorkloadSpec(
        "zipf_bf16", LayerDims(256, 4, 64, 64), 32, "powerlaw", 64, 1024,
        description="bf16, B=32, L~powerlaw(1.25) on [64,1024], d=256, 4x64/64, causal"),
    "ranking_cand": WorkloadSpec(
        "ranking_cand", LayerDims(512, 8, 64, 64), 16, "uniform", 512, 2048, candidates=512,
        description="bf16, B=16, history~U[512,2048] + 512 candidates, d=512, 8x64/64"),
    "sl_train": WorkloadSpec(
        "sl_train", LayerDims(512, 8, 128, 128), 64, "sl", 4096, 4096, sl_alpha=1.6, sl_max=4096,
        description="bf16, B=64, 4096 thinned by stochastic length a=1.6, d=512, 8x128/128"),
    "stack8_long": WorkloadSpec(
        "stack8_long", LayerDims(1024, 8, 128, 128, time_buckets=128, time_sub_bits=1), 8,
        "uniform", 4096, 8192, n_layers=8,
        description="bf16, 8 layers, B=8, L~U[4096,8192], d=1024, 8x128/128, 128 time buckets"),
    "len4k": WorkloadSpec(
        "len4k", LayerDims(512, 8, 128, 128), 16, "fixed", 4096, 4096,
        description="bf16, B=16, L=4096, d=512, 8x128/128, causal"),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(a.shape)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, np.float64).astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def _draw_lengths(spec: WorkloadSpec, rng, batch: int) -> np.ndarray:
    if spec.lengths == "uniform":
        return rng.integers(spec.lo, spec.hi, size=batch, endpoint=True).astype(np.int64)
    if spec.lengths == "fixed":
        return np.full(batch, spec.lo, np.int64)
    if spec.lengths == "sl":
        return np.full(batch, spec.sl_max, np.int64)
    if spec.lengths == "powerlaw":
        # inverse-CDF draw from p(L) ~ L^-1.25 on [lo, hi), floored
        e = 1.0 - 1.25
        u = rng.random(batch)
        a, b = spec.lo ** e, spec.hi ** e
        return np.floor((a + u * (b - a)) ** (1.0 / e)).astype(np.int64)
    raise ValueError(spec.lengths)


def stochastic_length_keep(n: int, n_max: int, alpha: float, u: float) -> int:
    """Length kept by stochastic length for a sequence of n tokens.

    Input shaping only (the HSTU paper's training-time sampler): when n exceeds
    n_max^(alpha/2) the sequence is cut to floor(n_max^(alpha/2)) tokens with
    probability 1 - n_max^alpha / n^2 (u is the uniform draw that decides);
    alpha = 2 never cuts.
    """
    thr = n_max ** (alpha / 2.0)
    if n > thr and u < 1.0 - (n_max ** alpha) / float(n * n):
        return int(np.floor(thr))
    return n


def draw_layer_params(rng, dims: LayerDims, random_ln: bool = False) -> Dict[str, np.ndarray]:
    d, H, dqk, dv = dims.d_model, dims.num_heads, dims.dqk, dims.dv
    n1, hdv = dims.n1, H * dv
    sd = 0.02
    p = {
        "w1": _cast(rng.normal(0.0, sd, (n1, d)), dims.dtype),
        "b1": _cast(rng.normal(0.0, sd, (n1,)), dims.dtype),
        "w2": _cast(rng.normal(0.0, sd, (d, hdv)), dims.dtype),
        "b2": _cast(rng.normal(0.0, sd, (d,)), dims.dtype),
        "pos_table": _cast(rng.normal(0.0, sd, (H, dims.pos_buckets)), dims.dtype),
        "time_table": _cast(rng.normal(0.0, sd, (H, dims.time_buckets)), dims.dtype),
    }
    if random_ln:
        p["ln_in_g"] = _cast(1.0 + rng.normal(0.0, 0.1, (d,)), dims.dtype)
        p["ln_in_b"] = _cast(rng.normal(0.0, 0.1, (d,)), dims.dtype)
        p["ln_av_g"] = _cast(1.0 + rng.normal(0.0, 0.1, (hdv,)), dims.dtype)
        p["ln_av_b"] = _cast(rng.normal(0.0, 0.1, (hdv,)), dims.dtype)
    else:
        p["ln_in_g"] = np.ones(d, np.float32)
        p["ln_in_b"] = np.zeros(d, np.float32)
        p["ln_av_g"] = np.ones(hdv, np.float32)
        p["ln_av_b"] = np.zeros(hdv, np.float32)
    if dims.num_types > 0:   # drawn last, so untyped workloads keep their draws
        nt = dims.num_types
        p["type_table"] = _cast(rng.normal(0.0, sd, (H, nt, nt)), dims.dtype)
    return p


def make_workload(name: str, seed: int = 0, batch: Optional[int] = None,
                  n_layers: Optional[int] = None, random_ln: bool = False,
                  dims: Optional[LayerDims] = None,
                  lengths: Optional[List[int]] = None,
                  candidates: Optional[List[int]] = None) -> Workload:
    """Draw one workload.  ``batch``/``n_layers``/``lengths`` shrink it for tests
    (same distributions); ``dims`` overrides flags such as time buckets."""
    spec = WORKLOADS[name]
    dims = dims or spec.dims
    rng = np.random.default_rng(seed)
    B = spec.batch if batch is None else batch
    L = n_layers if n_layers is not None else spec.n_layers

    # 1. lengths (history lengths when candidates are appended)
    if lengths is not None:
        base_len = np.asarray(lengths, np.int64)
        B = len(base_len)
    else:
        base_len = _draw_lengths(spec, rng, B)
    # 2. stochastic-length subsample choices (input shaping only)
    keep_idx = [None] * B
    if spec.lengths == "sl" and lengths is None:
        for b in range(B):
            u = rng.random()
            kept = stochastic_length_keep(int(base_len[b]), spec.sl_max, spec.sl_alpha, u)
            if kept < base_len[b]:
                keep_idx[b] = np.sort(rng.choice(int(base_len[b]), kept, replace=False))
    # 3. timestamp gaps for the full (un-thinned) histories
    hist_ts = []
    for b in range(B):
        gaps = rng.exponential(GAP_MEAN_S, int(base_len[b]))
        ts = EPOCH + np.floor(np.cumsum(gaps)).astype(np.int64)
        if keep_idx[b] is not None:
            ts = ts[keep_idx[b]]
        hist_ts.append(ts)
    # 4. candidates: one request time per sequence
    if candidates is not None:
        ncand = np.asarray(candidates, np.int64)
    else:
        ncand = np.full(B, spec.candidates, np.int64)
    has_cand = spec.candidates > 0 or candidates is not None
    ts_all = []
    for b in range(B):
        ts = hist_ts[b]
        m = int(ncand[b])
        if has_cand:
            req_gap = int(np.floor(rng.exponential(GAP_MEAN_S)))
            last = int(ts[-1]) if len(ts) else EPOCH
            ts = np.concatenate([ts, np.full(m, last + req_gap, np.int64)])
        ts_all.append(ts)
    lens = np.array([len(t) for t in ts_all], np.int64)
    off = np.zeros(B + 1, np.int64)
    off[1:] = np.cumsum(lens)
    T = int(off[-1])
    timestamps = np.concatenate(ts_all) if B else np.zeros(0, np.int64)
    # 5. activations
    x = _cast(rng.normal(0.0, 1.0, (T, dims.d_model)), dims.dtype)
    # 6. parameters, layer by layer
    layers = [draw_layer_params(rng, dims, random_ln) for _ in range(L)]
    # 7. token types: with two types, the history interleaves content (0) and
    #    action (1) tokens and every candidate is content; other counts draw
    #    uniformly (tests)
    types = None
    if dims.num_types > 0:
        if dims.num_types == 2:
            types = np.zeros(T, np.uint8)
            for b in range(B):
                nh = int(lens[b] - ncand[b]) if has_cand else int(lens[b])
                types[off[b]:off[b] + nh] = np.arange(nh) % 2
        else:
            types = rng.integers(0, dims.num_types, T).astype(np.uint8)
    return Workload(name, dims, x, off, timestamps.astype(np.int64),
                    ncand.astype(np.int32) if has_cand else None, layers, types)


def with_dims(w: Workload, **changes) -> Workload:
    """Same draws, different flags (e.g. residual off)."""
    return dataclasses.replace(w, dims=dataclasses.replace(w.dims, **changes))
