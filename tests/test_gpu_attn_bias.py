"""The attention kernel's own bias selection against the oracle's indices.

hstu_debug_attn_bias runs the forward attention kernel's block enumeration,
its per-(wave, key block) weight-mode classification (one time bucket per row,
two buckets split by a threshold, the 32-bit exact path, the 64-bit path) and
its per-pair bias lookup, and writes the bias each visited pair receives.  With
tables whose entries are distinct integers, time[h][b] in [0, 256) and
pos[h][p] = 512 (p + 1), every (position bucket, time bucket) pair has its own
sum, exact in bf16 and fp32, so the written bias names both buckets the
kernel used.  These must equal the oracle's bp(i, j) and bt(i, j)
(oracle.index_dump; page "4.4 Scaling Recommendation Models", section
"Generative Recommenders and HSTU", the bullets under the second equation;
page "HSTU: The First Exploration of the Scaling Law", 7.1.4 Innovation 1)
for every attended pair, and every masked pair must be NaN or never visited.
"""

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import _lib, layer, synth
from oracle import hstu_oracle as O

from edge_workloads import bucket_edge_workload, edge_workload
from gpu_helpers import say

NEG_LOG2E = -1.4426950408889634


def _decodable_tables(w):
    d = w.dims
    assert d.time_buckets <= 256 and d.pos_buckets <= 255
    h = np.arange(d.num_heads)[:, None]
    time_tab = ((np.arange(d.time_buckets)[None, :] + 17 * h) % 256).astype(np.float32)
    pos_tab = np.ascontiguousarray(np.broadcast_to(512.0 * (np.arange(d.pos_buckets)[None, :] + 1),
                                                   (d.num_heads, d.pos_buckets)), dtype=np.float32)
    return pos_tab, time_tab


def _rows(w, rng, extra=3):
    """Per sequence: its first rows, the 32-row wave and 128-row tile edges,
    the last history row and the first candidates, the last row, and a few
    random ones."""
    out = []
    for b in range(w.B):
        L = int(w.offsets[b + 1] - w.offsets[b])
        if L == 0:
            continue
        nh = L - (0 if w.num_candidates is None else int(w.num_candidates[b]))
        cand = {0, 1, 31, 32, 63, 64, 127, 128, 129, nh - 1, nh, nh + 1, L - 1}
        cand.update(rng.integers(0, L, extra).tolist())
        out += [(b, i) for i in sorted(c for c in cand if 0 <= c < L)]
    return out


def _workload(name):
    if name == "edge_wrap":
        w = edge_workload("bf16_s1")
        ts = w.timestamps.copy()
        ts[3] = -(1 << 62)          # int64-wrapping differences
        ts[4] = (1 << 62) + 5
        w.timestamps = ts
        return w
    if name == "edge_fp32":
        return edge_workload("fp32")
    if name.startswith("bucket_edges"):
        s = int(name[-1])
        return bucket_edge_workload(s, 129 if s else 9)
    return synth.make_workload(name, n_layers=1)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["edge_wrap", "edge_fp32", "bucket_edges_s0", "bucket_edges_s1",
                                  "bucket_edges_s2", "small_fp32", "zipf_bf16", "ranking_cand",
                                  "sl_train", "len4k", "stack8_long"])
def test_attention_kernel_buckets_match_oracle(name):
    w = _workload(name)
    rng = np.random.default_rng(3)
    rows = _rows(w, rng)
    max_len = int(np.max(np.diff(w.offsets)))
    say(f"attention bias {name}: {len(rows)} rows, keys up to {max_len}, "
        f"P={w.dims.pos_buckets} NB={w.dims.time_buckets} s={w.dims.time_sub_bits}")
    pos_tab, time_tab = _decodable_tables(w)
    dev = layer.to_device(w)
    tdt = _lib.torch_dtype(_lib.make_desc(w.dims))
    prm = {"pos_table": torch.from_numpy(pos_tab).to(tdt).cuda(),
           "time_table": torch.from_numpy(time_tab).to(tdt).cuda()}
    slot = np.full(w.T, -1, np.int32)
    for n, (b, i) in enumerate(rows):
        slot[w.offsets[b] + i] = n
    desc = _lib.make_desc(w.dims)
    got = _lib.debug_attn_bias(desc, dev["offsets"], dev["timestamps"], dev["num_candidates"], prm,
                               torch.from_numpy(slot).cuda(), len(rows), max_len)
    torch.cuda.synchronize()
    check_biases(w, rows, got.cpu().numpy(), pos_tab, time_tab)


def check_biases(w, rows, got, pos_tab, time_tab):
    """got [H, len(rows), max_len]: the kernel's biases times -log2 e."""
    got = got.astype(np.float64) / NEG_LOG2E
    qr, kr, sl, jj = [], [], [], []
    for n, (b, i) in enumerate(rows):
        s0, L = int(w.offsets[b]), int(w.offsets[b + 1] - w.offsets[b])
        qr.append(np.full(L, s0 + i))
        kr.append(s0 + np.arange(L))
        sl.append(np.full(L, n))
        jj.append(np.arange(L))
    qr, kr, sl, jj = map(np.concatenate, (qr, kr, sl, jj))
    ref = O.index_dump(w.offsets, w.timestamps, w.num_candidates, np.stack([qr, kr], 1), w.dims)
    att = ref["mask"] == 1
    g = got[:, sl, jj]                                         # [H, pairs]
    exp = time_tab[:, ref["bt"]] + pos_tab[:, ref["bp"]]       # [H, pairs]
    ga, ea = g[:, att], exp[:, att]
    bad = ~(np.abs(ga - ea) < 0.25)
    if bad.any():
        lines = []
        for h, k in np.argwhere(bad)[:8]:
            p = np.flatnonzero(att)[k]
            v = int(round(ga[h, k])) if np.isfinite(ga[h, k]) else -1
            lines.append(f"head {h}, seq {ref['b'][p]} i {ref['i'][p]} j {ref['j'][p]}: kernel {ga[h, k]:.3f} "
                         f"(bt {(v % 512 - 17 * h) % 256}, bp {v // 512 - 1}), oracle bt {ref['bt'][p]} "
                         f"bp {ref['bp'][p]}")
        raise AssertionError(f"{bad.sum()} of {bad.size} attended (head, pair)s with the wrong bias:\n  "
                             + "\n  ".join(lines))
    gm = g[:, ~att]
    assert np.all(np.isnan(gm) | np.isinf(gm)), "a masked pair was given a bias"
    say(f"  {int(att.sum())} attended and {int((~att).sum())} masked pairs per head agree")
