"""Gradients of one HSTU layer, float64 PyTorch autograd on the CPU — the
oracle of the backward pass.  TEST INFRASTRUCTURE ONLY.

The forward is the definition of oracle/hstu_oracle.py (pages and readings
listed there: "4.4 Scaling Recommendation Models", "Generative Recommenders
and HSTU" and its "Code" sketch; "HSTU: The First Exploration of the Scaling
Law", 7.1.4-7.1.5), written again with torch float64 operations so that
autograd differentiates it: gradients are those of L = sum(y * dy) with
respect to x and every parameter.  The integer indexing (positions, buckets,
mask) comes from oracle/hstu_oracle.py.  Training with this layer is the
pages' setting ([SRM] "Reported results" compares training cost; [FRC]
7.1.5 trains with stochastic length).  Pins (tests/test_grad_pins.py): the
forward equals the NumPy oracle's, and central finite differences in float64
match every gradient on tiny inputs.
"""

from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

from oracle import hstu_oracle as O

PARAMS = ("w1", "b1", "w2", "b2", "ln_in_g", "ln_in_b", "ln_av_g", "ln_av_b", "pos_table", "time_table")


def _indices(offsets, timestamps, num_candidates, cfg, b):
    off = np.asarray(offsets, np.int64)
    s0, s1 = int(off[b]), int(off[b + 1])
    L = s1 - s0
    m = 0 if num_candidates is None else int(num_candidates[b])
    nh = L - m
    loc = np.arange(L, dtype=np.int64)
    p = O.positions(loc, nh, cfg.cand_shared_pos)
    ts = np.asarray(timestamps, np.int64)[s0:s1]
    M = O.attend_mask(loc[:, None], loc[None, :], nh)
    bp = O.pos_bucket(p[:, None] - p[None, :], cfg.pos_buckets)
    bt = O.time_bucket(O.wrap_sub_i64(ts[:, None], ts[None, :]), cfg.time_buckets, cfg.time_sub_bits)
    N = L if cfg.norm_len == 0 else cfg.norm_len
    return s0, s1, torch.from_numpy(M), torch.from_numpy(bp), torch.from_numpy(bt), N


def attention(q, k, v, offsets, timestamps, num_candidates, prm, cfg):
    """AV [T, H*dv] from q, k [T, H, dqk] and v [T, H, dv] (torch float64)."""
    T, H, dv = v.shape
    B = len(offsets) - 1
    rows = []
    for b in range(B):
        s0, s1, M, bp, bt, N = _indices(offsets, timestamps, num_candidates, cfg, b)
        if s1 == s0:
            continue
        heads = []
        for h in range(H):
            S = q[s0:s1, h] @ k[s0:s1, h].T + prm["pos_table"][h][bp] + prm["time_table"][h][bt]
            A = torch.where(M, F.silu(S), torch.zeros((), dtype=S.dtype)) / N
            heads.append(A @ v[s0:s1, h])
        rows.append(torch.cat(heads, dim=1))
    return torch.cat(rows, dim=0) if rows else torch.zeros(0, H * dv, dtype=v.dtype)


def attention_grads(q, k, v, dav, offsets, timestamps, num_candidates, prm, cfg):
    """float64 NumPy gradients of sum(AV * dav) with respect to q, k [T, H, dqk],
    v [T, H, dv] and the position and time tables (the attention stage alone)."""
    qt, kt, vt = (torch.tensor(np.asarray(a, np.float64), requires_grad=True) for a in (q, k, v))
    pt = {n: torch.tensor(np.asarray(prm[n], np.float64), requires_grad=True) for n in ("pos_table", "time_table")}
    av = attention(qt, kt, vt, offsets, timestamps, num_candidates, pt, cfg)
    g = torch.autograd.grad((av * torch.from_numpy(np.asarray(dav, np.float64))).sum(),
                            [qt, kt, vt, pt["pos_table"], pt["time_table"]], allow_unused=True)
    names = ("q", "k", "v", "pos_table", "time_table")
    refs = (qt, kt, vt, pt["pos_table"], pt["time_table"])
    return {n: (np.zeros(r.shape) if x is None else x.numpy()) for n, x, r in zip(names, g, refs)}


def forward(x, offsets, timestamps, num_candidates, prm, cfg):
    """y [T, d] as a torch float64 graph; x and prm are torch float64 tensors."""
    T = x.shape[0]
    H, dqk, dv = cfg.num_heads, cfg.dqk, cfg.dv
    xin = F.layer_norm(x, (x.shape[1],), prm["ln_in_g"], prm["ln_in_b"], cfg.ln_eps) if cfg.input_norm else x
    act = F.silu(xin @ prm["w1"].T + prm["b1"])
    c0, c1, c2 = H * dv, 2 * H * dv, 2 * H * dv + H * dqk
    u = act[:, :c0]
    v = act[:, c0:c1].reshape(T, H, dv)
    q = act[:, c1:c2].reshape(T, H, dqk)
    k = act[:, c2:].reshape(T, H, dqk)
    av = attention(q, k, v, offsets, timestamps, num_candidates, prm, cfg)
    z = F.layer_norm(av, (H * dv,), prm["ln_av_g"], prm["ln_av_b"], cfg.ln_eps) * u
    y = z @ prm["w2"].T + prm["b2"]
    return y + x if cfg.residual else y


def layer_grads(x, offsets, timestamps, num_candidates, prm, cfg, dy):
    """float64 NumPy gradients of sum(y * dy): {"x": [T, d], name: like prm[name]}."""
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    pt = {n: torch.tensor(np.asarray(prm[n], np.float64), requires_grad=True) for n in PARAMS}
    y = forward(xt, offsets, timestamps, num_candidates, pt, cfg)
    gy = torch.from_numpy(np.asarray(dy, np.float64))
    names = ["x"] + list(PARAMS)
    grads = torch.autograd.grad((y * gy).sum(), [xt] + [pt[n] for n in PARAMS], allow_unused=True)
    out = {}
    for n, g in zip(names, grads):
        ref = xt if n == "x" else pt[n]
        out[n] = np.zeros(ref.shape) if g is None else g.numpy()
    return out
