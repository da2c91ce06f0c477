"""Scalar pure-Python HSTU layer for tiny inputs — TEST INFRASTRUCTURE ONLY.

A second, loop-by-loop formulation of the same definition as
oracle/hstu_oracle.py (sources and readings listed there: page "4.4 Scaling
Recommendation Models", section "Generative Recommenders and HSTU" and its
"Code" sketch; page "HSTU: The First Exploration of the Scaling Law", 7.1.4
and 7.1.5).  It shares no helper with the vectorised oracle: every sum is an
explicit loop over Python floats, ⌊log2⌋ comes from int.bit_length, the
sequence of a row from a linear scan, and SiLU from math.exp.
"""

from __future__ import annotations

import math


def _wrap64(v: int) -> int:
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >= (1 << 63) else v


def time_bucket(dt: int, nb: int, s: int) -> int:
    if dt <= 0:
        return 0
    k = dt.bit_length() - 1
    lead_and_below = dt >> (k - s) if k >= s else dt << (s - k)
    sub = lead_and_below - (1 << s)          # drop the leading one
    return min(nb - 1, 1 + k * (1 << s) + sub)


def pos_bucket(dp: int, P: int) -> int:
    R = (P - 1) // 2
    if dp > R:
        dp = R
    if dp < -R:
        dp = -R
    return dp + R


def _sig_mul(z: float) -> float:
    if z >= 0:
        return z / (1.0 + math.exp(-z))
    e = math.exp(z)
    return z * e / (1.0 + e)


def _ln(row, g, b, eps):
    n = len(row)
    mu = 0.0
    for a in row:
        mu += a
    mu /= n
    var = 0.0
    for a in row:
        var += (a - mu) * (a - mu)
    var /= n
    r = 1.0 / math.sqrt(var + eps)
    return [(row[c] - mu) * r * float(g[c]) + float(b[c]) for c in range(n)]


def layer(x, offsets, timestamps, num_candidates, prm, cfg, token_types=None):
    """Returns dict with av, z and y as nested Python lists (all rows).  With
    cfg.num_types > 0 the bias adds type_table[h][type of row t][type of key]."""
    typed = getattr(cfg, "num_types", 0) > 0
    T = len(x)
    d = cfg.d_model
    H, dqk, dv = cfg.num_heads, cfg.dqk, cfg.dv
    W1, b1, W2, b2 = prm["w1"], prm["b1"], prm["w2"], prm["b2"]
    n1 = len(W1)
    # projection, row by row
    act = []
    for t in range(T):
        xr = [float(a) for a in x[t]]
        if cfg.input_norm:
            xr = _ln(xr, prm["ln_in_g"], prm["ln_in_b"], cfg.ln_eps)
        r = []
        for n in range(n1):
            acc = float(b1[n])
            for c in range(d):
                acc += xr[c] * float(W1[n][c])
            r.append(_sig_mul(acc))
        act.append(r)
    U0, V0, Q0, K0 = 0, H * dv, 2 * H * dv, 2 * H * dv + H * dqk

    # sequence membership by linear scan
    seq_of, loc_of = [], []
    B = len(offsets) - 1
    for t in range(T):
        for b in range(B):
            if int(offsets[b]) <= t < int(offsets[b + 1]):
                seq_of.append(b)
                loc_of.append(t - int(offsets[b]))
                break

    av = [[0.0] * (H * dv) for _ in range(T)]
    for t in range(T):
        b = seq_of[t]
        i = loc_of[t]
        s0 = int(offsets[b])
        L = int(offsets[b + 1]) - s0
        m = 0 if num_candidates is None else int(num_candidates[b])
        nh = L - m
        N = L if cfg.norm_len == 0 else cfg.norm_len
        pi = min(i, nh) if cfg.cand_shared_pos else i
        for j in range(L):
            if j > i:
                continue
            if not (j < nh or j == i):
                continue
            pj = min(j, nh) if cfg.cand_shared_pos else j
            bp = pos_bucket(pi - pj, cfg.pos_buckets)
            dt = _wrap64(int(timestamps[t]) - int(timestamps[s0 + j]))
            bt = time_bucket(dt, cfg.time_buckets, cfg.time_sub_bits)
            for h in range(H):
                sc = 0.0
                for c in range(dqk):
                    sc += act[t][Q0 + h * dqk + c] * act[s0 + j][K0 + h * dqk + c]
                sc += float(prm["pos_table"][h][bp]) + float(prm["time_table"][h][bt])
                if typed:
                    sc += float(prm["type_table"][h][int(token_types[t])][int(token_types[s0 + j])])
                w = _sig_mul(sc) / N
                for c in range(dv):
                    av[t][h * dv + c] += w * act[s0 + j][V0 + h * dv + c]

    z, y = [], []
    for t in range(T):
        ln = _ln(av[t], prm["ln_av_g"], prm["ln_av_b"], cfg.ln_eps)
        zr = [ln[c] * act[t][U0 + c] for c in range(H * dv)]
        z.append(zr)
        yr = []
        for n in range(d):
            acc = float(b2[n])
            for c in range(H * dv):
                acc += zr[c] * float(W2[n][c])
            if cfg.residual:
                acc += float(x[t][n])
            yr.append(acc)
        y.append(yr)
    return {"av": av, "z": z, "y": y}
