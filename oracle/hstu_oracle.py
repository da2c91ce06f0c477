"""HSTU layer forward, float64 NumPy — the oracle.  TEST INFRASTRUCTURE ONLY.

Sources (cited by page title and section):
  [SRM]  page "4.4 Scaling Recommendation Models": section "Generative
         Recommenders and HSTU" — the three layer equations (split of the
         SiLU-activated f1 output into U, V, Q, K; AV = SiLU(QK^T + rab) V;
         Y = f2(Norm(AV) * U)), the bullets under them (pointwise SiLU weights
         with a constant normaliser such as the sequence length; gating in
         place of an FFN; a bias on position and time difference), the
         "Efficiency tricks" paragraph (variable-length kernels; candidates
         appended to the history that see the history but not each other);
         section "Code" (the HSTULayer sketch: LayerNorm before f1, f1 chunked
         as u, v, q, k, per-head bias added to q k^T, lower-triangular mask
         including the diagonal, division by n, LayerNorm over the merged
         heads, gate by u, f2, residual add).
  [FRC]  page "HSTU: The First Exploration of the Scaling Law": 7.1.4
         Innovation 1 (pointwise aggregation, LayerNorm(AV) * U), Innovation 2
         (bias from p_i - p_j and t_i - t_j); 7.1.5 M-FALCON layer 1 (batched
         candidates under a mask that hides candidates from each other).

Readings where the pages are silent or disagree (each is a flag or parameter):
  * normaliser N_b = L_b, the whole jagged sequence's length (norm_len > 0
    replaces it by a constant);
  * no 1/sqrt(d) scale on q.k;
  * input LayerNorm and residual present (flags), LayerNorm biased variance,
    eps = cfg.ln_eps (value not on the pages: parity unpinned for eps);
  * rab = pos_table[h, clamp(p_i - p_j, -R, R) + R] + time_table[h, bt(t_i - t_j)],
    R = (P - 1) / 2;
  * candidate positions: p(i) = min(i, n_b) when cand_shared_pos (every
    candidate sits at the next position after the history), else p(i) = i;
  * time bucket: int64 seconds, dt = t_query - t_key in wrapping two's-
    complement int64; dt <= 0 -> 0; else with k = floor(log2 dt),
    bt = min(NB - 1, 1 + k * 2^s + (the s bits below dt's leading one));
  * mask M_ij = (j <= i) and (j < n_b or j == i): causal with the diagonal,
    candidates see the history and themselves only;
  * token types ([FRC] 7.1.4 Innovation 2: the bias also depends on the two
    tokens' types, content or action): when cfg.num_types > 0 the bias gains
    the additive per-head term type_table[h, type_i, type_j] (query type
    first), one more table next to the position and time tables.

Pins (tests/): brute-force scalar loops (oracle/brute.py); an independent
dense torch formulation of the [SRM] "Code" layer; closed forms (prefix sums,
single-token sequences, constant rows); invariants (causality, batch
independence, candidate independence and permutation, M-FALCON equivalence);
exhaustive integer checks of the bucket and row-index functions against
second formulations and the hand-derived fixture tests/golden/time_buckets.txt.
"""

from __future__ import annotations

import numpy as np

I64 = np.int64


# ----------------------------------------------------------------- indexing
def token_index(offsets: np.ndarray, T: int):
    """Flat row -> (sequence b, local index i).  Empty sequences own no rows."""
    off = np.asarray(offsets, I64)
    rows = np.arange(T, dtype=I64)
    b = np.searchsorted(off, rows, side="right") - 1
    return b.astype(I64), rows - off[b]


def positions(i: np.ndarray, n_hist: int, shared: bool) -> np.ndarray:
    """Position used by the relative bias: candidates share position n_b."""
    i = np.asarray(i, I64)
    return np.minimum(i, n_hist) if shared else i


def pos_bucket(dp: np.ndarray, num_buckets: int) -> np.ndarray:
    """Relative-position table index: clamp(dp, -R, R) + R with R = (P-1)/2."""
    R = (num_buckets - 1) // 2
    return np.clip(np.asarray(dp, I64), -R, R) + R


def floor_log2(v: np.ndarray) -> np.ndarray:
    """floor(log2 v) for int64 v > 0, by binary search on shifts (exact)."""
    v = np.asarray(v, I64)
    k = np.zeros(v.shape, I64)
    for sh in (32, 16, 8, 4, 2, 1):
        hit = (v >> (k + sh)) > 0
        k = np.where(hit, k + sh, k)
    return k


def time_bucket(dt: np.ndarray, num_buckets: int, sub_bits: int) -> np.ndarray:
    """Log-bucketed time-difference index (see module header)."""
    dt = np.asarray(dt, I64)
    out = np.zeros(dt.shape, I64)
    pos = dt > 0
    d = dt[pos]
    k = floor_log2(d)
    s = sub_bits
    below = np.where(k >= s, d >> np.maximum(k - s, 0), d << np.maximum(s - k, 0))
    sub = below & ((1 << s) - 1)
    out[pos] = np.minimum(num_buckets - 1, 1 + (k << s) + sub)
    return out


def attend_mask(i: np.ndarray, j: np.ndarray, n_hist: int) -> np.ndarray:
    """Causal (diagonal included) + candidates see history and themselves."""
    i = np.asarray(i, I64)
    j = np.asarray(j, I64)
    return (j <= i) & ((j < n_hist) | (j == i))


def type_bias(table_h: np.ndarray, type_q: np.ndarray, type_k: np.ndarray) -> np.ndarray:
    """Token-type term of one head: table_h[type of query, type of key]."""
    return np.asarray(table_h, np.float64)[np.asarray(type_q, I64), np.asarray(type_k, I64)]


def wrap_sub_i64(a, b):
    """a - b in two's-complement int64 (numpy array subtraction wraps)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, I64) - np.asarray(b, I64)


# -------------------------------------------------------------- float parts
def silu(z: np.ndarray, dtype=np.float64) -> np.ndarray:
    """z * sigmoid(z), evaluated so that neither branch overflows."""
    z = np.asarray(z, dtype)
    out = np.empty_like(z)
    p = z >= 0
    out[p] = z[p] / (1.0 + np.exp(-z[p]))
    e = np.exp(z[~p])
    out[~p] = z[~p] * e / (1.0 + e)
    return out


def layer_norm(a: np.ndarray, gamma, beta, eps: float, dtype=np.float64) -> np.ndarray:
    """LayerNorm over the last axis, biased variance, affine gamma/beta."""
    a = np.asarray(a, dtype)
    mu = a.mean(axis=-1, keepdims=True)
    var = ((a - mu) ** 2).mean(axis=-1, keepdims=True)
    return (a - mu) / np.sqrt(var + eps) * np.asarray(gamma, dtype) \
        + np.asarray(beta, dtype)


def _f64(a, dtype=np.float64):
    return np.asarray(a, dtype)


# ------------------------------------------------------------------- layer
def project(x, prm, cfg, dtype=np.float64):
    """Steps 1-2: optional input LayerNorm, f1, SiLU, split into U, V, Q, K.

    Returns u [T, H*dv], v [T, H, dv], q [T, H, dqk], k [T, H, dqk].
    Head h owns the contiguous columns h*dh .. h*dh+dh-1 of each block.
    ``dtype``: float64 for parity; float32 only times the same steps.
    """
    x = _f64(x, dtype)
    T = x.shape[0]
    H, dqk, dv = cfg.num_heads, cfg.dqk, cfg.dv
    xin = layer_norm(x, prm["ln_in_g"], prm["ln_in_b"], cfg.ln_eps, dtype) if cfg.input_norm else x
    act = silu(xin @ _f64(prm["w1"], dtype).T + _f64(prm["b1"], dtype), dtype)
    c0, c1, c2 = H * dv, 2 * H * dv, 2 * H * dv + H * dqk
    u = act[:, :c0]
    v = act[:, c0:c1].reshape(T, H, dv)
    q = act[:, c1:c2].reshape(T, H, dqk)
    k = act[:, c2:].reshape(T, H, dqk)
    return u, v, q, k


def attention(q, k, v, offsets, timestamps, num_candidates, prm, cfg, rows=None,
              row_chunk: int = 256, token_types=None, dtype=np.float64):
    """Step 3: AV_i^h = (1/N_b) sum_{j: M_ij} SiLU(q_i.k_j + rab_ij^h) v_j^h.

    Returns AV [len(rows), H*dv] for the requested flat rows (all rows when
    ``rows`` is None).  Query rows are processed a chunk at a time only to
    bound memory; each row's sum is one matrix product over keys 0..i.
    With cfg.num_types > 0, rab gains type_table[h, type_i, type_j]
    (token_types: one type per flat row).  ``dtype``: float64 for parity;
    float32 only times the same steps.
    """
    typed = getattr(cfg, "num_types", 0) > 0
    if typed:
        ty_all = np.asarray(token_types, I64)
        wy = _f64(prm["type_table"], dtype)
    T, H, dqk = q.shape
    dv = v.shape[2]
    off = np.asarray(offsets, I64)
    ts_all = np.asarray(timestamps, I64)
    B = len(off) - 1
    q, k, v = _f64(q, dtype), _f64(k, dtype), _f64(v, dtype)
    wp = _f64(prm["pos_table"], dtype)
    wt = _f64(prm["time_table"], dtype)
    if rows is None:
        rows = np.arange(T, dtype=I64)
    rows = np.asarray(rows, I64)
    out = np.zeros((len(rows), H, dv), dtype)
    rb, _ = token_index(off, T)
    row_seq = rb[rows]
    for b in range(B):
        s0, s1 = int(off[b]), int(off[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        sel = np.nonzero(row_seq == b)[0]
        if len(sel) == 0:
            continue
        m = 0 if num_candidates is None else int(num_candidates[b])
        n_hist = L - m
        N = L if cfg.norm_len == 0 else cfg.norm_len
        loc = np.arange(L, dtype=I64)
        p = positions(loc, n_hist, cfg.cand_shared_pos)
        ts = ts_all[s0:s1]
        for c0 in range(0, len(sel), row_chunk):
            idx = sel[c0:c0 + row_chunk]
            ii = rows[idx] - s0
            kend = int(ii.max()) + 1
            jj = loc[:kend]
            M = attend_mask(ii[:, None], jj[None, :], n_hist)
            bp = pos_bucket(p[ii][:, None] - p[jj][None, :], cfg.pos_buckets)
            bt = time_bucket(wrap_sub_i64(ts[ii][:, None], ts[jj][None, :]),
                             cfg.time_buckets, cfg.time_sub_bits)
            for h in range(H):
                S = q[s0 + ii, h] @ k[s0:s0 + kend, h].T + wp[h][bp] + wt[h][bt]
                if typed:
                    S = S + type_bias(wy[h], ty_all[s0 + ii][:, None], ty_all[s0 + jj][None, :])
                A = np.where(M, silu(S, dtype), dtype(0.0)) / dtype(N)
                out[idx, h] = A @ v[s0:s0 + kend, h]
    return out.reshape(len(rows), H * dv)


def layer_forward(x, offsets, timestamps, num_candidates, prm, cfg, rows=None, token_types=None,
                  dtype=np.float64):
    """One HSTU layer.  Returns a dict of taps:

    u, v, q, k   projections for all rows;
    av           attention output (heads merged) for ``rows``;
    ln_av        LayerNorm(av) over the H*dv axis;
    z            ln_av * u;
    y            f2(z) (+ x when cfg.residual) for ``rows``.
    ``dtype``: float64 for parity; float32 only times the same steps.
    """
    x = _f64(x, dtype)
    T = x.shape[0]
    u, v, q, k = project(x, prm, cfg, dtype=dtype)
    sel = np.arange(T, dtype=I64) if rows is None else np.asarray(rows, I64)
    av = attention(q, k, v, offsets, timestamps, num_candidates, prm, cfg, rows=sel,
                   token_types=token_types, dtype=dtype)
    out = gate_and_project(av, u[sel], x[sel], prm, cfg, dtype=dtype)
    return {"u": u, "v": v, "q": q, "k": k, "av": av, "ln_av": out["ln_av"], "z": out["z"],
            "y": out["y"], "rows": sel}


def gate_and_project(av, u, x, prm, cfg, dtype=np.float64):
    """Steps 4-5: Z = LayerNorm(AV) * U over the merged heads, Y = Z W2^T + b2
    (+ x when cfg.residual).  Rows of av, u and x correspond one to one."""
    ln_av = layer_norm(_f64(av, dtype), prm["ln_av_g"], prm["ln_av_b"], cfg.ln_eps, dtype)
    z = ln_av * _f64(u, dtype)
    y = z @ _f64(prm["w2"], dtype).T + _f64(prm["b2"], dtype)
    if cfg.residual:
        y = y + _f64(x, dtype)
    return {"ln_av": ln_av, "z": z, "y": y}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each float64 element, as float64,
    rounding the float64 value directly (8 significant bits)."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                 # a = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: scale m to [128, 256) and round half to even
    return np.ldexp(np.round(m * 256.0), e - 8)


def stack_forward(x, offsets, timestamps, num_candidates, layers, cfg, io_dtype=None,
                  token_types=None):
    """Layers applied in order, each to the previous output (all rows).

    io_dtype="bf16": each layer's output is rounded to bf16 before it becomes
    the next layer's input, as in a stack whose layer inputs and outputs are
    bf16 tensors; every layer's arithmetic stays float64."""
    h = _f64(x)
    for prm in layers:
        h = layer_forward(h, offsets, timestamps, num_candidates, prm, cfg,
                          token_types=token_types)["y"]
        if io_dtype == "bf16":
            h = round_to_bf16(h)
    return h


def index_dump(offsets, timestamps, num_candidates, pairs, cfg):
    """Integer indexing for flat (query row, key row) pairs of one batch.

    Returns int64 arrays b, i, j, bp, bt and the mask bit; pairs whose key row
    is outside the query's sequence get b = -1 and zeros elsewhere.
    """
    off = np.asarray(offsets, I64)
    T = int(off[-1])
    pairs = np.asarray(pairs, I64).reshape(-1, 2)
    rb, ri = token_index(off, T)
    qr, kr = pairs[:, 0], pairs[:, 1]
    b = rb[qr]
    i = ri[qr]
    same = rb[kr] == b
    j = np.where(same, ri[kr], 0)
    L = off[b + 1] - off[b]
    m = np.zeros_like(L) if num_candidates is None else np.asarray(num_candidates, I64)[b]
    n_hist = L - m
    pi = positions(i, n_hist, cfg.cand_shared_pos)
    pj = positions(j, n_hist, cfg.cand_shared_pos)
    bp = pos_bucket(pi - pj, cfg.pos_buckets)
    ts = np.asarray(timestamps, I64)
    bt = time_bucket(wrap_sub_i64(ts[qr], ts[kr]), cfg.time_buckets, cfg.time_sub_bits)
    mk = attend_mask(i, j, n_hist).astype(I64)
    z = np.zeros_like(b)
    return {"b": np.where(same, b, -1), "i": np.where(same, i, z), "j": np.where(same, j, z),
            "bp": np.where(same, bp, z), "bt": np.where(same, bt, z),
            "mask": np.where(same, mk, z)}
