"""Device-side helpers above the C ABI: move a synthetic workload to the GPU and
run one layer or a stack of layers through hstu_layer_fwd.

The stack is a plain loop over hstu_layer_fwd calls (each layer's output is
the next layer's input, residual inside the layer), sharing one workspace;
layers after the first pass HSTU_REUSE_PLAN, since the attention plan depends
only on the batch metadata.
"""

from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

from . import _lib


def to_device(w, device="cuda") -> Dict[str, object]:
    """Device tensors for a synth.Workload (bf16 values are exact)."""
    dt = torch.bfloat16 if w.dims.dtype == "bf16" else torch.float32
    d = {
        "x": torch.from_numpy(np.ascontiguousarray(w.x)).to(device=device, dtype=dt),
        "offsets": torch.from_numpy(np.ascontiguousarray(w.offsets)).to(device),
        "timestamps": torch.from_numpy(np.ascontiguousarray(w.timestamps)).to(device),
        "num_candidates": (None if w.num_candidates is None else
                           torch.from_numpy(np.ascontiguousarray(w.num_candidates)).to(device)),
        "layers": [{k: torch.from_numpy(np.ascontiguousarray(v)).to(device=device, dtype=dt)
                    for k, v in prm.items()} for prm in w.layers],
        "token_types": (None if getattr(w, "token_types", None) is None else
                        torch.from_numpy(np.ascontiguousarray(w.token_types)).to(device)),
    }
    return d


class HSTUStack:
    """A stack of HSTU layers sharing one workspace; forward() enqueues
    len(layers) hstu_layer_fwd calls on torch's current stream."""

    def __init__(self, dims, layers: List[Dict[str, torch.Tensor]], flags_extra: int = 0):
        self.desc = _lib.make_desc(dims, flags_extra)
        # every layer after the first reuses the first layer's attention plan
        self.desc_reuse = _lib.make_desc(dims, flags_extra | _lib.HSTU_REUSE_PLAN)
        self.layers = layers
        self._weights = [_lib.make_weights(p) for p in layers]
        self._tables = [_lib.make_tables(p) for p in layers]
        self._ws: Optional[torch.Tensor] = None
        self._bufs: List[torch.Tensor] = []
        self._types: Optional[torch.Tensor] = None

    def workspace(self, T: int, B: int, device) -> torch.Tensor:
        need = _lib.workspace_size(self.desc, T, B)
        if self._ws is None or self._ws.numel() < need or self._ws.device != torch.device(device):
            self._ws = _lib.alloc_workspace(need, device)
        return self._ws

    def forward(self, x, offsets, timestamps, num_candidates=None, out=None,
                token_types=None) -> torch.Tensor:
        """token_types: [T] uint8 when the layers have a type table."""
        T, B = x.shape[0], offsets.shape[0] - 1
        ws = self.workspace(T, B, x.device)
        if token_types is not self._types:
            self._types = token_types
            self._tables = [_lib.make_tables(p, token_types) for p in self.layers]
        if len(self._bufs) != 2 or self._bufs[0].shape != x.shape or self._bufs[0].dtype != x.dtype:
            self._bufs = [torch.empty_like(x), torch.empty_like(x)]
        h = x
        for n, prm in enumerate(self.layers):
            last = n == len(self.layers) - 1
            dst = out if (last and out is not None) else self._bufs[n % 2]
            _lib.layer_fwd(self.desc if n == 0 else self.desc_reuse, h, offsets, timestamps,
                           num_candidates, prm, out=dst, workspace=ws, weights=self._weights[n],
                           tables=self._tables[n])
            h = dst
        return h


# ------------------------------------------------------------ cached ranking
def split_history(offsets: np.ndarray, num_candidates: Optional[np.ndarray]):
    """Host-side index arithmetic of a packed batch whose sequences end in
    candidates: returns (history rows, history offsets, candidate rows,
    candidate offsets, per-sequence candidate counts), all int64 NumPy."""
    off = np.asarray(offsets, np.int64)
    B = len(off) - 1
    L = np.diff(off)
    m = np.zeros(B, np.int64) if num_candidates is None else \
        np.minimum(np.maximum(np.asarray(num_candidates, np.int64), 0), L)
    n = L - m
    hrows = np.concatenate([np.arange(off[b], off[b] + n[b]) for b in range(B)] + [np.zeros(0, np.int64)])
    crows = np.concatenate([np.arange(off[b] + n[b], off[b + 1]) for b in range(B)] + [np.zeros(0, np.int64)])
    hoff = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    coff = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    return hrows.astype(np.int64), hoff, crows.astype(np.int64), coff, m


def candidate_microbatches(cand_offsets: np.ndarray, per_seq: int):
    """Splits every sequence's candidates (rows cand_offsets[b] ..
    cand_offsets[b+1]-1 of the packed candidates) into consecutive groups of at
    most `per_seq`; yields (rows, offsets) per micro-batch, sequences with no
    candidates left contributing empty ranges."""
    coff = np.asarray(cand_offsets, np.int64)
    m = np.diff(coff)
    nmb = int((m.max() + per_seq - 1) // per_seq) if len(m) and m.max() > 0 else 0
    for k in range(nmb):
        lo = np.minimum(m, k * per_seq)
        hi = np.minimum(m, (k + 1) * per_seq)
        rows = np.concatenate([np.arange(coff[b] + lo[b], coff[b] + hi[b]) for b in range(len(m))])
        yield rows.astype(np.int64), np.concatenate([[0], np.cumsum(hi - lo)]).astype(np.int64)


class CachedRanker:
    """Candidate scoring against a cached history for a stack of layers.

    encode_history() runs the stack over the history rows alone through the
    stage entry points and keeps every layer's K and V of those rows (history
    rows never see candidates, so these are the K, V of the full batch's history
    rows).  score() then pushes one micro-batch of candidates through every layer
    with hstu_cand_fwd against that layer's cache.  Needs HSTU_CAND_SHARED_POS
    (the dims' cand_shared_pos)."""

    def __init__(self, dims, layers: List[Dict[str, torch.Tensor]], flags_extra: int = 0):
        self.desc = _lib.make_desc(dims, flags_extra)
        self.layers = layers
        self._weights = [_lib.make_weights(p) for p in layers]
        self._tables = [_lib.make_tables(p) for p in layers]
        self.cache: List[Dict[str, torch.Tensor]] = []
        self._ws: Optional[torch.Tensor] = None

    def encode_history(self, x_hist, hist_offsets, hist_ts, need_output: bool = False,
                       hist_types=None):
        """Fills the per-layer K/V cache.  The last layer's attention and output
        stage only matter for the history's own output, returned when
        need_output (else None)."""
        self.hist_offsets, self.hist_ts, self.hist_types = hist_offsets, hist_ts, hist_types
        self.cache = []
        h = x_hist
        for n, prm in enumerate(self.layers):
            acts = _lib.proj_fwd(self.desc, h, prm)
            self.cache.append({"k": acts["k"], "v": acts["v"]})
            if n == len(self.layers) - 1 and not need_output:
                return None
            _lib.attn_fwd(self.desc, hist_offsets, hist_ts, None, prm, acts, token_types=hist_types)
            h, _ = _lib.out_fwd(self.desc, h, prm, acts)
        return h

    def score(self, x_cand, cand_offsets, cand_ts, num_candidates, out=None,
              cand_types=None) -> torch.Tensor:
        """The last layer's output rows of one candidate micro-batch;
        num_candidates[b] counts the sequence's candidates over all micro-batches."""
        Tc, B = x_cand.shape[0], cand_offsets.shape[0] - 1
        need = _lib.cand_workspace_size(self.desc, Tc, self.hist_ts.shape[0], B)
        if self._ws is None or self._ws.numel() < need or self._ws.device != x_cand.device:
            self._ws = _lib.alloc_workspace(need, x_cand.device)
        h = x_cand
        for n, prm in enumerate(self.layers):
            last = n == len(self.layers) - 1
            dst = out if (last and out is not None) else torch.empty_like(x_cand)
            tables = self._tables[n] if cand_types is None else \
                _lib.make_tables(prm, cand_types, self.hist_types)
            _lib.cand_fwd(self.desc, h, cand_offsets, cand_ts, num_candidates, self.hist_offsets,
                          self.hist_ts, self.cache[n]["k"], self.cache[n]["v"], prm, out=dst,
                          workspace=self._ws, weights=self._weights[n], tables=tables)
            h = dst
        return h
