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

    def workspace(self, T: int, B: int, device) -> torch.Tensor:
        need = _lib.workspace_size(self.desc, T, B)
        if self._ws is None or self._ws.numel() < need or self._ws.device != torch.device(device):
            self._ws = _lib.alloc_workspace(need, device)
        return self._ws

    def forward(self, x, offsets, timestamps, num_candidates=None, out=None) -> torch.Tensor:
        T, B = x.shape[0], offsets.shape[0] - 1
        ws = self.workspace(T, B, x.device)
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
