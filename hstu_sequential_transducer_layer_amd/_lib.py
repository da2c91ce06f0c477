"""ctypes binding of libhstu (include/hstu.h) — argument marshalling only.

Every step of the layer runs in the HIP kernels of libhstu.so; this module
turns torch device tensors into pointers, allocates caller-owned buffers
(workspace, outputs) with torch, and passes torch's current HIP stream.  There
is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu.so")

HSTU_OK, HSTU_ERR_INVALID_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE, HSTU_ERR_DEVICE = range(5)
HSTU_F32, HSTU_BF16 = 0, 1
HSTU_INPUT_NORM, HSTU_RESIDUAL, HSTU_CAND_SHARED_POS, HSTU_VALIDATE = 1, 2, 4, 8
HSTU_REUSE_PLAN = 1 << 4
HSTU_SAVED_FWD = 1 << 5

EXPORTS = [
    "hstu_workspace_size", "hstu_layer_fwd", "hstu_proj_workspace_size", "hstu_proj_fwd",
    "hstu_attn_workspace_size", "hstu_attn_fwd", "hstu_gate_fwd", "hstu_out_fwd",
    "hstu_cand_workspace_size", "hstu_cand_fwd", "hstu_bwd_workspace_size", "hstu_layer_fwd_train", "hstu_layer_bwd",
    "hstu_attn_bwd_workspace_size", "hstu_attn_bwd",
    "hstu_sl_workspace_size", "hstu_sl_sample",
    "hstu_gather_rows", "hstu_debug_indices", "hstu_debug_attn_bias",
    "hstu_status_str", "hstu_last_error", "hstu_layer_fwd_noalloc",
]
NOALLOC_SCRATCH_BYTES = 256 << 20


class HstuDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("dqk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("pos_buckets", ctypes.c_int32), ("time_buckets", ctypes.c_int32),
                ("time_sub_bits", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("flags", ctypes.c_uint32), ("ln_eps", ctypes.c_float),
                ("norm_len", ctypes.c_int32), ("num_types", ctypes.c_int32)]


class HstuWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w1", "b1", "w2", "b2", "ln_in_g", "ln_in_b", "ln_av_g", "ln_av_b")]


class HstuBiasTables(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_void_p), ("time", ctypes.c_void_p),
                ("pos_head_stride", ctypes.c_int32), ("time_head_stride", ctypes.c_int32),
                ("type", ctypes.c_void_p), ("type_head_stride", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("token_types", ctypes.c_void_p),
                ("hist_types", ctypes.c_void_p)]


GRAD_FIELDS = ("w1", "b1", "w2", "b2", "ln_in_g", "ln_in_b", "ln_av_g", "ln_av_b", "pos", "time")


class HstuGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class HstuActivations(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("v", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("av", ctypes.c_void_p), ("av_stats", ctypes.c_void_p)]


class HstuError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hstu status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libhstu.so (built by build_lib.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m hstu_sequential_transducer_layer_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER
    lib.hstu_workspace_size.argtypes = [P(HstuDesc), i64, i32]
    lib.hstu_workspace_size.restype = sz
    lib.hstu_proj_workspace_size.argtypes = [P(HstuDesc), i64]
    lib.hstu_proj_workspace_size.restype = sz
    lib.hstu_attn_workspace_size.argtypes = [P(HstuDesc), i64, i32]
    lib.hstu_attn_workspace_size.restype = sz
    lib.hstu_layer_fwd.argtypes = [P(HstuDesc), vp, vp, i32, i64, vp, vp, P(HstuWeights),
                                   P(HstuBiasTables), vp, vp, sz, vp]
    lib.hstu_layer_fwd_noalloc.argtypes = [P(HstuDesc), vp, vp, i32, i64, vp, vp, P(HstuWeights),
                                           P(HstuBiasTables), vp, vp]
    lib.hstu_proj_fwd.argtypes = [P(HstuDesc), vp, i64, P(HstuWeights), P(HstuActivations),
                                  vp, sz, vp]
    lib.hstu_attn_fwd.argtypes = [P(HstuDesc), vp, i32, i64, vp, vp, P(HstuBiasTables),
                                  P(HstuActivations), vp, sz, vp]
    lib.hstu_out_fwd.argtypes = [P(HstuDesc), vp, i64, P(HstuWeights), P(HstuActivations),
                                 vp, vp, vp]
    lib.hstu_gate_fwd.argtypes = [P(HstuDesc), i64, P(HstuWeights), P(HstuActivations), vp, vp]
    lib.hstu_cand_workspace_size.argtypes = [P(HstuDesc), i64, i64, i32]
    lib.hstu_cand_workspace_size.restype = sz
    lib.hstu_cand_fwd.argtypes = [P(HstuDesc), vp, vp, i32, i64, vp, vp, vp, i64, vp, vp, vp,
                                  P(HstuWeights), P(HstuBiasTables), vp, vp, sz, vp]
    lib.hstu_bwd_workspace_size.argtypes = [P(HstuDesc), i64, i32]
    lib.hstu_bwd_workspace_size.restype = sz
    lib.hstu_layer_fwd_train.argtypes = [P(HstuDesc), vp, vp, i32, i64, vp, vp, P(HstuWeights),
                                         P(HstuBiasTables), vp, vp, sz, vp]
    lib.hstu_layer_bwd.argtypes = [P(HstuDesc), vp, vp, i32, i64, vp, vp, P(HstuWeights), P(HstuBiasTables),
                                   vp, vp, P(HstuGrads), vp, sz, vp]
    lib.hstu_attn_bwd_workspace_size.argtypes = [P(HstuDesc), i64, i32]
    lib.hstu_attn_bwd_workspace_size.restype = sz
    lib.hstu_attn_bwd.argtypes = [P(HstuDesc), vp, i32, i64, vp, vp, P(HstuBiasTables), P(HstuActivations),
                                  vp, vp, vp, vp, vp, sz, vp]
    lib.hstu_sl_workspace_size.argtypes = [i32]
    lib.hstu_sl_workspace_size.restype = sz
    lib.hstu_sl_sample.argtypes = [vp, i32, i64, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.hstu_gather_rows.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp]
    lib.hstu_debug_indices.argtypes = [P(HstuDesc), vp, i32, i64, vp, vp, vp, i64, vp, vp]
    lib.hstu_debug_attn_bias.argtypes = [P(HstuDesc), vp, i32, i64, vp, vp, P(HstuBiasTables), vp, i32, i32, vp,
                                         vp, sz, vp]
    for f in ("hstu_layer_fwd", "hstu_proj_fwd", "hstu_attn_fwd", "hstu_gate_fwd", "hstu_out_fwd",
              "hstu_cand_fwd", "hstu_layer_fwd_train", "hstu_layer_bwd", "hstu_attn_bwd", "hstu_sl_sample",
              "hstu_gather_rows", "hstu_debug_indices", "hstu_debug_attn_bias", "hstu_layer_fwd_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    lib.hstu_status_str.argtypes = [ctypes.c_int]
    lib.hstu_status_str.restype = ctypes.c_char_p
    lib.hstu_last_error.argtypes = []
    lib.hstu_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != HSTU_OK:
        raise HstuError(status, load().hstu_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_desc(dims, flags_extra: int = 0) -> HstuDesc:
    """HstuDesc from any object with the LayerDims attributes."""
    flags = flags_extra
    if dims.input_norm:
        flags |= HSTU_INPUT_NORM
    if dims.residual:
        flags |= HSTU_RESIDUAL
    if dims.cand_shared_pos:
        flags |= HSTU_CAND_SHARED_POS
    return HstuDesc(dims.d_model, dims.num_heads, dims.dqk, dims.dv, dims.pos_buckets,
                    dims.time_buckets, dims.time_sub_bits,
                    HSTU_BF16 if dims.dtype == "bf16" else HSTU_F32, flags,
                    float(dims.ln_eps), int(dims.norm_len), int(getattr(dims, "num_types", 0)))


def torch_dtype(desc: HstuDesc) -> torch.dtype:
    return torch.bfloat16 if desc.dtype == HSTU_BF16 else torch.float32


def make_weights(prm: Dict[str, torch.Tensor]) -> HstuWeights:
    return HstuWeights(*[_ptr(prm.get(n)) for n in
                         ("w1", "b1", "w2", "b2", "ln_in_g", "ln_in_b", "ln_av_g", "ln_av_b")])


def make_tables(prm: Dict[str, torch.Tensor], token_types: Optional[torch.Tensor] = None,
                hist_types: Optional[torch.Tensor] = None) -> HstuBiasTables:
    """Tables of one layer; the token-type fields are filled when the layer
    has a "type_table" ([H, NT, NT], or [NT, NT] shared across heads)."""
    pos, tim = prm["pos_table"], prm["time_table"]
    typ = prm.get("type_table")
    for name, t in (("pos_table", pos), ("time_table", tim), ("type_table", typ)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (rows of the table one after another)")
    tstride = 0
    if typ is not None and typ.dim() == 3:
        tstride = typ.shape[1] * typ.shape[2]
    return HstuBiasTables(_ptr(pos), _ptr(tim),
                          pos.shape[-1] if pos.dim() == 2 else 0,
                          tim.shape[-1] if tim.dim() == 2 else 0,
                          _ptr(typ), tstride, 0, _ptr(token_types), _ptr(hist_types))


def workspace_size(desc: HstuDesc, T: int, B: int) -> int:
    return int(load().hstu_workspace_size(ctypes.byref(desc), T, B))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def layer_fwd(desc: HstuDesc, x: torch.Tensor, seq_offsets: torch.Tensor,
              timestamps: torch.Tensor, num_candidates: Optional[torch.Tensor],
              prm: Dict[str, torch.Tensor], out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, weights: Optional[HstuWeights] = None,
              tables: Optional[HstuBiasTables] = None,
              token_types: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_layer_fwd on torch's current stream; returns `out` ([T, d])."""
    lib = load()
    T, B = x.shape[0], seq_offsets.shape[0] - 1
    if out is None:
        out = torch.empty_like(x)
    need = workspace_size(desc, T, B)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, x.device)
    w = weights if weights is not None else make_weights(prm)
    t = tables if tables is not None else make_tables(prm, token_types)
    _check(lib.hstu_layer_fwd(ctypes.byref(desc), _ptr(x), _ptr(seq_offsets), B, T,
                              _ptr(timestamps), _ptr(num_candidates), ctypes.byref(w),
                              ctypes.byref(t), _ptr(out), _ptr(workspace), workspace.numel(),
                              _stream()))
    return out


def layer_fwd_noalloc(desc: HstuDesc, x: torch.Tensor, seq_offsets: torch.Tensor,
                      timestamps: torch.Tensor, num_candidates: Optional[torch.Tensor],
                      prm: Dict[str, torch.Tensor], out: torch.Tensor,
                      weights: Optional[HstuWeights] = None,
                      tables: Optional[HstuBiasTables] = None) -> torch.Tensor:
    """hstu_layer_fwd_noalloc on torch's current stream (the library's own
    per-GPU scratch, no workspace); writes and returns `out` ([T, d])."""
    lib = load()
    T, B = x.shape[0], seq_offsets.shape[0] - 1
    w = weights if weights is not None else make_weights(prm)
    t = tables if tables is not None else make_tables(prm)
    _check(lib.hstu_layer_fwd_noalloc(ctypes.byref(desc), _ptr(x), _ptr(seq_offsets), B, T,
                                      _ptr(timestamps), _ptr(num_candidates), ctypes.byref(w),
                                      ctypes.byref(t), _ptr(out), _stream()))
    return out


def alloc_activations(desc: HstuDesc, T: int, device) -> Dict[str, torch.Tensor]:
    dt = torch_dtype(desc)
    H, dqk, dv = desc.num_heads, desc.dqk, desc.dv
    return {
        "u": torch.empty(T, H * dv, dtype=dt, device=device),
        "v": torch.empty(H, T, dv, dtype=dt, device=device),
        "q": torch.empty(H, T, dqk, dtype=dt, device=device),
        "k": torch.empty(H, T, dqk, dtype=dt, device=device),
        "av": torch.empty(T, H * dv, dtype=dt, device=device),
        "av_stats": torch.empty(T, H, 2, dtype=torch.float32, device=device),
    }


def _acts(a: Dict[str, torch.Tensor]) -> HstuActivations:
    return HstuActivations(*[_ptr(a.get(n)) for n in ("u", "v", "q", "k", "av", "av_stats")])


def proj_workspace_size(desc: HstuDesc, T: int) -> int:
    return int(load().hstu_proj_workspace_size(ctypes.byref(desc), T))


def proj_fwd(desc: HstuDesc, x: torch.Tensor, prm: Dict[str, torch.Tensor],
             acts: Optional[Dict[str, torch.Tensor]] = None,
             workspace: Optional[torch.Tensor] = None,
             weights: Optional[HstuWeights] = None) -> Dict[str, torch.Tensor]:
    lib = load()
    T = x.shape[0]
    acts = acts or alloc_activations(desc, T, x.device)
    need = proj_workspace_size(desc, T)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        alloc_workspace(need, x.device)
    a = _acts(acts)
    w = weights if weights is not None else make_weights(prm)
    _check(lib.hstu_proj_fwd(ctypes.byref(desc), _ptr(x), T, ctypes.byref(w), ctypes.byref(a),
                             _ptr(ws), ws.numel(), _stream()))
    return acts


def attn_workspace_size(desc: HstuDesc, T: int, B: int) -> int:
    return int(load().hstu_attn_workspace_size(ctypes.byref(desc), T, B))


def attn_fwd(desc: HstuDesc, seq_offsets, timestamps, num_candidates, prm, acts, workspace=None,
             token_types=None):
    lib = load()
    T, B = acts["u"].shape[0], seq_offsets.shape[0] - 1
    need = attn_workspace_size(desc, T, B)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        alloc_workspace(need, acts["u"].device)
    a, t = _acts(acts), make_tables(prm, token_types)
    _check(lib.hstu_attn_fwd(ctypes.byref(desc), _ptr(seq_offsets), B, T, _ptr(timestamps),
                             _ptr(num_candidates), ctypes.byref(t), ctypes.byref(a), _ptr(ws),
                             ws.numel(), _stream()))
    return acts


def gate_fwd(desc: HstuDesc, prm, acts, z=None):
    """Stage 3a (Z = LayerNorm(AV) * U); returns z, allocating it when not given."""
    lib = load()
    T = acts["u"].shape[0]
    if z is None:
        z = torch.empty_like(acts["u"])
    a, w = _acts(acts), make_weights(prm)
    _check(lib.hstu_gate_fwd(ctypes.byref(desc), T, ctypes.byref(w), ctypes.byref(a), _ptr(z), _stream()))
    return z


def out_fwd(desc: HstuDesc, x, prm, acts, out=None, z=None):
    """Stage 3; returns (out, z), allocating either when not given."""
    lib = load()
    T = acts["u"].shape[0]
    if out is None:
        out = torch.empty(T, desc.d_model, dtype=torch_dtype(desc), device=acts["u"].device)
    if z is None:
        z = torch.empty_like(acts["u"])
    a, w = _acts(acts), make_weights(prm)
    _check(lib.hstu_out_fwd(ctypes.byref(desc), _ptr(x), T, ctypes.byref(w), ctypes.byref(a),
                            _ptr(out), _ptr(z), _stream()))
    return out, z


def cand_workspace_size(desc: HstuDesc, Tc: int, Th: int, B: int) -> int:
    return int(load().hstu_cand_workspace_size(ctypes.byref(desc), Tc, Th, B))


def cand_fwd(desc: HstuDesc, x_cand: torch.Tensor, cand_offsets: torch.Tensor,
             cand_ts: torch.Tensor, num_candidates: torch.Tensor, hist_offsets: torch.Tensor,
             hist_ts: torch.Tensor, hist_k: torch.Tensor, hist_v: torch.Tensor,
             prm: Dict[str, torch.Tensor], out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, weights: Optional[HstuWeights] = None,
             tables: Optional[HstuBiasTables] = None, cand_types: Optional[torch.Tensor] = None,
             hist_types: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_cand_fwd on torch's current stream; returns `out` ([Tc, d])."""
    lib = load()
    Tc, B = x_cand.shape[0], cand_offsets.shape[0] - 1
    Th = hist_ts.shape[0]
    if out is None:
        out = torch.empty_like(x_cand)
    need = cand_workspace_size(desc, Tc, Th, B)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, x_cand.device)
    w = weights if weights is not None else make_weights(prm)
    t = tables if tables is not None else make_tables(prm, cand_types, hist_types)
    _check(lib.hstu_cand_fwd(ctypes.byref(desc), _ptr(x_cand), _ptr(cand_offsets), B, Tc,
                             _ptr(cand_ts), _ptr(num_candidates), _ptr(hist_offsets), Th,
                             _ptr(hist_ts), _ptr(hist_k), _ptr(hist_v), ctypes.byref(w),
                             ctypes.byref(t), _ptr(out), _ptr(workspace), workspace.numel(),
                             _stream()))
    return out


def bwd_workspace_size(desc: HstuDesc, T: int, B: int) -> int:
    return int(load().hstu_bwd_workspace_size(ctypes.byref(desc), T, B))


def layer_fwd_train(desc: HstuDesc, x: torch.Tensor, seq_offsets: torch.Tensor, timestamps: torch.Tensor,
                    num_candidates: Optional[torch.Tensor], prm: Dict[str, torch.Tensor],
                    workspace: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_layer_fwd_train: the layer forward into a backward workspace (kept
    for layer_bwd with HSTU_SAVED_FWD); returns `out`."""
    lib = load()
    T, B = x.shape[0], seq_offsets.shape[0] - 1
    if out is None:
        out = torch.empty_like(x)
    w, t = make_weights(prm), make_tables(prm)
    _check(lib.hstu_layer_fwd_train(ctypes.byref(desc), _ptr(x), _ptr(seq_offsets), B, T, _ptr(timestamps),
                                    _ptr(num_candidates), ctypes.byref(w), ctypes.byref(t), _ptr(out),
                                    _ptr(workspace), workspace.numel(), _stream()))
    return out


def layer_bwd(desc: HstuDesc, x: torch.Tensor, seq_offsets: torch.Tensor, timestamps: torch.Tensor,
              num_candidates: Optional[torch.Tensor], prm: Dict[str, torch.Tensor], dy: torch.Tensor,
              dx: Optional[torch.Tensor] = None, grads: Optional[Dict[str, torch.Tensor]] = None,
              workspace: Optional[torch.Tensor] = None):
    """hstu_layer_bwd; returns (dx, grads) with grads[name] fp32 shaped like
    the parameter (pos/time like the tables)."""
    lib = load()
    T, B = x.shape[0], seq_offsets.shape[0] - 1
    dev = x.device
    if dx is None:
        dx = torch.empty_like(x)
    if grads is None:
        shape = {"w1": prm["w1"].shape, "b1": prm["b1"].shape, "w2": prm["w2"].shape, "b2": prm["b2"].shape,
                 "ln_in_g": prm["ln_in_g"].shape, "ln_in_b": prm["ln_in_b"].shape,
                 "ln_av_g": prm["ln_av_g"].shape, "ln_av_b": prm["ln_av_b"].shape,
                 "pos": prm["pos_table"].shape, "time": prm["time_table"].shape}
        grads = {n: torch.empty(shape[n], dtype=torch.float32, device=dev) for n in GRAD_FIELDS}
    need = bwd_workspace_size(desc, T, B)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, dev)
    g = HstuGrads(*[_ptr(grads[n]) for n in GRAD_FIELDS])
    w, t = make_weights(prm), make_tables(prm)
    _check(lib.hstu_layer_bwd(ctypes.byref(desc), _ptr(x), _ptr(seq_offsets), B, T, _ptr(timestamps),
                              _ptr(num_candidates), ctypes.byref(w), ctypes.byref(t), _ptr(dy), _ptr(dx),
                              ctypes.byref(g), _ptr(workspace), workspace.numel(), _stream()))
    return dx, grads


def attn_bwd(desc: HstuDesc, seq_offsets, timestamps, num_candidates, prm, acts, dav: torch.Tensor):
    """hstu_attn_bwd; returns (dqkv [T, N1] fp32 with the v, q, k column blocks
    written, dpos, dtime)."""
    lib = load()
    T, B = dav.shape[0], seq_offsets.shape[0] - 1
    dev = dav.device
    n1 = 2 * desc.num_heads * (desc.dqk + desc.dv)
    dqkv = torch.zeros(T, n1, dtype=torch.float32, device=dev)
    dpos = torch.empty(prm["pos_table"].shape, dtype=torch.float32, device=dev)
    dtime = torch.empty(prm["time_table"].shape, dtype=torch.float32, device=dev)
    need = int(lib.hstu_attn_bwd_workspace_size(ctypes.byref(desc), T, B))
    ws = alloc_workspace(need, dev)
    a, t = _acts(acts), make_tables(prm)
    _check(lib.hstu_attn_bwd(ctypes.byref(desc), _ptr(seq_offsets), B, T, _ptr(timestamps),
                             _ptr(num_candidates), ctypes.byref(t), ctypes.byref(a), _ptr(dav), _ptr(dqkv),
                             _ptr(dpos), _ptr(dtime), _ptr(ws), ws.numel(), _stream()))
    return dqkv, dpos, dtime


def sl_sample(seq_offsets: torch.Tensor, u: torch.Tensor, keys: torch.Tensor, max_len: int,
              alpha: float, out_offsets: Optional[torch.Tensor] = None,
              out_rows: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """hstu_sl_sample; returns (out_offsets [B+1], out_rows [T]) device tensors
    (out_rows valid up to out_offsets[B])."""
    lib = load()
    B, T = seq_offsets.shape[0] - 1, keys.shape[0]
    dev = seq_offsets.device
    if out_offsets is None:
        out_offsets = torch.empty(B + 1, dtype=torch.int64, device=dev)
    if out_rows is None:
        out_rows = torch.empty(max(T, 1), dtype=torch.int64, device=dev)
    need = int(lib.hstu_sl_workspace_size(B))
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, dev)
    _check(lib.hstu_sl_sample(_ptr(seq_offsets), B, T, int(max_len), float(alpha), _ptr(u), _ptr(keys),
                              _ptr(out_offsets), _ptr(out_rows), _ptr(workspace), workspace.numel(),
                              _stream()))
    return out_offsets, out_rows


def gather_rows(src: torch.Tensor, rows: torch.Tensor, num_rows: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_gather_rows over src's first dimension; num_rows: a one-element
    device tensor (e.g. out_offsets[-1:]).  out has src's shape (rows past
    *num_rows untouched)."""
    lib = load()
    if out is None:
        out = torch.empty_like(src)
    n = src.shape[0]
    row_bytes = src.element_size() * (src.numel() // max(n, 1))
    _check(lib.hstu_gather_rows(_ptr(src), n, row_bytes, _ptr(rows), _ptr(num_rows), out.shape[0],
                                _ptr(out), _stream()))
    return out


def debug_indices(desc: HstuDesc, seq_offsets, timestamps, num_candidates, pairs: torch.Tensor):
    lib = load()
    T, B = timestamps.shape[0], seq_offsets.shape[0] - 1
    n = pairs.shape[0]
    out = torch.empty(n, 6, dtype=torch.int64, device=pairs.device)
    _check(lib.hstu_debug_indices(ctypes.byref(desc), _ptr(seq_offsets), B, T, _ptr(timestamps),
                                  _ptr(num_candidates), _ptr(pairs), n, _ptr(out), _stream()))
    return out


def debug_attn_bias(desc: HstuDesc, seq_offsets, timestamps, num_candidates, prm, slot: torch.Tensor,
                    n_slots: int, max_len: int, fill: float = float("inf")):
    """hstu_debug_attn_bias: the attention kernel's per-pair biases (times
    -log2 e; NaN where masked) of the rows with slot[row] >= 0, as a float32
    [H, n_slots, max_len] tensor first filled with `fill` (entries the kernel
    does not visit keep it)."""
    lib = load()
    T, B = timestamps.shape[0], seq_offsets.shape[0] - 1
    need = attn_workspace_size(desc, T, B)
    ws = alloc_workspace(need, timestamps.device)
    out = torch.full((desc.num_heads, n_slots, max_len), fill, dtype=torch.float32, device=timestamps.device)
    t = make_tables(prm)
    _check(lib.hstu_debug_attn_bias(ctypes.byref(desc), _ptr(seq_offsets), B, T, _ptr(timestamps),
                                    _ptr(num_candidates), ctypes.byref(t), _ptr(slot), n_slots, max_len,
                                    _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out
