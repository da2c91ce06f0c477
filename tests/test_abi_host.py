"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/hstu.h declares, sizes its workspace as documented, and
rejects bad arguments with the documented status before touching a device."""

import ctypes
import os
import re

import pytest

from hstu_sequential_transducer_layer_amd import _lib, build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        build_lib.build(verbose=False)
    return _lib.load()


def _declared():
    src = open(HEADER).read()
    return re.findall(r"^\s*(?:size_t|hstu_status|const char\*)\s+(hstu_\w+)\(", src, re.M)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def _desc(**kw):
    base = dict(d_model=512, num_heads=8, dqk=128, dv=128, pos_buckets=129, time_buckets=64,
                time_sub_bits=0, dtype=_lib.HSTU_BF16,
                flags=_lib.HSTU_INPUT_NORM | _lib.HSTU_RESIDUAL | _lib.HSTU_CAND_SHARED_POS,
                ln_eps=1e-5, norm_len=0)
    base.update(kw)
    return _lib.HstuDesc(**base)


def test_workspace_size_matches_layout(lib):
    T, B = 57291, 64
    d = _desc()
    e, H, dv, dq, dm = 2, 8, 128, 128, 512
    a = lambda n: (n + 255) // 256 * 256
    tiles = (T + 127) // 128 + B
    kblocks = (T + 63) // 64 + B
    # work list, key-block list, two counters, per-sequence tile / key-block bases
    # and history split, per-row offsets (+64 pad), per-row stats pair
    attn = a(tiles * 8) + a(kblocks * 8) + a(8) + 3 * a((B + 1) * 4) + a((T + 64) * 4) + a(T * 16) \
        + a((T + 64) * 4)   # key rows' token types
    want = (a(T * dm * e) + a(T * H * dv * e) * 3 + a(T * H * dq * e) * 2 + a(T * H * 8)
            + attn)
    assert _lib.workspace_size(d, T, B) == want
    d2 = _desc(flags=_lib.HSTU_RESIDUAL)     # no input LayerNorm buffer
    assert _lib.workspace_size(d2, T, B) == want - a(T * dm * e)
    assert _lib.workspace_size(_desc(dqk=48), T, B) == 0
    assert lib.hstu_attn_workspace_size(ctypes.byref(d), T, B) == attn
    assert lib.hstu_proj_workspace_size(ctypes.byref(d), T) == a(T * dm * e)


FAKE = 0x10000   # aligned non-null host address: validation never dereferences it


def _call(lib, desc, T=1000, B=4, x=FAKE, off=FAKE, ts=FAKE, nc=None, weights=None,
          tables=None, out=FAKE, ws=FAKE, ws_bytes=None):
    w = weights or _lib.HstuWeights(*([FAKE] * 8))
    t = tables or _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.hstu_layer_fwd(ctypes.byref(desc), x, off, B, T, ts, nc, ctypes.byref(w),
                              ctypes.byref(t), out, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("dqk", 48, _lib.HSTU_ERR_UNSUPPORTED),
    ("dv", 256, _lib.HSTU_ERR_UNSUPPORTED),
    ("d_model", 100, _lib.HSTU_ERR_UNSUPPORTED),
    ("num_heads", 0, _lib.HSTU_ERR_UNSUPPORTED),
    ("pos_buckets", 128, _lib.HSTU_ERR_INVALID_ARG),
    ("time_buckets", 0, _lib.HSTU_ERR_INVALID_ARG),
    ("time_sub_bits", 5, _lib.HSTU_ERR_INVALID_ARG),
    ("dtype", 7, _lib.HSTU_ERR_UNSUPPORTED),
    ("flags", 1 << 9, _lib.HSTU_ERR_INVALID_ARG),
    ("ln_eps", 0.0, _lib.HSTU_ERR_INVALID_ARG),
    ("norm_len", -1, _lib.HSTU_ERR_INVALID_ARG),
    ("num_types", 17, _lib.HSTU_ERR_UNSUPPORTED),
    ("num_types", -1, _lib.HSTU_ERR_UNSUPPORTED),
])
def test_bad_descriptor(lib, field, value, status):
    assert _call(lib, _desc(**{field: value})) == status
    assert lib.hstu_last_error().decode() != ""


def test_fp32_wide_heads_unsupported(lib):
    assert _call(lib, _desc(dtype=_lib.HSTU_F32)) == _lib.HSTU_ERR_UNSUPPORTED


def test_bad_pointers_and_sizes(lib):
    d = _desc()
    assert _call(lib, d, x=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, x=FAKE + 2) == _lib.HSTU_ERR_INVALID_ARG        # misaligned
    assert _call(lib, d, out=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, off=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, off=FAKE + 4) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, ts=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, nc=FAKE + 2) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, T=-1) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, B=-1) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, B=0) == _lib.HSTU_ERR_INVALID_ARG
    w = _lib.HstuWeights(*([FAKE] * 7 + [None]))
    assert _call(lib, d, weights=w) == _lib.HSTU_ERR_INVALID_ARG
    t = _lib.HstuBiasTables(FAKE, FAKE, 100, 64)                       # stride < P
    assert _call(lib, d, tables=t) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert _call(lib, d, ws_bytes=1000) == _lib.HSTU_ERR_WORKSPACE
    assert _call(lib, d, ws=FAKE + 16) == _lib.HSTU_ERR_WORKSPACE       # not 256-aligned
    assert _call(lib, d, T=0, B=0) == _lib.HSTU_OK                      # nothing to do


def test_input_norm_weights_only_required_with_flag(lib):
    d = _desc(flags=_lib.HSTU_RESIDUAL)
    w = _lib.HstuWeights(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE)
    # all checks pass; the call then fails (or succeeds) at the device, never with INVALID_ARG
    assert _call(lib, d, weights=w, T=0, B=1) == _lib.HSTU_OK
    d2 = _desc()
    assert _call(lib, d2, weights=w) == _lib.HSTU_ERR_INVALID_ARG


def test_stage3_entry_points_check_arguments(lib):
    d = _desc()
    w = _lib.HstuWeights(*([FAKE] * 8))
    a = _lib.HstuActivations(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    R = ctypes.byref
    # z is required by both; NULL or misaligned is rejected before any launch
    assert lib.hstu_gate_fwd(R(d), 100, R(w), R(a), None, None) == _lib.HSTU_ERR_INVALID_ARG
    assert lib.hstu_gate_fwd(R(d), 100, R(w), R(a), FAKE + 8, None) == _lib.HSTU_ERR_INVALID_ARG
    assert lib.hstu_out_fwd(R(d), FAKE, 100, R(w), R(a), FAKE, None, None) == _lib.HSTU_ERR_INVALID_ARG
    assert lib.hstu_out_fwd(R(d), FAKE, 100, R(w), R(a), None, FAKE, None) == _lib.HSTU_ERR_INVALID_ARG
    a_bad = _lib.HstuActivations(FAKE, FAKE, FAKE, FAKE, None, FAKE)    # no av
    assert lib.hstu_gate_fwd(R(d), 100, R(w), R(a_bad), FAKE, None) == _lib.HSTU_ERR_INVALID_ARG
    w_bad = _lib.HstuWeights(*([FAKE] * 6 + [None, FAKE]))             # no ln_av_g
    assert lib.hstu_gate_fwd(R(d), 100, R(w_bad), R(a), FAKE, None) == _lib.HSTU_ERR_INVALID_ARG
    assert lib.hstu_gate_fwd(R(d), -1, R(w), R(a), FAKE, None) == _lib.HSTU_ERR_INVALID_ARG
    assert lib.hstu_gate_fwd(R(d), 0, R(w), R(a), FAKE, None) == _lib.HSTU_OK   # nothing to do


def test_status_strings(lib):
    for s in range(5):
        assert lib.hstu_status_str(s).decode()
    assert lib.hstu_status_str(99).decode() == "unknown status"


def test_cand_workspace_size_matches_layout(lib):
    Tc, Th, B = 3000, 57291, 64
    d = _desc()
    e, H, dv, dq, dm = 2, 8, 128, 128, 512
    a = lambda n: (n + 255) // 256 * 256
    # work items (query tiles x up to 8 history chunks) over the candidates, key
    # blocks / offsets / stats over the history, then the fp32 partial AV of up
    # to 8 chunks per candidate row
    attn = (a(((Tc + 127) // 128 + B) * 8 * 8) + a(((Th + 63) // 64 + B) * 8) + a(8) + 3 * a((B + 1) * 4)
            + a((Th + 64) * 4) + a(Th * 16) + a((Th + 64) * 4))
    part = a(8 * Tc * H * dv * 4)
    want = (a(Tc * dm * e) + a(Tc * H * dv * e) * 3 + a(Tc * H * dq * e) * 2 + a(Tc * H * 8)
            + attn + part)
    assert _lib.cand_workspace_size(d, Tc, Th, B) == want
    assert _lib.cand_workspace_size(d, Tc, -1, B) == 0


def _cand(lib, desc, Tc=100, Th=1000, B=4, x=FAKE, coff=FAKE, cts=FAKE, m=FAKE, hoff=FAKE,
          hts=FAKE, hk=FAKE, hv=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    w = _lib.HstuWeights(*([FAKE] * 8))
    t = _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    R = ctypes.byref
    return lib.hstu_cand_fwd(R(desc), x, coff, B, Tc, cts, m, hoff, Th, hts, hk, hv, R(w), R(t),
                             out, ws, ws_bytes, None)


def test_cand_entry_point_checks_arguments(lib):
    d = _desc()
    no_shared = _desc(flags=_lib.HSTU_INPUT_NORM | _lib.HSTU_RESIDUAL)
    assert _cand(lib, no_shared) == _lib.HSTU_ERR_UNSUPPORTED
    assert "SHARED_POS" in lib.hstu_last_error().decode()
    for kw in (dict(x=None), dict(out=None), dict(m=None), dict(m=FAKE + 2), dict(hk=None),
               dict(hv=FAKE + 8), dict(coff=None), dict(hts=None), dict(cts=FAKE + 4),
               dict(Th=-1), dict(Tc=-1), dict(B=0)):
        assert _cand(lib, d, **kw) == _lib.HSTU_ERR_INVALID_ARG, kw
    assert _cand(lib, d, ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert _cand(lib, d, ws_bytes=4096) == _lib.HSTU_ERR_WORKSPACE
    assert _cand(lib, d, Tc=0, x=None, out=None) == _lib.HSTU_OK        # nothing to score
    # no history: the cache pointers are not needed (the call then reaches the
    # device only through a workspace check, which fails here)
    assert _cand(lib, d, Th=0, hk=None, hv=None, hts=None, ws_bytes=4096) == _lib.HSTU_ERR_WORKSPACE
    assert _cand(lib, d, hoff=None) == _lib.HSTU_ERR_INVALID_ARG


def test_type_table_fields_checked(lib):
    d = _desc(num_types=2)
    T4 = lambda **kw: _lib.HstuBiasTables(**{**dict(pos=FAKE, time=FAKE, pos_head_stride=129,
                                                    time_head_stride=64, type=FAKE, type_head_stride=4,
                                                    reserved=0, token_types=FAKE, hist_types=FAKE), **kw})
    assert _call(lib, d, tables=T4(), ws=None) == _lib.HSTU_ERR_WORKSPACE       # all type fields valid
    assert _call(lib, d, tables=T4(type=None)) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, tables=T4(type=FAKE + 1)) == _lib.HSTU_ERR_INVALID_ARG  # misaligned bf16
    assert _call(lib, d, tables=T4(token_types=None)) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, tables=T4(type_head_stride=3)) == _lib.HSTU_ERR_INVALID_ARG
    assert _call(lib, d, tables=T4(type_head_stride=0), ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert _call(lib, d, tables=T4(reserved=1)) == _lib.HSTU_ERR_INVALID_ARG
    # untyped layers ignore every type field
    assert _call(lib, _desc(), tables=T4(type=None, token_types=None, reserved=5), ws=None) == \
        _lib.HSTU_ERR_WORKSPACE


def test_sl_entry_points_check_arguments(lib):
    ws = lambda n: n
    call = lambda **kw: lib.hstu_sl_sample(*[{**dict(off=FAKE, B=4, T=100, N=4096, a=1.6, u=FAKE, keys=FAKE,
                                                     oo=FAKE, orows=FAKE, ws=FAKE, wb=1 << 20), **kw}[k]
                                             for k in ("off", "B", "T", "N", "a", "u", "keys", "oo", "orows",
                                                       "ws", "wb")], None)
    assert lib.hstu_sl_workspace_size(4) == 256
    assert call(a=0.0) == _lib.HSTU_ERR_INVALID_ARG
    assert call(a=2.5) == _lib.HSTU_ERR_INVALID_ARG
    assert call(N=0) == _lib.HSTU_ERR_INVALID_ARG
    assert call(keys=None) == _lib.HSTU_ERR_INVALID_ARG
    assert call(u=FAKE + 2) == _lib.HSTU_ERR_INVALID_ARG
    assert call(orows=None) == _lib.HSTU_ERR_INVALID_ARG
    assert call(ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert call(T=-1) == _lib.HSTU_ERR_INVALID_ARG
    g = lambda **kw: lib.hstu_gather_rows(*[{**dict(src=FAKE, sr=10, rb=64, rows=FAKE, n=FAKE, mr=10, dst=FAKE),
                                            **kw}[k] for k in ("src", "sr", "rb", "rows", "n", "mr", "dst")], None)
    assert g(rows=None) == _lib.HSTU_ERR_INVALID_ARG
    assert g(n=FAKE + 4) == _lib.HSTU_ERR_INVALID_ARG
    assert g(sr=0) == _lib.HSTU_ERR_INVALID_ARG
    assert g(rb=-8) == _lib.HSTU_ERR_INVALID_ARG
    assert g(mr=0, src=None) == _lib.HSTU_OK                            # nothing to copy


def test_bwd_entry_point_checks_arguments(lib):
    R = ctypes.byref
    gr = _lib.HstuGrads(*([FAKE] * 10))
    w = _lib.HstuWeights(*([FAKE] * 8))
    t = _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    call = lambda d, gg=gr, dy=FAKE, ws=FAKE, wb=1 << 40: lib.hstu_layer_bwd(
        R(d), FAKE, FAKE, 4, 1000, FAKE, None, R(w), R(t), dy, FAKE, R(gg), ws, wb, None)
    assert call(_desc(dqk=64, dv=128)) == _lib.HSTU_ERR_UNSUPPORTED          # dqk != dv
    assert call(_desc(num_types=2)) == _lib.HSTU_ERR_UNSUPPORTED
    assert call(_desc(), dy=None) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), gg=_lib.HstuGrads(*([FAKE] * 9 + [None]))) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.hstu_bwd_workspace_size(R(_desc()), 1000, 4) > lib.hstu_workspace_size(R(_desc()), 1000, 4)
    assert lib.hstu_bwd_workspace_size(R(_desc(dqk=64, dv=32)), 1000, 4) == 0
    # the LayerNorm backward kernels' per-workgroup column sums cover 2048 columns
    assert call(_desc(d_model=4096)) == _lib.HSTU_ERR_UNSUPPORTED
    assert call(_desc(num_heads=32, dqk=128, dv=128)) == _lib.HSTU_ERR_UNSUPPORTED
    assert lib.hstu_bwd_workspace_size(R(_desc(d_model=4096)), 1000, 4) == 0
    assert lib.hstu_bwd_workspace_size(R(_desc(d_model=2048, num_heads=16)), 1000, 4) > 0


def test_fwd_train_entry_point_checks_arguments(lib):
    R = ctypes.byref
    w = _lib.HstuWeights(*([FAKE] * 8))
    t = _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    call = lambda d, x=FAKE, out=FAKE, ws=FAKE, wb=1 << 40: lib.hstu_layer_fwd_train(
        R(d), x, FAKE, 4, 1000, FAKE, None, R(w), R(t), out, ws, wb, None)
    assert call(_desc(dqk=64, dv=128)) == _lib.HSTU_ERR_UNSUPPORTED          # the backward's limits
    assert call(_desc(num_types=2)) == _lib.HSTU_ERR_UNSUPPORTED
    assert call(_desc(), x=None) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), out=FAKE + 8) == _lib.HSTU_ERR_INVALID_ARG          # misaligned
    assert call(_desc(), ws=None) == _lib.HSTU_ERR_WORKSPACE
    need = lib.hstu_bwd_workspace_size(R(_desc()), 1000, 4)
    assert call(_desc(), wb=need - 1) == _lib.HSTU_ERR_WORKSPACE             # a backward workspace
    # the saved-forward flag is a known flag bit
    flags = _lib.HSTU_INPUT_NORM | _lib.HSTU_RESIDUAL | _lib.HSTU_CAND_SHARED_POS | _lib.HSTU_SAVED_FWD
    assert lib.hstu_bwd_workspace_size(R(_desc(flags=flags)), 1000, 4) == need


def test_attn_bwd_entry_point_checks_arguments(lib):
    R = ctypes.byref
    a = _lib.HstuActivations(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    t = _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    call = lambda d, dav=FAKE, acts=a, ws=FAKE: lib.hstu_attn_bwd(R(d), FAKE, 4, 1000, FAKE, None, R(t), R(acts),
                                                                   dav, FAKE, FAKE, FAKE, ws, 1 << 40, None)
    assert call(_desc(dqk=64, dv=128)) == _lib.HSTU_ERR_UNSUPPORTED
    assert call(_desc(), dav=None) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), acts=_lib.HstuActivations(FAKE, FAKE, None, FAKE, FAKE, FAKE)) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert lib.hstu_attn_bwd_workspace_size(R(_desc()), 1000, 4) >= lib.hstu_attn_workspace_size(R(_desc()), 1000, 4)


def test_debug_attn_bias_checks_arguments(lib):
    R = ctypes.byref
    t = _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    call = lambda d, n_slots=4, max_len=100, slot=FAKE, out=FAKE, ws=FAKE, T=1000: lib.hstu_debug_attn_bias(
        R(d), FAKE, 4, T, FAKE, None, R(t), slot, n_slots, max_len, out, ws, 1 << 40, None)
    assert call(_desc(num_types=2)) == _lib.HSTU_ERR_UNSUPPORTED
    assert call(_desc(), n_slots=-1) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), max_len=-1) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), slot=None) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), out=FAKE + 2) == _lib.HSTU_ERR_INVALID_ARG
    assert call(_desc(), ws=None) == _lib.HSTU_ERR_WORKSPACE
    assert call(_desc(), n_slots=0, slot=None, out=None, ws=None) == _lib.HSTU_OK
    assert call(_desc(), T=0) == _lib.HSTU_OK


def _call_noalloc(lib, desc, T=1000, B=4, x=FAKE, off=FAKE, ts=FAKE, nc=None, out=FAKE):
    w = _lib.HstuWeights(*([FAKE] * 8))
    t = _lib.HstuBiasTables(FAKE, FAKE, 129, 64)
    return lib.hstu_layer_fwd_noalloc(ctypes.byref(desc), x, off, B, T, ts, nc, ctypes.byref(w),
                                      ctypes.byref(t), out, None)


def test_noalloc_rejects_before_touching_a_device(lib):
    """hstu_layer_fwd_noalloc: argument checks, HSTU_VALIDATE, and inputs whose
    workspace exceeds the library's scratch array are refused on the host."""
    d = _desc()
    need = lib.hstu_workspace_size(ctypes.byref(d), 200000, 4)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(lib, d, T=200000) == _lib.HSTU_ERR_WORKSPACE
    assert str(_lib.NOALLOC_SCRATCH_BYTES) in lib.hstu_last_error().decode()
    assert _call_noalloc(lib, _desc(flags=_lib.HSTU_VALIDATE)) == _lib.HSTU_ERR_INVALID_ARG
    assert _call_noalloc(lib, d, x=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _call_noalloc(lib, d, off=FAKE + 4) == _lib.HSTU_ERR_INVALID_ARG
    assert _call_noalloc(lib, _desc(dqk=48)) == _lib.HSTU_ERR_UNSUPPORTED
    assert _call_noalloc(lib, d, T=0) == _lib.HSTU_OK
