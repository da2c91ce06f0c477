"""hstu_layer_fwd_noalloc (the entry point for callers that cannot allocate)
against hstu_layer_fwd: the same kernels on the same arguments, with the
workspace taken from the library's per-GPU scratch array, so the outputs must
agree bit for bit.  Two calls in a row, the second on a smaller batch (the
array keeps the first call's contents); a third call after a regular
hstu_layer_fwd on other data; and a batch whose workspace exceeds the array is
refused."""

import numpy as np
import pytest
import torch

from hstu_sequential_transducer_layer_amd import _lib, layer, synth

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _both(w):
    dev = layer.to_device(w)
    desc = _lib.make_desc(w.dims)
    args = (dev["x"], dev["offsets"], dev["timestamps"], dev["num_candidates"], dev["layers"][0])
    T, B = w.T, w.B
    assert _lib.workspace_size(desc, T, B) <= _lib.NOALLOC_SCRATCH_BYTES
    out_na = torch.full_like(dev["x"], float("nan"))
    _lib.layer_fwd_noalloc(desc, *args, out=out_na)
    ref = _lib.layer_fwd(desc, *args)
    torch.cuda.synchronize()
    return out_na.float().cpu().numpy(), ref.float().cpu().numpy()


@pytest.mark.parametrize("first,second", [
    (("ranking_cand", 6), ("ranking_cand", 2)),
    (("sl_train", 8), ("zipf_bf16", 5)),
    (("small_fp32", None), ("small_fp32", 2)),
])
def test_noalloc_matches_layer_fwd(first, second):
    for name, batch in (first, second):
        w = synth.make_workload(name, batch=batch, seed=1)
        say(f"noalloc vs layer_fwd: {name}, B={w.B}, T={w.T}")
        got, ref = _both(w)
        assert np.all(np.isfinite(got))
        np.testing.assert_array_equal(got, ref)


def test_noalloc_after_other_work_and_oversize():
    w = synth.make_workload("ranking_cand", batch=3, seed=2)
    other = synth.make_workload("zipf_bf16", batch=7, seed=4)
    dev_o = layer.to_device(other)
    _lib.layer_fwd(_lib.make_desc(other.dims), dev_o["x"], dev_o["offsets"], dev_o["timestamps"], None,
                   dev_o["layers"][0])
    got, ref = _both(w)
    np.testing.assert_array_equal(got, ref)
    big = synth.make_workload("len4k", batch=16)
    dev = layer.to_device(big)
    desc = _lib.make_desc(big.dims)
    assert _lib.workspace_size(desc, big.T, big.B) > _lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(_lib.HstuError) as e:
        _lib.layer_fwd_noalloc(desc, dev["x"], dev["offsets"], dev["timestamps"], None, dev["layers"][0],
                               out=torch.empty_like(dev["x"]))
    assert e.value.status == _lib.HSTU_ERR_WORKSPACE
    torch.cuda.synchronize()
