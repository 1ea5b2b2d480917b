"""sfnn_layer_noalloc, the layer call that allocates nothing (its workspace is
the library's per-GPU scratch array), against sfnn_layer with a caller
workspace, through the C ABI.  Two calls in a row, the second on a smaller
input, each checked against sfnn_layer (same kernels: identical bits) and
against the oracle (compaction bit-exact, FFN output within 2e-3)."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as sg
import oracle
import synth
from gpu_util import DEV, gpu_layer, rel_err, to_dev, upload_layer

pytestmark = pytest.mark.gpu


def _noalloc(pred, ffn, x):
    B = x.shape[0]
    f, d = ffn.d_ff, ffn.d_model
    mask = torch.zeros((B, f // 64), dtype=torch.uint64, device=DEV)
    ids = torch.full((f,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((4,), -1, dtype=torch.int32, device=DEV)
    y = torch.full((B, d), float("nan"), dtype=torch.float32, device=DEV)
    sg.sfnn_layer_noalloc(pred, ffn, to_dev(x), B, y, mask, ids, cnt)
    torch.cuda.synchronize()
    c = int(cnt[0].item())
    return dict(y=y.cpu().numpy(), mask=mask.cpu().numpy(), ids=ids.cpu().numpy()[:c], count=c)


def _case(spec, lay, B, stream):
    x = synth.make_tokens(spec, B, stream=stream)
    pred, ffn = upload_layer(lay)
    assert sg.sfnn_workspace_bytes(pred, ffn, B) <= sg.SFNN_NOALLOC_SCRATCH_BYTES
    got = _noalloc(pred, ffn, x)
    ref = gpu_layer(pred, ffn, x)
    assert got["count"] == ref["count"]
    assert np.array_equal(got["mask"], ref["mask"])
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.array_equal(got["y"].view(np.uint32), ref["y"].view(np.uint32))
    # the oracle on the mask the kernels chose: ids bit-exact, y within 2e-3
    rid, rc, _ = oracle.compact(got["mask"], B, spec.d_ff)
    assert rc == got["count"] and np.array_equal(rid, got["ids"])
    m = oracle.unpack_mask(got["mask"], spec.d_ff)
    assert rel_err(got["y"], oracle.masked_ffn(lay, x, m)) <= 2e-3
    return got


def test_noalloc_layer_two_calls_second_smaller():
    big = synth.config("c2")
    small = synth.config("c1")
    lay_big = synth.make_layer(big, layer=0)
    lay_small = synth.make_layer(small, layer=0)
    first = _case(big, lay_big, 4, stream=31)
    second = _case(small, lay_small, 1, stream=32)
    assert first["count"] > second["count"] > 0
    # and the same layer again at a smaller batch, after the smaller shape
    _case(big, lay_big, 1, stream=33)


def test_noalloc_rejects_beyond_scratch():
    spec = synth.config("c1")
    lay = synth.make_layer(spec, layer=0)
    pred, ffn = upload_layer(lay)
    big = sg._lib.sfnn_ffn(12288, 49152, sg.SFNN_I4G128, 0, 1 << 20, None, 1 << 20, 1 << 20, None, 1 << 20,
                           None, None, None)
    bigp = sg._lib.sfnn_pred(12288, 49152, 1024, sg.SFNN_F16, 1 << 20, 1 << 20, 1 << 20)
    L = sg.load()
    import ctypes
    assert L.sfnn_layer_noalloc(ctypes.byref(bigp), ctypes.byref(big), 1 << 20, 64, 1 << 20, None, None, None,
                                None) == 5
    # a valid call afterwards still works
    x = synth.make_tokens(spec, 1, stream=34)
    got = _noalloc(pred, ffn, x)
    assert np.isfinite(got["y"]).all() and got["count"] > 0
