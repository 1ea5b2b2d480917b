"""Dense hot prefix of the predictor (sfnn_pred.hot_prefix) through the C ABI.

The leading mask words are set for every token and their logits read +inf.
The prefix's W2^T rows and thresholds are NaN-poisoned here, which shows they
are not read.  The rest of the mask and of the logits is bitwise that of the
same call without the prefix (the other mask words run the same kernels), and
layers match the oracle run with the same prefix.
"""
import numpy as np
import pytest

import oracle
import synth
from activation_sparse_gemv_amd import Pred
from gpu_util import band_check, gpu_layer, gpu_predict, rel_err, to_dev, upload_layer

pytestmark = pytest.mark.gpu

TOL = 2e-3
ALL = np.uint64(0xFFFFFFFFFFFFFFFF)


def _poisoned_pred(lay, hot):
    w2 = lay.w2_t.copy()
    tau = lay.tau.copy()
    w2[:hot] = np.nan
    tau[:hot] = np.nan
    return Pred(to_dev(lay.w1_t), to_dev(w2), to_dev(tau), hot_prefix=hot)


# f16 at batches 1 and 3 and f32 take the per-row kernels, f16 at 9 and 40
# the matrix cores (40: two token passes, the union ORed over both)
@pytest.mark.parametrize("pdt,B", [("f16", 1), ("f16", 3), ("f16", 9), ("f16", 40), ("f32", 1), ("f32", 6)])
@pytest.mark.parametrize("hot", [64, 1024, 3072])
def test_predict_hot_prefix(pdt, B, hot):
    spec = synth.config("c1", wtype=pdt, pred_dtype=pdt)  # d_model 768, d_ff 3072, rank 128
    f = spec.d_ff
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, B, stream=40 + B)
    p0, _ = upload_layer(lay, predictor=True)
    m0, l0 = gpu_predict(p0, x, f)
    mh, lh = gpu_predict(_poisoned_pred(lay, hot), x, f)
    W = hot // 64
    assert (mh[:, :W] == ALL).all()
    assert np.isposinf(lh[:, :hot]).all()
    assert np.array_equal(mh[:, W:], m0[:, W:])
    assert np.array_equal(lh[:, hot:].view(np.uint32), l0[:, hot:].view(np.uint32))
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x, hot_prefix=hot)
    assert np.array_equal(oracle.unpack_mask(mh, f)[:, :hot], ob[:, :hot])
    ol0, _ = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    band_check(m0, l0, ol0, oracle.guard_band(lay.w1_t, lay.w2_t, x), lay.tau, f)


@pytest.mark.parametrize("wtype,B", [("f16", 1), ("f16", 4), ("f16", 9), ("i4g128", 1), ("i4g128", 4),
                                     ("f32", 2)])
def test_layer_hot_prefix(wtype, B):
    spec = synth.config("c3", d_model=1024, d_ff=8192, rank=128, wtype=wtype,
                        pred_dtype="f32" if wtype == "f32" else "f16")
    f, hot = spec.d_ff, 1024
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, B, stream=60 + B)
    _, ffn = upload_layer(lay)
    out = gpu_layer(_poisoned_pred(lay, hot), ffn, x)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x, hot_prefix=hot)
    band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
    gb = oracle.unpack_mask(out["mask"], f)
    assert gb[:, :hot].all()
    outside = np.abs(ol - lay.tau[None, :].astype(np.float64)) > band
    assert not ((gb != ob) & outside).any()
    rid, rc, _ = oracle.compact(out["mask"], B, f)
    assert out["count"] == rc and np.array_equal(out["ids"], rid)
    assert np.array_equal(out["ids"][:hot], np.arange(hot))
    ref = oracle.masked_ffn(lay, x, gb)
    for b in range(B):
        assert rel_err(out["y"][b], ref[b]) <= TOL, b


@pytest.mark.parametrize("B", [1, 9])
def test_layer_all_hot_is_dense(B):
    """A prefix of d_ff takes every neuron: the layer is the dense FFN."""
    spec = synth.config("c2", d_model=1024, d_ff=4096, rank=128)
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, B, stream=80 + B)
    _, ffn = upload_layer(lay)
    out = gpu_layer(_poisoned_pred(lay, spec.d_ff), ffn, x)
    assert out["count"] == spec.d_ff and (out["mask"] == ALL).all()
    ref = oracle.dense_ffn(lay, x)
    for b in range(B):
        assert rel_err(out["y"][b], ref[b]) <= TOL, b
