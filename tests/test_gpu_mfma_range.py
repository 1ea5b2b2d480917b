"""Range of the matrix-core FFN paths: activations far outside fp16's range.

The matrix-core kernels carry h (INT4: h times the row's scale) as two fp16
planes.  Each token is scaled by a power of two chosen from its largest |h|
before the split and scaled back after the products, so neither plane
overflows (fp16's largest finite value is 65504) and small activations keep
their low bits.  These layers are drawn so that max |h| reaches about 1e5 and
more (weights and inputs scaled up), or stays near 1e-4 (scaled down); the bar
is the usual 2e-3 normwise relative error per token against the float64
oracle, on the sparse and the dense entry points, with one token tile (batch
8) and two (batch 20).  Unscaled, the large cases would overflow the high plane.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import gpu_dense_ffn, gpu_sparse_ffn, rel_err, upload_layer

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _scaled_layer(wtype, act, wscale, xscale, seed):
    """A layer whose up / gate products are wscale times the drawn ones, and
    biases wscale * xscale times (so inputs scaled by xscale keep the drawn
    sparsity pattern)."""
    spec = synth.config("c2", d_model=512, d_ff=1088, rank=64, wtype=wtype, act=act, pred_dtype="f16")
    lay = synth.make_layer(spec, layer=seed, predictor=False)
    for k in ("up", "gate"):
        if wtype == "i4g128":
            s = getattr(lay, "s_" + k)
            if s is not None:
                setattr(lay, "s_" + k, (s.astype(np.float32) * wscale).astype(np.float16))
        else:
            w = getattr(lay, "w_" + k)
            if w is not None:
                setattr(lay, "w_" + k, (w.astype(np.float32) * wscale).astype(np.float16))
        b = getattr(lay, "b_" + k)
        if b is not None:
            setattr(lay, "b_" + k, (b.astype(np.float32) * (wscale * xscale)).astype(np.float16))
    return lay


def _h_max(lay, x):
    """Largest |h| over every neuron and token (the magnitude the test is about)."""
    def rows(k):
        if lay.spec.wtype == "i4g128":
            return oracle.dequant_int4(getattr(lay, "q_" + k), getattr(lay, "s_" + k))
        return getattr(lay, "w_" + k).astype(np.float64)
    xs = x.astype(np.float64)
    up = xs @ rows("up").T + (0 if lay.b_up is None else lay.b_up.astype(np.float64))
    if lay.spec.act == "relu":
        return float(np.abs(np.maximum(up, 0)).max())
    gt = xs @ rows("gate").T + (0 if lay.b_gate is None else lay.b_gate.astype(np.float64))
    return float(np.abs(np.maximum(gt, 0) * up).max())


@pytest.mark.parametrize("wtype,act,wscale,xscale,lo,hi", [
    ("f16", "relu", 1000.0, 64.0, 6.6e4, 1e7),  # biases near fp16's limit cap the ReLU case
    ("f16", "reglu", 50.0, 8.0, 1e5, 1e9),
    ("i4g128", "relu", 1000.0, 64.0, 6.6e4, 1e7),
    ("i4g128", "reglu", 50.0, 8.0, 1e5, 1e9),
    ("f16", "relu", 1e-2, 1e-2, 1e-6, 1e-3),
    ("i4g128", "relu", 1e-2, 1e-2, 1e-6, 1e-3),
])
@pytest.mark.parametrize("B", [8, 20])
def test_mfma_ffn_outside_fp16_range(wtype, act, wscale, xscale, lo, hi, B):
    lay = _scaled_layer(wtype, act, wscale, xscale, seed=B)
    x = (synth.make_tokens(lay.spec, B, stream=600 + B).astype(np.float32) * xscale).astype(np.float16)
    hm = _h_max(lay, x)
    assert lo <= hm <= hi, hm  # the workload is what the test says it is
    _, ffn = upload_layer(lay, predictor=False)
    ffn.mfma_min_batch = 1  # the matrix-core path at this batch
    words = synth.random_masks(B, lay.spec.d_ff, 0.3, seed=610 + B)
    y = gpu_sparse_ffn(ffn, x, words)
    ref = oracle.masked_ffn(lay, x, words)
    assert np.isfinite(y).all()
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b
    yd = gpu_dense_ffn(ffn, x)
    refd = oracle.dense_ffn(lay, x)
    assert np.isfinite(yd).all()
    for b in range(B):
        assert rel_err(yd[b], refd[b]) <= TOL, b
