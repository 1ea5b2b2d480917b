"""Parity of the matrix-core predictor (k_pred1_mfma + k_pred2_mfma, fp16
predictors at batches of 8 or more) with the float64 oracle, through the C ABI.

Bars as for the per-row predictor kernels: on integer-grid layers every
intermediate is an integer below 2^22, so logits and masks equal the oracle
bitwise; on random layers a mask bit may differ from the oracle's only inside
the fp32 rounding band of its logit (the two-plane fp16 form of z keeps 22
bits, far inside that band), and it always equals the threshold of the
logits the GPU returns.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import gpu_layer, gpu_predict, rel_err, upload_layer
from test_gpu_parity import _pred_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B", [8, 17, 40, 64])
def test_mfma_predict_integer_grid_bitwise(B):
    # rank 136: ragged against the 16-row stage-1 tiles and the 32-wide
    # stage-2 steps; d_model 640: 10 column pairs over 8 wavefronts
    lay = synth.make_grid_layer(640, 2112, 136, wtype="f16", seed=3)
    x = synth.make_grid_tokens(640, B, seed=B)
    pred, _ = upload_layer(lay)
    words, lg = gpu_predict(pred, x, 2112)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    assert np.array_equal(lg.astype(np.float64), ol)
    assert np.array_equal(words, oracle.pack_mask(ob))


@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_mfma_predict_opt6_7b_full_size(B):
    _pred_case(synth.config("c2"), B, stream=60 + B)


def test_mfma_predict_wide_d_model_b32():
    # the OPT-175B predictor's d_model (12288: 192 column pairs) at batch 32
    _pred_case(synth.config("c2", d_model=12288, d_ff=8192), 32, stream=70)


def test_mfma_predict_small_rank():
    # rank 8: one K block per row, three of four lane groups idle in stage 2
    _pred_case(synth.config("c2", d_model=256, d_ff=1024, rank=8), 12, stream=71)


def test_mfma_predict_union_over_two_passes():
    """Batch 40 runs as passes of 32 and 8 tokens; the union mask that the
    layer's FFN compacts is the OR of both passes' masks."""
    spec = synth.config("c2", d_model=512, d_ff=2048, rank=64)
    lay = synth.make_layer(spec, layer=0)
    B = 40
    x = synth.make_tokens(spec, B, stream=72)
    pred, ffn = upload_layer(lay)
    pred.dense_min_batch = -1
    out = gpu_layer(pred, ffn, x)
    rid, rc, _ = oracle.compact(out["mask"], B, 2048)
    assert out["count"] == rc and np.array_equal(out["ids"], rid)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
    outside = np.abs(ol - lay.tau[None, :].astype(np.float64)) > band
    gb = oracle.unpack_mask(out["mask"], 2048)
    assert not ((gb != ob) & outside).any()
    ref = oracle.masked_ffn(lay, x, out["mask"])
    for b in range(B):
        assert rel_err(out["y"][b], ref[b]) <= 2e-3, b


def test_mfma_predict_deterministic():
    spec = synth.config("c2", d_model=1024, d_ff=4096, rank=256)
    lay = synth.make_layer(spec, layer=1)
    x = synth.make_tokens(spec, 24, stream=73)
    pred, _ = upload_layer(lay)
    w1, l1 = gpu_predict(pred, x, 4096)
    w2, l2 = gpu_predict(pred, x, 4096)
    assert np.array_equal(w1, w2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("lookahead", [False, True])
def test_mfma_predict_stack_b20(lookahead):
    # the residual chain's layer input comes from the RMSNorm launch in front
    # of stage 1; two token tiles per pass
    from test_gpu_stack import _stack_case
    spec = synth.config("c2", d_model=768, d_ff=3072, rank=96, n_layers=3)
    _stack_case(spec, 3, 20, seed=12, lookahead=lookahead)


@pytest.mark.parametrize("B", [9, 20])
def test_mfma_predict_split_stage1_integer_grid_bitwise(B):
    # d_model 8192: stage 1 runs in two d_model slices whose partial z are
    # added by the reduce launch; on the integer grid every sum is exact
    lay = synth.make_grid_layer(8192, 1024, 64, wtype="f16", seed=9)
    x = synth.make_grid_tokens(8192, B, seed=90 + B)
    pred, _ = upload_layer(lay)
    words, lg = gpu_predict(pred, x, 1024)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    assert np.abs(ol).max() < 2 ** 24
    assert np.array_equal(lg.astype(np.float64), ol)
    assert np.array_equal(words, oracle.pack_mask(ob))
