"""The dense switch of sfnn_layer / sfnn_stack_decode (sfnn_pred.dense_min_batch).

Past the crossover batch the union of the tokens' active neurons covers most
of d_ff and the calls run the dense FFN instead (53ai.com sparsity survey,
DejaVu section: contextual sparsity is per token, so a batch's union grows
with its size).  The dense FFN is the masked FFN under an all-ones mask, so
the oracle here is oracle.dense_ffn, and the reported mask / ids / count are
the all-ones mask, 0..d_ff-1 and d_ff.  The switch is off unless the
descriptor sets a positive threshold (the stack's per-layer mix is covered
in test_gpu_stack.py).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gpu_dense_ffn, gpu_layer, gpu_stack, rel_err, upload_layer

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _check_dense_report(out, B, f):
    assert np.array_equal(out["mask"], np.full((B, f // 64), np.uint64(2 ** 64 - 1)))
    assert out["count"] == f and np.array_equal(out["ids"], np.arange(f, dtype=np.int32))


def _dense_layer_case(lay, x, dense_min_batch=16, check_tokens=None):
    f = lay.spec.d_ff
    B = x.shape[0]
    pred, ffn = upload_layer(lay)
    pred.dense_min_batch = dense_min_batch
    out = gpu_layer(pred, ffn, x)
    _check_dense_report(out, B, f)
    # the same kernels as the dense entry point: bitwise equal
    assert np.array_equal(out["y"], gpu_dense_ffn(ffn, x))
    toks = range(B) if check_tokens is None else check_tokens
    for b in toks:
        ref = oracle.dense_ffn(lay, x[b:b + 1])[0]
        assert rel_err(out["y"][b], ref) <= TOL, b
    return out


@pytest.mark.parametrize("wtype,act", [("f16", "relu"), ("f16", "reglu"), ("i4g128", "relu"), ("f32", "relu")])
def test_layer_switches_at_threshold(wtype, act):
    spec = synth.config("c4" if act == "reglu" else "c2", d_model=512, d_ff=2048, rank=64, wtype=wtype,
                        pred_dtype="f32" if wtype == "f32" else "f16")
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 16, stream=300)
    _dense_layer_case(lay, x)


@pytest.mark.parametrize("thr,B", [(16, 15), (0, 40)])
def test_layer_below_threshold_or_default_stays_sparse(thr, B):
    spec = synth.config("c2", d_model=512, d_ff=2048, rank=64)
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, B, stream=301)
    pred, ffn = upload_layer(lay)
    pred.dense_min_batch = thr
    out = gpu_layer(pred, ffn, x)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
    gb = oracle.unpack_mask(out["mask"], 2048)
    outside = np.abs(ol - lay.tau[None, :].astype(np.float64)) > band
    assert not ((gb != ob) & outside).any()
    rid, rc, _ = oracle.compact(out["mask"], B, 2048)
    assert out["count"] == rc and np.array_equal(out["ids"][:rc], rid)
    assert not gb.all()  # the predictor's masks, not all ones
    ref = oracle.masked_ffn(lay, x, out["mask"])
    for b in range(B):
        assert rel_err(out["y"][b], ref[b]) <= TOL, b


@pytest.mark.parametrize("thr,B,dense", [(4, 4, True), (4, 3, False), (-1, 40, False), (0, 40, False),
                                         (40, 40, True), (1, 1, True)])
def test_layer_threshold_field(thr, B, dense):
    spec = synth.config("c5", d_model=768, d_ff=3072, rank=64)
    lay = synth.make_layer(spec, layer=1)
    x = synth.make_tokens(spec, B, stream=302 + B)
    if dense:
        _dense_layer_case(lay, x, dense_min_batch=thr, check_tokens=[0, B - 1])
        return
    pred, ffn = upload_layer(lay)
    pred.dense_min_batch = thr
    out = gpu_layer(pred, ffn, x)
    rid, rc, _ = oracle.compact(out["mask"], B, 3072)
    assert out["count"] == rc and np.array_equal(out["ids"][:rc], rid)
    assert not oracle.unpack_mask(out["mask"], 3072).all()
    ref = oracle.masked_ffn(lay, x, out["mask"])
    for b in (0, B - 1):
        assert rel_err(out["y"][b], ref[b]) <= TOL, b


def test_layer_opt6_7b_full_size_b16_dense():
    """OPT-6.7B layer at batch 16 (past its crossover): the dense FFN on the
    matrix cores; three tokens checked against the oracle's dense FFN, all
    of them bitwise against the dense entry point."""
    spec = synth.config("c2")
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 16, stream=303)
    _dense_layer_case(lay, x, check_tokens=[0, 7, 15])


def test_layer_opt175b_int4_shape_b32_dense():
    """OPT-175B's INT4-g128 layout and rank at batch 32, d_model / d_ff cut
    to a quarter so the oracle's dense FFN over all rows stays quick."""
    spec = synth.config("c5", d_model=3072, d_ff=12288)
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 32, stream=304)
    _dense_layer_case(lay, x, check_tokens=[0, 15, 31])


@pytest.mark.parametrize("lookahead", [False, True])
@pytest.mark.parametrize("cfg,B", [("c2", 16), ("c4", 20), ("c5", 32)])
def test_stack_dense(cfg, B, lookahead):
    spec = synth.config(cfg, d_model=768, d_ff=3072, rank=64, n_layers=3)
    L = 3
    lays = [synth.make_layer(spec, layer=l, seed=5) for l in range(L)]
    dev = [upload_layer(lay) for lay in lays]
    for pred, _ in dev:
        pred.dense_min_batch = 16
    r_in = synth.make_tokens(spec, B, stream=310 + B, dtype=np.float32) * np.float32(3.0)
    out = gpu_stack(dev, r_in, 1e-6, torch.float16, flags=1 if lookahead else 0)
    f = spec.d_ff
    r = r_in.astype(np.float32).copy()
    for l, lay in enumerate(lays):
        x = out["x"][l]
        _, x_ref = oracle.residual_rmsnorm(r, np.zeros_like(r), 1e-6)
        assert rel_err(x, x_ref) <= 1e-3, l
        xs = x.astype(spec.x_dtype)
        _check_dense_report(dict(mask=out["mask"][l], ids=out["ids"][l], count=out["count"][l]), B, f)
        ref = oracle.dense_ffn(lay, xs)
        for b in range(B):
            assert rel_err(out["y"][l][b], ref[b]) <= TOL, (l, b)
        # bitwise the single-layer call on the captured input (also dense at this batch)
        one = gpu_layer(dev[l][0], dev[l][1], xs)
        assert np.array_equal(one["y"], out["y"][l]), l
        r = (r + out["y"][l]).astype(np.float32)
    assert np.array_equal(out["r_out"], r)
