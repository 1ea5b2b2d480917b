"""Parity of the residual-stack entry point (sfnn_stack_decode) with the
oracle, layer by layer, on the inputs the GPU captured for each layer.

For every layer l: the captured input x_l is the RMS-normalised residual
r_l = r_in + y_0 + ... + y_{l-1} (fp32 adds in that order); its mask is the
predictor's threshold outside the rounding band (of x_l, or with the
look-ahead flag of x_{l-1} for l >= 1); ids/count are the compaction of that
mask, bit-exact; y_l matches the oracle's masked FFN of x_l within 2e-3; and
without look-ahead y_l is bitwise what sfnn_layer returns for the same x_l.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gpu_layer, gpu_stack, rel_err, upload_layer

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _stack_case(spec, L, B, seed=0, lookahead=False, mfma_min_batch=0, hot_prefix=0, dense_layers=(),
                down_bias=False):
    """dense_layers: layers whose dense switch is set at this batch (the
    others stay sparse).  down_bias: a nonzero b_down on every layer (the
    generated layers have none), so the bias and the residual meet in the
    same output columns."""
    lays = [synth.make_layer(spec, layer=l, seed=seed) for l in range(L)]
    if down_bias:
        for l, lay in enumerate(lays):
            g = np.random.default_rng(900 + l)
            lay.b_down = (g.normal(0.0, 0.1, spec.d_model)).astype(lay.b_down.dtype)
    dev = [upload_layer(lay) for lay in lays]
    for l, (pred, ffn) in enumerate(dev):
        ffn.mfma_min_batch = mfma_min_batch
        pred.hot_prefix = hot_prefix
        pred.dense_min_batch = B if l in dense_layers else -1
    r_in = synth.make_tokens(spec, B, stream=200 + B, dtype=np.float32) * np.float32(3.0)
    xdt = torch.float32 if spec.wtype == "f32" else torch.float16
    out = gpu_stack(dev, r_in, 1e-6, xdt, flags=1 if lookahead else 0)
    f = spec.d_ff
    r = r_in.astype(np.float32).copy()
    for l, lay in enumerate(lays):
        x = out["x"][l]
        # the layer input is the RMS-normalised running residual
        _, x_ref = oracle.residual_rmsnorm(r, np.zeros_like(r), 1e-6)
        assert rel_err(x, x_ref) <= (1e-6 if spec.wtype == "f32" else 1e-3), l
        xs = x.astype(spec.x_dtype)
        assert np.array_equal(xs.astype(np.float32), x)
        if l in dense_layers:
            # no predictor: all-ones mask, every id, the dense FFN
            assert np.array_equal(out["mask"][l], np.full((B, f // 64), np.uint64(2 ** 64 - 1))), l
            assert out["count"][l] == f and np.array_equal(out["ids"][l], np.arange(f, dtype=np.int32)), l
            ref = oracle.dense_ffn(lay, xs)
            for b in range(B):
                assert rel_err(out["y"][l][b], ref[b]) <= TOL, (l, b)
            one = gpu_layer(dev[l][0], dev[l][1], xs)
            assert np.array_equal(one["y"], out["y"][l]), l
            r = (r + out["y"][l]).astype(np.float32)
            continue
        # mask: threshold of the predictor on its input (x_l, or x_{l-1} when
        # looking ahead), outside the fp32 rounding band
        xp = xs if (not lookahead or l == 0) else out["x"][l - 1].astype(spec.x_dtype)
        ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, xp, hot_prefix=hot_prefix)
        band = oracle.guard_band(lay.w1_t, lay.w2_t, xp)
        gb = oracle.unpack_mask(out["mask"][l], f)
        outside = np.abs(ol - lay.tau[None, :].astype(np.float64)) > band
        assert not ((gb != ob) & outside).any(), l
        # inside the band a bit may go either way, but only for a handful of neurons
        assert ((gb != ob) & ~outside).sum() <= max(1, int(1e-4 * gb.size)), l
        # ids / count: compaction of the GPU's own mask, bit-exact
        rid, rc, _ = oracle.compact(out["mask"][l], B, f)
        assert out["count"][l] == rc and np.array_equal(out["ids"][l][:rc], rid), l
        # y: the oracle's masked FFN on the same input and mask
        ref = oracle.masked_ffn(lay, xs, out["mask"][l])
        for b in range(B):
            assert rel_err(out["y"][l][b], ref[b]) <= TOL, (l, b)
        # and bitwise the single-layer entry point on the captured input
        if not lookahead:
            one = gpu_layer(dev[l][0], dev[l][1], xs)
            assert np.array_equal(one["y"], out["y"][l]), l
            assert np.array_equal(one["mask"], out["mask"][l]), l
        r = (r + out["y"][l]).astype(np.float32)
    assert np.array_equal(out["r_out"], r)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_stack_fp16_relu(B):
    _stack_case(synth.config("c2", d_model=1024, d_ff=4096, rank=128, n_layers=3), 3, B)


@pytest.mark.parametrize("B", [1, 4])
def test_stack_fp16_reglu_zipf(B):
    _stack_case(synth.config("c4", d_model=768, d_ff=2048, rank=64, n_layers=3), 3, B)


@pytest.mark.parametrize("B", [1, 2, 9])
def test_stack_int4(B):
    _stack_case(synth.config("c5", d_model=1536, d_ff=3072, rank=128, n_layers=2), 2, B)


def test_stack_fp32_opt125m_shape():
    _stack_case(synth.config("c1", n_layers=2), 2, 1)


def test_stack_opt6_7b_full_width_two_layers():
    """Full OPT-6.7B layer shape (d_model 4096, d_ff 16384, rank 1024), 2 layers, batch 1."""
    _stack_case(synth.config("c2"), 2, 1)


def test_stack_single_layer_and_aliasing():
    spec = synth.config("c2", d_model=512, d_ff=1024, rank=64, n_layers=1)
    lay = synth.make_layer(spec, layer=0)
    pred, ffn = upload_layer(lay)
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import to_dev, workspace
    r_in = synth.make_tokens(spec, 2, stream=9, dtype=np.float32)
    out = gpu_stack([(pred, ffn)], r_in)
    # r_out may alias r_in
    r = to_dev(r_in)
    ws = workspace(pred, ffn, 2)
    sg.sfnn_stack_decode(sg.Stack([(pred, ffn)]), 2, r, r, 1e-6, ws)
    torch.cuda.synchronize()
    assert np.array_equal(r.cpu().numpy(), out["r_out"])


# ---------------------------------------------------------------------------
# look-ahead predictor: batches 1 and 2 run the fused two-launch schedule,
# larger batches the same schedule as separate launches
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B", [1, 2, 3])
def test_stack_lookahead_fp16_relu(B):
    _stack_case(synth.config("c2", d_model=1024, d_ff=4096, rank=128, n_layers=3), 3, B, lookahead=True)


@pytest.mark.parametrize("B", [1, 2, 5])
def test_stack_lookahead_fp16_reglu_zipf(B):
    _stack_case(synth.config("c4", d_model=768, d_ff=2048, rank=64, n_layers=3), 3, B, lookahead=True)


@pytest.mark.parametrize("B", [1, 2, 4])
def test_stack_lookahead_int4(B):
    _stack_case(synth.config("c5", d_model=1536, d_ff=3072, rank=128, n_layers=3), 3, B, lookahead=True)


@pytest.mark.parametrize("B", [1, 3])
def test_stack_lookahead_fp32(B):
    _stack_case(synth.config("c1", n_layers=2), 2, B, lookahead=True)


def test_stack_lookahead_single_layer():
    _stack_case(synth.config("c2", d_model=512, d_ff=1024, rank=64, n_layers=1), 1, 1, lookahead=True)


def test_stack_lookahead_opt6_7b_full_width():
    """Full OPT-6.7B layer shape, 3 layers, batch 1 (the fused schedule at bench shape)."""
    _stack_case(synth.config("c2"), 3, 1, lookahead=True)


def test_stack_lookahead_int4_wide():
    """d_model 12288 INT4 (32 columns per thread in the down projection), 2 layers."""
    _stack_case(synth.config("c5", d_ff=4096, rank=256, n_layers=2), 2, 1, lookahead=True)


@pytest.mark.parametrize("lookahead", [False, True])
@pytest.mark.parametrize("cfg,kw,B", [
    ("c2", dict(d_model=1024, d_ff=4096, rank=128, n_layers=3), 1),
    ("c2", dict(d_model=1024, d_ff=4096, rank=128, n_layers=3), 2),
    ("c5", dict(d_model=1536, d_ff=3072, rank=128, n_layers=3), 1),
    ("c4", dict(d_model=768, d_ff=2048, rank=64, n_layers=3), 9),
])
def test_stack_down_bias(cfg, kw, B, lookahead):
    """A nonzero down-projection bias through the whole stack: y_l = b_down +
    the gated rows, r_{l+1} = r_l + y_l, per-row and matrix-core batches."""
    _stack_case(synth.config(cfg, **kw), 3, B, lookahead=lookahead, down_bias=True)


@pytest.mark.parametrize("cfg,kw,B", [
    ("c2", dict(d_model=1024, d_ff=4096, rank=128, n_layers=3), 1),
    ("c4", dict(d_model=768, d_ff=2048, rank=64, n_layers=3), 2),
    ("c5", dict(d_model=1536, d_ff=3072, rank=128, n_layers=3), 1),
    ("c5", dict(d_model=1536, d_ff=3072, rank=128, n_layers=3), 4),
])
def test_stack_lookahead_deterministic(cfg, kw, B):
    """Two runs of the look-ahead stack on the same inputs agree bit for bit
    (every reduction has a fixed order; how the launches' workgroups are
    scheduled on the CUs must not show in the results)."""
    spec = synth.config(cfg, **kw)
    lays = [synth.make_layer(spec, layer=l) for l in range(spec.n_layers)]
    dev = [upload_layer(lay) for lay in lays]
    for pred, ffn in dev:
        pred.dense_min_batch = -1
    r_in = synth.make_tokens(spec, B, stream=310 + B, dtype=np.float32) * np.float32(3.0)
    xdt = torch.float32 if spec.wtype == "f32" else torch.float16
    a = gpu_stack(dev, r_in, 1e-6, xdt, flags=1)
    b = gpu_stack(dev, r_in, 1e-6, xdt, flags=1)
    assert np.isfinite(a["r_out"]).all()
    for k in ("r_out", "x", "y", "mask", "ids", "count"):
        assert np.array_equal(a[k], b[k], equal_nan=(k in ("x", "y"))), k


# dense hot prefix (the first neurons taken for every token): per-layer and
# look-ahead schedules, per-row and matrix-core batches
@pytest.mark.parametrize("B", [1, 9])
def test_stack_hot_prefix(B):
    _stack_case(synth.config("c4", d_model=768, d_ff=2048, rank=64, n_layers=3), 3, B, hot_prefix=512)


@pytest.mark.parametrize("B", [1, 2, 9])
def test_stack_lookahead_hot_prefix(B):
    _stack_case(synth.config("c2", d_model=1024, d_ff=4096, rank=128, n_layers=3), 3, B, lookahead=True,
                hot_prefix=1024)


# per-layer dense switch: a step mixes dense layers (no predictor) with
# sparse ones; with look-ahead, a sparse layer still predicts from the input
# of the layer before it, dense or not
@pytest.mark.parametrize("lookahead", [False, True])
@pytest.mark.parametrize("B,dense_layers", [(1, (1,)), (2, (0, 2)), (4, (1, 3)), (9, (0,)), (9, (3,))])
def test_stack_mixed_dense_fp16(B, dense_layers, lookahead):
    _stack_case(synth.config("c2", d_model=1024, d_ff=4096, rank=128, n_layers=4), 4, B, lookahead=lookahead,
                dense_layers=dense_layers)


@pytest.mark.parametrize("B,dense_layers", [(1, (0,)), (3, (1,))])
def test_stack_mixed_dense_int4_lookahead(B, dense_layers):
    _stack_case(synth.config("c5", d_model=1536, d_ff=3072, rank=128, n_layers=3), 3, B, lookahead=True,
                dense_layers=dense_layers)


def test_stack_mixed_dense_fp32_lookahead():
    _stack_case(synth.config("c1", n_layers=3), 3, 2, lookahead=True, dense_layers=(1,))


def test_stack_mixed_dense_reglu_hot_prefix_lookahead():
    _stack_case(synth.config("c4", d_model=768, d_ff=2048, rank=64, n_layers=3), 3, 2, lookahead=True,
                hot_prefix=512, dense_layers=(2,))


def test_stack_bad_flags_rejected():
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import workspace
    spec = synth.config("c2", d_model=512, d_ff=1024, rank=64, n_layers=1)
    pred, ffn = upload_layer(synth.make_layer(spec, layer=0))
    r = torch.zeros((1, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(sg.SfnnError):
        sg.sfnn_stack_decode(sg.Stack([(pred, ffn)]), 1, r, r, 1e-6, workspace(pred, ffn, 1), flags=6)
