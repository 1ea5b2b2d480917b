"""Parity of the INT4-g128 matrix-core FFN path (k_up_mfma_i4 + k_down_mfma_i4
+ k_sum) with the float64 oracle, through the C ABI.

The path is selected per call by batch size (the FFN descriptor's
mfma_min_batch); these tests force it on (threshold 1) or off (-1).  No weight
is rounded on this path (nibbles enter the matrix cores as fp16 integers, the
group scales are applied in fp32), so the bars are those of the per-row
kernels: 2e-3 normwise relative error per token on random layers, bit-exact on
integer-grid layers (power-of-two scales, every intermediate an integer below
2^22), and bitwise run-to-run determinism.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import gpu_dense_ffn, gpu_sparse_ffn, rel_err, upload_layer
from test_gpu_parity import TOL, _ffn_layer

pytestmark = pytest.mark.gpu

ON, OFF = 1, -1


def _up(lay, thr):
    _, ffn = upload_layer(lay, predictor=False)
    ffn.mfma_min_batch = thr
    return ffn


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("B", [1, 5, 16, 17, 32, 33])
def test_mfma_i4_sparse_ffn_random_masks(act, B):
    # d 640: 5 scale groups over 8 wavefronts (3 idle) and 5 column
    # workgroups (an odd count: the XCD pairing leaves the tail unpaired);
    # d_ff 1088: |U| ragged against the 64- and 96-row up workgroups and 32-slot steps
    lay = _ffn_layer("i4g128", act)
    x = synth.make_tokens(lay.spec, B, stream=240 + B)
    words = synth.random_masks(B, lay.spec.d_ff, 0.1, seed=200 + B)
    ffn = _up(lay, ON)
    y = gpu_sparse_ffn(ffn, x, words)
    ref = oracle.masked_ffn(lay, x, words)
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_mfma_i4_matches_rows_path(act):
    lay = _ffn_layer("i4g128", act, d=2048, f=4096, seed=4)
    B = 16
    x = synth.make_tokens(lay.spec, B, stream=250)
    words = synth.random_masks(B, 4096, 0.2, seed=250)
    ffn = _up(lay, OFF)
    ref = oracle.masked_ffn(lay, x, words)
    y_rows = gpu_sparse_ffn(ffn, x, words)
    ffn.mfma_min_batch = ON
    y_mfma = gpu_sparse_ffn(ffn, x, words)
    for b in range(B):
        assert rel_err(y_rows[b], ref[b]) <= TOL, b
        assert rel_err(y_mfma[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("B", [8, 32])
def test_mfma_i4_dense_ffn(act, B):
    lay = _ffn_layer("i4g128", act, d=1024, f=2048, seed=2)
    x = synth.make_tokens(lay.spec, B, stream=260 + B)
    ffn = _up(lay, ON)
    y = gpu_dense_ffn(ffn, x)
    ref = oracle.dense_ffn(lay, x)
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("B", [6, 17, 40])
def test_mfma_i4_integer_grid_bitwise(act, B):
    d, f = (256, 1088) if act == "relu" else (128, 576)
    lay = synth.make_grid_layer(d, f, 32, act=act, wtype="i4g128", seed=30 + B)
    x = synth.make_grid_tokens(d, B, seed=30 + B, dtype=np.float16)
    words = synth.random_masks(B, f, 0.3, seed=30 + B)
    ffn = _up(lay, ON)
    ref = oracle.masked_ffn(lay, x, words, return_f64=True)
    assert np.abs(ref).max() < 2 ** 22
    y = gpu_sparse_ffn(ffn, x, words)
    yd = gpu_dense_ffn(ffn, x)
    ffn.mfma_min_batch = OFF
    y_rows = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(y.astype(np.float64), ref)
    assert np.array_equal(yd.astype(np.float64), oracle.dense_ffn(lay, x, return_f64=True))
    assert np.array_equal(y, y_rows)  # the two paths agree bitwise on the grid


def test_mfma_i4_rows_outside_union_never_read():
    """NaN scales and biases on every row outside the union change nothing."""
    lay = _ffn_layer("i4g128", "reglu")
    B, f = 9, lay.spec.d_ff
    x = synth.make_tokens(lay.spec, B, stream=270)
    words = synth.random_masks(B, f, 0.05, seed=270)
    words[:, 0] &= ~np.uint64(1)  # keep row 0 out of the union
    ffn = _up(lay, ON)
    y_clean = gpu_sparse_ffn(ffn, x, words)
    _, _, uni = oracle.compact(words, B, f)
    off = ~oracle.unpack_mask(uni[None], f)[0]
    assert off[0]  # row 0 is outside the union: padding slots must not read it
    for name in ("s_up", "s_gate", "s_down_t", "b_up", "b_gate"):
        a = getattr(lay, name).copy()
        a[off] = np.float16(np.nan)
        setattr(lay, name, a)
    ffn2 = _up(lay, ON)
    y_poison = gpu_sparse_ffn(ffn2, x, words)
    assert np.isfinite(y_poison).all()
    assert np.array_equal(y_clean, y_poison)


def test_mfma_i4_empty_set_gives_bias_bitwise():
    lay = _ffn_layer("i4g128", "relu")
    lay.b_down = (np.arange(lay.spec.d_model) % 7 - 3).astype(np.float16) * np.float16(0.25)
    B = 12
    x = synth.make_tokens(lay.spec, B, stream=280)
    words = np.zeros((B, lay.spec.d_ff // 64), dtype=np.uint64)
    ffn = _up(lay, ON)
    y = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(y, np.tile(lay.b_down.astype(np.float32), (B, 1)))


def test_mfma_i4_deterministic_run_to_run():
    lay = _ffn_layer("i4g128", "reglu", d=1024, f=4096)
    B = 24
    x = synth.make_tokens(lay.spec, B, stream=290)
    words = synth.random_masks(B, 4096, 0.2, seed=290)
    ffn = _up(lay, ON)
    a = gpu_sparse_ffn(ffn, x, words)
    b = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("lookahead", [False, True])
def test_mfma_i4_stack_b12(lookahead):
    from test_gpu_stack import _stack_case
    spec = synth.config("c5", d_model=768, d_ff=3072, rank=64, n_layers=3)
    _stack_case(spec, 3, 12, seed=13, lookahead=lookahead, mfma_min_batch=ON)
