"""Parity of the matrix-core FFN path (k_up_mfma + k_down_mfma + k_sum) with the
float64 oracle, through the C ABI.

The path is selected per call by batch size (the FFN descriptor's
mfma_min_batch); these tests force it on (threshold 1) or off (-1).
Bars as for the per-row kernels: 2e-3 normwise relative error per token on
random layers, bit-exact on integer-grid layers (every intermediate an integer
below 2^22, so fp32 accumulation in any order and the two-part fp16 h are
exact), and bitwise run-to-run determinism.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import gpu_dense_ffn, gpu_sparse_ffn, rel_err, to_dev, upload_layer
from test_gpu_parity import TOL, _ffn_layer, _layer_case, full_layer

pytestmark = pytest.mark.gpu


ON, OFF = 1, -1  # mfma_min_batch: matrix cores for every batch / never


def _up(lay, thr):
    _, ffn = upload_layer(lay, predictor=False)
    ffn.mfma_min_batch = thr
    return ffn


def test_descriptor_threshold_round_trips():
    lay = _ffn_layer("f16", "relu", d=128, f=64)
    ffn = _up(lay, 0)
    assert ffn.mfma_min_batch == 0 and ffn.c.mfma_min_batch == 0
    ffn.mfma_min_batch = 5
    assert ffn.c.mfma_min_batch == 5


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("B", [1, 5, 16, 17, 32, 33, 64])
def test_mfma_sparse_ffn_random_masks(act, B):
    # d 640: 10 column pairs over 8 wavefronts; d_ff 1088: 34 row workgroups,
    # |U| ragged against the 32-slot steps
    lay = _ffn_layer("f16", act)
    x = synth.make_tokens(lay.spec, B, stream=140 + B)
    words = synth.random_masks(B, lay.spec.d_ff, 0.1, seed=100 + B)
    ffn = _up(lay, ON)
    y = gpu_sparse_ffn(ffn, x, words)
    ref = oracle.masked_ffn(lay, x, words)
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_mfma_matches_rows_path(act):
    """Both paths on the same call, each within the bar of the oracle."""
    lay = _ffn_layer("f16", act, d=1024, f=4096, seed=4)
    B = 16
    x = synth.make_tokens(lay.spec, B, stream=150)
    words = synth.random_masks(B, 4096, 0.2, seed=150)
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
def test_mfma_dense_ffn(act, B):
    lay = _ffn_layer("f16", act, d=1024, f=2048, seed=2)
    x = synth.make_tokens(lay.spec, B, stream=160 + B)
    ffn = _up(lay, ON)
    y = gpu_dense_ffn(ffn, x)
    ref = oracle.dense_ffn(lay, x)
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("B", [6, 17, 40])
def test_mfma_integer_grid_bitwise(act, B):
    d, f = (256, 1088) if act == "relu" else (128, 576)
    lay = synth.make_grid_layer(d, f, 32, act=act, wtype="f16", seed=20 + B)
    x = synth.make_grid_tokens(d, B, seed=20 + B, dtype=np.float16)
    words = synth.random_masks(B, f, 0.3, seed=20 + B)
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


def test_mfma_rows_outside_union_never_read():
    """NaN in every row and bias outside the union changes nothing, bitwise."""
    lay = _ffn_layer("f16", "reglu")
    B, f = 9, lay.spec.d_ff
    x = synth.make_tokens(lay.spec, B, stream=170)
    words = synth.random_masks(B, f, 0.05, seed=170)
    words[:, 0] &= ~np.uint64(1)  # keep row 0 out of the union
    ffn = _up(lay, ON)
    y_clean = gpu_sparse_ffn(ffn, x, words)
    _, _, uni = oracle.compact(words, B, f)
    off = ~oracle.unpack_mask(uni[None], f)[0]
    assert off[0]  # row 0 is outside the union: padding slots must not read it
    for name in ("w_up", "w_gate", "w_down_t", "b_up", "b_gate"):
        a = getattr(lay, name).copy()
        a[off] = np.float16(np.nan)
        setattr(lay, name, a)
    ffn2 = _up(lay, ON)
    y_poison = gpu_sparse_ffn(ffn2, x, words)
    assert np.isfinite(y_poison).all()
    assert np.array_equal(y_clean, y_poison)


def test_mfma_empty_set_gives_bias_bitwise():
    lay = _ffn_layer("f16", "relu")
    lay.b_down = (np.arange(lay.spec.d_model) % 7 - 3).astype(np.float16) * np.float16(0.25)
    B = 12
    x = synth.make_tokens(lay.spec, B, stream=180)
    words = np.zeros((B, lay.spec.d_ff // 64), dtype=np.uint64)
    ffn = _up(lay, ON)
    y = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(y, np.tile(lay.b_down.astype(np.float32), (B, 1)))


def test_mfma_out_of_range_ids_skipped_and_count_clamped():
    import torch
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import workspace
    lay = _ffn_layer("f16", "relu", d=256, f=1024)
    B = 3
    x = synth.make_tokens(lay.spec, B, stream=185)
    ffn = _up(lay, ON)
    ws = workspace(None, ffn, B)
    xd = to_dev(x)
    # ids 5, 1<<20 (out of range), -3 (out of range), 9: only 5 and 9 contribute
    ids = to_dev(np.array([5, 1 << 20, -3, 9] + [0] * 1020, dtype=np.int32))
    cnt = to_dev(np.array([4, 0, 0, 0], dtype=np.int32))
    y = torch.empty((B, 256), dtype=torch.float32, device="cuda")
    sg.sfnn_sparse_ffn(ffn, xd, B, ids, cnt, None, y, ws)
    m = np.zeros((B, 1024), dtype=bool)
    m[:, [5, 9]] = True
    ref = oracle.masked_ffn(lay, x, m)
    for b in range(B):
        assert rel_err(y.cpu().numpy()[b], ref[b]) <= TOL
    ids = to_dev(np.arange(1024, dtype=np.int32))
    cnt = to_dev(np.array([5000, 0, 0, 0], dtype=np.int32))
    sg.sfnn_sparse_ffn(ffn, xd, B, ids, cnt, None, y, ws)
    ref = oracle.dense_ffn(lay, x)
    for b in range(B):
        assert rel_err(y.cpu().numpy()[b], ref[b]) <= TOL


def test_mfma_deterministic_run_to_run():
    lay = _ffn_layer("f16", "reglu", d=1024, f=4096)
    B = 24
    x = synth.make_tokens(lay.spec, B, stream=190)
    words = synth.random_masks(B, 4096, 0.2, seed=190)
    ffn = _up(lay, ON)
    a = gpu_sparse_ffn(ffn, x, words)
    b = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(a, b)


def test_mfma_layer_opt6_7b_full_size_b32():
    spec = synth.config("c2")
    lay = full_layer("c2")
    x = synth.make_tokens(spec, 32, stream=5)
    _layer_case(lay, x, check_tokens=[0, 13, 31], mfma_min_batch=ON)


def test_mfma_layer_llama_reglu70b_full_size_b16():
    spec = synth.config("c4")
    lay = full_layer("c4")
    x = synth.make_tokens(spec, 16, stream=6)
    _layer_case(lay, x, check_tokens=[0, 15], mfma_min_batch=ON)


@pytest.mark.parametrize("lookahead", [False, True])
def test_mfma_stack_fp16_relu_b9(lookahead):
    from test_gpu_stack import _stack_case
    spec = synth.config("c2", d_model=512, d_ff=2048, rank=64, n_layers=3)
    _stack_case(spec, 3, 9, seed=11, lookahead=lookahead, mfma_min_batch=ON)


def test_rows_path_still_covers_large_batches():
    lay = _ffn_layer("f16", "relu")
    B = 17
    x = synth.make_tokens(lay.spec, B, stream=195)
    words = synth.random_masks(B, lay.spec.d_ff, 0.1, seed=195)
    ffn = _up(lay, OFF)
    y = gpu_sparse_ffn(ffn, x, words)
    ref = oracle.masked_ffn(lay, x, words)
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("lookahead", [False, True])
def test_mfma_stack_few_partial_rows_b9(lookahead):
    # d_model 1024: the matrix-core down projection writes 32 partial rows per
    # token, which the wide sum adds (with the residual) instead of k_sum
    from test_gpu_stack import _stack_case
    spec = synth.config("c2", d_model=1024, d_ff=2048, rank=64, n_layers=2)
    _stack_case(spec, 2, 9, seed=14, lookahead=lookahead, mfma_min_batch=ON)
