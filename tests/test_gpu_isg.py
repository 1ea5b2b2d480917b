"""Parity of the input-sparse GEMV (relufication stage 2: ReLU after the
normalisation layer, [53ai] 第二阶段——插入新的ReLU) with the float64 oracle,
through the C ABI.

Bars: the listed inputs J and their count are bit-exact; y within 2e-3
normwise relative error per token (fp32 accumulation in a different order
than the oracle's); bit-exact on integer-grid inputs (every partial sum an
integer below 2^24); rows of w_t outside J are never read (NaN there changes
nothing); bitwise run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as sg
import oracle
import synth
from gpu_util import rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _run(w_t, bias, x):
    B, n_in = x.shape
    n_out = w_t.shape[1]
    op = sg.Isg(to_dev(w_t), to_dev(bias))
    ws = torch.empty(sg.sfnn_isg_workspace_bytes(op, B), dtype=torch.uint8, device="cuda")
    y = torch.full((B, n_out), float("nan"), dtype=torch.float32, device="cuda")
    cols = torch.full((n_in,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    sg.sfnn_input_sparse_gemv(op, to_dev(x), B, y, ws, cols, cnt)
    torch.cuda.synchronize()
    c = int(cnt[0].item())
    return y.cpu().numpy(), cols.cpu().numpy(), c


def _case(n_in, n_out, B, density, wtype, seed, bias=True):
    w_t, b = synth.make_isg_weights(n_in, n_out, wtype, seed=seed, key=seed, bias=bias)
    x = synth.make_relu_inputs(n_in, B, density, seed=seed, stream=B,
                               dtype=np.float32 if wtype == "f32" else np.float16)
    return w_t, b, x


@pytest.mark.parametrize("wtype", ["f16", "f32"])
@pytest.mark.parametrize("B", [1, 3, 8, 9, 17, 33])
@pytest.mark.parametrize("density", [0.5, 0.1])
def test_isg_random(wtype, B, density):
    # n_in 640 (10 mask words), n_out 2176: one full 2048-column block and a
    # ragged one; fp16 from 4 tokens takes the matrix cores (passes of 32),
    # fp32 the per-row kernel (passes of 8)
    w_t, b, x = _case(640, 2176, B, density, wtype, seed=B)
    y, cols, c = _run(w_t, b, x)
    ref, J = oracle.input_sparse_gemv(w_t, x, b)
    assert c == len(J) and np.array_equal(cols[:c], J)
    assert np.all(cols[c:] == -7)
    for t in range(B):
        assert rel_err(y[t], ref[t]) <= TOL, t


@pytest.mark.parametrize("B", [1, 16])
def test_isg_opt6_7b_up_projection_shape(B):
    """d_model 4096 -> d_ff 16384, the up projection of OPT-6.7B, half the
    inputs zero (a plain ReLU of a normalised input)."""
    w_t, b, x = _case(4096, 16384, B, 0.5, "f16", seed=40 + B, bias=False)
    y, cols, c = _run(w_t, b, x)
    ref, J = oracle.input_sparse_gemv(w_t, x, b)
    assert c == len(J) and np.array_equal(cols[:c], J)
    for t in range(B):
        assert rel_err(y[t], ref[t]) <= TOL, t


@pytest.mark.parametrize("wtype", ["f16", "f32"])
@pytest.mark.parametrize("B", [1, 5, 12])
def test_isg_integer_grid_bitwise(wtype, B):
    g = np.random.default_rng(50 + B)
    dt = np.float32 if wtype == "f32" else np.float16
    w_t = g.integers(-2, 3, (512, 1024)).astype(dt)
    bias = g.integers(-8, 9, 1024).astype(dt)
    x = (g.integers(-2, 3, (B, 512)) * (g.random((B, 512)) < 0.3)).astype(dt)
    y, cols, c = _run(w_t, bias, x)
    ref, J = oracle.input_sparse_gemv(w_t, x, bias, return_f64=True)
    assert c == len(J) and np.array_equal(cols[:c], J)
    assert np.array_equal(y.astype(np.float64), ref)


def test_isg_unlisted_rows_never_read():
    w_t, b, x = _case(1024, 2048, 4, 0.1, "f16", seed=60)
    y, cols, c = _run(w_t, b, x)
    off = np.ones(1024, dtype=bool)
    off[cols[:c]] = False
    assert off.any()
    w2 = w_t.copy()
    w2[off] = np.float16(np.nan)
    y2, cols2, c2 = _run(w2, b, x)
    assert np.isfinite(y2).all() and c2 == c
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("wt,B", [("f16", 1), ("f16", 2), ("f32", 3), ("f16", 5)])
def test_isg_unlisted_rows_never_read_row0_off(wt, B):
    """Per-row kernel (fp16 below 4 tokens, fp32) and matrix cores: input 0 is
    zero for every token and its row is NaN; the slots past each workgroup's
    share of the list must re-read a listed row, never row 0."""
    w_t, b, x = _case(1024, 2048, B, 0.3, wt, seed=62 + B)
    x[:, 0] = 0
    y, cols, c = _run(w_t, b, x)
    off = np.ones(1024, dtype=bool)
    off[cols[:c]] = False
    assert off[0]
    w2 = w_t.copy()
    w2[off] = np.nan
    y2, _, c2 = _run(w2, b, x)
    assert np.isfinite(y2).all() and c2 == c
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("B", [3, 6])
def test_isg_zero_input_gives_bias_bitwise(B):
    w_t, b, _ = _case(256, 512, 1, 0.5, "f16", seed=61)
    x = np.zeros((B, 256), dtype=np.float16)
    x[1, 7] = np.float16(-0.0)  # a negative zero is a zero input
    y, cols, c = _run(w_t, b, x)
    assert c == 0
    assert np.array_equal(y, np.tile(b.astype(np.float32), (B, 1)))


def test_isg_dense_input_and_no_bias():
    w_t, _, x = _case(384, 640, 6, 1.0, "f32", seed=62, bias=False)
    y, cols, c = _run(w_t, None, x)
    ref, J = oracle.input_sparse_gemv(w_t, x, None)
    assert c == 384 and np.array_equal(cols[:c], np.arange(384))
    for t in range(6):
        assert rel_err(y[t], ref[t]) <= TOL, t


def test_isg_deterministic():
    w_t, b, x = _case(2048, 4096, 8, 0.3, "f16", seed=63)
    a = _run(w_t, b, x)[0]
    c = _run(w_t, b, x)[0]
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


# Single-launch form: every workgroup lists the nonzero inputs itself (per-row
# path, n_in <= 16384, no row groups); past those limits the mask, compaction
# and GEMV launches.  Both sides of each limit, with the list reported.
@pytest.mark.parametrize("wtype,n_in,n_out,B", [
    ("f16", 16384, 256, 1),    # largest list the LDS holds
    ("f16", 16448, 256, 1),    # one mask word more: three launches
    ("f16", 8192, 16384, 2),   # long rows: 8192 x 128-byte tiles stay within one row group
    ("f16", 9216, 12288, 1),   # 9216 x 128-byte tiles pass 1 MB: row groups, three launches
    ("f32", 8192, 512, 8),     # fp32, eight tokens a pass
    ("f32", 8192, 4352, 8),    # fp32 128-byte tiles x eight tokens: the largest reduction buffer
    ("f16", 64, 128, 3),       # one mask word
])
def test_isg_single_launch_limits(wtype, n_in, n_out, B):
    w_t, b, x = _case(n_in, n_out, B, 0.3, wtype, seed=n_in + B)
    y, cols, c = _run(w_t, b, x)
    ref, J = oracle.input_sparse_gemv(w_t, x, b)
    assert c == len(J) and np.array_equal(cols[:c], J)
    assert np.all(cols[c:] == -7)
    for t in range(B):
        assert rel_err(y[t], ref[t]) <= TOL, t


def test_isg_single_launch_all_zero_and_nan_inputs():
    """An all-zero batch lists nothing (y = bias bitwise); a NaN input is not a
    zero, so its row is listed; -0.0 is a zero."""
    w_t, b, x = _case(1024, 512, 1, 0.3, "f16", seed=71)
    z = np.zeros_like(x)
    y, cols, c = _run(w_t, b, z)
    assert c == 0 and np.array_equal(y[0], b.astype(np.float32))
    x2 = np.zeros_like(x)
    x2[0, 5] = np.float16(-0.0)
    x2[0, 700] = np.float16(np.nan)
    x2[0, 1023] = np.float16(2.0)
    y2, cols2, c2 = _run(w_t, b, x2)
    assert c2 == 2 and np.array_equal(cols2[:2], [700, 1023])
    assert np.isnan(y2[0]).all()
