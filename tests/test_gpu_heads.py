"""Head-gated attention projections through the C ABI against the oracle:
per-token head sets (the pages report up to 80% of heads skipped), fp16 and
fp32, batches 1 to 33, ragged head counts; rows of unused heads NaN-poisoned
(not read), outputs of heads off for a token exactly 0 (Q/K/V) or absent
(output projection); all heads = the dense projections; determinism."""
import numpy as np
import pytest
import torch

import oracle
import synth
import activation_sparse_gemv_amd as sg
from gpu_util import rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _run(w_qkv, b_qkv, w_o_t, b_o, hd, x, attn, words):
    op = sg.Heads(to_dev(w_qkv), to_dev(w_o_t), hd, to_dev(b_qkv), to_dev(b_o))
    B = x.shape[0]
    qkv = torch.full((B, w_qkv.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((B, w_o_t.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    hm = to_dev(words)
    ws = torch.empty(sg.sfnn_heads_workspace_bytes(op, B), dtype=torch.uint8, device="cuda")
    sg.sfnn_head_qkv(op, to_dev(x), B, hm, qkv)
    sg.sfnn_head_out(op, to_dev(attn), B, hm, y, ws)
    torch.cuda.synchronize()
    return qkv.cpu().numpy(), y.cpu().numpy()


def _case(d, H, hd, B, density, wtype="f16", seed=0, poison=True):
    w_qkv, b_qkv, w_o_t, b_o = synth.make_head_weights(d, H, hd, wtype, seed=seed)
    bits, words = synth.make_head_masks(B, H, density, seed=seed + B)
    xdt = np.float32 if wtype == "f32" else np.float16
    x = synth.make_relu_inputs(d, B, 1.0, seed=seed, stream=1, dtype=xdt)
    attn = synth.make_relu_inputs(H * hd, B, 1.0, seed=seed, stream=2, dtype=xdt)
    unused = ~bits.any(axis=0)
    attn_p = attn.copy()
    attn_p[np.repeat(~bits, hd, axis=1)] = np.nan   # entries of heads off for a token are not used
    wq_p, wo_p = w_qkv.copy(), w_o_t.copy()
    if poison:
        for h in np.flatnonzero(unused):
            for blk in range(3):
                wq_p[blk * H * hd + h * hd:blk * H * hd + (h + 1) * hd] = np.nan
            wo_p[h * hd:(h + 1) * hd] = np.nan
    qkv, y = _run(wq_p, b_qkv, wo_p, b_o, hd, x, attn_p, words)
    rq = oracle.head_qkv(w_qkv, b_qkv, x, bits, hd, return_f64=True)
    ry = oracle.head_out(w_o_t, b_o, attn, bits, hd, return_f64=True)
    off = rq == 0.0
    assert np.array_equal(qkv[off], np.zeros(int(off.sum()), dtype=np.float32)) and np.isfinite(qkv).all()
    for t in range(B):
        if bits[t].any():
            assert rel_err(qkv[t], rq[t]) <= TOL, t
        assert rel_err(y[t], ry[t]) <= TOL, t
    return bits, qkv, y


@pytest.mark.parametrize("B", [1, 2, 3, 8, 33])
@pytest.mark.parametrize("density", [0.2, 0.5])
def test_heads_opt6_7b_shape(B, density):
    """OPT-6.7B attention: d_model 4096, 32 heads of 128."""
    _case(4096, 32, 128, B, density)


@pytest.mark.parametrize("d,H,hd,B", [(768, 12, 64, 5), (1024, 24, 8, 3), (2048, 80, 64, 2), (16384, 8, 64, 2)])
def test_heads_ragged_shapes(d, H, hd, B):
    """12 heads of 64 (OPT-125M), head_dim 8, 80 heads (two mask words), d_model 16384."""
    _case(d, H, hd, B, 0.4, seed=d)


@pytest.mark.parametrize("B", [1, 4])
def test_heads_fp32(B):
    _case(768, 12, 64, B, 0.5, wtype="f32", seed=3)


@pytest.mark.parametrize("wtype,d,H,hd,B", [("f16", 16384, 8, 64, 5), ("f16", 12288, 16, 128, 8),
                                            ("f16", 12288, 16, 128, 11), ("f32", 4096, 8, 64, 8)])
def test_heads_qkv_chunked_x(wtype, d, H, hd, B):
    """x staged in several d_model chunks (8 tokens of a wide d_model do not fit
    64 KB at once), including a ragged last token group."""
    _case(d, H, hd, B, 0.5, wtype=wtype, seed=d + B)


def test_heads_all_and_none():
    d, H, hd, B = 1024, 16, 64, 3
    w_qkv, b_qkv, w_o_t, b_o = synth.make_head_weights(d, H, hd, "f16", seed=9)
    x = synth.make_relu_inputs(d, B, 1.0, seed=9, stream=1, dtype=np.float16)
    attn = synth.make_relu_inputs(H * hd, B, 1.0, seed=9, stream=2, dtype=np.float16)
    on = np.ones((B, 64), dtype=bool)
    qkv, y = _run(w_qkv, b_qkv, w_o_t, b_o, hd, x, attn, synth.pack_bits(on))
    dq = x.astype(np.float64) @ w_qkv.T.astype(np.float64) + b_qkv
    dy = attn.astype(np.float64) @ w_o_t.astype(np.float64) + b_o
    for t in range(B):
        assert rel_err(qkv[t], dq[t]) <= TOL and rel_err(y[t], dy[t]) <= TOL
    none = synth.pack_bits(np.zeros((B, 64), dtype=bool))
    qkv0, y0 = _run(w_qkv, b_qkv, w_o_t, b_o, hd, x, attn, none)
    assert not qkv0.any()
    assert np.array_equal(y0, np.tile(b_o.astype(np.float32), (B, 1)))


def test_heads_deterministic():
    a = _case(4096, 32, 128, 8, 0.3, seed=11)
    b = _case(4096, 32, 128, 8, 0.3, seed=11)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


# The output projection around the input-sparse GEMV's size limits (16384
# attention inputs, 96 heads of 128 as in OPT-175B, head_dim 8), fp16 and
# fp32, with unused heads' rows and off entries NaN-poisoned.
@pytest.mark.parametrize("wtype,d,H,hd,B", [
    ("f16", 1024, 96, 128, 1),    # OPT-175B's 96 heads of 128, d_model cut for the oracle
    ("f16", 1024, 128, 128, 2),   # 16384 inputs: the largest single-launch list
    ("f16", 1024, 130, 128, 1),   # 16640 inputs: gate + GEMV
    ("f32", 1024, 64, 128, 6),    # fp32, 6 tokens in one pass
    ("f16", 2048, 40, 8, 3),      # head_dim 8: 8 heads per mask word of 64 rows
])
def test_heads_out_single_launch_limits(wtype, d, H, hd, B):
    _case(d, H, hd, B, 0.3, wtype=wtype, seed=H + B)
