"""Every entry point can be captured in a HIP graph (no host synchronisation,
no allocation, no memset nodes): capture once, then replay several times with
new inputs copied into the captured buffers between replays (eager work and a
synchronisation in between), and check every replay bitwise against the eager
call on the same input.  The calls are deterministic, so bitwise is the bar.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as sg
import synth
from activation_sparse_gemv_amd.device import to_dev, upload_layer, workspace

pytestmark = pytest.mark.gpu


def _replays(run, set_input, inputs):
    """Capture run() once; for each input: eager result, then graph result."""
    set_input(inputs[0])
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    torch.cuda.synchronize()
    def raw(t):  # bit patterns, comparable for every dtype used here
        return t.view(torch.int64) if t.dtype == torch.uint64 else (t.view(torch.uint8) if t.dtype.is_floating_point else t)

    for inp in inputs:
        set_input(inp)
        eager = [raw(o).clone() for o in run()]
        torch.cuda.synchronize()
        for o in outs:  # poison the outputs, so a replay that writes nothing fails
            if o.dtype.is_floating_point:
                o.fill_(float("nan"))
            else:
                raw(o).fill_(123)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a, raw(b))


@pytest.mark.parametrize("B", [1, 9])
def test_graph_layer(B):
    spec = synth.config("c2", d_model=1024, d_ff=4096, rank=128)
    lay = synth.make_layer(spec, layer=0)
    pred, ffn = upload_layer(lay)
    pred.dense_min_batch = 16
    f, d = spec.d_ff, spec.d_model
    x = torch.empty((B, d), dtype=torch.float16, device="cuda")
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    mask = torch.zeros((B, f // 64), dtype=torch.uint64, device="cuda")
    ids = torch.empty(f, dtype=torch.int32, device="cuda")
    cnt = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = workspace(pred, ffn, B)

    def run():
        sg.sfnn_layer(pred, ffn, x, B, y, mask, ids, cnt, ws)
        return [y, mask, cnt[:1]]

    inputs = [synth.make_tokens(spec, B, stream=300 + k) for k in range(3)]
    _replays(run, lambda a: x.copy_(to_dev(a)), inputs)


def test_graph_stack_lookahead():
    spec = synth.config("c2", d_model=768, d_ff=3072, rank=96, n_layers=3)
    lays = [synth.make_layer(spec, layer=l) for l in range(3)]
    dev = [upload_layer(l) for l in lays]
    st = sg.Stack(dev)
    B = 1
    r_in = torch.empty((B, 768), dtype=torch.float32, device="cuda")
    r_out = torch.empty((B, 768), dtype=torch.float32, device="cuda")
    ws = workspace(dev[0][0], dev[0][1], B)

    def run():
        sg.sfnn_stack_decode(st, B, r_in, r_out, 1e-6, ws, flags=sg.SFNN_STACK_LOOKAHEAD)
        return [r_out]

    inputs = [synth.make_tokens(spec, B, stream=310 + k, dtype=np.float32) * np.float32(3.0) for k in range(3)]
    _replays(run, lambda a: r_in.copy_(to_dev(a)), inputs)


@pytest.mark.parametrize("B", [1, 9])
def test_graph_stack_lookahead_hot_prefix(B):
    """Look-ahead stack with a dense hot prefix; batch 9 runs the matrix-core predictor."""
    spec = synth.config("c2", d_model=768, d_ff=3072, rank=96, n_layers=3)
    lays = [synth.make_layer(spec, layer=l) for l in range(3)]
    dev = [upload_layer(l) for l in lays]
    for pred, _ in dev:
        pred.hot_prefix = 512
    st = sg.Stack(dev)
    r_in = torch.empty((B, 768), dtype=torch.float32, device="cuda")
    r_out = torch.empty((B, 768), dtype=torch.float32, device="cuda")
    mc = torch.zeros((3, B, 3072 // 64), dtype=torch.uint64, device="cuda")
    ws = workspace(dev[0][0], dev[0][1], B)

    def run():
        sg.sfnn_stack_decode(st, B, r_in, r_out, 1e-6, ws, flags=sg.SFNN_STACK_LOOKAHEAD, mask_cap=mc)
        return [r_out, mc]

    inputs = [synth.make_tokens(spec, B, stream=320 + k, dtype=np.float32) * np.float32(3.0) for k in range(3)]
    _replays(run, lambda a: r_in.copy_(to_dev(a)), inputs)


@pytest.mark.parametrize("B", [1, 6])
def test_graph_input_sparse_gemv(B):
    w_t, b = synth.make_isg_weights(1024, 2048, "f16", seed=5, key=5)
    op = sg.Isg(to_dev(w_t), to_dev(b))
    x = torch.empty((B, 1024), dtype=torch.float16, device="cuda")
    y = torch.empty((B, 2048), dtype=torch.float32, device="cuda")
    cols = torch.empty(1024, dtype=torch.int32, device="cuda")
    cnt = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(sg.sfnn_isg_workspace_bytes(op, B), dtype=torch.uint8, device="cuda")

    def run():
        sg.sfnn_input_sparse_gemv(op, x, B, y, ws, cols, cnt)
        return [y, cnt[:1]]

    inputs = [synth.make_relu_inputs(1024, B, 0.3, seed=k, stream=B) for k in range(3)]
    _replays(run, lambda a: x.copy_(to_dev(a)), inputs)


@pytest.mark.parametrize("B", [1, 8])
def test_graph_head_projections(B):
    d, H, hd = 1024, 16, 64
    w_qkv, b_qkv, w_o_t, b_o = synth.make_head_weights(d, H, hd, "f16", seed=13)
    op = sg.Heads(to_dev(w_qkv), to_dev(w_o_t), hd, to_dev(b_qkv), to_dev(b_o))
    x = torch.empty((B, d), dtype=torch.float16, device="cuda")
    attn = torch.empty((B, H * hd), dtype=torch.float16, device="cuda")
    hm = torch.zeros((B, 1), dtype=torch.uint64, device="cuda")
    qkv = torch.empty((B, 3 * H * hd), dtype=torch.float32, device="cuda")
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(sg.sfnn_heads_workspace_bytes(op, B), dtype=torch.uint8, device="cuda")

    def run():
        sg.sfnn_head_qkv(op, x, B, hm, qkv)
        sg.sfnn_head_out(op, attn, B, hm, y, ws)
        return [qkv, y]

    def set_input(k):
        x.copy_(to_dev(synth.make_relu_inputs(d, B, 1.0, seed=k, stream=1)))
        attn.copy_(to_dev(synth.make_relu_inputs(H * hd, B, 1.0, seed=k, stream=2)))
        hm.copy_(to_dev(synth.make_head_masks(B, H, 0.3, seed=k)[1]))

    _replays(run, set_input, [330, 331, 332])


@pytest.mark.parametrize("wtype", ["f16", "i4g128"])
def test_graph_layer_dense_switch(wtype):
    """Past the dense switch (batch 16): the fill of the reported mask / ids /
    count is a kernel, so the call captures and replays like the sparse one."""
    B = 16
    spec = synth.config("c2", d_model=512, d_ff=2048, rank=64, wtype=wtype)
    lay = synth.make_layer(spec, layer=0)
    pred, ffn = upload_layer(lay)
    pred.dense_min_batch = 16
    f, d = spec.d_ff, spec.d_model
    x = torch.empty((B, d), dtype=torch.float16, device="cuda")
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    mask = torch.zeros((B, f // 64), dtype=torch.uint64, device="cuda")
    ids = torch.empty(f, dtype=torch.int32, device="cuda")
    cnt = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = workspace(pred, ffn, B)

    def run():
        sg.sfnn_layer(pred, ffn, x, B, y, mask, ids, cnt, ws)
        return [y, mask, ids, cnt[:1]]

    inputs = [synth.make_tokens(spec, B, stream=320 + k) for k in range(3)]
    _replays(run, lambda a: x.copy_(to_dev(a)), inputs)


@pytest.mark.parametrize("dense_layers", [(0, 1, 2), (1,)])
def test_graph_stack_dense_switch(dense_layers):
    """Every layer dense, or one dense layer between sparse ones (the
    look-ahead schedule then runs stage by stage)."""
    B = 20
    spec = synth.config("c2", d_model=768, d_ff=3072, rank=96, n_layers=3)
    lays = [synth.make_layer(spec, layer=l) for l in range(3)]
    dev = [upload_layer(l) for l in lays]
    for l, (pred, _) in enumerate(dev):
        pred.dense_min_batch = 16 if l in dense_layers else 0
    st = sg.Stack(dev)
    d, f = spec.d_model, spec.d_ff
    r_in = torch.empty((B, d), dtype=torch.float32, device="cuda")
    r_out = torch.empty((B, d), dtype=torch.float32, device="cuda")
    mc = torch.zeros((3, B, f // 64), dtype=torch.uint64, device="cuda")
    cc = torch.empty(3, dtype=torch.int32, device="cuda")
    ws = workspace(dev[0][0], dev[0][1], B)

    def run():
        sg.sfnn_stack_decode(st, B, r_in, r_out, 1e-6, ws, flags=sg.SFNN_STACK_LOOKAHEAD, mask_cap=mc,
                             count_cap=cc)
        return [r_out, mc, cc]

    inputs = [synth.make_tokens(spec, B, stream=330 + k, dtype=np.float32) for k in range(3)]
    _replays(run, lambda a: r_in.copy_(to_dev(a)), inputs)
