"""GPU parity of the helpers around the hot path: the residual + RMSNorm stack
step, offline fire counting, hot-first relayout (and that a relaid-out layer
computes the same outputs), and the bandwidth probes."""
import numpy as np
import pytest
import torch

import activation_sparse_gemv_amd as sg
import oracle
import synth
from gpu_util import gpu_layer, gpu_sparse_ffn, rel_err, to_dev, upload_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,d", [(1, 4096), (3, 640), (64, 128)])
@pytest.mark.parametrize("xt", [torch.float16, torch.float32])
def test_residual_rmsnorm(B, d, xt):
    g = np.random.default_rng(B)
    r = g.normal(0, 2, (B, d)).astype(np.float32)
    y = g.normal(0, 1, (B, d)).astype(np.float32)
    rd, yd = to_dev(r), to_dev(y)
    x = torch.empty((B, d), dtype=xt, device="cuda")
    sg.sfnn_residual_rmsnorm(rd, yd, rd, B, d, 1e-6, x)
    r_ref, x_ref = oracle.residual_rmsnorm(r, y, 1e-6)
    assert np.array_equal(rd.cpu().numpy(), (r + y))       # one fp32 add, exactly rounded
    tol = 1e-6 if xt == torch.float32 else 1e-3
    assert rel_err(x.float().cpu().numpy(), x_ref) <= tol
    # y = NULL copies r_in
    r2 = torch.empty_like(rd)
    sg.sfnn_residual_rmsnorm(yd, None, r2, B, d, 1e-6, x)
    assert np.array_equal(r2.cpu().numpy(), y)


@pytest.mark.parametrize("f,n", [(64, 1), (4096, 37), (28672, 256)])
def test_fire_counts(f, n):
    words = synth.random_masks(n, f, 0.2, seed=n)
    counts = torch.full((f,), 5, dtype=torch.int32, device="cuda")
    sg.sfnn_fire_counts(to_dev(words), n, f, counts)
    got = counts.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, oracle.fire_counts(words, f).astype(np.int64) + 5)


def test_gather_rows_and_hot_first_relayout_preserves_outputs():
    spec = synth.config("c3", d_model=512, d_ff=2048, rank=64)
    lay = synth.make_layer(spec, layer=0)
    f = spec.d_ff
    # profile: predicted masks of 128 seeded tokens
    xp = synth.make_tokens(spec, 128, stream=5)
    _, mp = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, xp)
    words = oracle.pack_mask(mp)
    counts = torch.zeros(f, dtype=torch.int32, device="cuda")
    sg.sfnn_fire_counts(to_dev(words), 128, f, counts)
    ch = counts.cpu().numpy().view(np.uint32).copy()
    perm = np.empty(f, dtype=np.int32)
    sg.sfnn_hot_first_perm(ch, f, perm)
    assert np.array_equal(perm, oracle.hot_first_perm(oracle.fire_counts(words, f)))
    pred, ffn = upload_layer(lay)
    x = synth.make_tokens(spec, 2, stream=6)
    before = gpu_layer(pred, ffn, x)
    pd = to_dev(perm)
    for t in [ffn.t["w_up"], ffn.t["w_down_t"], ffn.t["b_up"], pred.w2_t, pred.tau]:
        src = t.clone()
        sg.sfnn_gather_rows(src, pd, f, t.numel() * t.element_size() // f, t)
        ref = src.cpu().numpy()[perm]
        torch.cuda.synchronize()
        assert np.array_equal(t.cpu().numpy(), ref)
    after = gpu_layer(pred, ffn, x)
    assert np.array_equal(oracle.unpack_mask(after["mask"], f), oracle.unpack_mask(before["mask"], f)[:, perm])
    assert after["count"] == before["count"]
    assert list(after["ids"]) == list(oracle.permute_layer_ids(perm, before["ids"]))
    assert rel_err(after["y"], before["y"]) <= 1e-5
    # hot neurons now lead: the first quarter of the layout holds most of the fires
    hot_share = oracle.fire_counts(oracle.pack_mask(mp[:, perm]), f)[: f // 4].sum() / mp.sum()
    assert hot_share > 0.5


def test_probes_run():
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(buf)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    sg.sfnn_probe_read(buf, buf.numel() * 4, sink)
    sg.sfnn_probe_copy(buf, dst, buf.numel() * 4)
    torch.cuda.synchronize()
    assert torch.equal(buf, dst)
