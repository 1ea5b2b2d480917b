"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
host-generated inputs and bring the results back as numpy arrays."""
from __future__ import annotations

import numpy as np
import torch

import activation_sparse_gemv_amd as sg
from activation_sparse_gemv_amd.device import to_dev, upload_layer, workspace

DEV = "cuda"


def rel_err(got, ref) -> float:
    """Normwise relative error ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def gpu_compact(words: np.ndarray, batch: int, f: int):
    m = to_dev(words.reshape(batch, f // 64))
    ids = torch.full((f,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((4,), -1, dtype=torch.int32, device=DEV)
    uni = torch.zeros(f // 64, dtype=torch.uint64, device=DEV)
    sg.sfnn_compact(m, batch, f, ids, cnt, uni)
    torch.cuda.synchronize()
    c = int(cnt[0].item())
    return ids.cpu().numpy(), c, uni.cpu().numpy()


def gpu_predict(pred, x: np.ndarray, f: int, with_logits=True):
    B = x.shape[0]
    xd = to_dev(x)
    mask = torch.zeros((B, f // 64), dtype=torch.uint64, device=DEV)
    logits = torch.zeros((B, f), dtype=torch.float32, device=DEV) if with_logits else None
    ws = workspace(pred, None, B)
    sg.sfnn_predict(pred, xd, B, mask, logits, ws)
    torch.cuda.synchronize()
    return mask.cpu().numpy(), (logits.cpu().numpy() if with_logits else None)


def gpu_sparse_ffn(ffn, x: np.ndarray, words: np.ndarray, gate=True):
    """Compaction + sparse FFN on the given per-token masks (packed words)."""
    B = x.shape[0]
    f, d = ffn.d_ff, ffn.d_model
    xd = to_dev(x)
    m = to_dev(words.reshape(B, f // 64))
    ids = torch.empty(f, dtype=torch.int32, device=DEV)
    cnt = torch.empty(4, dtype=torch.int32, device=DEV)
    y = torch.full((B, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(None, ffn, B)
    sg.sfnn_compact(m, B, f, ids, cnt)
    sg.sfnn_sparse_ffn(ffn, xd, B, ids, cnt, m if gate else None, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_dense_ffn(ffn, x: np.ndarray):
    B = x.shape[0]
    y = torch.full((B, ffn.d_model), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(None, ffn, B)
    sg.sfnn_dense_ffn(ffn, to_dev(x), B, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_layer(pred, ffn, x: np.ndarray):
    B = x.shape[0]
    f, d = ffn.d_ff, ffn.d_model
    mask = torch.zeros((B, f // 64), dtype=torch.uint64, device=DEV)
    ids = torch.empty(f, dtype=torch.int32, device=DEV)
    cnt = torch.empty(4, dtype=torch.int32, device=DEV)
    y = torch.full((B, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(pred, ffn, B)
    sg.sfnn_layer(pred, ffn, to_dev(x), B, y, mask, ids, cnt, ws)
    torch.cuda.synchronize()
    c = int(cnt[0].item())
    return dict(y=y.cpu().numpy(), mask=mask.cpu().numpy(), ids=ids.cpu().numpy()[:c], count=c)


def band_check(gpu_words, gpu_logits, ora_logits, band, tau, f):
    """Mask parity under the guard-band rule.

    Returns the number of bits inside the band that differ (allowed) after
    asserting (a) the GPU mask is exactly the threshold of the GPU's own fp32
    logits and (b) every bit outside the band equals the oracle's.
    """
    import oracle
    gb = oracle.unpack_mask(gpu_words, f)
    own = gpu_logits > tau[None, :].astype(np.float32)
    assert np.array_equal(gb, own), "mask is not the threshold of the kernel's own logits"
    ob = ora_logits > tau[None, :].astype(np.float64)
    outside = np.abs(ora_logits - tau[None, :].astype(np.float64)) > band
    bad = (gb != ob) & outside
    assert not bad.any(), f"{int(bad.sum())} mask bits differ outside the rounding band"
    assert (np.abs(gpu_logits - ora_logits) <= band + 1e-30).all(), "logit error above the bound"
    return int(((gb != ob) & ~outside).sum())


def gpu_stack(layers_dev, r_in: np.ndarray, eps: float = 1e-6, xdtype=torch.float16, flags: int = 0):
    """sfnn_stack_decode over uploaded layers with every per-layer capture on."""
    L = len(layers_dev)
    B, d = r_in.shape
    pred0, ffn0 = layers_dev[0]
    f = ffn0.d_ff
    st = sg.Stack(layers_dev)
    rin = to_dev(r_in.astype(np.float32))
    rout = torch.full((B, d), float("nan"), dtype=torch.float32, device=DEV)
    xc = torch.full((L, B, d), float("nan"), dtype=xdtype, device=DEV)
    yc = torch.full((L, B, d), float("nan"), dtype=torch.float32, device=DEV)
    mc = torch.zeros((L, B, f // 64), dtype=torch.uint64, device=DEV)
    ic = torch.full((L, f), -7, dtype=torch.int32, device=DEV)
    cc = torch.full((L + 3,), -1, dtype=torch.int32, device=DEV)
    ws = workspace(pred0, ffn0, B)
    sg.sfnn_stack_decode(st, B, rin, rout, eps, ws, flags=flags, x_cap=xc, y_cap=yc, mask_cap=mc, ids_cap=ic,
                         count_cap=cc)
    torch.cuda.synchronize()
    return dict(r_out=rout.cpu().numpy(), x=xc.float().cpu().numpy(), y=yc.cpu().numpy(), mask=mc.cpu().numpy(),
                ids=ic.cpu().numpy(), count=cc.cpu().numpy()[:L])
