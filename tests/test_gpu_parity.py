"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bars: compaction ids/count/union bit-exact; masks bit-exact outside the fp32
rounding band of the predictor (and exactly the threshold of the kernel's own
logits); FFN outputs within 2e-3 normwise relative error (fp16 weights, fp32
accumulation); bit-exact everywhere on integer-grid layers where every
intermediate is an integer below 2^24.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (band_check, gpu_compact, gpu_dense_ffn, gpu_layer, gpu_predict, gpu_sparse_ffn, rel_err,
                      to_dev, upload_layer)

pytestmark = pytest.mark.gpu

TOL = 2e-3
_LAYERS = {}


def full_layer(name):
    """Full-size layer 0 of a workload, drawn once per test session."""
    if name not in _LAYERS:
        _LAYERS.clear()
        _LAYERS[name] = synth.make_layer(synth.config(name), layer=0)
    return _LAYERS[name]


# ---------------------------------------------------------------------------
# compaction: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("f", [64, 1088, 49152, 65536])
@pytest.mark.parametrize("B", [1, 3, 64])
@pytest.mark.parametrize("density", [0.0, 1e-4, 0.1, 0.5, 1.0])
def test_compact_random(f, B, density):
    words = synth.random_masks(B, f, density, seed=f + B)
    ids, c, uni = gpu_compact(words, B, f)
    rid, rc, runi = oracle.compact(words, B, f)
    assert c == rc
    assert np.array_equal(ids[:c], rid)
    assert np.all(ids[c:] == -7), "entries past count must be left untouched"
    assert np.array_equal(uni, runi)


def test_compact_pages_example():
    bits = np.zeros((1, 64), dtype=bool)
    bits[0, [3, 4, 5]] = True
    ids, c, _ = gpu_compact(synth.pack_bits(bits), 1, 64)
    assert c == 3 and list(ids[:3]) == [3, 4, 5]


@pytest.mark.parametrize("bit", [0, 63, 64, 16383, 65535])
def test_compact_single_bit(bit):
    f = 65536
    bits = np.zeros((2, f), dtype=bool)
    bits[1, bit] = True
    ids, c, _ = gpu_compact(synth.pack_bits(bits), 2, f)
    assert c == 1 and ids[0] == bit


# ---------------------------------------------------------------------------
# predictor: bit-exact masks outside the rounding band
# ---------------------------------------------------------------------------

def _pred_case(spec, B, stream):
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, B, stream=stream)
    pred, _ = upload_layer(lay)
    words, lg = gpu_predict(pred, x, spec.d_ff)
    ol, _ = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
    flips = band_check(words, lg, ol, band, lay.tau, spec.d_ff)
    assert flips <= max(1, B * spec.d_ff // 10000)
    return lay, x, words


@pytest.mark.parametrize("B", [1, 4, 9])
def test_predict_opt125m_fp32(B):
    _pred_case(synth.config("c1"), B, stream=10 + B)


@pytest.mark.parametrize("B", [1, 8, 33])
def test_predict_fp16_ragged(B):
    _pred_case(synth.config("c2", d_model=1152, d_ff=4160, rank=264), B, stream=20 + B)


def test_predict_opt6_7b_full_size():
    _pred_case(synth.config("c2"), 1, stream=30)


@pytest.mark.parametrize("wtype", ["f32", "f16"])
@pytest.mark.parametrize("B", [1, 5])
def test_predict_integer_grid_exact(wtype, B):
    lay = synth.make_grid_layer(512, 2048, 128, wtype=wtype)
    x = synth.make_grid_tokens(512, B, dtype=np.float32 if wtype == "f32" else np.float16)
    pred, _ = upload_layer(lay)
    words, lg = gpu_predict(pred, x, 2048)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    assert np.array_equal(lg.astype(np.float64), ol)
    assert np.array_equal(words, oracle.pack_mask(ob))


# ---------------------------------------------------------------------------
# sparse FFN on given masks
# ---------------------------------------------------------------------------

def _ffn_layer(wtype, act, d=640, f=1088, seed=0):
    spec = synth.config("c2", d_model=d, d_ff=f, rank=64, wtype=wtype, act=act,
                        pred_dtype="f32" if wtype == "f32" else "f16")
    return synth.make_layer(spec, layer=seed, predictor=False)


@pytest.mark.parametrize("wtype,act", [("f32", "relu"), ("f16", "relu"), ("f16", "reglu"),
                                       ("i4g128", "relu"), ("i4g128", "reglu")])
@pytest.mark.parametrize("B", [1, 3, 8, 9, 17, 32])
def test_sparse_ffn_random_masks(wtype, act, B):
    lay = _ffn_layer(wtype, act)
    x = synth.make_tokens(lay.spec, B, stream=40 + B)
    words = synth.random_masks(B, lay.spec.d_ff, 0.1, seed=B)
    _, ffn = upload_layer(lay, predictor=False)
    y = gpu_sparse_ffn(ffn, x, words)
    ref = oracle.masked_ffn(lay, x, words)
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL, b


@pytest.mark.parametrize("wtype", ["f32", "f16", "i4g128"])
def test_sparse_ffn_ungated_union(wtype):
    lay = _ffn_layer(wtype, "relu")
    B, f = 4, lay.spec.d_ff
    x = synth.make_tokens(lay.spec, B, stream=50)
    words = synth.random_masks(B, f, 0.1, seed=7)
    _, ffn = upload_layer(lay, predictor=False)
    y = gpu_sparse_ffn(ffn, x, words, gate=False)
    _, _, uni = oracle.compact(words, B, f)
    ref = oracle.masked_ffn(lay, x, np.tile(uni, (B, 1)))
    for b in range(B):
        assert rel_err(y[b], ref[b]) <= TOL


@pytest.mark.parametrize("wtype,act", [("f32", "relu"), ("f16", "relu"), ("f16", "reglu"), ("i4g128", "relu"),
                                       ("i4g128", "reglu")])
def test_dense_ffn(wtype, act):
    lay = _ffn_layer(wtype, act)
    x = synth.make_tokens(lay.spec, 3, stream=60)
    _, ffn = upload_layer(lay, predictor=False)
    y = gpu_dense_ffn(ffn, x)
    ref = oracle.dense_ffn(lay, x)
    for b in range(3):
        assert rel_err(y[b], ref[b]) <= TOL


@pytest.mark.parametrize("wtype,act", [("f32", "relu"), ("f16", "relu"), ("f16", "reglu"), ("i4g128", "relu"),
                                       ("i4g128", "reglu")])
@pytest.mark.parametrize("B", [1, 6, 17])
def test_sparse_ffn_integer_grid_bitwise(wtype, act, B):
    d, f = (256, 1088) if act == "relu" else (128, 576)
    lay = synth.make_grid_layer(d, f, 32, act=act, wtype=wtype, seed=B)
    x = synth.make_grid_tokens(d, B, seed=B, dtype=np.float32 if wtype == "f32" else np.float16)
    words = synth.random_masks(B, f, 0.3, seed=B)
    _, ffn = upload_layer(lay, predictor=False)
    y = gpu_sparse_ffn(ffn, x, words)
    ref = oracle.masked_ffn(lay, x, words, return_f64=True)
    assert np.abs(ref).max() < 2 ** 22
    assert np.array_equal(y.astype(np.float64), ref)
    # batch invariance, bitwise on the grid
    y0 = gpu_sparse_ffn(ffn, x[:1], words[:1])
    assert np.array_equal(y0[0], y[0])
    # dense on the grid
    yd = gpu_dense_ffn(ffn, x)
    assert np.array_equal(yd.astype(np.float64), oracle.dense_ffn(lay, x, return_f64=True))


def test_inactive_rows_nan_poison_bitwise():
    """Rows outside the union are never read: NaN there changes nothing."""
    lay = _ffn_layer("f16", "reglu")
    B, f = 3, lay.spec.d_ff
    x = synth.make_tokens(lay.spec, B, stream=70)
    words = synth.random_masks(B, f, 0.1, seed=70)
    _, ffn = upload_layer(lay, predictor=False)
    y_clean = gpu_sparse_ffn(ffn, x, words)
    _, _, uni = oracle.compact(words, B, f)
    off = ~oracle.unpack_mask(uni[None], f)[0]
    for name in ("w_up", "w_gate", "w_down_t"):
        a = getattr(lay, name).copy()
        a[off] = np.float16(np.nan)
        setattr(lay, name, a)
    for name in ("b_up", "b_gate"):
        a = getattr(lay, name).copy()
        a[off] = np.float16(np.nan)
        setattr(lay, name, a)
    _, ffn2 = upload_layer(lay, predictor=False)
    y_poison = gpu_sparse_ffn(ffn2, x, words)
    assert np.isfinite(y_poison).all()
    assert np.array_equal(y_clean, y_poison)


@pytest.mark.parametrize("wtype", ["f16", "i4g128"])
def test_empty_set_gives_bias_bitwise(wtype):
    lay = _ffn_layer(wtype, "relu")
    lay.b_down = (np.arange(lay.spec.d_model) % 7 - 3).astype(np.float16) * np.float16(0.25)
    B = 2
    x = synth.make_tokens(lay.spec, B, stream=80)
    words = np.zeros((B, lay.spec.d_ff // 64), dtype=np.uint64)
    _, ffn = upload_layer(lay, predictor=False)
    y = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(y, np.tile(lay.b_down.astype(np.float32), (B, 1)))


def test_superset_of_true_active_equals_dense():
    lay = _ffn_layer("f16", "relu")
    B, f = 2, lay.spec.d_ff
    x = synth.make_tokens(lay.spec, B, stream=90)
    t = oracle.true_active(lay, x)
    rng = np.random.default_rng(3)
    dense_ref = oracle.dense_ffn(lay, x)
    _, ffn = upload_layer(lay, predictor=False)
    for extra in (0.0, 0.1, 1.0):
        m = t | (rng.random(t.shape) < extra)
        y = gpu_sparse_ffn(ffn, x, synth.pack_bits(m))
        for b in range(B):
            assert rel_err(y[b], dense_ref[b]) <= TOL


def test_out_of_range_ids_skipped_and_count_clamped():
    import torch
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import workspace
    lay = _ffn_layer("f16", "relu", d=256, f=1024)
    x = synth.make_tokens(lay.spec, 1, stream=95)
    _, ffn = upload_layer(lay, predictor=False)
    ws = workspace(None, ffn, 1)
    xd = to_dev(x)
    # ids 5, 1<<20 (out of range), 9 -> only 5 and 9 contribute
    ids = to_dev(np.array([5, 1 << 20, 9] + [0] * 1021, dtype=np.int32))
    cnt = to_dev(np.array([3, 0, 0, 0], dtype=np.int32))
    y = torch.empty((1, 256), dtype=torch.float32, device="cuda")
    sg.sfnn_sparse_ffn(ffn, xd, 1, ids, cnt, None, y, ws)
    m = np.zeros((1, 1024), dtype=bool)
    m[0, [5, 9]] = True
    assert rel_err(y.cpu().numpy()[0], oracle.masked_ffn(lay, x, m)[0]) <= TOL
    # count above d_ff is clamped to d_ff
    ids = to_dev(np.arange(1024, dtype=np.int32))
    cnt = to_dev(np.array([5000, 0, 0, 0], dtype=np.int32))
    sg.sfnn_sparse_ffn(ffn, xd, 1, ids, cnt, None, y, ws)
    assert rel_err(y.cpu().numpy()[0], oracle.dense_ffn(lay, x)[0]) <= TOL


def test_deterministic_run_to_run():
    lay = _ffn_layer("f16", "reglu", d=1024, f=4096)
    B = 4
    x = synth.make_tokens(lay.spec, B, stream=99)
    words = synth.random_masks(B, 4096, 0.2, seed=99)
    _, ffn = upload_layer(lay, predictor=False)
    a = gpu_sparse_ffn(ffn, x, words)
    b = gpu_sparse_ffn(ffn, x, words)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# whole layer: predict -> compact -> sparse FFN
# ---------------------------------------------------------------------------

def _layer_case(lay, x, check_tokens=None, max_flip_frac=1e-4, mfma_min_batch=0):
    spec = lay.spec
    f = spec.d_ff
    pred, ffn = upload_layer(lay)
    ffn.mfma_min_batch = mfma_min_batch
    pred.dense_min_batch = -1  # the sparse path at every batch (the dense switch has its own tests)
    out = gpu_layer(pred, ffn, x)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
    gb = oracle.unpack_mask(out["mask"], f)
    ob_in = ob != gb
    outside = np.abs(ol - lay.tau[None, :].astype(np.float64)) > band
    assert not (ob_in & outside).any()
    assert ob_in.sum() <= max(1, int(max_flip_frac * ob.size))
    # ids / count: the compaction of the GPU's own mask, bit-exact
    rid, rc, _ = oracle.compact(out["mask"], x.shape[0], f)
    assert out["count"] == rc and np.array_equal(out["ids"], rid)
    toks = range(x.shape[0]) if check_tokens is None else check_tokens
    for b in toks:
        # the GPU's own mask (checked above against the oracle's outside the band)
        ref = oracle.masked_ffn(lay, x[b:b + 1], gb[b:b + 1])[0]
        assert rel_err(out["y"][b], ref) <= TOL, b
    return out


# The matrix-core FFN compacts the union inside its first kernel (every
# workgroup scans the mask words for its own slots): an empty union, a full
# one, an odd number of mask words (d_ff 1088: 17), ragged last slots and
# several 32-token passes, fp16 (32-slot workgroups) and INT4 (64- and
# 128-slot workgroups).
@pytest.mark.parametrize("wtype,act,B", [("f16", "relu", 8), ("f16", "reglu", 40), ("i4g128", "relu", 3),
                                         ("i4g128", "relu", 20), ("i4g128", "reglu", 33)])
@pytest.mark.parametrize("tau", ["empty", "full", "calibrated"])
def test_layer_matrix_core_union_edges(wtype, act, B, tau):
    spec = synth.config("c4" if act == "reglu" else "c2", d_model=640, d_ff=1088, rank=64, wtype=wtype, act=act)
    lay = synth.make_layer(spec, layer=2)
    f = spec.d_ff
    if tau == "empty":
        lay.tau = np.full(f, np.inf, dtype=np.float32)
        lay.b_down = ((np.arange(spec.d_model) % 7 - 3) * 0.25).astype(lay.b_down.dtype)
    elif tau == "full":
        lay.tau = np.full(f, -np.inf, dtype=np.float32)
    x = synth.make_tokens(spec, B, stream=120 + B)
    out = _layer_case(lay, x)
    if tau == "empty":
        assert out["count"] == 0
        assert np.array_equal(out["y"], np.tile(lay.b_down.astype(np.float32), (B, 1)))
    elif tau == "full":
        assert out["count"] == f and np.array_equal(out["ids"], np.arange(f, dtype=np.int32))
        ref = oracle.dense_ffn(lay, x)
        for b in range(B):
            assert rel_err(out["y"][b], ref[b]) <= TOL, b


def test_layer_opt125m_64_decode_vectors():
    spec = synth.config("c1")
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 64, stream=0)
    pred, ffn = upload_layer(lay)
    for t in range(64):
        out = gpu_layer(pred, ffn, x[t:t + 1])
        ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x[t:t + 1])
        band = oracle.guard_band(lay.w1_t, lay.w2_t, x[t:t + 1])
        gb = oracle.unpack_mask(out["mask"], spec.d_ff)
        assert not ((gb != ob) & (np.abs(ol - lay.tau.astype(np.float64)) > band)).any()
        if np.array_equal(gb, ob):
            rid, rc, _ = oracle.compact(oracle.pack_mask(ob), 1, spec.d_ff)
            assert out["count"] == rc and np.array_equal(out["ids"], rid)
            assert rel_err(out["y"][0], oracle.masked_ffn(lay, x[t:t + 1], ob)[0]) <= TOL


@pytest.mark.parametrize("act,wtype", [("relu", "f16"), ("reglu", "f16"), ("relu", "i4g128"), ("relu", "f32")])
@pytest.mark.parametrize("B", [1, 7])
def test_layer_integer_grid_bitwise(act, wtype, B):
    d, f, r = (256, 1024, 64) if act == "relu" else (128, 512, 64)
    lay = synth.make_grid_layer(d, f, r, act=act, wtype=wtype, seed=3 + B)
    x = synth.make_grid_tokens(d, B, seed=B, dtype=np.float32 if wtype == "f32" else np.float16)
    pred, ffn = upload_layer(lay)
    out = gpu_layer(pred, ffn, x)
    ol, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    assert np.array_equal(out["mask"], oracle.pack_mask(ob))
    rid, rc, _ = oracle.compact(oracle.pack_mask(ob), B, f)
    assert out["count"] == rc and np.array_equal(out["ids"], rid)
    ref = oracle.masked_ffn(lay, x, ob, return_f64=True)
    assert np.array_equal(out["y"].astype(np.float64), ref)


def test_layer_opt6_7b_full_size_b1():
    spec = synth.config("c2")
    lay = full_layer("c2")
    x = synth.make_tokens(spec, 1, stream=1)
    _layer_case(lay, x)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_layer_opt30b_zipf_full_size(B):
    spec = synth.config("c3")
    lay = full_layer("c3")
    x = synth.make_tokens(spec, B, stream=2)
    _layer_case(lay, x)  # every token's y


@pytest.mark.parametrize("B", [1, 8])
def test_layer_llama_reglu70b_full_size(B):
    spec = synth.config("c4")
    lay = full_layer("c4")
    x = synth.make_tokens(spec, B, stream=3)
    _layer_case(lay, x, check_tokens=[0, B - 1])


@pytest.mark.parametrize("B", [1, 2, 4, 32])
def test_layer_opt175b_int4_full_size(B):
    spec = synth.config("c5")
    lay = full_layer("c5")
    x = synth.make_tokens(spec, B, stream=4)
    _layer_case(lay, x)  # every token's y


@pytest.mark.parametrize("wtype", ["f16", "i4g128"])
@pytest.mark.parametrize("B", [1, 9])
def test_layer_max_d_model(wtype, B):
    """d_model 16384, the largest the ABI accepts: 128 INT4 scale groups per
    row, 256 column pairs in the matrix-core kernels, four d_model slices in
    predictor stage 1; per-row kernels at batch 1, matrix cores at 9."""
    spec = synth.config("c2", d_model=16384, d_ff=2048, rank=256, wtype=wtype,
                        pred_dtype="f16")
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, B, stream=17)
    _layer_case(lay, x, check_tokens=[0, B - 1])
