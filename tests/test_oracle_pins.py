"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle itself re-typed.

* brute force on tiny shapes (literal per-element loops)
* the pages' one-layer example (3/4/5 predicted, 3/5/7 hot)
* zero rows contribute nothing; a superset of the true active set gives the dense result
* closed forms: empty set, single neuron, all-ones = textbook matrix chain
* exact integer arithmetic on integer-grid layers
* permutation and batch invariance
* INT4 nibble layout decoded by hand; quantise/dequantise round trip
* predictor closed form; fp32 evaluation stays inside the guard band
* dense hot prefix: the pages' example in hot-first order; prefix 0 and f
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from synth import LayerSpec, Layer


def tiny_layer(d, f, r, act="relu", wtype="f32", seed=0, density=0.3):
    g = np.random.default_rng(seed)
    spec = LayerSpec("tiny", 0, d, f, r, wtype, act, "f32", 1, "uniform", density)
    lay = Layer(spec=spec, probs=np.full(f, density), w1_t=g.normal(0, 0.5, (r, d)),
                w2_t=g.normal(0, 0.5, (f, r)), tau=g.normal(0, 0.5, f).astype(np.float32))
    if wtype == "i4g128":
        lay.q_up, lay.s_up = synth.quant_int4_g128(g.normal(0, 0.3, (f, d)))
        lay.q_down_t, lay.s_down_t = synth.quant_int4_g128(g.normal(0, 0.3, (f, d)))
        if act == "reglu":
            lay.q_gate, lay.s_gate = synth.quant_int4_g128(g.normal(0, 0.3, (f, d)))
    else:
        lay.w_up = g.normal(0, 0.5, (f, d))
        lay.w_down_t = g.normal(0, 0.5, (f, d))
        if act == "reglu":
            lay.w_gate = g.normal(0, 0.5, (f, d))
    lay.b_up = g.normal(0, 0.5, f)
    if act == "reglu":
        lay.b_gate = g.normal(0, 0.5, f)
    lay.b_down = g.normal(0, 0.5, d)
    return lay


# ---------------------------------------------------------------------------
# literal brute force
# ---------------------------------------------------------------------------

def _nibble_weight(lay, which, i, k):
    q = getattr(lay, "q_" + which)
    s = getattr(lay, "s_" + which)
    byte = int(q[i][k // 2])
    nib = (byte >> (4 * (k % 2))) & 15
    v = nib - 16 if nib >= 8 else nib
    return v * float(s[i][k // 128])


def _w(lay, which, i, k):
    w = getattr(lay, "w_" + which)
    if w is not None:
        return float(w[i][k])
    return _nibble_weight(lay, which, i, k)


def brute_predict(lay, xb):
    d, f, r = lay.spec.d_model, lay.spec.d_ff, lay.spec.rank
    z = [sum(float(lay.w1_t[j][k]) * float(xb[k]) for k in range(d)) for j in range(r)]
    logits = [sum(float(lay.w2_t[i][j]) * z[j] for j in range(r)) for i in range(f)]
    return logits, [logits[i] > float(lay.tau[i]) for i in range(f)]


def brute_ffn(lay, xb, active):
    d, f = lay.spec.d_model, lay.spec.d_ff
    y = [float(lay.b_down[c]) for c in range(d)]
    for i in range(f):
        if not active[i]:
            continue
        a = sum(_w(lay, "up", i, k) * float(xb[k]) for k in range(d)) + float(lay.b_up[i])
        if lay.spec.act == "relu":
            h = a if a > 0 else 0.0
        else:
            g = sum(_w(lay, "gate", i, k) * float(xb[k]) for k in range(d)) + float(lay.b_gate[i])
            h = (g if g > 0 else 0.0) * a
        for c in range(d):
            y[c] += h * _w(lay, "down_t", i, c)
    return y


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("B", [1, 3])
def test_brute_force_predict_and_masked_ffn(act, B):
    d, f, r = 16, 64, 8
    lay = tiny_layer(d, f, r, act=act, seed=B)
    x = np.random.default_rng(7 + B).normal(0, 1, (B, d))
    logits, bits = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    y = oracle.masked_ffn(lay, x, bits, return_f64=True)
    for b in range(B):
        bl, bb = brute_predict(lay, x[b])
        np.testing.assert_allclose(logits[b], bl, rtol=1e-12, atol=1e-12)
        assert list(bits[b]) == bb
        np.testing.assert_allclose(y[b], brute_ffn(lay, x[b], bb), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_brute_force_int4(act):
    d, f, r = 128, 16, 8
    lay = tiny_layer(d, f, r, act=act, wtype="i4g128", seed=3)
    x = np.random.default_rng(11).normal(0, 1, (2, d))
    bits = np.random.default_rng(12).random((2, f)) < 0.5
    y = oracle.masked_ffn(lay, x, bits, return_f64=True)
    for b in range(2):
        np.testing.assert_allclose(y[b], brute_ffn(lay, x[b], bits[b]), rtol=1e-12, atol=1e-12)


def brute_compact(words, batch, f):
    ids = []
    for i in range(f):
        w, j = divmod(i, 64)
        if any((int(words[b][w]) >> j) & 1 for b in range(batch)):
            ids.append(i)
    return ids


@pytest.mark.parametrize("density", [0.0, 1e-4, 0.1, 0.5, 1.0])
@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_compact_brute_force(density, B):
    f = 1024
    words = synth.random_masks(B, f, density, seed=B)
    ids, count, union = oracle.compact(words, B, f)
    ref = brute_compact(words, B, f)
    assert list(ids) == ref and count == len(ref)
    assert list(oracle.unpack_mask(union[None], f)[0].nonzero()[0]) == ref


@pytest.mark.parametrize("bit", [0, 63, 64, 4095])
def test_compact_single_bits(bit):
    f = 4096
    bits = np.zeros((1, f), dtype=bool)
    bits[0, bit] = True
    words = synth.pack_bits(bits)
    ids, count, _ = oracle.compact(words, 1, f)
    assert count == 1 and ids[0] == bit


def test_mask_pack_layout_by_hand():
    # neuron 0 -> bit 0 of word 0, neuron 65 -> bit 1 of word 1 (LSB first)
    bits = np.zeros((1, 128), dtype=bool)
    bits[0, [0, 65, 127]] = True
    w = oracle.pack_mask(bits)
    assert int(w[0, 0]) == 1 and int(w[0, 1]) == (1 << 1) | (1 << 63)
    assert np.array_equal(oracle.unpack_mask(w, 128), bits)
    assert np.array_equal(synth.pack_bits(bits), w)


# ---------------------------------------------------------------------------
# the pages' worked example
# ---------------------------------------------------------------------------

def test_powerinfer_toy_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "powerinfer_toy_example.json")))
    f = g["d_ff"]
    bits = np.zeros((1, f), dtype=bool)
    bits[0, g["predicted"]] = True
    words = oracle.pack_mask(bits)
    assert int(words[0, 0]) == int(g["mask_word_hex"], 16)
    ids, count, _ = oracle.compact(words, 1, f)
    assert list(ids) == g["predicted"] and count == 3
    hot = set(g["hot"])
    assert sorted(set(ids) & hot) == g["predicted_and_hot"]
    assert sorted(set(ids) - hot) == g["predicted_not_hot"]
    assert sorted(hot - set(ids)) == g["hot_not_predicted"]
    counts = np.zeros(f, dtype=np.uint32)
    counts[g["hot"]] = 10
    perm = oracle.hot_first_perm(counts)
    assert list(perm[:3]) == [3, 5, 7] and list(perm[3:7]) == [0, 1, 2, 4]
    assert list(oracle.permute_layer_ids(perm, ids)) == g["hot_first_positions_of_predicted"]


def test_fire_counts_and_hot_first_ties():
    f = 128
    bits = np.zeros((3, f), dtype=bool)
    bits[:, 5] = True
    bits[:2, 70] = True
    bits[:2, 9] = True
    bits[0, 127] = True
    c = oracle.fire_counts(oracle.pack_mask(bits), f)
    assert c[5] == 3 and c[70] == 2 and c[9] == 2 and c[127] == 1 and c.sum() == 8
    perm = oracle.hot_first_perm(c)
    assert list(perm[:5]) == [5, 9, 70, 127, 0]
    assert sorted(perm) == list(range(f))


# ---------------------------------------------------------------------------
# invariants the pages fix
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("extra", [0.0, 0.1, 1.0])
def test_superset_of_true_active_equals_dense_bitwise(act, extra):
    """[53ai] 验证上下文稀疏存在: recomputing with only the recorded set gives the same output."""
    lay = tiny_layer(32, 256, 8, act=act, seed=5)
    x = np.random.default_rng(3).normal(0, 1, (4, 32))
    t = oracle.true_active(lay, x)
    assert 0 < t.sum() < t.size
    m = t | (np.random.default_rng(4).random(t.shape) < extra)
    ym = oracle.masked_ffn(lay, x, m)
    yd = oracle.dense_ffn(lay, x)
    assert np.array_equal(ym, yd)
    # dropping one truly active neuron of token 0 must change its output
    i = int(np.flatnonzero(t[0])[0])
    m2 = m.copy()
    m2[0, i] = False
    assert not np.array_equal(oracle.masked_ffn(lay, x, m2)[0], yd[0])


def test_inactive_rows_contribute_nothing_nan_poison():
    """[53ai] 激活稀疏: rows outside the active set are neither read nor multiplied."""
    lay = tiny_layer(32, 256, 8, act="reglu", seed=6)
    x = np.random.default_rng(1).normal(0, 1, (2, 32))
    _, bits = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    y0 = oracle.masked_ffn(lay, x, bits)
    off = ~(bits[0] | bits[1])
    for name in ("w_up", "w_gate", "w_down_t"):
        getattr(lay, name)[off] = np.nan
    lay.b_up[off] = np.nan
    lay.b_gate[off] = np.nan
    y1 = oracle.masked_ffn(lay, x, bits)
    assert np.isfinite(y1).all() and np.array_equal(y0, y1)


def test_empty_set_gives_bias_exactly():
    lay = tiny_layer(16, 64, 8, seed=8)
    x = np.random.default_rng(2).normal(0, 1, (3, 16))
    y = oracle.masked_ffn(lay, x, np.zeros((3, 64), dtype=bool))
    assert np.array_equal(y, np.tile(lay.b_down.astype(np.float32), (3, 1)))


def test_single_neuron_hand_worked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "single_neuron.json")))
    for c in g["cases"]:
        spec = LayerSpec("one", 0, 2, 64, 8, "f32", c["act"], "f32", 1, "uniform", 0.1)
        lay = Layer(spec=spec, probs=None, w1_t=None, w2_t=None, tau=None)
        f = 64
        lay.w_up = np.zeros((f, 2)); lay.w_up[17] = c["w_up"]
        lay.w_down_t = np.zeros((f, 2)); lay.w_down_t[17] = c["w_down_col"]
        lay.b_up = np.zeros(f); lay.b_up[17] = c["b_up"]
        if c["act"] == "reglu":
            lay.w_gate = np.zeros((f, 2)); lay.w_gate[17] = c["w_gate"]
            lay.b_gate = np.zeros(f); lay.b_gate[17] = c["b_gate"]
        lay.b_down = np.array(c["b_down"])
        m = np.zeros((1, f), dtype=bool)
        m[0, 17] = True
        y = oracle.masked_ffn(lay, np.array([c["x"]]), m, return_f64=True)
        assert np.array_equal(y[0], np.array(c["y"]))


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_all_ones_equals_textbook_matrix_chain(act):
    lay = tiny_layer(48, 320, 8, act=act, seed=9)
    x = np.random.default_rng(5).normal(0, 1, (3, 48))
    W_up = lay.w_up                        # [f][d]
    W_down = lay.w_down_t.T                # conventional [d][f]
    pre = x @ W_up.T + lay.b_up
    if act == "relu":
        h = np.maximum(pre, 0)
    else:
        h = np.maximum(x @ lay.w_gate.T + lay.b_gate, 0) * pre
    ref = h @ W_down.T + lay.b_down
    np.testing.assert_allclose(oracle.dense_ffn(lay, x, return_f64=True), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_integer_grid_exact(act):
    d, f, r = (128, 512, 32) if act == "relu" else (128, 256, 32)
    lay = synth.make_grid_layer(d, f, r, act=act, wtype="f32")
    x = synth.make_grid_tokens(d, 3, dtype=np.float32)
    xi = x.astype(np.int64)
    z = xi @ lay.w1_t.astype(np.int64).T
    logit = z @ lay.w2_t.astype(np.int64).T
    bits_ref = (2 * logit) > (2 * lay.tau.astype(np.float64)).astype(np.int64)
    logits, bits = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    assert np.array_equal(logits, logit.astype(np.float64)) and np.array_equal(bits, bits_ref)
    up = xi @ lay.w_up.astype(np.int64).T + lay.b_up.astype(np.int64)
    if act == "relu":
        h = np.maximum(up, 0)
    else:
        h = np.maximum(xi @ lay.w_gate.astype(np.int64).T + lay.b_gate.astype(np.int64), 0) * up
    h = np.where(bits, h, 0)
    y = h @ lay.w_down_t.astype(np.int64) + lay.b_down.astype(np.int64)
    assert np.abs(y).max() < 2 ** 24
    assert np.array_equal(oracle.masked_ffn(lay, x, bits, return_f64=True), y.astype(np.float64))


def test_permutation_invariance():
    lay = tiny_layer(32, 256, 8, act="relu", seed=10)
    x = np.random.default_rng(6).normal(0, 1, (2, 32))
    _, bits = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    y = oracle.masked_ffn(lay, x, bits, return_f64=True)
    perm = np.random.default_rng(7).permutation(256)
    lay2 = tiny_layer(32, 256, 8, act="relu", seed=10)
    for name in ("w_up", "w_down_t", "b_up", "w2_t", "tau"):
        setattr(lay2, name, getattr(lay, name)[perm])
    _, bits2 = oracle.predict(lay2.w1_t, lay2.w2_t, lay2.tau, x)
    assert np.array_equal(bits2, bits[:, perm])
    y2 = oracle.masked_ffn(lay2, x, bits2, return_f64=True)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)


def test_batch_invariance():
    lay = tiny_layer(32, 256, 8, act="reglu", seed=11)
    x = np.random.default_rng(8).normal(0, 1, (5, 32))
    _, bits = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    y = oracle.masked_ffn(lay, x, bits)
    for b in range(5):
        assert np.array_equal(oracle.masked_ffn(lay, x[b:b + 1], bits[b:b + 1])[0], y[b])


# ---------------------------------------------------------------------------
# INT4 format
# ---------------------------------------------------------------------------

def test_int4_nibbles_by_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int4_nibbles.json")))
    q = np.zeros((1, 64), dtype=np.uint8)
    raw = [int(h, 16) for h in g["bytes_hex"]]
    q[0, :len(raw)] = raw
    s = np.array([[g["scale"]]], dtype=np.float16)
    w = oracle.dequant_int4(q, s)
    vals = g["values_by_hand"]
    assert list(w[0, :len(vals)]) == [v * g["scale"] for v in vals]
    assert not w[0, len(vals):].any()


def test_int4_roundtrip():
    g = np.random.default_rng(0)
    s = (2.0 ** g.integers(-8, 0, size=(8, 4)))
    qv = g.integers(-7, 8, size=(8, 512))
    qv[:, ::128] = 7                      # every group reaches max|q| = 7 so s = amax / 7
    w = qv * np.repeat(s, 128, axis=1)
    q, s16 = synth.quant_int4_g128(w)
    assert np.array_equal(oracle.dequant_int4(q, s16), w)
    wr = g.normal(0, 0.02, (16, 256))
    q, s16 = synth.quant_int4_g128(wr)
    deq = oracle.dequant_int4(q, s16)
    half_step = np.repeat(s16.astype(np.float64), 128, axis=1) / 2
    assert (np.abs(deq - wr) <= half_step * (1 + 1e-3)).all()


# ---------------------------------------------------------------------------
# predictor closed form and rounding band
# ---------------------------------------------------------------------------

def test_predictor_closed_form():
    d, r, f = 12, 4, 64
    w1_t = np.zeros((r, d)); w1_t[:, :r] = np.eye(r)     # z = x[:r]
    sel = np.arange(f) % r
    scale = 1.0 + np.arange(f) / 8.0
    w2_t = np.zeros((f, r)); w2_t[np.arange(f), sel] = scale
    tau = np.where(np.arange(f) % 2 == 0, 0.0, 1.0)
    x = np.array([[0.5, -1.0, 2.0, 0.25] + [9.0] * (d - r)])
    logits, bits = oracle.predict(w1_t, w2_t, tau, x)
    expect = scale * x[0, sel]
    assert np.array_equal(logits[0], expect)
    assert np.array_equal(bits[0], expect > tau)


def test_hot_prefix_toy_example(golden_dir):
    """The pages' example in hot-first order with a dense hot prefix of the 3
    hot neurons: the computed set is hot | predicted = {3, 4, 5, 7}, so hot
    neuron 7, which the predictor skips for this input, is computed too."""
    g = json.load(open(os.path.join(golden_dir, "powerinfer_toy_example.json")))
    f = g["d_ff"]
    counts = np.zeros(f, dtype=np.uint32)
    counts[g["hot"]] = 10
    perm = oracle.hot_first_perm(counts)          # position p holds neuron perm[p]
    eye = np.eye(f)
    x = np.zeros((1, f))
    x[0, g["hot_first_positions_of_predicted"]] = 1.0   # logit = x, tau = 0.5
    tau = np.full(f, 0.5)
    _, plain = oracle.predict(eye, eye, tau, x)
    assert sorted(perm[plain[0]]) == g["predicted"]
    logits, bits = oracle.predict(eye, eye, tau, x, hot_prefix=len(g["hot"]))
    assert sorted(perm[bits[0]]) == sorted(set(g["hot"]) | set(g["predicted"])) == [3, 4, 5, 7]
    assert np.isposinf(logits[0, :3]).all() and np.array_equal(logits[0, 3:], x[0, 3:])


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_hot_prefix_bounds(act):
    """Prefix 0 is the plain predictor; prefix f selects every neuron, so the
    layer is the dense FFN (the matrix chain pinned above) whatever tau holds;
    a partial prefix sets its bits even for tau = +inf or NaN and leaves the
    rest of the logits and bits untouched."""
    lay = tiny_layer(32, 256, 8, act=act, seed=11)
    x = np.random.default_rng(12).normal(0, 1, (3, 32))
    l0, b0 = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    lz, bz = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x, hot_prefix=0)
    assert np.array_equal(l0, lz) and np.array_equal(b0, bz)
    assert 0 < b0.sum() < b0.size
    _, ball = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x, hot_prefix=256)
    assert ball.all()
    assert np.array_equal(oracle.masked_ffn(lay, x, ball), oracle.dense_ffn(lay, x))
    tau = lay.tau.copy()
    tau[:64] = np.inf
    tau[64:128] = np.nan
    lh, bh = oracle.predict(lay.w1_t, lay.w2_t, tau, x, hot_prefix=128)
    assert bh[:, :128].all() and np.isposinf(lh[:, :128]).all()
    assert np.array_equal(lh[:, 128:], l0[:, 128:]) and np.array_equal(bh[:, 128:], b0[:, 128:])
    # ReLU: the prefix adds neurons whose exact output may be zero; over a
    # superset of the true active set the layer stays the dense one
    if act == "relu":
        t = oracle.true_active(lay, x)
        _, bp = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x, hot_prefix=64)
        assert np.array_equal(oracle.masked_ffn(lay, x, bp | t), oracle.dense_ffn(lay, x))


def test_guard_band_covers_fp32_evaluation():
    lay = synth.make_layer(synth.config("c1"), layer=0)
    x = synth.make_tokens(lay.spec, 8)
    logits, _ = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
    x32 = x.astype(np.float32)
    z32 = np.empty((8, lay.spec.rank), dtype=np.float32)
    for j in range(lay.spec.rank):          # sequential fp32 order
        acc = np.zeros(8, dtype=np.float32)
        for k in range(0, lay.spec.d_model, 64):
            acc = acc + (x32[:, k:k + 64] * lay.w1_t[j, k:k + 64]).sum(axis=1, dtype=np.float32)
        z32[:, j] = acc
    l32 = (z32 @ lay.w2_t.T.astype(np.float32)).astype(np.float64)
    assert (np.abs(l32 - logits) <= band).all()
    assert band.max() < 1e-2 * np.abs(logits).max()


# ---------------------------------------------------------------------------
# stack step
# ---------------------------------------------------------------------------

def test_residual_rmsnorm_closed_form():
    r = np.zeros((1, 8))
    y = np.full((1, 8), 3.0)
    r2, x2 = oracle.residual_rmsnorm(r, y, eps=1e-6)
    assert np.array_equal(r2, y)
    np.testing.assert_allclose(x2, 3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-15)
    g = np.random.default_rng(0).normal(0, 5, (3, 64))
    _, xg = oracle.residual_rmsnorm(g, np.zeros_like(g), eps=0.0)
    np.testing.assert_allclose((xg ** 2).mean(axis=1), 1.0, rtol=1e-12)


# ---------------------------------------------------------------------------
# input-sparse GEMV (relufication stage 2, [53ai] 第二阶段——插入新的ReLU)
# ---------------------------------------------------------------------------

def _isg_case(n_in, n_out, B, density, seed):
    g = np.random.default_rng(seed)
    w_t = g.normal(0, 0.5, (n_in, n_out))
    bias = g.normal(0, 0.5, n_out)
    x = g.normal(0, 1, (B, n_in)) * (g.random((B, n_in)) < density)
    return w_t, bias, x


@pytest.mark.parametrize("B,density", [(1, 0.3), (3, 0.5), (2, 0.0), (4, 1.0)])
def test_isg_brute_force(B, density):
    """Literal loops over every input (zero or not) give the same y and J."""
    w_t, bias, x = _isg_case(12, 7, B, density, seed=B)
    y, J = oracle.input_sparse_gemv(w_t, x, bias, return_f64=True)
    ref = np.zeros((B, 7))
    for b in range(B):
        for o in range(7):
            acc = bias[o]
            for j in range(12):
                acc += x[b, j] * w_t[j, o]
            ref[b, o] = acc
    assert np.allclose(y, ref, rtol=0, atol=1e-12)
    cols = [j for j in range(12) if any(x[b, j] != 0 for b in range(B))]
    assert list(J) == cols


def test_isg_equals_dense_matmul():
    """The skipped columns carry exact zeros: y is the textbook product."""
    w_t, bias, x = _isg_case(256, 96, 5, 0.2, seed=7)
    y, J = oracle.input_sparse_gemv(w_t, x, bias, return_f64=True)
    dense = x @ w_t + bias[None, :]
    scale = np.abs(x) @ np.abs(w_t) + np.abs(bias)[None, :]
    assert np.all(np.abs(y - dense) <= 1e-13 * scale)
    assert len(J) < 256


def test_isg_closed_forms():
    w_t, bias, _ = _isg_case(32, 16, 1, 0.0, seed=3)
    # no nonzero input: the bias alone, nothing read
    y, J = oracle.input_sparse_gemv(w_t, np.zeros((2, 32)), bias, return_f64=True)
    assert len(J) == 0 and np.array_equal(y, np.tile(bias, (2, 1)))
    # one nonzero input: bias + x_j times row j of w_t
    x = np.zeros((1, 32))
    x[0, 9] = -1.75
    y, J = oracle.input_sparse_gemv(w_t, x, bias, return_f64=True)
    assert list(J) == [9] and np.array_equal(y[0], bias + (-1.75) * w_t[9])
    # no bias: the product alone
    y, _ = oracle.input_sparse_gemv(w_t, x, None, return_f64=True)
    assert np.array_equal(y[0], (-1.75) * w_t[9])


def test_isg_unused_rows_never_read():
    """Rows of w_t outside J (no token has a nonzero input there) may hold NaN."""
    w_t, bias, x = _isg_case(64, 24, 3, 0.25, seed=11)
    y, J = oracle.input_sparse_gemv(w_t, x, bias)
    poisoned = w_t.copy()
    off = np.ones(64, dtype=bool)
    off[J] = False
    assert off.any()
    poisoned[off] = np.nan
    y2, J2 = oracle.input_sparse_gemv(poisoned, x, bias)
    assert np.array_equal(J, J2) and np.array_equal(y, y2)


def test_isg_signed_zero_and_nan_inputs():
    w_t, bias, _ = _isg_case(8, 4, 1, 0.0, seed=5)
    x = np.zeros((1, 8))
    x[0, 2] = -0.0   # a negative zero is a zero input: its column is skipped
    x[0, 5] = np.nan  # a NaN is not zero: its column is read
    y, J = oracle.input_sparse_gemv(w_t, x, bias, return_f64=True)
    assert list(J) == [5] and np.isnan(y).all()


def test_relu_inputs_density():
    """The generator's entries are nonzero with the requested probability
    (99.9% binomial interval over 64 x 4096 draws) and never negative."""
    for density in (0.5, 0.3, 0.1):
        x = synth.make_relu_inputs(4096, 64, density, dtype=np.float32)
        n = x.size
        k = int((x != 0).sum())
        sd = np.sqrt(n * density * (1 - density))
        assert abs(k - n * density) <= 3.3 * sd, density
        assert (x >= 0).all()
    # density 1: the dense input, negative values kept
    x = synth.make_relu_inputs(512, 4, 1.0, dtype=np.float32)
    assert (x < 0).any() and (x != 0).all()


# ---------------------------------------------------------------------------
# head-gated attention projections
# ---------------------------------------------------------------------------

def _heads(d, H, hd, seed):
    g = np.random.default_rng(seed)
    return (g.normal(0, 0.5, (3 * H * hd, d)), g.normal(0, 0.5, 3 * H * hd),
            g.normal(0, 0.5, (H * hd, d)), g.normal(0, 0.5, d))


def test_head_qkv_brute_force():
    d, H, hd, B = 6, 3, 2, 2
    w, b, _, _ = _heads(d, H, hd, 1)
    x = np.random.default_rng(2).normal(0, 1, (B, d))
    bits = np.array([[True, False, True], [False, False, True]])
    out = oracle.head_qkv(w, b, x, bits, hd, return_f64=True)
    for t in range(B):
        for blk in range(3):                      # q, k, v blocks
            for h in range(H):
                for i in range(hd):
                    r = blk * H * hd + h * hd + i
                    ref = b[r]
                    for k in range(d):
                        ref += w[r, k] * x[t, k]
                    assert out[t, r] == (pytest.approx(ref, rel=1e-12, abs=1e-12) if bits[t, h] else 0.0)


def test_head_out_brute_force():
    d, H, hd, B = 5, 3, 2, 2
    _, _, wo, bo = _heads(d, H, hd, 3)
    a = np.random.default_rng(4).normal(0, 1, (B, H * hd))
    bits = np.array([[True, True, False], [False, True, False]])
    y = oracle.head_out(wo, bo, a, bits, hd, return_f64=True)
    for t in range(B):
        for c in range(d):
            ref = bo[c]
            for h in range(H):
                if bits[t, h]:
                    for i in range(hd):
                        ref += a[t, h * hd + i] * wo[h * hd + i, c]
            assert y[t, c] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_head_projections_closed_forms():
    """All heads: the dense projections (x W^T + b, attn W_o + b_o); no heads:
    zeros and b_o exactly; rows of unused heads are never read (NaN-poisoned);
    the output projection equals the input-sparse GEMV of the head-masked
    attention output."""
    d, H, hd, B = 16, 4, 8, 3
    w, b, wo, bo = _heads(d, H, hd, 5)
    x = np.random.default_rng(6).normal(0, 1, (B, d))
    a = np.random.default_rng(7).normal(0, 1, (B, H * hd))
    on = np.ones((B, H), dtype=bool)
    off = np.zeros((B, H), dtype=bool)
    assert np.allclose(oracle.head_qkv(w, b, x, on, hd, True), x @ w.T + b, rtol=1e-13, atol=1e-13)
    assert np.allclose(oracle.head_out(wo, bo, a, on, hd, True), a @ wo + bo, rtol=1e-13, atol=1e-13)
    assert not oracle.head_qkv(w, b, x, off, hd, True).any()
    assert np.array_equal(oracle.head_out(wo, bo, a, off, hd, True), np.tile(bo, (B, 1)))
    bits = np.array([[True, False, False, True], [False, False, False, True], [True, False, False, False]])
    wo_p = wo.copy()
    wo_p[hd:3 * hd] = np.nan                      # heads 1 and 2: used by no token
    assert np.array_equal(oracle.head_out(wo_p, bo, a, bits, hd, True), oracle.head_out(wo, bo, a, bits, hd, True))
    gated = a * np.repeat(bits, hd, axis=1)
    y_isg, _ = oracle.input_sparse_gemv(wo, gated, bo, return_f64=True)
    assert np.allclose(oracle.head_out(wo, bo, a, bits, hd, True), y_isg, rtol=1e-13, atol=1e-13)
