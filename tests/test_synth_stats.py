"""Statistics of the seeded workloads, checked against the pages' figures and
closed forms (the generator is test and bench infrastructure).

* ReLU layers at ~90% sparsity (53ai.com survey, section 激活稀疏的可行性).
* Power law: 26% / 43% of the neurons carry 80% of the activations, about 20%
  of OPT-30B's neurons fire per token (hexiedandong.com PowerInfer repost,
  power-law paragraph; 53ai.com survey, section 性能对比).
* The union over a batch grows like mean_i 1 - (1 - p_i)^B, i.e. sparsity decays
  with batch while the union grows sub-linearly under the power law
  (53ai.com survey, section 工程效果 / throughput paragraph).
"""
import numpy as np
import pytest

import oracle
import synth


def _ci(p, n, z=3.29):
    return z * np.sqrt(p * (1 - p) / n)


def test_relu_bias_calibration_fire_rate():
    spec = synth.config("c1")
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 1024, stream=5)
    t = oracle.true_active(lay, x)
    rate = t.mean()
    assert abs(rate - 0.1) < _ci(0.1, t.size) * 3
    per_neuron = t.mean(axis=0)
    # per-neuron rates within a 99.9% binomial interval for almost every neuron
    ok = np.abs(per_neuron - 0.1) <= _ci(0.1, x.shape[0])
    assert ok.mean() > 0.99


def test_predictor_threshold_calibration_fire_rate():
    spec = synth.config("c1")
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 2048, stream=6)
    _, m = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
    assert abs(m.mean() - 0.1) < 4 * _ci(0.1, m.size)
    ok = np.abs(m.mean(axis=0) - 0.1) <= _ci(0.1, x.shape[0])
    assert ok.mean() > 0.99


@pytest.mark.parametrize("n,phi,rho,s_expect", [(28672, 0.26, 0.2, 1.674), (28672, 0.43, 0.1, 0.903)])
def test_zipf_profile_matches_page_shares(n, phi, rho, s_expect):
    p, s, c = synth.zipf_probs(n, phi, rho)
    k = int(round(phi * n))
    assert abs(p[:k].sum() / p.sum() - 0.80) < 1e-6
    assert abs(p.mean() - rho) < 1e-6
    assert np.all(np.diff(p) <= 0) and p.max() <= 1.0 and p.min() > 0
    assert abs(s - s_expect) < 5e-3


def test_zipf_layer_is_not_hot_first_but_profile_recovers_it():
    spec = synth.config("c3", d_model=128, d_ff=1024, rank=64)
    p = synth.workload._probs_for(spec, 0, 0)
    assert abs(p.mean() - 0.2) < 1e-6
    assert not np.all(np.diff(p) <= 0)          # natural layout is scattered
    # profiling masks drawn at these rates recover a hot-first order
    words = synth.random_masks(4000, 1024, 0.0, seed=1, probs=p)
    perm = oracle.hot_first_perm(oracle.fire_counts(words, 1024))
    top = perm[:100]
    assert p[top].mean() > np.sort(p)[::-1][:100].mean() * 0.9


@pytest.mark.parametrize("B", [1, 2, 4, 32])
def test_union_law_uniform(B):
    f, trials = 4096, 64
    sizes = []
    for t in range(trials):
        w = synth.random_masks(B, f, 0.1, seed=1000 * B + t)
        sizes.append(oracle.compact(w, B, f)[1] / f)
    expect = synth.union_density(np.full(f, 0.1), B)
    assert abs(expect - {1: 0.1, 2: 0.19, 4: 0.3439, 32: 1 - 0.9 ** 32}[B]) < 1e-12
    assert abs(np.mean(sizes) - expect) < 4 * np.std(sizes) / np.sqrt(trials) + 1e-3


def test_union_law_power_law_is_sublinear():
    p, _, _ = synth.zipf_probs(28672, 0.26, 0.2)
    u = [synth.union_density(p, b) for b in (1, 4, 16)]
    assert abs(u[0] - 0.2) < 1e-9 and abs(u[1] - 0.368) < 2e-3 and abs(u[2] - 0.647) < 2e-3
    uni = [synth.union_density(np.full(28672, 0.2), b) for b in (1, 4, 16)]
    assert u[1] < uni[1] and u[2] < uni[2]          # power law keeps the union smaller
    w = synth.random_masks(16, 28672, 0.0, seed=3, probs=p)
    got = oracle.compact(w, 16, 28672)[1] / 28672
    assert abs(got - u[2]) < 0.01


def test_seeded_layers_are_reproducible_and_distinct():
    spec = synth.config("c2", d_model=256, d_ff=1024, rank=64)
    a = synth.make_layer(spec, layer=0)
    b = synth.make_layer(spec, layer=0)
    c = synth.make_layer(spec, layer=1)
    assert np.array_equal(a.w_up, b.w_up) and np.array_equal(a.tau, b.tau)
    assert not np.array_equal(a.w_up, c.w_up)
    assert a.w_up.dtype == np.float16 and a.b_up.dtype == np.float16 and a.tau.dtype == np.float32
    assert abs(float(a.w_up.astype(np.float64).std()) - 0.02) < 1e-3


def test_int4_layer_shapes_and_grid_layer_bounds():
    spec = synth.config("c5", d_model=256, d_ff=512, rank=64)
    lay = synth.make_layer(spec, layer=0)
    assert lay.q_up.shape == (512, 128) and lay.s_up.shape == (512, 2) and lay.w_up is None
    g = synth.make_grid_layer(256, 1024, 64, act="relu", wtype="i4g128")
    w = oracle.dequant_int4(g.q_up, g.s_up)
    assert np.abs(w).max() <= 4 and np.all(w * 2 == np.round(w * 2))
