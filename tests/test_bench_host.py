"""Host-side logic of bench.py (no GPU): the rule that sizes the dense hot prefix."""
import importlib.util
import os

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_auto_hot_prefix_rule():
    """A mask word joins the prefix while sum(1 - u_i) FFN rows < 64 predictor
    rows, from the front, stopping at the first word that fails."""
    b = _bench()
    spec = synth.config("c3", d_model=1024, d_ff=4096, rank=128)   # fp16: FFN row 4 KB, predictor row 260 B
    ffn_row, pred_row = 2 * 1024 * 2, 128 * 2 + 4
    limit = 64 * pred_row / ffn_row                                 # misses a word may hold: 4.06
    u = np.zeros(4096)
    assert b._auto_hot_prefix(spec, u) == 0
    u[:] = 1.0
    assert b._auto_hot_prefix(spec, u) == 4096
    u[:] = 0.0
    u[:128] = 1.0
    u[128:192] = 1.0 - 4.0 / 64                                     # 4 misses: joins
    u[192:256] = 1.0 - 5.0 / 64                                     # 5 misses: stops here
    u[256:] = 1.0
    assert 4.0 < limit < 5.0
    assert b._auto_hot_prefix(spec, u) == 192


def test_row_sample_is_the_first_neurons():
    """The dense-FFN row sample is the layer cut to its first k neurons: its
    dense output equals the full layer's masked FFN over those neurons."""
    import oracle
    b = _bench()
    spec = synth.config("c1", d_model=256, d_ff=512, rank=32)
    lay = synth.make_layer(spec, layer=0)
    x = synth.make_tokens(spec, 2, stream=3)
    sub = b._row_sample(lay, 128)
    assert sub.spec.d_ff == 128 and sub.w_up.shape == (128, 256) and lay.w_up.shape == (512, 256)
    bits = np.zeros((2, 512), dtype=bool)
    bits[:, :128] = True
    assert np.array_equal(oracle.dense_ffn(sub, x), oracle.masked_ffn(lay, x, bits))


def test_cpu_baseline_fields():
    """The CPU baseline reports the cores this process may use and both the
    sparse and the dense oracle rates (a tiny layer, a short budget)."""
    b = _bench()
    spec = synth.config("c1", d_model=256, d_ff=512, rank=32)
    hosts = [synth.make_layer(spec, layer=l) for l in range(2)]
    r = b._cpu_baseline(hosts, spec, 1, 4, 0.5)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["cores"] == len(os.sched_getaffinity(0))
    assert r["value"] > 0 and r["dense_ffn_tokens_s"] > 0
    assert r["dense_ffn_ms_per_layer"] > 0 and "median" in r["sample"]
