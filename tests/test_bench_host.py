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
