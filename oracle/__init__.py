"""CPU oracle for the predictor-gated sparse FFN.  TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product library never
does, and this package imports nothing from it.  See ``oracle/ffn.py`` for
what each function follows.
"""
from .ffn import (  # noqa: F401
    unpack_mask,
    pack_mask,
    predict,
    guard_band,
    compact,
    dequant_int4,
    rows_f64,
    masked_ffn,
    dense_ffn,
    true_active,
    fire_counts,
    hot_first_perm,
    permute_layer_ids,
    residual_rmsnorm,
    input_sparse_gemv,
    head_qkv,
    head_out,
)
