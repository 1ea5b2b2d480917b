"""Seeded synthetic workloads for the predictor-gated sparse FFN.

This package only *draws* inputs: weights, biases, thresholds, token vectors
and integer-grid fixtures.  It holds none of the method's arithmetic (no
prediction, no compaction, no FFN) so that both the CPU oracle and the HIP
path can consume the very same bytes without sharing any computation.
"""
from .workload import (  # noqa: F401
    CONFIGS,
    LayerSpec,
    Layer,
    config,
    make_layer,
    make_tokens,
    make_grid_layer,
    make_grid_tokens,
    zipf_probs,
    uniform_probs,
    union_density,
    layer_probs,
    quant_int4_g128,
    random_masks,
    pack_bits,
    make_isg_weights,
    make_relu_inputs,
    make_head_weights,
    make_head_masks,
)
