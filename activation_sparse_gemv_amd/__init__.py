"""activation_sparse_gemv_amd: predictor-gated activation-sparse FFN decoding
for MI355X (gfx950), as a C-ABI library (libsfnn.so) plus this thin binding.

The entry points keep their C names (see include/sfnn.h):
sfnn_predict, sfnn_compact, sfnn_sparse_ffn, sfnn_layer, sfnn_layer_noalloc, sfnn_stack_decode, sfnn_dense_ffn,
sfnn_residual_rmsnorm, sfnn_fire_counts, sfnn_hot_first_perm, sfnn_dense_min_batch,
sfnn_gather_rows, sfnn_workspace_bytes, sfnn_input_sparse_gemv, sfnn_isg_workspace_bytes,
sfnn_head_qkv, sfnn_head_out, sfnn_heads_workspace_bytes.
"""
from ._lib import (  # noqa: F401
    EXPORTS, FFN, LIB_PATH, Pred, SFNN_F16, SFNN_F32, SFNN_I4G128, SFNN_RELU, SFNN_REGLU, SfnnError, load,
    sfnn_compact, sfnn_dense_ffn, sfnn_dense_min_batch, sfnn_fire_counts, sfnn_gather_rows, sfnn_hot_first_perm, sfnn_layer,
    sfnn_layer_noalloc, SFNN_NOALLOC_SCRATCH_BYTES,
    sfnn_predict, sfnn_probe_copy, sfnn_stack_decode, Stack, SFNN_STACK_LOOKAHEAD, sfnn_probe_read, sfnn_residual_rmsnorm, sfnn_sparse_ffn, sfnn_status_str,
    sfnn_version, sfnn_workspace_bytes, Isg, sfnn_input_sparse_gemv, sfnn_isg_workspace_bytes,
    Heads, sfnn_head_qkv, sfnn_head_out, sfnn_heads_workspace_bytes,
)
