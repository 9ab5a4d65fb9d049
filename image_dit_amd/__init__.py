"""MI355X-native training-free block-sparse attention forward.

The product is the HIP library ``libsparse_attn.so`` (C ABI in
``include/sparse_attn.h``); this package is its thin Python binding plus a
helper that sequences the four entry points over torch-allocated buffers.
"""

from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, SA_BF16, SA_ERR_CAPACITY, SA_ERR_EMPTY_ROW, SA_ERR_HIP, SA_ERR_INVALID_ARGUMENT,
    SA_ERR_UNSUPPORTED, SA_F32, SA_MAX_KEY_BLOCKS, SA_OK, SA_ORDER_HILBERT, SA_ORDER_IDENTITY,
    SA_ORDER_WINDOW, SA_PV_GROUP_ROWS, SaAttnParams, SaLayout, SaMaskParams, SparseAttnError, lib,
    make_attn_params, make_layout, make_mask_params, sa_permute, sa_plan_permutation, sa_plan_tile_window,
    sa_predict_mask, sa_predict_mask_ex, sa_predict_mask_gather_noalloc, SA_NOALLOC_SCRATCH_BYTES,
    sa_predict_workspace_bytes, sa_predict_workspace_offsets, sa_sparse_attn_fwd, sa_status_string,
    sa_unpermute, SA_FP8_KEY_ROWS, sa_quantize_fp8, sa_sparse_attn_fwd_qk8, sa_predict_mask_gather,
    sa_sparse_attn_fwd_gather, sa_predict_mask_qk8)
from .pipeline import PathConfig, SparseAttentionPath, config_from_workload  # noqa: F401
