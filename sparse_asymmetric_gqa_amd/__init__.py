"""libsaga: SAGA top-N decode attention for AMD MI355X (gfx950).

The C ABI (include/saga.h) is bound 1:1 by `_binding` (same names); `tensors`
adds torch-tensor convenience wrappers. Importing fails if libsaga.so has not
been built: there is no CPU or eager fallback.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, SAGA_BF16, SAGA_ERR_HIP, SAGA_ERR_INVALID_ARG, SAGA_ERR_TOO_LARGE,
    SAGA_ERR_UNSUPPORTED, SAGA_ERR_WORKSPACE, SAGA_F32, SAGA_OK, SagaError, lib, saga_atopn_attn, saga_atopn_calibrate,
    saga_atopn_workspace_size, saga_debug_fallback_rows, saga_debug_gather_rows,
    saga_debug_stream_read,
    saga_debug_scores, saga_decode_attn, saga_decode_attn_noalloc, saga_decode_attn_timed,
    saga_noalloc_scratch_bytes,
    saga_dense_attn, saga_dense_workspace_size, saga_sparq_attn, saga_sparq_workspace_size,
    saga_status_string, saga_workspace_size, status_string, SAGA_MERGE_KEY, SAGA_MERGE_LOGIT,
    SAGA_MERGE_SEQUENTIAL, saga_key_merge, saga_key_merge_timed, saga_key_merge_workspace_size,
    saga_merge_permute)
from .tensors import (  # noqa: F401
    atopn_attn, atopn_calibrate, atopn_workspace_size, debug_scores, decode_attn, dense_attn,
    dense_workspace_size, key_merge, key_merge_workspace_size, merge_permute, new_workspace,
    sparq_attn, sparq_workspace_size, workspace_size)
