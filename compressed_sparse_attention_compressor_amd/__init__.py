"""Compressed sparse attention (CSA / HCA / CSA2) on MI355X (gfx950).

The compute path is libcsa.so (hand-written HIP kernels behind the C ABI of
include/csa.h); this package only marshals torch tensors into it.
"""

from ._lib import CacheT, CsaError, lib  # noqa: F401
from .ops import (  # noqa: F401
    D,
    D_NOPE,
    D_ROPE,
    Cache,
    compress,
    compress_hidden,
    compress_index_scores,
    compress_index_topk,
    hca_dense_attn,
    index_scores,
    index_pool,
    index_topk,
    layer_stack,
    CSA2_FULL,
    CSA2_REINDEX,
    CSA2_REUSE,
    CAND_AUTO,
    CAND_SCAN,
    CAND_SELECTION,
    CAND_POOL,
    topk,
    sparse_attn,
    sparse_attn_w8,
    hca_dense_attn_w8,
    swa_encode,
    workspace_bytes,
    WS_DENSE_ATTN,
    WS_INDEX_POOL,
    WS_INDEX_TOPK,
    WS_SPARSE_ATTN,
    WS_TOPK,
    FLAG_CAND,
    FLAG_ENTRIES,
    FLAG_IDX_ORDER,
    FLAG_IDX_RANGE,
    FLAG_WINDOW,
    read_device_flags,
)
