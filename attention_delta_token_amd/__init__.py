"""DASH (Delta Attention Selective Halting) prefill hot path for AMD Instinct MI355X.

The computation lives in the HIP library ``libdash.so`` (C ABI in
``include/dash.h``); this package is its thin Python binding plus drivers that
chain the calls into whole stacks.
"""
from ._lib import (  # noqa: F401
    DASH_BF16, DASH_F32, DASH_KV_ACTIVE, DASH_KV_ALL, DASH_OP_ATTN_ACTIVE, DASH_OP_ATTN_LAYER, DASH_OP_SELECT,
    DASH_SEL_ORDER_STAT, DASH_SEL_THRESHOLD, DASH_SEL_TOPK, DashError, EXPORTED, LIB_PATH,
    dash_attn_active, dash_attn_layer, dash_attn_layer_noalloc, dash_compact, dash_compact_many, dash_compact_batch, dash_score,
    dash_attn_layer_varlen, dash_select_ragged, dash_attn_active_varlen, dash_attn_active_gather, dash_decode, DASH_OP_DECODE, dash_select, dash_workspace_size, keep_count, percentile_rank, select_status, load, make_shape,
    version, workspace, trace_start, trace_select, trace_stop, trace_read,
)
