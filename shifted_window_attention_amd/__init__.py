"""MI355X (gfx950) shifted-window multi-head self-attention.

A thin ctypes binding over libswinattn.so: every function here only marshals
arguments (tensor data pointers, sizes, the current HIP stream) to the C ABI
declared in include/swin_attn.h, include/swin_block.h, include/swin_offload.h and
include/swin_route.h, under the same names. All computation runs in
the library's HIP kernels; there is no fallback. If the library has not been
built, importing the binding raises.
"""
import ctypes
import os

from .native import (  # noqa: F401
    SWIN_BF16, SWIN_F32, SWIN_OK, SWIN_PERIODIC_LAT, SWIN_PERIODIC_LEVEL, SWIN_PERIODIC_LON, SwinAttnDesc,
    SwinAttnStats, SwinError, lib, make_desc, swin_attn_bwd, swin_attn_bwd_noalloc, swin_attn_fwd, swin_attn_host_index_map,
    swin_attn_host_stats, swin_attn_index_map, swin_attn_plan_create, swin_attn_plan_destroy, swin_attn_plan_stats, swin_attn_sizes,
    swin_attn_plan_flags, swin_block_plan_flags, SWIN_FLAG_DT_SATURATED,
    swin_attn_sizes_recompute, swin_attn_fwd_recompute, swin_attn_bwd_recompute,
    swin_status_string, swin_window_gather, swin_window_scatter, swin_attn_trace_events, swin_attn_trace_cursor, Plan,
    SwinBlockDesc, SwinBlockParams, SwinBlockGrads, make_block_desc, swin_block_plan_create, swin_block_plan_destroy,
    swin_block_sizes, swin_block_fwd, swin_block_bwd, BlockPlan,
    PinnedBuffer, swin_offload_create, swin_offload_destroy, swin_offload_store, swin_offload_load, swin_offload_wait,
    swin_offload_query, swin_offload_sync, swin_offload_bytes,
    SWIN_LAYOUT_STRIPES, SWIN_LAYOUT_WINDOWS, SwinRankLayout, make_rank_layout, swin_route_host_tables, RoutePlan,
    swin_route_pack, swin_route_unpack, swin_route_loopback,
)
