"""Batch- and chunk-invariant attention over a paged KV cache on MI355X.

A thin ctypes binding of ``libbia.so`` (declared in ``include/bia.h``). The
functions keep the C names; they only turn torch tensors into device
pointers, numpy arrays into host pointers and torch streams into HIP stream
handles. Every step of the computation runs in the library's HIP kernels;
there is no fallback: if the library is missing or a call fails, an exception
says so.

Typical use::

    plan = bia_plan_create(BIA_MODE_PREFILL, qo_indptr, kv_indptr, page_table,
                           num_qo_heads=32, num_kv_heads=8, head_dim=128,
                           num_pages=pool_pages, split_size=BIA_PREFILL_SPLIT)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    bia_prefill_paged(plan, q, k_pool, v_pool, page_table_dev, sm_scale,
                      out, lse, ws)
"""
from __future__ import annotations

from ._lib import (BIA_DECODE_SPLIT, BIA_KV_TILE, BIA_MODE_DECODE,
                   BIA_MLA_MAX_SPLIT, BIA_MLA_QK_DIM, BIA_MLA_V_DIM, BIA_MODE_PREFILL,
                   BIA_PAGE_SIZE,
                   BIA_PLAN_MLA, BIA_PLAN_STRICT_CHUNK_ALIGN,
                   BIA_PREFILL_SPLIT, BIA_Q_TILE_ROWS, BIA_STATIC_WORKSPACE_BYTES,
                   BiaError, DecodeGraph, Plan,
                   bia_append_paged_kv, bia_decode_graph_create,
                   bia_decode_graph_destroy, bia_decode_graph_read_flags,
                   bia_decode_graph_run, bia_decode_graph_workspace_bytes,
                   bia_decode_paged, bia_decode_paged_static,
                   bia_last_error, bia_merge_states, bia_mla_decode_paged,
                   bia_mla_prefill_paged, bia_plan_create,
                   bia_plan_destroy, bia_plan_workspace_bytes,
                   bia_prefill_chunk_align, bia_prefill_paged, lib_path,
                   load_library)

__all__ = [
    "BIA_DECODE_SPLIT", "BIA_KV_TILE", "BIA_MLA_MAX_SPLIT", "BIA_MLA_QK_DIM", "BIA_MLA_V_DIM",
    "BIA_MODE_DECODE",
    "BIA_MODE_PREFILL", "BIA_PAGE_SIZE", "BIA_PLAN_MLA", "BIA_PLAN_STRICT_CHUNK_ALIGN", "BIA_PREFILL_SPLIT", "BIA_Q_TILE_ROWS",
    "BIA_STATIC_WORKSPACE_BYTES", "BiaError", "DecodeGraph", "Plan", "bia_append_paged_kv", "bia_decode_graph_create",
    "bia_decode_graph_destroy", "bia_decode_graph_read_flags", "bia_decode_graph_run",
    "bia_decode_graph_workspace_bytes", "bia_decode_paged", "bia_decode_paged_static", "bia_last_error",
    "bia_merge_states", "bia_mla_decode_paged", "bia_mla_prefill_paged", "bia_plan_create",
    "bia_plan_destroy", "bia_plan_workspace_bytes", "bia_prefill_chunk_align",
    "bia_prefill_paged", "lib_path", "load_library",
]
