"""MI355X-native grouped int4-dequant MoE layer.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/moe_int4.h (libmoe_int4.so); this package is the thin ctypes binding.
"""
from .binding import (ABLATIONS, GRAPH_CONCURRENT, Layer, LayerGraph, ablation_workspace_bytes, alloc_routing, alloc_workspace,
                      OVERFLOW_H, OVERFLOW_O, OVERFLOW_X, grouped_gemm_int4, layer_forward, layer_forward_ablation,
                      layer_forward_checked, layer_forward_noalloc, layer_forward_router, load, max_blocks,
                      prefill_chunked, route, route_workspace_bytes, router_logits, router_topk, status_string,
                      prepared_bytes, workspace_bytes, workspace_layout)

__all__ = ["ABLATIONS", "GRAPH_CONCURRENT", "Layer", "LayerGraph", "ablation_workspace_bytes", "alloc_routing", "alloc_workspace",
           "OVERFLOW_H", "OVERFLOW_O", "OVERFLOW_X", "grouped_gemm_int4", "layer_forward", "layer_forward_ablation",
           "layer_forward_checked", "layer_forward_noalloc", "layer_forward_router", "load", "max_blocks",
           "prefill_chunked", "route", "route_workspace_bytes", "router_logits", "router_topk", "status_string",
           "prepared_bytes", "workspace_bytes", "workspace_layout"]
