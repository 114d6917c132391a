"""MI355X-native grouped int4-dequant MoE layer.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/moe_int4.h (libmoe_int4.so); this package is the thin ctypes binding.
"""
import os as _os

# Kernel arguments in device memory: without this the HIP runtime may keep
# them in host memory, where every workgroup of a launch reads them across
# the host link (a 2048-token layer call measured 3 % slower, an eager
# one-token decode step 18 % slower). The runtime reads it when it starts, so
# it applies when this package is imported before anything initialises the
# GPU; a value the caller set is kept.
_os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

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
