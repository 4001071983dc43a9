"""Routed fp8 MoE FFN layer for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI declared
in include/moe_ffn.h (libmoe_ffn.so); this package is the thin Python
binding with the same entry points (route, ffn_fp8, layer, layer_static,
quant_fp8, pack_weights, add_rmsnorm, layer_add_rmsnorm, sum_partials,
prefetch_experts), plus the host-side route-ahead set measures
(route_ahead).
"""
from ._lib import (EXPORTS, STATIC_WS_BYTES, MAX_EXPERTS, MAX_ROWS, MAX_TOPK, SMALL_ROWS, SMALL_ROWS_WIDE, split_rows,
                   MOE_EINVAL, MOE_ELAUNCH, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_OK, PREFETCH_DOWN, PREFETCH_GATE_UP,
                   WEIGHTS_PACKED, WEIGHTS_ROW_MAJOR, Dims, Experts, MoeError, Routing, Shared, Taps, add_rmsnorm,
                   ffn_fp8, layer, layer_add_rmsnorm, layer_static, load, pack_experts, pack_shared, pack_weights,
                   prefetch_experts, quant_fp8, route, sum_partials, workspace, workspace_bytes)
from . import route_ahead

__all__ = [
    "EXPORTS", "STATIC_WS_BYTES", "MAX_EXPERTS", "MAX_ROWS", "MAX_TOPK", "SMALL_ROWS", "SMALL_ROWS_WIDE", "split_rows",
    "MOE_EINVAL", "MOE_ELAUNCH", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE", "MOE_OK", "PREFETCH_DOWN", "PREFETCH_GATE_UP",
    "WEIGHTS_PACKED", "WEIGHTS_ROW_MAJOR", "Dims", "Experts", "MoeError", "Routing", "Shared", "Taps", "add_rmsnorm",
    "ffn_fp8", "layer", "layer_add_rmsnorm", "layer_static", "load", "pack_experts", "pack_shared", "pack_weights",
    "prefetch_experts", "quant_fp8", "route", "route_ahead", "sum_partials", "workspace", "workspace_bytes",
]
