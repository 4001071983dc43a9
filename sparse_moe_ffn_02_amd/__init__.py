"""Routed fp8 MoE FFN layer for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI declared
in include/moe_ffn.h (libmoe_ffn.so); this package is the thin Python
binding with the same entry points (route, ffn_fp8, layer, quant_fp8,
pack_weights, add_rmsnorm, layer_add_rmsnorm).
"""
from ._lib import (EXPORTS, STATIC_WS_BYTES, MAX_EXPERTS, MAX_ROWS, MAX_TOPK, SMALL_ROWS, SMALL_ROWS_WIDE, split_rows, MOE_EINVAL, MOE_ELAUNCH, MOE_EUNSUPPORTED,
                   MOE_EWORKSPACE, MOE_OK, WEIGHTS_PACKED, WEIGHTS_ROW_MAJOR, Dims, Experts, MoeError, Routing, Shared, Taps, add_rmsnorm, ffn_fp8,
                   layer, layer_add_rmsnorm, layer_static, load, pack_experts, pack_shared, pack_weights, quant_fp8, route, sum_partials,
                   workspace, workspace_bytes)

__all__ = [
    "EXPORTS", "STATIC_WS_BYTES", "MAX_EXPERTS", "MAX_ROWS", "MAX_TOPK", "SMALL_ROWS", "SMALL_ROWS_WIDE", "split_rows", "MOE_EINVAL", "MOE_ELAUNCH", "MOE_EUNSUPPORTED",
    "MOE_EWORKSPACE", "MOE_OK", "WEIGHTS_PACKED", "WEIGHTS_ROW_MAJOR", "Dims", "Experts", "MoeError", "Routing", "Shared", "Taps", "add_rmsnorm",
    "ffn_fp8", "layer", "layer_add_rmsnorm", "layer_static", "load", "pack_experts", "pack_shared", "pack_weights", "quant_fp8", "route", "sum_partials", "workspace", "workspace_bytes",
]
