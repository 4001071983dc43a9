"""ctypes binding of libmoe_ffn.so: argument marshalling only.

Each function takes torch tensors that already live on the GPU, passes their
device addresses and torch's current HIP stream to the C ABI, and raises
MoeError on a non-zero status.  No step of the layer runs here.  If the
library has not been built, loading fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_ffn.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_ELAUNCH = range(5)
WEIGHTS_ROW_MAJOR = 0            # checkpoint layout (refused by the layer calls)
WEIGHTS_PACKED = 0x4B43504D      # rearranged by moe_pack_weights
MAX_ROWS, MAX_EXPERTS, MAX_TOPK, MAX_INTER = 16384, 256, 16, 8192
SMALL_ROWS = 24      # steps of up to this many rows take the split small-step kernels (inter <= 512)
SMALL_ROWS_WIDE = 16 # the same for wider experts (inter > 512)
NARROW_INTER = 512


def split_rows(inter: int) -> int:
    """Most rows of a step that takes the split small-step kernels."""
    return SMALL_ROWS if inter <= NARROW_INTER else SMALL_ROWS_WIDE


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class CDims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("routed_scale", C.c_float)]


class CRouter(C.Structure):
    _fields_ = [("w", C.c_void_p), ("bias", C.c_void_p)]


class CExperts(C.Structure):
    _fields_ = [("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p), ("layout", C.c_uint32)]


class CShared(C.Structure):
    _fields_ = [("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p), ("layout", C.c_uint32)]


class CRouting(C.Structure):
    _fields_ = [("topk_ids", C.c_void_p), ("topk_w", C.c_void_p), ("n_union", C.c_void_p),
                ("union_ids", C.c_void_p), ("offs", C.c_void_p), ("rows", C.c_void_p), ("slot_of", C.c_void_p)]


class CTaps(C.Structure):
    _fields_ = [("x_codes", C.c_void_p), ("x_scales", C.c_void_p), ("h_codes", C.c_void_p),
                ("h_scales", C.c_void_p)]


EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_ffn_fp8", "moe_layer", "moe_layer_static", "moe_quant_fp8",
           "moe_pack_weights", "moe_add_rmsnorm", "moe_layer_add_rmsnorm", "moe_sum_partials", "moe_prefetch_experts", "moe_trace_set",
           "moe_kernel_name", "moe_status_str")
STATIC_WS_BYTES = 64 << 20       # MOE_STATIC_WS_BYTES: the static workspace of moe_layer_static

_lib = None


def load() -> C.CDLL:
    """Load the library once.  Raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_ffn_02_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    lib.moe_workspace_bytes.argtypes = [C.POINTER(CDims), C.c_int32]
    lib.moe_workspace_bytes.restype = C.c_size_t
    lib.moe_route.argtypes = [C.POINTER(CDims), C.c_int32, P, P, C.POINTER(CRouter), C.POINTER(CRouting), P,
                              C.c_size_t, P]
    lib.moe_ffn_fp8.argtypes = [C.POINTER(CDims), C.c_int32, P, P, C.POINTER(CRouting), C.POINTER(CExperts), P,
                                C.POINTER(CTaps), P, C.c_size_t, P]
    lib.moe_layer.argtypes = [C.POINTER(CDims), C.c_int32, P, P, C.POINTER(CRouter), C.POINTER(CExperts),
                              C.POINTER(CShared), P, C.POINTER(CRouting), C.POINTER(CTaps), P, C.c_size_t, P]
    lib.moe_layer_static.argtypes = [C.POINTER(CDims), C.c_int32, P, P, C.POINTER(CRouter), C.POINTER(CExperts),
                                     C.POINTER(CShared), P, C.POINTER(CRouting), C.POINTER(CTaps), P]
    lib.moe_add_rmsnorm.argtypes = [C.c_int32, C.c_int32, P, P, P, P, C.c_float, P, P, P]
    lib.moe_sum_partials.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, P, P]
    lib.moe_prefetch_experts.argtypes = [C.POINTER(CDims), P, P, C.POINTER(CExperts), C.c_uint32, C.c_int64,
                                         C.c_int32, P, P]
    lib.moe_layer_add_rmsnorm.argtypes = [C.POINTER(CDims), C.c_int32, P, P, C.POINTER(CRouter),
                                          C.POINTER(CExperts), C.POINTER(CShared), P, P, C.c_float, P, P, P,
                                          C.POINTER(CRouting), C.POINTER(CTaps), P, C.c_size_t, P]
    lib.moe_quant_fp8.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P, P, P]
    lib.moe_pack_weights.argtypes = [P, P, C.c_int64, C.c_int32, C.c_int32, P]
    lib.moe_trace_set.argtypes = [P, C.c_int32, P, P]
    lib.moe_trace_set.restype = C.c_int
    lib.moe_kernel_name.argtypes = [C.c_int32]
    lib.moe_kernel_name.restype = C.c_char_p
    lib.moe_status_str.argtypes = [C.c_int]
    lib.moe_status_str.restype = C.c_char_p
    for f in ("moe_route", "moe_ffn_fp8", "moe_layer", "moe_layer_static", "moe_quant_fp8", "moe_pack_weights",
              "moe_add_rmsnorm", "moe_layer_add_rmsnorm", "moe_sum_partials"):
        getattr(lib, f).restype = C.c_int
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    # without a visible GPU every call fails its checks or its first launch
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0


def _check(st: int) -> None:
    if st != MOE_OK:
        raise MoeError(st, load().moe_status_str(st).decode())


@dataclass(frozen=True)
class Dims:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    routed_scale: float = 2.5

    def c(self) -> CDims:
        return CDims(self.hidden, self.n_experts, self.top_k, self.inter, self.shared_inter, self.routed_scale)


@dataclass
class Routing:
    """Device buffers of one step's routing (layout of moe_routing)."""
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    n_union: torch.Tensor
    union_ids: torch.Tensor
    offs: torch.Tensor
    rows: torch.Tensor
    slot_of: torch.Tensor

    @staticmethod
    def empty(dims: Dims, m: int, device="cuda") -> "Routing":
        i32 = dict(dtype=torch.int32, device=device)
        return Routing(torch.empty((m, dims.top_k), **i32), torch.empty((m, dims.top_k), dtype=torch.float32,
                                                                          device=device),
                       torch.empty(1, **i32), torch.empty(dims.n_experts, **i32),
                       torch.empty(dims.n_experts + 1, **i32), torch.empty(max(1, m * dims.top_k), **i32),
                       torch.empty((m, dims.top_k), **i32))

    def c(self) -> CRouting:
        return CRouting(*(_ptr(t) for t in (self.topk_ids, self.topk_w, self.n_union, self.union_ids, self.offs,
                                            self.rows, self.slot_of)))


@dataclass
class Experts:
    """Routed expert weights.  The layer calls take them packed (pack_experts
    returns layout=WEIGHTS_PACKED); row-major checkpoint tensors are refused."""
    w_gate: torch.Tensor   # uint8 [E, I, H]
    w_up: torch.Tensor
    w_down: torch.Tensor   # uint8 [E, H, I]
    s_gate: torch.Tensor   # f32 [E, I/128, H/128]
    s_up: torch.Tensor
    s_down: torch.Tensor
    layout: int = WEIGHTS_ROW_MAJOR

    def c(self) -> CExperts:
        return CExperts(*(_ptr(t) for t in (self.w_gate, self.w_up, self.w_down, self.s_gate, self.s_up,
                                            self.s_down)), self.layout)


@dataclass
class Shared:
    """Shared-expert weights (bf16 bits); packed by pack_shared."""
    w_gate: torch.Tensor   # bf16 bits (int16/uint16) [I_s, H]
    w_up: torch.Tensor
    w_down: torch.Tensor   # [H, I_s]
    layout: int = WEIGHTS_ROW_MAJOR

    def c(self) -> CShared:
        return CShared(_ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down), self.layout)


@dataclass
class Taps:
    x_codes: Optional[torch.Tensor] = None
    x_scales: Optional[torch.Tensor] = None
    h_codes: Optional[torch.Tensor] = None
    h_scales: Optional[torch.Tensor] = None

    @staticmethod
    def empty(dims: Dims, m: int, device="cuda") -> "Taps":
        u8 = dict(dtype=torch.uint8, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        s = max(1, m * dims.top_k)
        return Taps(torch.empty((m, dims.hidden), **u8), torch.empty((m, dims.hidden // 128), **f32),
                    torch.empty((s, dims.inter), **u8), torch.empty((s, dims.inter // 128), **f32))

    def c(self) -> CTaps:
        return CTaps(_ptr(self.x_codes), _ptr(self.x_scales), _ptr(self.h_codes), _ptr(self.h_scales))


def workspace_bytes(dims: Dims, max_rows: int) -> int:
    d = dims.c()
    return int(load().moe_workspace_bytes(C.byref(d), max_rows))


def workspace(dims: Dims, max_rows: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(dims, max_rows)
    if n == 0:
        raise MoeError(MOE_EINVAL, "invalid dims or row count for the workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def route(dims: Dims, x: torch.Tensor, row_mask: Optional[torch.Tensor], router_w: torch.Tensor,
          bias: torch.Tensor, out: Routing, ws: torch.Tensor) -> None:
    d = dims.c()
    r = CRouter(_ptr(router_w), _ptr(bias))
    o = out.c()
    _check(load().moe_route(C.byref(d), x.shape[0], _ptr(x), _ptr(row_mask), C.byref(r), C.byref(o), _ptr(ws),
                            ws.numel(), _stream()))


def ffn_fp8(dims: Dims, x: torch.Tensor, row_mask: Optional[torch.Tensor], routing: Routing, experts: Experts,
            y: torch.Tensor, ws: torch.Tensor, taps: Optional[Taps] = None) -> None:
    d = dims.c()
    rt = routing.c()
    ew = experts.c()
    tp = taps.c() if taps is not None else None
    _check(load().moe_ffn_fp8(C.byref(d), x.shape[0], _ptr(x), _ptr(row_mask), C.byref(rt), C.byref(ew), _ptr(y),
                              C.byref(tp) if tp is not None else None, _ptr(ws), ws.numel(), _stream()))


def layer(dims: Dims, x: torch.Tensor, row_mask: Optional[torch.Tensor], router_w: torch.Tensor, bias: torch.Tensor,
          experts: Experts, shared: Optional[Shared], y: torch.Tensor, routing: Routing, ws: torch.Tensor,
          taps: Optional[Taps] = None) -> None:
    d = dims.c()
    r = CRouter(_ptr(router_w), _ptr(bias))
    ew = experts.c()
    sw = shared.c() if shared is not None else None
    rt = routing.c()
    tp = taps.c() if taps is not None else None
    _check(load().moe_layer(C.byref(d), x.shape[0], _ptr(x), _ptr(row_mask), C.byref(r), C.byref(ew),
                            C.byref(sw) if sw is not None else None, _ptr(y), C.byref(rt),
                            C.byref(tp) if tp is not None else None, _ptr(ws), ws.numel(), _stream()))


def layer_static(dims: Dims, x: torch.Tensor, row_mask: Optional[torch.Tensor], router_w: torch.Tensor,
                 bias: torch.Tensor, experts: Experts, shared: Optional[Shared], y: torch.Tensor, routing: Routing,
                 taps: Optional[Taps] = None) -> None:
    """moe_layer_static: the layer in the library's static per-GPU workspace
    (no workspace argument, nothing allocated by the call)."""
    d = dims.c()
    r = CRouter(_ptr(router_w), _ptr(bias))
    ew = experts.c()
    sw = shared.c() if shared is not None else None
    rt = routing.c()
    tp = taps.c() if taps is not None else None
    _check(load().moe_layer_static(C.byref(d), x.shape[0], _ptr(x), _ptr(row_mask), C.byref(r), C.byref(ew),
                                   C.byref(sw) if sw is not None else None, _ptr(y), C.byref(rt),
                                   C.byref(tp) if tp is not None else None, _stream()))


def add_rmsnorm(y: torch.Tensor, row_mask: Optional[torch.Tensor], residual: torch.Tensor, gamma: torch.Tensor,
                eps: float, residual_out: torch.Tensor, out: torch.Tensor) -> None:
    """moe_add_rmsnorm on bf16 [M, H] tensors (uint16 bits or bfloat16)."""
    m, h = y.shape
    _check(load().moe_add_rmsnorm(m, h, _ptr(y), _ptr(row_mask), _ptr(residual), _ptr(gamma), eps,
                                  _ptr(residual_out), _ptr(out), _stream()))


def layer_add_rmsnorm(dims: Dims, x: torch.Tensor, row_mask: Optional[torch.Tensor], router_w: torch.Tensor,
                      bias: torch.Tensor, experts: Experts, shared: Optional[Shared], residual: torch.Tensor,
                      gamma: torch.Tensor, eps: float, y: Optional[torch.Tensor], residual_out: torch.Tensor,
                      out: torch.Tensor, routing: Routing, ws: torch.Tensor, taps: Optional[Taps] = None) -> None:
    """moe_layer_add_rmsnorm: the layer with the residual add + RMSNorm in its combine."""
    d = dims.c()
    r = CRouter(_ptr(router_w), _ptr(bias))
    ew = experts.c()
    sw = shared.c() if shared is not None else None
    rt = routing.c()
    tp = taps.c() if taps is not None else None
    _check(load().moe_layer_add_rmsnorm(C.byref(d), x.shape[0], _ptr(x), _ptr(row_mask), C.byref(r), C.byref(ew),
                                        C.byref(sw) if sw is not None else None, _ptr(residual), _ptr(gamma), eps,
                                        _ptr(y), _ptr(residual_out), _ptr(out), C.byref(rt),
                                        C.byref(tp) if tp is not None else None, _ptr(ws), ws.numel(), _stream()))


def sum_partials(parts: torch.Tensor, row_mask: Optional[torch.Tensor], y: torch.Tensor) -> None:
    """moe_sum_partials: parts bf16 bits [M, nsrc, H] -> y [M, H], float32 sum in
    ascending source order, one bf16 rounding."""
    m, nsrc, h = parts.shape
    _check(load().moe_sum_partials(m, h, nsrc, _ptr(parts), _ptr(row_mask), _ptr(y), _stream()))


PREFETCH_GATE_UP = 1     # MOE_PREFETCH_GATE_UP
PREFETCH_DOWN = 2        # MOE_PREFETCH_DOWN


def prefetch_experts(dims: Dims, n_union: torch.Tensor, union_ids: torch.Tensor, experts: Experts, parts: int,
                     max_bytes: int, workgroups: int = 0, checksum: Optional[torch.Tensor] = None) -> None:
    """moe_prefetch_experts: read the listed experts' packed matrices (the
    first *n_union entries of union_ids, device int32) ahead of use; checksum
    (int32 [1], cleared by the caller) receives the 32-bit word sum of the
    bytes read."""
    d = dims.c()
    ew = experts.c()
    _check(load().moe_prefetch_experts(C.byref(d), _ptr(n_union), _ptr(union_ids), C.byref(ew), parts, max_bytes,
                                       workgroups, _ptr(checksum), _stream()))


def pack_weights(src: torch.Tensor, dst: torch.Tensor, is_bf16: bool) -> None:
    """moe_pack_weights on a row-major weight tensor [..., rows, K] (e4m3 codes
    or bf16 bits) into dst (same shape and size) on the current stream."""
    row_bytes = src.shape[-1] * src.element_size()
    rows = src.numel() * src.element_size() // row_bytes
    _check(load().moe_pack_weights(_ptr(src), _ptr(dst), rows, row_bytes, 1 if is_bf16 else 0, _stream()))


def _packed(t: torch.Tensor, is_bf16: bool) -> torch.Tensor:
    out = torch.empty_like(t)
    pack_weights(t, out, is_bf16)
    return out


def pack_experts(row_major: Experts) -> Experts:
    """Packed copies of row-major expert weights (scales are shared, not copied)."""
    if row_major.layout != WEIGHTS_ROW_MAJOR:
        raise MoeError(MOE_EINVAL, "pack_experts takes row-major weights")
    return Experts(_packed(row_major.w_gate, False), _packed(row_major.w_up, False), _packed(row_major.w_down, False),
                   row_major.s_gate, row_major.s_up, row_major.s_down, WEIGHTS_PACKED)


def pack_shared(row_major: Shared) -> Shared:
    """Packed copies of row-major bf16 shared-expert weights."""
    if row_major.layout != WEIGHTS_ROW_MAJOR:
        raise MoeError(MOE_EINVAL, "pack_shared takes row-major weights")
    return Shared(_packed(row_major.w_gate, True), _packed(row_major.w_up, True), _packed(row_major.w_down, True),
                  WEIGHTS_PACKED)


def quant_fp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor) -> None:
    """x: fp32 or bf16-bits (int16/uint16) [rows, cols] -> codes uint8, scales f32 [rows, cols/128]."""
    is_bf16 = 1 if x.dtype in (torch.int16, torch.uint16, torch.bfloat16) else 0
    if not is_bf16 and x.dtype != torch.float32:
        raise MoeError(MOE_EINVAL, "quant_fp8 takes float32 or bf16 input")
    _check(load().moe_quant_fp8(_ptr(x), is_bf16, x.shape[0], x.shape[1], _ptr(codes), _ptr(scales), _stream()))
