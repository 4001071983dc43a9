"""CPU oracle of the routed fp8 MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Plain float64 numpy with its own exact fp8/bf16 codecs.  It shares no code,
headers or tables with the HIP path, and the HIP path never imports it.
Only the tests, the smoke check and the CPU-baseline leg of the benchmark
may import or run anything in this package.

Pins (see tests/test_oracle_*.py): the e4m3/bf16 codecs against their closed
forms and torch's library casts over every code and every rounding midpoint;
the quantization rule against exactly representable blocks; routing against a
library sort in the bias-free special case and the k = E case; the block GEMM
against a library float64 matmul of dequantized matrices; the whole layer
against a brute-force dense evaluation of every expert on every row masked by
the top-k, written without the union or row compaction; and the layer
invariants (row slot permutation, companion rows, pad rows zero under NaN
poison, repeat determinism); the residual add + RMSNorm epilogue against its
closed form on constant rows, scale invariance, a library RMSNorm and
library bf16 casts; the fixed-order sum of tensor-parallel partials against
exact integer sums, a float64 sum within the rounding bound, a case whose
result depends on the order, and pad rows.  No function is left unpinned.
"""
from .codec import (E4M3_TABLE, decode_bf16, decode_e4m3, encode_bf16, encode_e4m3)
from .norm import add_residual, add_rmsnorm, rmsnorm
from .tp import sum_partials
from .moe_layer import (BLOCK, ExpertOut, LayerOut, Routing, block_gemm, ffn, layer, quant_1x128,
                    quant_rows, route, routed_expert, shared_expert, sigmoid, silu, union)

__all__ = [
    "E4M3_TABLE", "decode_bf16", "decode_e4m3", "encode_bf16", "encode_e4m3",
    "BLOCK", "ExpertOut", "LayerOut", "Routing", "block_gemm", "ffn", "layer", "quant_1x128",
    "quant_rows", "route", "routed_expert", "shared_expert", "sigmoid", "silu", "union",
    "add_residual", "add_rmsnorm", "rmsnorm", "sum_partials",
]
