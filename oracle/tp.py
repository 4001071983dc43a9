"""Plain CPU oracle of the fixed-order sum of tensor-parallel partial outputs
(test infrastructure).

Under tensor parallelism over the expert inter dimension every rank holds a
slice of each expert's (and the shared expert's) intermediate columns and
produces a partial layer output for every row; the partials are summed per
row in a fixed source order, from one region laid out row by row and source by
source, so the Dp8 and the span row mappings give the same bits (openinfer PR
#610, description: the reduce-scatter region holds [parity][row][src][hidden];
"Gates": same fixed-order reductions under both mappings).  The parity
dimension alternates buffers between steps across ranks and has no role on one
GPU.  Readings (the pages name the layout and the fixed order, not the
arithmetic): each partial is the rank's bf16 layer output; the sum is taken in
float32, sources in ascending order, and rounded once to bf16; pad rows are
+0.0 and their partials are never read.
"""
from __future__ import annotations

import numpy as np

from .codec import decode_bf16, encode_bf16


def sum_partials(parts_bits: np.ndarray, row_mask: np.ndarray) -> np.ndarray:
    """parts_bits: bf16 bits [M, nsrc, H]; returns bf16 bits [M, H] of
    y[r] = bf16( (((0 + fl32(p[r,0])) + fl32(p[r,1])) + ...) ), float32 adds in
    ascending source order; pad rows +0.0."""
    m, nsrc, h = parts_bits.shape
    real = np.asarray(row_mask) != 0
    acc = np.zeros((m, h), dtype=np.float32)
    for s in range(nsrc):                                   # ascending source order
        v = decode_bf16(parts_bits[:, s, :]).astype(np.float32)
        acc[real] = (acc[real] + v[real]).astype(np.float32)
    out = encode_bf16(acc)
    out[~real] = 0
    return out
