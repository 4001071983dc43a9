"""Plain CPU oracle of the residual add + RMSNorm epilogue (test infrastructure).

The step after the layer on the pages: the layer output is added to the
residual stream and the sum is RMS-normalized for the next layer's input, in
one fused pass (mstar PR #388: the "kernel switches" note fuses each
all-reduce with the next add + RMSNorm, and its "Tests" list checks that the
fused wiring emits what the unfused ops do).  The pages name the fusion, not
its arithmetic.  Readings:

* the add: r_new = bf16_rne(fl32(r) + fl32(y)), y being the layer's bf16
  output and r the bf16 residual, added once in float32 (as a separate add
  kernel between two bf16 tensors would);
* the norm: out = r_new / sqrt(mean over the row of r_new^2 + eps) * gamma,
  evaluated here in float64 from the bf16 values of r_new and gamma, and
  returned before rounding (the device rounds its float32 value to bf16);
* pad rows: r_new = out = +0.0; their residual and y are never read.
"""
from __future__ import annotations

import numpy as np

from .codec import decode_bf16, encode_bf16


def add_residual(y_bits: np.ndarray, r_bits: np.ndarray, row_mask: np.ndarray) -> np.ndarray:
    """bf16 bits of r_new = bf16_rne(fl32(r) + fl32(y)); pad rows +0.0."""
    y = decode_bf16(y_bits).astype(np.float32)
    r = decode_bf16(r_bits).astype(np.float32)
    s = np.zeros(y.shape, dtype=np.float32)
    real = row_mask.astype(bool)
    s[real] = r[real] + y[real]                  # one float32 addition per element
    out = encode_bf16(s)
    out[~real] = 0
    return out


def rmsnorm(r_new_bits: np.ndarray, gamma_bits: np.ndarray, eps: float, row_mask: np.ndarray) -> np.ndarray:
    """float64 out[r, h] = v[r, h] / sqrt(mean_h v[r, h]^2 + eps) * gamma[h], v = r_new; pad rows 0."""
    v = decode_bf16(r_new_bits).astype(np.float64)
    g = decode_bf16(gamma_bits).astype(np.float64)
    ms = np.mean(v * v, axis=1)
    inv = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    out = v * inv[:, None] * g[None, :]
    out[~row_mask.astype(bool)] = 0.0
    return out


def add_rmsnorm(y_bits: np.ndarray, r_bits: np.ndarray, gamma_bits: np.ndarray, eps: float,
                row_mask: np.ndarray):
    """(r_new bf16 bits, float64 normalized output) of the fused epilogue."""
    r_new = add_residual(y_bits, r_bits, row_mask)
    return r_new, rmsnorm(r_new, gamma_bits, eps, row_mask)
