"""Exact number codecs used by the oracle (test infrastructure only).

* e4m3 (OCP FP8 "e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, S.1111.111 is NaN, largest finite value 448) -- the
  format of the routed-expert weights and of the activation codes (the fp8
  checkpoint of MoE-Infinity PR #140, commit "native FP8 e4m3 block-scale
  dequant kernel ... bit-exact vs python"; activations quantized to e4m3 per
  128 columns in mstar PR #388, FlashInfer crossover note).
* bf16: the upper 16 bits of an IEEE binary32.

Decoding is exact in float64.  Encoding rounds to nearest, ties to even.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of every code, from the closed form above
E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Round finite values to the nearest e4m3 code, ties to even, saturating.

    Magnitudes at or above 448 map to 448 (code 0x7E); the sign is kept, so
    -0.0 encodes as 0x80.  Inputs must not be NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("encode_e4m3: NaN input")
    neg = np.signbit(v)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    sat = a >= E4M3_MAX
    sub = a < 2.0 ** -6
    # subnormal range: the grid is multiples of 2^-9; a rounded count of 8 is
    # exactly the smallest normal, whose code is also 8.
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub & ~sat
    if nrm.any():
        an = a[nrm]
        ex = np.floor(np.log2(an)).astype(np.int64)
        # guard the floor(log2) against rounding at exact powers of two
        ex = np.where(np.ldexp(1.0, ex) > an, ex - 1, ex)
        ex = np.where(np.ldexp(1.0, ex + 1) <= an, ex + 1, ex)
        q = np.rint(np.ldexp(an, 3 - ex)).astype(np.int64)    # in [8, 16]
        code[nrm] = ((ex + 7) << 3) + (q - 8)                   # q == 16 carries
    code[sat] = 0x7E
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def encode_bf16(v: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to bf16 (nearest, ties to even) -> uint16 bits.

    Overflow goes to infinity (round to nearest), NaN stays NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    fin = np.isfinite(v)
    a = v[fin]
    m, e = np.frexp(a)                       # a = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits; below 2^-126 the grid is fixed at 2^-133
    e_eff = np.maximum(e, -125)
    r = np.ldexp(np.rint(np.ldexp(a, 8 - e_eff)), e_eff - 8)
    out[fin] = r
    out[~fin] = v[~fin]
    with np.errstate(over="ignore"):
        f32 = out.astype(np.float32)         # exact for every finite rounded value below 2^128
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(v)
    bits[nan] = 0x7FC0
    return bits
