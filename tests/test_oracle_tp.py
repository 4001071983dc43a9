"""Pins of oracle.sum_partials (fixed-order sum of tensor-parallel partials)
against what arithmetic fixes, independent of its own formula."""
import numpy as np
import pytest
import torch

import oracle
from oracle import tp as tpmod


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_integer_partials_sum_exactly():
    """Small integers are exact in bf16 and in every float32 partial sum, so
    the result is the exact sum rounded once to bf16 (torch's cast)."""
    rng = np.random.default_rng(1)
    v = rng.integers(-100, 100, size=(5, 8, 64)).astype(np.float32)
    out = oracle.sum_partials(bf16(v), np.ones(5, np.uint8))
    assert np.array_equal(out, bf16(v.sum(axis=1)))


def test_matches_float64_sum_within_rounding():
    """|y - sum| <= the float32 sum's error bound (nsrc ulp of the running
    magnitudes) plus one bf16 rounding of the result."""
    rng = np.random.default_rng(2)
    v = rng.standard_normal((16, 8, 512)).astype(np.float32)
    bits = bf16(v)
    exact = oracle.decode_bf16(bits).sum(axis=1)
    absum = np.abs(oracle.decode_bf16(bits)).sum(axis=1)
    out = oracle.decode_bf16(oracle.sum_partials(bits, np.ones(16, np.uint8)))
    bound = 8 * 2.0 ** -24 * absum + 2.0 ** -8 * np.abs(exact) + 1e-30
    assert np.all(np.abs(out - exact) <= bound)


def test_ascending_source_order():
    """2^24 + 1 rounds back to 2^24 in float32, so the order decides the bits:
    sources (2^24, 1, -2^24) sum to 0 in ascending order (1 in the order 0, 2, 1)."""
    parts = np.zeros((1, 3, 4), np.float32)
    parts[0, 0], parts[0, 1], parts[0, 2] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    out = oracle.decode_bf16(oracle.sum_partials(bf16(parts), np.ones(1, np.uint8)))
    assert np.all(out == 0.0)
    out2 = oracle.decode_bf16(oracle.sum_partials(bf16(parts[:, [0, 2, 1]]), np.ones(1, np.uint8)))
    assert np.all(out2 == 1.0)


def test_pad_rows_zero_and_never_read():
    v = np.ones((3, 4, 8), np.float32)
    bits = bf16(v)
    bits[1] = 0x7FC0                                      # NaN partials of a pad row
    out = oracle.sum_partials(bits, np.array([1, 0, 1], np.uint8))
    assert not out[1].any()
    assert np.all(oracle.decode_bf16(out[[0, 2]]) == 4.0)


def test_planted_order_mistake_fails_the_pin(monkeypatch):
    """A reversed source order (a plausible slip) is caught by the order pin."""
    real = tpmod.sum_partials

    def reversed_order(parts_bits, row_mask):
        return real(parts_bits[:, ::-1, :], row_mask)
    monkeypatch.setattr(oracle, "sum_partials", reversed_order)
    with pytest.raises(AssertionError):
        test_ascending_source_order()
