"""Pins of the residual add + RMSNorm oracle (CPU only).

Each test checks the oracle against something other than itself: library
bf16 casts, a library RMSNorm, the closed form on constant rows and the
scale invariance of the normalization; planted mistakes fail them.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import decode_bf16
from synth import to_bf16_bits


def _bits(rng, shape, scale=1.0):
    return to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _torch_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_add_residual_matches_library_casts():
    rng = np.random.default_rng(11)
    m, h = 9, 640
    y, r = _bits(rng, (m, h)), _bits(rng, (m, h), 4.0)
    # exponent gaps of 20-30 binades, where the float32 sum itself rounds
    y[0, :64] = to_bf16_bits(np.float32(1.0) + np.zeros(64, np.float32))
    r[0, :64] = to_bf16_bits(np.ldexp(rng.uniform(1, 2, 64), -rng.integers(20, 30, 64)).astype(np.float32))
    mask = np.ones(m, np.uint8)
    mask[4] = 0
    got = oracle.add_residual(y, r, mask)
    ty = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16).float()
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16).float()
    want = _torch_bits((tr + ty).to(torch.bfloat16))
    real = mask.astype(bool)
    assert np.array_equal(got[real], want[real])
    assert not got[~real].any()


@pytest.mark.parametrize("h", [128, 640, 6144])
def test_rmsnorm_constant_rows_closed_form(h):
    # a row of one value c: mean(c^2) = c^2 exactly, so with eps = 0 the
    # normalized row is sign(c) * gamma (up to the rounding of 1 / |c| and
    # the two products)
    rng = np.random.default_rng(h)
    c = to_bf16_bits(rng.standard_normal(5).astype(np.float32) * np.float32(3.0))
    v = np.repeat(c[:, None], h, axis=1)
    g = _bits(rng, (h,))
    out = oracle.rmsnorm(v, g, 0.0, np.ones(5, np.uint8))
    want = np.sign(decode_bf16(c))[:, None] * decode_bf16(g)[None, :]
    assert np.all(np.abs(out - want) <= 4 * 2.0 ** -52 * np.abs(want))


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(3)
    v = _bits(rng, (6, 512))
    g = _bits(rng, (512,))
    mask = np.ones(6, np.uint8)
    base = oracle.rmsnorm(v, g, 0.0, mask)
    for k in (-7, 3, 11):
        vk = to_bf16_bits((decode_bf16(v) * np.float32(2.0 ** k)).astype(np.float32))
        assert np.allclose(oracle.rmsnorm(vk, g, 0.0, mask), base, rtol=1e-15, atol=0)


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_rmsnorm_matches_library(eps):
    rng = np.random.default_rng(5)
    v = _bits(rng, (7, 768), 0.3)
    g = _bits(rng, (768,))
    mask = np.ones(7, np.uint8)
    mask[2] = 0
    out = oracle.rmsnorm(v, g, eps, mask)
    tv = torch.from_numpy(decode_bf16(v).astype(np.float64))
    tg = torch.from_numpy(decode_bf16(g).astype(np.float64))
    lib = F.rms_norm(tv, (768,), weight=tg, eps=float(np.float32(eps))).numpy()
    real = mask.astype(bool)
    assert np.allclose(out[real], lib[real], rtol=1e-12, atol=1e-300)
    assert not out[~real].any()


def test_planted_mistakes_fail_the_pins():
    """A sum in place of the mean breaks the closed form; a dropped eps breaks
    the library comparison at a large eps."""
    rng = np.random.default_rng(8)
    h = 256
    c = to_bf16_bits(np.array([1.5, -0.25], np.float32))
    v = np.repeat(c[:, None], h, axis=1)
    g = to_bf16_bits(np.ones(h, np.float32))
    vv = decode_bf16(v).astype(np.float64)
    summed = vv / np.sqrt(np.sum(vv * vv, axis=1))[:, None]
    assert not np.array_equal(summed, oracle.rmsnorm(v, g, 0.0, np.ones(2, np.uint8)))
    w = _bits(rng, (3, h))
    wv = decode_bf16(w).astype(np.float64)
    no_eps = wv / np.sqrt(np.mean(wv * wv, axis=1))[:, None]
    lib = F.rms_norm(torch.from_numpy(wv), (h,), eps=0.5).numpy()
    assert not np.allclose(no_eps, lib, rtol=1e-12)
    assert np.allclose(oracle.rmsnorm(w, g, 0.5, np.ones(3, np.uint8)), lib, rtol=1e-12)
