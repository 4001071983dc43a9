"""Pins of the oracle's fp8 e4m3 and bf16 codecs (CPU only).

Pinned against: torch's float8_e4m3fn / bfloat16 casts (library routines),
every code of the format, every round-to-nearest-even midpoint, and a
brute-force nearest-neighbour search.
"""
import numpy as np
import pytest
import torch

from oracle import E4M3_TABLE, decode_bf16, decode_e4m3, encode_bf16, encode_e4m3


def test_decode_all_codes_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = decode_e4m3(np.arange(256, dtype=np.uint8))
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])
    # signed zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0])


def test_decode_spot_values():
    assert E4M3_TABLE[0x7E] == 448.0
    assert E4M3_TABLE[0x08] == 2.0 ** -6        # smallest normal
    assert E4M3_TABLE[0x01] == 2.0 ** -9        # smallest subnormal
    assert E4M3_TABLE[0x38] == 1.0
    assert E4M3_TABLE[0xB8] == -1.0


def test_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes).astype(np.float32)), codes)


def _positive_finite_codes():
    return [c for c in range(0, 0x7F)]


def test_encode_midpoints_ties_to_even():
    pos = _positive_finite_codes()
    for c in pos[:-1]:
        lo, hi = E4M3_TABLE[c], E4M3_TABLE[c + 1]
        mid = np.float32((lo + hi) / 2)           # exact in fp32
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        for sign in (1, -1):
            got = encode_e4m3(np.array([sign * mid], dtype=np.float32))[0]
            assert got == (even | (0x80 if sign < 0 else 0)), (c, sign)
            below = np.nextafter(np.float32(sign * mid), np.float32(0))
            above = np.nextafter(np.float32(sign * mid), np.float32(sign * np.inf))
            s = 0x80 if sign < 0 else 0
            assert encode_e4m3(np.array([below], np.float32))[0] == (c | s)
            assert encode_e4m3(np.array([above], np.float32))[0] == ((c + 1) | s)


def test_encode_saturates():
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e30, -448.0, -1e9], dtype=np.float32)
    assert list(encode_e4m3(v)) == [0x7E] * 6 + [0xFE] * 2


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    parts = [rng.uniform(-448, 448, 200_000),
             rng.normal(0, 1, 200_000),
             rng.uniform(-2 ** -6, 2 ** -6, 100_000),      # subnormal range
             np.ldexp(rng.uniform(-2, 2, 100_000), rng.integers(-12, 9, 100_000))]
    v = np.clip(np.concatenate(parts), -448, 448).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = encode_e4m3(v)
    assert np.array_equal(ours, lib)


def test_encode_rejects_nan():
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.nan], dtype=np.float32))


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = decode_bf16(bits)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_bf16_encode_matches_torch_fp32():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.normal(0, 1, 300_000),
        np.ldexp(rng.uniform(-2, 2, 100_000), rng.integers(-140, 127, 100_000)),
    ]).astype(np.float32)
    # add exact bf16 midpoints (ties) around a spread of exponents
    base = rng.integers(0, 1 << 15, 50_000, dtype=np.uint32) << np.uint32(16)
    mids = (base | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, mids[np.isfinite(mids)]])
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(encode_bf16(v), lib)


def test_bf16_encode_fp64_single_rounding_brute_force():
    """float64 inputs round once, to the nearest bf16 (ties to even)."""
    rng = np.random.default_rng(11)
    v = rng.normal(0, 3, 20_000)
    got = encode_bf16(v)
    # brute force: the two bf16 neighbours by bit pattern
    f32 = v.astype(np.float32).view(np.uint32)
    for i in range(v.size):
        hi16 = int(f32[i] >> 16)
        cands = [hi16 - 1, hi16, hi16 + 1]
        vals = [float(decode_bf16(np.array([c], dtype=np.uint16))[0]) for c in cands]
        d = [abs(x - v[i]) for x in vals]
        best = min(d)
        winners = [c for c, di in zip(cands, d) if di == best]
        want = winners[0] if len(winners) == 1 else [c for c in winners if c % 2 == 0][0]
        assert got[i] == want, (v[i], got[i], want)


def test_bf16_encode_specials():
    v = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.5e38], dtype=np.float64)
    b = encode_bf16(v)
    assert b[0] == 0x0000 and b[1] == 0x8000
    assert b[2] == 0x7F80 and b[3] == 0xFF80
    assert b[4] == 0x7FC0
    assert b[5] == 0x7F80          # rounds past the largest finite bf16
