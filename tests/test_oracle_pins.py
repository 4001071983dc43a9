"""Pins of the oracle's quantization rule, router, union and block GEMM (CPU only).

Each test checks the oracle against something other than itself: exactly
representable inputs, a library sort or matmul, exhaustive subset search,
exact integer arithmetic, or a mathematical identity.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import decode_bf16, decode_e4m3, encode_e4m3
from synth import to_bf16_bits


# ---------------------------------------------------------------- quant rule

def test_quant_exact_blocks_roundtrip():
    rng = np.random.default_rng(0)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    rows, k = 6, 512
    codes = rng.choice(finite, size=(rows, k)).astype(np.uint8)
    p = rng.integers(-20, 20, size=(rows, k // 128))
    for r in range(rows):
        for b in range(k // 128):
            codes[r, b * 128 + rng.integers(0, 128)] = 0x7E if rng.random() < 0.5 else 0xFE
    s = np.ldexp(1.0, p).astype(np.float32)
    v = (decode_e4m3(codes) * np.repeat(s, 128, axis=1)).astype(np.float32)
    q, sc = oracle.quant_1x128(v)
    assert np.array_equal(sc, s)
    assert np.array_equal(q, codes)


def test_quant_zero_block():
    v = np.zeros((2, 256), dtype=np.float32)
    v[1, 128:] = np.linspace(-3, 3, 128, dtype=np.float32)
    q, s = oracle.quant_1x128(v)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert not q[0].any() and not q[1, :128].any()
    assert s[1, 1] == np.float32(np.float32(3.0) / np.float32(448.0))


def test_quant_error_bound():
    """|v - dec(q) s| <= 2^-4 |v| (normal range) or s * 2^-10 (subnormal range)."""
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((64, 1024)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    q, s = oracle.quant_1x128(v)
    se = np.repeat(s.astype(np.float64), 128, axis=1)
    back = decode_e4m3(q) * se
    err = np.abs(back - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, se * 2.0 ** -10) * (1 + 1e-6)
    assert (err <= bound).all()
    # the block maximum maps to +-448
    amax_code = np.abs(decode_e4m3(q)).reshape(64, 8, 128).max(axis=2)
    assert (amax_code == 448.0).all()


# ---------------------------------------------------------------- router

def _router_case(m, h, e, seed, bias_scale=0.1):
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32))
    wr = to_bf16_bits((rng.standard_normal((e, h)) / np.sqrt(h)).astype(np.float32))
    b = (rng.standard_normal(e) * bias_scale).astype(np.float32)
    return x, wr, b


def test_route_zero_bias_is_topk_of_logits():
    x, wr, _ = _router_case(16, 256, 32, 5)
    ids, w, _ = oracle.route(x, np.ones(16, np.uint8), wr, np.zeros(32, np.float32), 6)
    l = decode_bf16(x) @ decode_bf16(wr).T        # library matmul, independent of the oracle's
    for r in range(16):
        want = np.sort(np.argsort(-l[r], kind="stable")[:6])
        assert np.array_equal(ids[r], want)


def test_route_matches_subset_search():
    """The selected set maximizes the summed biased score (exhaustive search)."""
    x, wr, b = _router_case(12, 128, 9, 6, bias_scale=0.3)
    ids, w, _ = oracle.route(x, np.ones(12, np.uint8), wr, b, 3, 2.5)
    l = decode_bf16(x) @ decode_bf16(wr).T
    sig = expit(l)                                 # library sigmoid
    c = sig + b.astype(np.float64)
    for r in range(12):
        best = max(itertools.combinations(range(9), 3), key=lambda s: sum(c[r, j] for j in s))
        assert tuple(ids[r]) == best
        # weights use the unbiased sigmoid of the selected experts
        ws = 2.5 * sig[r, list(best)] / sig[r, list(best)].sum()
        assert np.allclose(w[r], ws, rtol=1e-14, atol=0)


def test_route_bias_changes_selection_not_weights():
    x, wr, _ = _router_case(4, 128, 8, 9)
    b = np.zeros(8, np.float32)
    b[7] = 10.0                                     # forces expert 7 into every row
    ids, w, _ = oracle.route(x, np.ones(4, np.uint8), wr, b, 2, 2.5)
    sig = expit(decode_bf16(x) @ decode_bf16(wr).T)
    for r in range(4):
        assert 7 in ids[r]
        assert np.allclose(w[r], 2.5 * sig[r, ids[r]] / sig[r, ids[r]].sum(), rtol=1e-14)


def test_route_k_equals_e_and_weight_sum():
    x, wr, b = _router_case(8, 128, 8, 2)
    ids, w, _ = oracle.route(x, np.ones(8, np.uint8), wr, b, 8, 2.5)
    assert (ids == np.arange(8)).all()
    assert np.allclose(w.sum(axis=1), 2.5, rtol=0, atol=8 * 2.5 * 2 ** -52)


def test_route_ties_go_to_lower_id_and_pads():
    x = np.zeros((3, 128), np.uint16)             # all-zero rows: every logit is 0
    wr = to_bf16_bits(np.random.default_rng(0).standard_normal((10, 128)).astype(np.float32))
    mask = np.array([1, 0, 1], np.uint8)
    ids, w, _ = oracle.route(x, mask, wr, np.zeros(10, np.float32), 4, 2.5)
    assert (ids[0] == [0, 1, 2, 3]).all() and (ids[2] == [0, 1, 2, 3]).all()
    assert (ids[1] == -1).all() and (w[1] == 0).all()
    assert np.allclose(w[0], 2.5 / 4, rtol=0, atol=1e-15)


def test_sigmoid_silu_identities():
    g = np.linspace(-30, 30, 2001)
    assert np.allclose(oracle.sigmoid(g), expit(g), rtol=1e-15, atol=1e-300)
    # silu(g) - silu(-g) == g ; silu(0) == 0 ; silu(g) -> g for large g
    assert np.allclose(oracle.silu(g) - oracle.silu(-g), g, rtol=1e-14, atol=1e-14)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert oracle.silu(np.array([-800.0]))[0] == 0.0


# ---------------------------------------------------------------- union

def test_union_brute_force():
    rng = np.random.default_rng(4)
    m, k, e = 11, 3, 20
    ids = np.stack([np.sort(rng.choice(e, k, replace=False)) for _ in range(m)]).astype(np.int32)
    mask = np.ones(m, np.uint8)
    mask[[3, 8]] = 0
    ids[[3, 8]] = -1
    rt = oracle.union(ids, np.zeros((m, k)), mask)
    real = [r for r in range(m) if mask[r]]
    assert list(rt.union_ids) == sorted({int(x) for r in real for x in ids[r]})
    assert rt.offs[0] == 0 and rt.offs[-1] == len(real) * k
    for u, ex in enumerate(rt.union_ids):
        got = list(rt.rows[rt.offs[u]:rt.offs[u + 1]])
        assert got == [r for r in real if ex in ids[r]]
    for r in real:
        for j in range(k):
            s = rt.slot_of[r, j]
            assert rt.rows[s] == r
            u = np.searchsorted(rt.offs, s, side="right") - 1
            assert rt.union_ids[u] == ids[r, j]
    assert (rt.slot_of[[3, 8]] == -1).all()


# ---------------------------------------------------------------- block GEMM

def _rand_codes(rng, shape):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return rng.choice(finite, size=shape).astype(np.uint8)


def test_block_gemm_vs_dequantized_matmul():
    rng = np.random.default_rng(8)
    m, n, k = 5, 256, 384
    a = _rand_codes(rng, (m, k))
    w = _rand_codes(rng, (n, k))
    sa = np.exp(rng.uniform(-5, 5, (m, k // 128))).astype(np.float32)
    sw = np.exp(rng.uniform(-5, 5, (n // 128, k // 128))).astype(np.float32)
    got = oracle.block_gemm(a, sa, w, sw)
    ad = decode_e4m3(a) * np.repeat(sa.astype(np.float64), 128, axis=1)
    wd = decode_e4m3(w) * np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)
    want = ad @ wd.T
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_block_gemm_inner_sums_exact():
    """With unit scales the result equals exact integer arithmetic."""
    rng = np.random.default_rng(9)
    m, n, k = 3, 128, 256
    a = _rand_codes(rng, (m, k))
    w = _rand_codes(rng, (n, k))
    ones_a = np.ones((m, k // 128), np.float32)
    ones_w = np.ones((n // 128, k // 128), np.float32)
    got = oracle.block_gemm(a, ones_a, w, ones_w)
    ai = (decode_e4m3(a) * 512).astype(np.int64)      # every e4m3 value is a multiple of 2^-9
    wi = (decode_e4m3(w) * 512).astype(np.int64)
    for i in range(m):
        for j in range(0, n, 17):
            exact = sum(int(ai[i, h]) * int(wi[j, h]) for h in range(k))
            assert got[i, j] == exact / 2 ** 18
