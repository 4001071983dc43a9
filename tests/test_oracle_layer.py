"""Whole-layer pins of the oracle on the tiny configuration (CPU only).

The reference here is a brute-force dense evaluation written without the
union, the row compaction or the per-block GEMM: the router by exhaustive
subset search with a library sigmoid, every expert on every row with library
float64 matmuls of dequantized matrices, and the combine masked by the top-k.
Planted mistakes in the oracle must make the comparison fail.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import oracle.moe_layer as OL
import synth
from oracle import decode_bf16, decode_e4m3


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    lay = synth.make_layer(cfg, threads=4)
    x, mask = synth.activations(cfg)
    return cfg, lay, x, mask


def _expert_fn(lay):
    def get(e):
        return {"gate": lay.w_gate[e], "s_gate": lay.s_gate[e], "up": lay.w_up[e], "s_up": lay.s_up[e],
                "down": lay.w_down[e], "s_down": lay.s_down[e]}
    return get


def run_oracle(cfg, lay, x, mask, rows=None):
    d = cfg.dims
    return oracle.layer(x, mask, lay.router_w, lay.bias, d.top_k, d.routed_scale, _expert_fn(lay),
                        lay.shared or None, rows=rows)


def _deq(codes, scales, bn=128, bk=128):
    s = np.repeat(np.repeat(scales.astype(np.float64), bn, axis=0), bk, axis=1)
    return decode_e4m3(codes) * s


def dense_reference(cfg, lay, x, mask):
    """Every expert on every real row, combined with the top-k mask."""
    d = cfg.dims
    real = np.flatnonzero(mask)
    xf = decode_bf16(x[real])
    l = xf @ decode_bf16(lay.router_w).T
    sig = expit(l)
    c = sig + lay.bias.astype(np.float64)
    sel = np.zeros((len(real), d.n_experts), bool)
    wfull = np.zeros((len(real), d.n_experts))
    for i in range(len(real)):
        best = max(itertools.combinations(range(d.n_experts), d.top_k),
                   key=lambda s: (sum(c[i, j] for j in s), [-j for j in s]))
        sel[i, list(best)] = True
        wfull[i, list(best)] = d.routed_scale * sig[i, list(best)] / sig[i, list(best)].sum()
    xq, xs = oracle.quant_1x128(xf.astype(np.float32))
    xd = decode_e4m3(xq) * np.repeat(xs.astype(np.float64), 128, axis=1)
    y = np.zeros((len(real), d.hidden))
    hcodes = {}
    for e in range(d.n_experts):                                   # ascending id
        g = xd @ _deq(lay.w_gate[e], lay.s_gate[e]).T
        u = xd @ _deq(lay.w_up[e], lay.s_up[e]).T
        h = (g * expit(g) * u).astype(np.float32)
        hq, hs = oracle.quant_1x128(h)
        dd = (decode_e4m3(hq) * np.repeat(hs.astype(np.float64), 128, axis=1)) @ _deq(lay.w_down[e], lay.s_down[e]).T
        for i in range(len(real)):
            if sel[i, e]:
                y[i] = y[i] + wfull[i, e] * dd[i]
                hcodes[(int(real[i]), e)] = hq[i]
    # shared expert via torch float64 and torch's bf16 cast
    xs64 = torch.from_numpy(xf)
    sg = torch.from_numpy(decode_bf16(lay.shared["gate"]))
    su = torch.from_numpy(decode_bf16(lay.shared["up"]))
    sd = torch.from_numpy(decode_bf16(lay.shared["down"]))
    gs = xs64 @ sg.T
    us = xs64 @ su.T
    hs_ = (torch.nn.functional.silu(gs) * us).float().to(torch.bfloat16).double()
    y = y + (hs_ @ sd.T).numpy()
    return real, sel, y, hcodes


def _matches_dense(cfg, lay, x, mask, out):
    real, sel, y, hcodes = dense_reference(cfg, lay, x, mask)
    for i, r in enumerate(real):
        got = np.zeros(cfg.dims.n_experts, bool)
        got[out.routing.ids[r]] = True
        if not np.array_equal(got, sel[i]):
            return False
        ref = out.y_ref[r]
        if np.abs(ref - y[i]).max() > 1e-9 * np.abs(y[i]).max():
            return False
    return True


def test_layer_equals_dense_brute_force(tiny):
    cfg, lay, x, mask = tiny
    out = run_oracle(cfg, lay, x, mask)
    real, sel, y, hcodes = dense_reference(cfg, lay, x, mask)
    for i, r in enumerate(real):
        assert set(out.routing.ids[r]) == set(np.flatnonzero(sel[i]))
        scale = np.abs(y[i]).max()
        assert np.abs(out.y_ref[r] - y[i]).max() <= 1e-9 * scale
        for j, e in enumerate(out.routing.ids[r]):
            s = out.routing.slot_of[r, j]
            assert np.array_equal(out.h_codes[s], hcodes[(int(r), int(e))])
    ybits = oracle.encode_bf16(y)
    assert np.array_equal(out.y_bits[real], ybits)


def test_layer_dense_pin_catches_planted_mistakes(tiny, monkeypatch):
    cfg, lay, x, mask = tiny
    assert _matches_dense(cfg, lay, x, mask, run_oracle(cfg, lay, x, mask))

    real_route = OL.route

    def route_without_bias(xb, m, wr, b, k, sc=2.5):
        return real_route(xb, m, wr, np.zeros_like(b), k, sc)

    mistakes = {
        "selection ignores the correction bias": ("route", route_without_bias),
        "first K-block scale reused for every block": (
            "block_gemm", lambda a, sa, w, sw: oracle.block_gemm(
                a, np.repeat(sa[:, :1], sa.shape[1], 1), w, np.repeat(sw[:, :1], sw.shape[1], 1))),
        "sign error in SiLU": ("silu", lambda g: np.asarray(g, np.float64) / (1.0 + np.exp(np.asarray(g, np.float64)))),
        "shared expert dropped": ("shared_expert", lambda xb, sw: np.zeros((xb.shape[0], xb.shape[1]))),
        "up projection uses gate weights": (
            "routed_expert", lambda xq, xs, ew: oracle.routed_expert(xq, xs, dict(ew, up=ew["gate"], s_up=ew["s_gate"]))),
    }
    for name, (attr, fn) in mistakes.items():
        with monkeypatch.context() as mp:
            mp.setattr(OL, attr, fn)
            out = run_oracle(cfg, lay, x, mask)
        assert not _matches_dense(cfg, lay, x, mask, out), name


def test_invariant_row_permutation(tiny):
    cfg, lay, x, mask = tiny
    base = run_oracle(cfg, lay, x, mask)
    perm = np.array([5, 2, 7, 0, 3, 6, 1, 4])
    out = run_oracle(cfg, lay, x[perm], mask[perm])
    assert np.array_equal(out.y_bits, base.y_bits[perm])
    assert np.array_equal(out.routing.ids, base.routing.ids[perm])


def test_invariant_companion_rows_and_nan_pads(tiny):
    cfg, lay, x, mask = tiny
    base = run_oracle(cfg, lay, x, mask)
    x2 = x.copy()
    rng = np.random.default_rng(99)
    x2[[1, 4]] = synth.to_bf16_bits(rng.standard_normal((2, x.shape[1])).astype(np.float32))
    m2 = mask.copy()
    m2[[2, 6]] = 0
    x2[[2, 6]] = 0x7FC0                                # NaN-poisoned pads
    out = run_oracle(cfg, lay, x2, m2)
    for r in (0, 3, 5, 7):
        assert np.array_equal(out.y_bits[r], base.y_bits[r])
    assert not out.y_bits[[2, 6]].any()
    assert (out.routing.ids[[2, 6]] == -1).all()


def test_invariant_repeat_and_row_subset(tiny):
    cfg, lay, x, mask = tiny
    a = run_oracle(cfg, lay, x, mask)
    b = run_oracle(cfg, lay, x, mask)
    assert np.array_equal(a.y_bits, b.y_bits)
    c = run_oracle(cfg, lay, x, mask, rows=[3])
    assert np.array_equal(c.y_bits[3], a.y_bits[3])


def test_all_rows_pad():
    cfg = synth.CONFIGS["tiny"]
    lay = synth.make_layer(cfg, threads=2)
    x, _ = synth.activations(cfg)
    mask = np.zeros(8, np.uint8)
    out = run_oracle(cfg, lay, x, mask)
    assert out.routing.n_union == 0
    assert not out.y_bits.any()
