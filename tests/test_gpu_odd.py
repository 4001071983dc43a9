"""GPU parity on an edge-shape layer: hidden 640 (not a multiple of 256 or
512: the float64 logit chunks end part-way, the 256-column down tiles end
part-way), 40 experts (not a multiple of 64: top-k lanes and union words
partly empty), top-6, inter 384 (three 128-blocks), a one-block shared
expert.  Both execution paths: an 8-row step (split) and a 150-row step
(tiled) that carries the same 8 rows first."""
import dataclasses

import numpy as np
import pytest
import torch

import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import (GpuLayer, assert_routing_equal, assert_y_close, compare_h_codes, run_layer, run_oracle,
                      say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def odd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()
    cfg = synth.CONFIGS["odd"]
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    x, mask = synth.activations(cfg)
    return cfg, gl, x, mask


def _check(gl, x, mask):
    g = run_layer(gl, x, mask)
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    real = mask != 0
    assert np.array_equal(g["x_codes"][real], o.x_codes[real])
    assert np.array_equal(g["x_scales"][real], o.x_scales[real])
    bad, n = compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    assert not g["y"][~real].any()
    return g, err, bad, n


def test_odd_split_step(odd):
    cfg, gl, x, mask = odd
    say("odd layer M=8 (split)")
    _, err, bad, n = _check(gl, x, mask)
    say(f"odd split: max row rel err {err:.3e}, h code flips {bad}/{n}")


def test_odd_tiled_step_and_row_identity(odd):
    cfg, gl, x, mask = odd
    m = 150
    rng = np.random.default_rng(77)
    xl = synth.to_bf16_bits(rng.standard_normal((m, cfg.dims.hidden)).astype(np.float32))
    ml = np.ones(m, np.uint8)
    xl[:8], ml[:8] = x, mask               # the 8-row step's rows first
    ml[100] = 0
    xl[100] = 0x7FC0
    say("odd layer M=150 (tiled)")
    g, err, bad, n = _check(gl, xl, ml)
    say(f"odd tiled: max row rel err {err:.3e}, h code flips {bad}/{n}")
    small = run_layer(gl, x, mask)
    assert np.array_equal(g["y"][:8], small["y"])
    assert np.array_equal(g["ids"][:8], small["ids"])


@pytest.fixture(scope="module")
def narrow():
    """The smallest legal hidden size, 128: one K-block, so the first of the
    two gate/up K segments is empty, and a one-block shared expert."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()
    base = synth.CONFIGS["odd"]
    cfg = dataclasses.replace(base, dims=dataclasses.replace(base.dims, hidden=128), seed=1007)
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    return cfg, gl


@pytest.mark.parametrize("m", [8, 20, 60])        # split, split with two row halves, tiled
def test_narrow_hidden(narrow, m):
    cfg, gl = narrow
    x, mask = synth.activations(synth.with_rows(cfg, m))
    mask = mask.copy()
    x = x.copy()
    mask[m // 2] = 0
    x[m // 2] = 0x7FC0
    say(f"hidden 128 layer M={m}")
    g, err, bad, n = _check(gl, x, mask)
    say(f"hidden 128 M={m}: max row rel err {err:.3e}, h code flips {bad}/{n}")
