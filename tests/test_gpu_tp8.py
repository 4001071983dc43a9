"""GPU parity at one TP8 rank's share of the GLM layer (hidden 6144, 256
experts top-8, expert inter 256 = 2048 / 8, shared inter 256), the shape of
the rank-share token sweep: span-decode rows at 1 and 10 tokens (small-step
path) and 20 tokens (tiled path), against the oracle, and each step's first
row bit-identical to the 1-token step."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import (GpuLayer, assert_routing_equal, assert_y_close, compare_h_codes, run_layer, run_oracle,
                      say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rank_layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()
    cfg = synth.CONFIGS["tp8rank"]
    return cfg, GpuLayer(synth.make_layer(cfg, threads=8))


@pytest.mark.parametrize("m", [1, 10, 20])
def test_tp8_rank_share(rank_layer, m):
    cfg, gl = rank_layer
    x, mask = synth.activations(synth.with_rows(cfg, m))
    say(f"tp8 rank share M={m}")
    g = run_layer(gl, x, mask)
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    assert np.array_equal(g["x_codes"], o.x_codes)
    bad, n = compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    say(f"tp8 rank M={m}: |U|={g['n_union']}, max row rel err {err:.3e}, h code flips {bad}/{n}")
    if m > 1:
        one = run_layer(gl, x[:1], mask[:1])
        assert np.array_equal(g["y"][:1], one["y"])
