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


def tp8_shards(lay: synth.Layer, n: int = 8):
    """The n tensor-parallel shards of one layer: shard s holds every routed
    expert's inter columns [s I/n, (s+1) I/n) (gate/up rows, down columns, with
    their 128x128 scale blocks) and the shared expert's likewise; the router is
    every shard's."""
    d = lay.dims
    si, ss = d.inter // n, d.shared_inter // n
    bi, bs = si // 128, ss // 128
    out = []
    for s in range(n):
        ri, rs = slice(s * si, (s + 1) * si), slice(s * ss, (s + 1) * ss)
        sd = synth.Dims(d.hidden, d.n_experts, d.top_k, si, ss, d.routed_scale)
        c = np.ascontiguousarray
        out.append(synth.Layer(
            sd, lay.router_w, lay.bias,
            c(lay.w_gate[:, ri, :]), c(lay.w_up[:, ri, :]), c(lay.w_down[:, :, ri]),
            c(lay.s_gate[:, s * bi:(s + 1) * bi, :]), c(lay.s_up[:, s * bi:(s + 1) * bi, :]),
            c(lay.s_down[:, :, s * bi:(s + 1) * bi]),
            {"gate": c(lay.shared["gate"][rs, :]), "up": c(lay.shared["up"][rs, :]),
             "down": c(lay.shared["down"][:, rs])}))
    return out


def test_tp8_shards_fixed_order_partials():
    """One GLM layer (the span-8 seed) as its 8 TP8 shards (expert inter 2048 / 8
    per shard) run in turn on one GPU, their partial outputs written into a
    [row][src][H] region and summed in ascending source order
    (moe_sum_partials): within 2e-2 per row of the oracle's sum of the shards'
    float64 outputs, the sum itself bit-identical to the oracle's fixed-order sum
    of the same partials, pad rows zero, and the DP8 rows' bits unchanged when
    they ride in span slots beside other rows."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from gpu_util import np16, t16, t8
    cfg = synth.CONFIGS["span8"]
    say("tp8 shards: generating the GLM layer")
    shards = tp8_shards(synth.make_layer(cfg))
    gls = [GpuLayer(sh) for sh in shards]
    say("tp8 shards: uploaded")
    xs, ms = synth.activations(cfg)
    xd, md = synth.activations(synth.CONFIGS["dp8"])

    def run_tp8(x, mask):
        m = x.shape[0]
        parts = np.zeros((m, len(gls), cfg.dims.hidden), np.uint16)
        for s, gl in enumerate(gls):
            parts[:, s, :] = run_layer(gl, x, mask)["y"]
        y = torch.empty((m, cfg.dims.hidden), dtype=torch.int16, device="cuda")
        moe.sum_partials(t16(parts), t8(mask), y)
        torch.cuda.synchronize()
        return parts, np16(y)

    for name, x, mask in (("span8", xs, ms), ("dp8", xd, md)):
        parts, y = run_tp8(x, mask)
        assert np.array_equal(y, oracle.sum_partials(parts, mask)), f"{name}: fixed-order sum differs"
        real = np.flatnonzero(mask)
        ref = np.zeros((x.shape[0], cfg.dims.hidden))
        for sh in shards:
            o = oracle.layer(x, mask, sh.router_w, sh.bias, sh.dims.top_k, sh.dims.routed_scale,
                             lambda e, sh=sh: {"gate": sh.w_gate[e], "s_gate": sh.s_gate[e], "up": sh.w_up[e],
                                               "s_up": sh.s_up[e], "down": sh.w_down[e], "s_down": sh.s_down[e]},
                             sh.shared)
            ref[real] += o.y_ref[real]
        yd = oracle.decode_bf16(y[real])
        err = np.abs(yd - ref[real]).max(axis=1) / np.abs(ref[real]).max(axis=1)
        say(f"tp8 shards {name}: max row rel err {err.max():.3e}")
        assert (err <= 2e-2).all()
        assert not y[mask == 0].any()
        if name == "dp8":
            # the same real rows in span-style slots, span rows as companions
            placed = np.array([6, 0, 3, 7, 1])
            mix = xs.copy()
            mix[placed] = x[real]
            _, ymix = run_tp8(mix, np.ones(8, np.uint8))
            assert np.array_equal(ymix[placed], y[real])
