"""GPU parity at the full GLM-5.2 layer size (H=6144, 256 experts top-8,
I=2048, shared I=2048), in the launch configuration the benchmark times.

Routing, union, compaction and x codes are compared bit-exactly on every row.
Output rows and h codes are compared on every row for the 8-row steps and, for
the prefill chunks, on rows chosen to cover every union expert and every tile
position class (the oracle evaluates a row from its experts alone, so a
sample is exact for that row).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_02_amd as moe
import synth
from prefetch_util import expected_checksum, prefetch_checksum
from gpu_util import (GpuLayer, assert_routing_equal, assert_y_close, compare_h_codes, cover_rows, np16,
                      rescale_rows, run_layer, run_oracle, say, t16)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

_cache = {}


def glm_layer(name):
    cfg = synth.CONFIGS[name]
    key = (cfg.seed, 0)
    if key not in _cache:
        if not torch.cuda.is_available():
            pytest.skip("no GPU")
        _cache.clear()
        torch.cuda.empty_cache()
        say(f"generating layer seed={cfg.seed}")
        _cache[key] = GpuLayer(synth.make_layer(cfg))
        say("layer ready")
    return cfg, _cache[key]


def test_span8_decode_step():
    cfg, gl = glm_layer("span8")
    x, mask = synth.activations(cfg)
    say("span8: M=8, all rows real")
    g = run_layer(gl, x, mask)
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    assert np.array_equal(g["x_codes"], o.x_codes) and np.array_equal(g["x_scales"], o.x_scales)
    bad, n = compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    say(f"span8: |U|={g['n_union']}, max row rel err {err:.3e}, h flips {bad}/{n}")


def test_span8_route_ahead_prefetch_reads_the_union():
    """At full size, in the grid the benchmark uses: the prefetch of a routed
    span-8 union reads exactly those experts' packed gate/up (and down)
    bytes, capped as asked, checked through its word-sum checksum."""
    cfg, gl = glm_layer("span8")
    x, mask = synth.activations(cfg)
    d = gl.dims
    rt = moe.Routing.empty(d, cfg.rows)
    moe.route(d, t16(x), torch.from_numpy(mask).cuda(), gl.router_w, gl.bias, rt, moe.workspace(d, cfg.rows))
    torch.cuda.synchronize()
    ids = [int(e) for e in rt.union_ids[:int(rt.n_union.item())].cpu()]
    say(f"span8 prefetch: |U|={len(ids)}")
    both = moe.PREFETCH_GATE_UP | moe.PREFETCH_DOWN
    for parts, cap, wg in ((moe.PREFETCH_GATE_UP, 1 << 40, 256), (moe.PREFETCH_GATE_UP, 128 << 20, 64),
                           (both, 300 << 20, 0)):
        got = prefetch_checksum(d, rt.n_union, rt.union_ids, gl.experts, parts, cap, wg)
        assert got == expected_checksum(gl.experts, ids, parts, cap, d.n_experts), (parts, cap, wg)


def test_dp8_decode_step_pads_and_placement():
    cfg, gl = glm_layer("dp8")
    x, mask = synth.activations(cfg, pad_fill="nan")
    xz, _ = synth.activations(cfg, pad_fill="zero")
    say("dp8: M=8, pads at", cfg.pad_slots)
    g = run_layer(gl, x, mask)
    gz = run_layer(gl, xz, mask)
    assert np.array_equal(g["y"], gz["y"])
    assert not g["y"][list(cfg.pad_slots)].any()
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    say(f"dp8: |U|={g['n_union']}, max row rel err {err:.3e}")
    # the same real rows carried in span-style slots of another step, with
    # span rows as companions, keep their bits
    xs, _ = synth.activations(synth.CONFIGS["span8"])
    real = np.flatnonzero(mask)
    placed = np.array([6, 0, 3, 7, 1])
    mix = xs.copy()
    mix[placed] = x[real]
    h = run_layer(gl, mix, np.ones(8, np.uint8))
    assert np.array_equal(h["y"][placed], g["y"][real])


def test_prefill512_chunk():
    cfg, gl = glm_layer("prefill512")
    glz = gl.with_bias(synth.router_bias(cfg))          # Zipf-skewed bias, same expert weights
    x, mask = synth.activations(cfg)
    say("prefill512: M=512")
    g = run_layer(glz, x, mask)
    sample = cover_rows(g["offs"], g["rows"], extra=(0, 1, 255, 511))
    say(f"prefill512: oracle on {len(sample)} rows covering all {g['n_union']} union experts")
    o = run_oracle(glz, x, mask, rows=sample)
    assert_routing_equal(g, o.routing, mask)
    assert np.array_equal(g["x_codes"], o.x_codes) and np.array_equal(g["x_scales"], o.x_scales)
    compare_h_codes(g["h_codes"], g["h_scales"], o, glz)
    err = assert_y_close(g["y"], o, rows=sample)
    loads = np.diff(o.routing.offs)
    say(f"prefill512: |U|={g['n_union']}, loads min/mean/max {loads.min()}/{loads.mean():.1f}/{loads.max()}, "
        f"sampled max row rel err {err:.3e}")
    # the sampled rows equal the same rows run as an 8-row decode step
    pick = [0, 1, 255, 511, 2, 3, 4, 5]
    d = run_layer(glz, x[pick], mask[pick])
    assert np.array_equal(d["y"][:4], g["y"][[0, 1, 255, 511]])
    # a repeat gives the same bits everywhere (no read of unsettled or racing data)
    g2 = run_layer(glz, x, mask)
    assert np.array_equal(g2["y"], g["y"]) and np.array_equal(g2["h_codes"], g["h_codes"])


def test_prefill4096_chain_of_4_layers():
    """The 4096-token chunk through 4 stacked layers with independent seeded
    weights: layer l + 1 takes layer l's GPU output rescaled per row to unit
    RMS.  Each layer is compared with the oracle run on the GPU's own input to
    that layer: routing, union and x codes on every row; y and h codes on rows
    covering every union expert and tile position class."""
    cfg = synth.CONFIGS["prefill4096x4"]
    x, mask = synth.activations(cfg, layer=0)
    for l in range(cfg.n_layers):
        _cache.clear()
        torch.cuda.empty_cache()
        say(f"prefill4096 layer {l}: generating weights")
        gl = GpuLayer(synth.make_layer(cfg, layer=l))
        g = run_layer(gl, x, mask)
        sample = cover_rows(g["offs"], g["rows"], extra=(7, 2048, 4095))
        say(f"prefill4096 layer {l}: |U|={g['n_union']}, oracle on {len(sample)} rows")
        o = run_oracle(gl, x, mask, rows=sample)
        assert_routing_equal(g, o.routing, mask)
        assert np.array_equal(g["x_codes"], o.x_codes) and np.array_equal(g["x_scales"], o.x_scales)
        compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
        err = assert_y_close(g["y"], o, rows=sample)
        loads = np.diff(o.routing.offs)
        say(f"prefill4096 layer {l}: sampled max row rel err {err:.3e}, expert rows max {loads.max()}")
        del gl
        if l + 1 < cfg.n_layers:
            yb = t16(g["y"])
            xn = np16(rescale_rows(yb))
            # the link itself: r_new is y, out is y at unit RMS (oracle in float64, bf16 rounding + fp32 sums)
            r_new, ref = oracle.add_rmsnorm(g["y"], np.zeros_like(g["y"]), np.full(g["y"].shape[1], 0x3F80, np.uint16),
                                            1e-6, mask)
            assert np.array_equal(r_new, np.where(g["y"] == 0x8000, 0, g["y"]))
            got = oracle.decode_bf16(xn)
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
            rms = np.sqrt(np.mean(got * got, axis=1))
            assert np.all(np.abs(rms - 1.0) < 1e-2)
            x = xn


def test_span8_and_dp8_steps_share_a_workspace():
    """The span-8 and the DP8 step (different unions) alternate on one
    workspace, as consecutive decode steps do; each equals its own fresh run."""
    cfg, gl = glm_layer("span8")
    xs, ms = synth.activations(cfg)
    xd, md = synth.activations(synth.CONFIGS["dp8"])
    ref = {"s": run_layer(gl, xs, ms)["y"], "d": run_layer(gl, xd, md)["y"]}
    d = gl.dims
    ws = moe.workspace(d, 8)
    rt = moe.Routing.empty(d, 8)
    y = torch.empty((8, d.hidden), dtype=torch.int16, device="cuda")
    for k, x, mk in (("s", xs, ms), ("d", xd, md), ("s", xs, ms), ("d", xd, md)):
        moe.layer(d, t16(x), torch.from_numpy(mk).cuda(), gl.router_w, gl.bias, gl.experts, gl.shared, y, rt, ws)
        torch.cuda.synchronize()
        assert np.array_equal(np16(y), ref[k]), k
