"""moe_layer captured into a HIP graph: every replay, with eager work and
synchronizations between replays and new inputs copied into the captured
buffers, matches the eager result bit for bit."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import GpuLayer, np16, say, t16, t8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [8, 40])
def test_graph_replays_match_eager(m):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.CONFIGS["tiny"]
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    d = gl.dims
    rng = np.random.default_rng(m)
    inputs = [synth.to_bf16_bits(rng.standard_normal((m, d.hidden)).astype(np.float32)) for _ in range(4)]
    masks = [np.ones(m, np.uint8) for _ in range(4)]
    masks[2][[1, m - 1]] = 0
    say(f"graph M={m}")
    x = torch.zeros((m, d.hidden), dtype=torch.int16, device="cuda")
    mk = torch.ones(m, dtype=torch.uint8, device="cuda")
    y = torch.zeros((m, d.hidden), dtype=torch.int16, device="cuda")
    rt = moe.Routing.empty(d, m)
    ws = moe.workspace(d, m)

    def call():
        moe.layer(d, x, mk, gl.router_w, gl.bias, gl.experts, gl.shared, y, rt, ws)

    eager = []
    for xi, mi in zip(inputs, masks):
        x.copy_(t16(xi))
        mk.copy_(t8(mi))
        call()
        torch.cuda.synchronize()
        eager.append(np16(y).copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for i, (xi, mi) in enumerate(zip(inputs, masks)):
            x.copy_(t16(xi))
            mk.copy_(t8(mi))
            y.fill_(-1)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(np16(y), eager[i]), f"replay {rep} input {i} differs"
            # eager work between replays
            call()
            torch.cuda.synchronize()
            assert np.array_equal(np16(y), eager[i])


@pytest.mark.parametrize("m", [8, 40])
def test_graph_fused_norm_replays_match_eager(m):
    """moe_layer_add_rmsnorm (fused epilogue) and moe_layer + moe_add_rmsnorm
    captured into graphs: every replay equals the eager outputs (y, r_new, out)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.CONFIGS["tiny"]
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    d = gl.dims
    rng = np.random.default_rng(100 + m)
    inputs = [synth.to_bf16_bits(rng.standard_normal((m, d.hidden)).astype(np.float32)) for _ in range(3)]
    res_np, gam_np = synth.norm_inputs(cfg, rows=m)
    say(f"graph fused norm M={m}")
    x = torch.zeros((m, d.hidden), dtype=torch.int16, device="cuda")
    mk = torch.ones(m, dtype=torch.uint8, device="cuda")
    mk[m // 2] = 0
    res, gam = t16(res_np), t16(gam_np)
    y = torch.zeros((m, d.hidden), dtype=torch.int16, device="cuda")
    r_out = torch.zeros_like(y)
    out = torch.zeros_like(y)
    rt = moe.Routing.empty(d, m)
    ws = moe.workspace(d, m)

    def fused():
        moe.layer_add_rmsnorm(d, x, mk, gl.router_w, gl.bias, gl.experts, gl.shared, res, gam, 1e-6, y, r_out, out,
                              rt, ws)

    def unfused():
        moe.layer(d, x, mk, gl.router_w, gl.bias, gl.experts, gl.shared, y, rt, ws)
        moe.add_rmsnorm(y, mk, res, gam, 1e-6, r_out, out)

    def snap():
        return np16(y).copy(), np16(r_out).copy(), np16(out).copy()

    for call in (fused, unfused):
        eager = []
        for xi in inputs:
            x.copy_(t16(xi))
            call()
            torch.cuda.synchronize()
            eager.append(snap())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        for rep in range(3):
            for i, xi in enumerate(inputs):
                x.copy_(t16(xi))
                y.fill_(-1)
                r_out.fill_(-1)
                out.fill_(-1)
                g.replay()
                torch.cuda.synchronize()
                got = snap()
                assert all(np.array_equal(a, b) for a, b in zip(got, eager[i])), \
                    f"{call.__name__} replay {rep} input {i} differs"
                call()                                    # eager work between replays
                torch.cuda.synchronize()
        del g
