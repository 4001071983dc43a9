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
