"""moe_route on its own (both routing paths: the small-step logits +
select/union kernels for M <= 32 and the large-step logits, top-k and
chunked-union kernels above) against the oracle's routing, and against the
routing that moe_layer writes for the same rows (one per-logit procedure)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import GpuLayer, assert_routing_equal, run_layer, say, t16, t8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layers():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()
    out = {}
    for name in ("tiny", "odd"):
        cfg = synth.CONFIGS[name]
        out[name] = (cfg, GpuLayer(synth.make_layer(cfg, threads=4)))
    return out


def _route(gl, x_bits, mask):
    m = x_bits.shape[0]
    d = gl.dims
    ws = moe.workspace(d, m)
    rt = moe.Routing.empty(d, m)
    for t in (rt.topk_ids, rt.union_ids, rt.offs, rt.rows, rt.slot_of, rt.n_union):
        t.fill_(-7)
    moe.route(d, t16(x_bits), t8(mask), gl.router_w, gl.bias, rt, ws)
    torch.cuda.synchronize()
    return dict(ids=rt.topk_ids.cpu().numpy(), w=rt.topk_w.cpu().numpy(), n_union=int(rt.n_union.item()),
                union_ids=rt.union_ids.cpu().numpy()[:int(rt.n_union.item())],
                offs=rt.offs.cpu().numpy()[:int(rt.n_union.item()) + 1], rows=rt.rows.cpu().numpy(),
                slot_of=rt.slot_of.cpu().numpy())


@pytest.mark.parametrize("name", ["tiny", "odd"])
@pytest.mark.parametrize("m", [1, 6, 16, 17, 32, 33, 90])
def test_route_matches_oracle_and_layer(layers, name, m):
    cfg, gl = layers[name]
    d = cfg.dims
    rng = np.random.default_rng(500 + m)
    x = synth.to_bf16_bits(rng.standard_normal((m, d.hidden)).astype(np.float32))
    mask = np.ones(m, np.uint8)
    if m > 2:
        mask[m // 3] = 0
        x[m // 3] = 0x7FC0                  # pad rows are never read
    say(f"route {name} M={m}")
    g = _route(gl, x, mask)
    ids, w, _ = oracle.route(x, mask, gl.host.router_w, gl.host.bias, d.top_k, d.routed_scale)
    o = oracle.union(ids, w, mask)
    assert_routing_equal(g, o, mask)
    lay = run_layer(gl, x, mask)
    for k in ("ids", "w", "slot_of"):
        assert np.array_equal(g[k], lay[k]), k
    assert g["n_union"] == lay["n_union"]
    assert np.array_equal(g["union_ids"], lay["union_ids"])
