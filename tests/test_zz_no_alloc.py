"""moe_layer_static -- the layer entry point that allocates nothing (its
workspace is a static per-GPU array inside the library) -- against moe_layer
with a caller workspace: the same kernels, so the same bits.  Two calls in a
row, the second with fewer rows (the array keeps the first call's contents),
on the tiled and on the split path; and a step too large for the array is
refused."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import GpuLayer, np16, say, t8, t16

pytestmark = pytest.mark.gpu


def _run(gl, x, mask, static):
    d = gl.dims
    m = x.shape[0]
    y = torch.full((m, d.hidden), -1, dtype=torch.int16, device="cuda")
    rt = moe.Routing.empty(d, m)
    tp = moe.Taps.empty(d, m)
    xt, mk = t16(x), t8(mask)
    if static:
        moe.layer_static(d, xt, mk, gl.router_w, gl.bias, gl.experts, gl.shared, y, rt, tp)
    else:
        ws = moe.workspace(d, m)
        moe.layer(d, xt, mk, gl.router_w, gl.bias, gl.experts, gl.shared, y, rt, ws, tp)
    torch.cuda.synchronize()
    nu = int(rt.n_union.item())
    out = dict(y=np16(y), ids=rt.topk_ids.cpu().numpy(), w=rt.topk_w.cpu().numpy().view(np.uint32), nu=nu,
               union=rt.union_ids.cpu().numpy()[:nu], offs=rt.offs.cpu().numpy()[:nu + 1],
               slot_of=rt.slot_of.cpu().numpy(), xq=tp.x_codes.cpu().numpy(), xs=tp.x_scales.cpu().numpy())
    slots = int(out["offs"][-1]) if nu else 0
    out["rows"] = rt.rows.cpu().numpy()[:slots]
    out["hq"] = tp.h_codes.cpu().numpy()[:slots]
    out["hs"] = tp.h_scales.cpu().numpy()[:slots]
    return out


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_static_entry_point_matches_layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.CONFIGS["tiny"]
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    rng = np.random.default_rng(2024)
    big = synth.to_bf16_bits(rng.standard_normal((40, cfg.dims.hidden)).astype(np.float32))
    mbig = np.ones(40, np.uint8)
    mbig[[3, 17]] = 0
    big[[3, 17]] = 0x7FC0                         # pads, never read
    small, msmall = synth.activations(cfg)
    msmall = msmall.copy()
    msmall[5] = 0
    small = small.copy()
    small[5] = 0x7FC0
    for name, x, mask in (("40 rows (tiled)", big, mbig), ("8 rows (split)", small, msmall)):
        say(f"moe_layer_static: {name}")
        s = _run(gl, x, mask, static=True)
        r = _run(gl, x, mask, static=False)
        _same(s, r)
        assert not s["y"][mask == 0].any()
    # a step too large for the static array is refused before any launch
    d = gl.dims
    m = 16384
    assert moe.workspace_bytes(d, m) > moe.STATIC_WS_BYTES
    y = torch.empty((m, d.hidden), dtype=torch.int16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.layer_static(d, torch.zeros((m, d.hidden), dtype=torch.int16, device="cuda"), None, gl.router_w,
                         gl.bias, gl.experts, gl.shared, y, moe.Routing.empty(d, m))
    assert ei.value.status == moe.MOE_EWORKSPACE
