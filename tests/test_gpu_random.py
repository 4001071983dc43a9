"""Randomized parity sweep: seeded draws of small layer shapes (hidden,
expert count, top-k, expert and shared-expert widths), step sizes on both
sides of every path switch (split small steps, tiled steps, the all-float64
and the certified router), row recipes, pad patterns and router biases.
Every row is compared with the oracle: routing, union and x codes bit for
bit, h codes within the MFMA error interval, y within the layer tolerance."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import (GpuLayer, assert_routing_equal, assert_y_close, compare_h_codes, run_layer, run_oracle,
                      say)

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([8, 16, 40, 64, 256, 256]))
        H = int(rng.choice([128, 256, 384, 640] if E == 256 else [128, 256, 384, 640, 1024]))
        I = int(rng.choice([128, 256] if E == 256 else [128, 256, 384, 512]))
        K = int(rng.choice([k for k in (1, 2, 4, 6, 8) if k <= E]))
        Is = int(rng.choice([0, 128, 256]))
        M = int(rng.choice([1, 2, 5, 8, 13, 16, 17, 24, 25, 40, 129, 600, 700]))
        pads = tuple(int(p) for p in np.flatnonzero(rng.random(M) < 0.2)) if M > 1 else ()
        if len(pads) == M:
            pads = pads[1:]
        kind = "span" if rng.random() < 0.3 else "iid"
        bias = "zipf" if rng.random() < 0.3 else "normal"
        d = synth.Dims(hidden=H, n_experts=E, top_k=K, inter=I, shared_inter=Is)
        out.append(synth.Config(f"rand{i}", d, M, 3000 + i, row_kind=kind, pad_slots=pads, bias_kind=bias))
    return out


CASES = _cases()


@pytest.mark.parametrize("cfg", CASES, ids=[f"{c.name}-H{c.dims.hidden}-E{c.dims.n_experts}-k{c.dims.top_k}"
                                            f"-I{c.dims.inter}-S{c.dims.shared_inter}-M{c.rows}" for c in CASES])
def test_random_shape_parity(cfg):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()
    say(f"random case {cfg.name}: dims {cfg.dims} M={cfg.rows} pads={len(cfg.pad_slots)} {cfg.row_kind} "
        f"{cfg.bias_kind}")
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    x, mask = synth.activations(cfg)
    g = run_layer(gl, x, mask)
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    real = mask != 0
    assert np.array_equal(g["x_codes"][real], o.x_codes[real])
    assert np.array_equal(g["x_scales"][real], o.x_scales[real])
    bad, n = compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    assert (g["y"][~real] == 0).all()
    say(f"  |U|={g['n_union']} max row rel err {err:.3e} h flips {bad}/{n}")
