"""The certified selection of larger steps (more than 512 rows: MFMA
estimates with an error bound, float64 logits only for the candidates) gives
the ids and weights of the all-float64 selection bit for bit.

Inputs are built on the host to sit where an estimate could mislead: router
rows that are exact or one-ulp copies of each other (scores tied or nearly
tied at the k-th place, with equal biases), rows with a wide dynamic range,
rows that saturate the sigmoid (ties at 0 and 1), zero rows, rows that
cancel (large sum |x| |w| against a small logit), rows holding an infinity
(the non-finite path), and pad rows poisoned with NaN.  The same rows are
routed once as one step (certified path) and again in 128-row steps (every
logit in float64); ids and fp32 weights must match exactly, and the finite
rows must also match the oracle (ids exactly, weights within one fp32
rounding).  Three independent draws of the 256 rows below make one
768-row step.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_02_amd as moe
from gpu_util import say

pytestmark = pytest.mark.gpu

DIMS = {"tiny": (512, 16, 4), "odd": (640, 40, 6), "glm": (6144, 256, 8)}


def bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def router(h, e, rng):
    w = bf16(rng.standard_normal((e, h)) / np.sqrt(h))
    b = (rng.standard_normal(e) * 0.01).astype(np.float32)
    for j in range(e):
        if j % 4 == 1:                      # one-ulp copy of the previous expert
            w[j] = w[j - 1]
            k = rng.integers(h)
            w[j, k] = w[j - 1, k] + (1 if w[j - 1, k] & 0x7F80 else 0)
            b[j] = b[j - 1]
        elif j % 4 == 2:                    # exact copy of expert j - 2
            w[j] = w[j - 2]
            b[j] = b[j - 2]
    return w, b


def rows(h, wr, rng):
    blocks = []
    blocks.append(rng.standard_normal((64, h)))                                       # plain
    blocks.append(rng.standard_normal((64, h)) * np.exp2(rng.integers(-8, 9, (64, h))))   # wide range
    blocks.append(rng.standard_normal((32, h)) * 64.0)                                # saturated sigmoid
    blocks.append(np.zeros((32, h)))                                                  # zero rows
    w0 = oracle.decode_bf16(wr[0])
    r = rng.standard_normal((32, h)) * 50.0
    r -= np.outer(r @ w0 / (w0 @ w0), w0)                                             # cancels against expert 0
    blocks.append(r)
    inf = rng.standard_normal((16, h))
    inf[np.arange(16), rng.integers(h, size=16)] = np.inf                             # non-finite rows
    blocks.append(inf)
    blocks.append(np.zeros((16, h)))                                                  # pads (NaN bits below)
    x = bf16(np.concatenate(blocks))
    mask = np.ones(x.shape[0], np.uint8)
    mask[-16:] = 0
    x[-16:] = 0x7FC0
    finite = np.ones(x.shape[0], bool)
    finite[224:240] = False
    return x, mask, finite


def route(d, x, mask, wr, b, split=None):
    m = x.shape[0]
    parts = [(0, m)] if split is None else [(s, min(s + split, m)) for s in range(0, m, split)]
    ids, w = [], []
    for lo, hi in parts:
        rt = moe.Routing.empty(d, hi - lo)
        moe.route(d, torch.from_numpy(x[lo:hi].view(np.int16)).cuda(), torch.from_numpy(mask[lo:hi]).cuda(),
                  torch.from_numpy(wr.view(np.int16)).cuda(), torch.from_numpy(b).cuda(), rt, moe.workspace(d, hi - lo))
        torch.cuda.synchronize()
        ids.append(rt.topk_ids.cpu().numpy())
        w.append(rt.topk_w.cpu().numpy())
    return np.concatenate(ids), np.concatenate(w)


@pytest.mark.parametrize("name", list(DIMS))
def test_certified_selection_equals_float64_selection(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h, e, k = DIMS[name]
    rng = np.random.default_rng(4242 + h)
    d = moe.Dims(h, e, k, 256, 0)
    wr, b = router(h, e, rng)
    parts = [rows(h, wr, rng) for _ in range(3)]           # 768 rows: the certified path
    x = np.concatenate([p[0] for p in parts])
    mask = np.concatenate([p[1] for p in parts])
    finite = np.concatenate([p[2] for p in parts])
    say(f"certified routing {name}: M={x.shape[0]} H={h} E={e} k={k}")
    ids_c, w_c = route(d, x, mask, wr, b)
    ids_f, w_f = route(d, x, mask, wr, b, split=128)
    assert np.array_equal(ids_c, ids_f)
    assert np.array_equal(w_c.view(np.int32), w_f.view(np.int32))
    keep = finite & (mask != 0)
    o_ids, o_w, _ = oracle.route(x[keep], np.ones(keep.sum(), np.uint8), wr, b, k)
    assert np.array_equal(ids_c[keep], o_ids)
    ref = o_w.astype(np.float32)
    assert np.all(np.abs(w_c[keep].astype(np.float64) - o_w) <= np.spacing(np.abs(ref)).astype(np.float64))
    # the constructed ties really sit at the decision: some rows pick one expert of a tied pair only
    split_pairs = sum(1 for r in ids_c[keep] for j in range(0, e - 2, 4) if (j in r) != (j + 2 in r))
    say(f"  rows x tied pairs split by the k-th place: {split_pairs}")
    assert (ids_c[mask == 0] == -1).all()
