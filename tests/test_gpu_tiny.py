"""GPU parity of the HIP path against the CPU oracle on the tiny layer
(H=512, 16 experts top-4, I=256, shared I=256) and on ragged / edge row
counts.  Every call goes through the C ABI (libmoe_ffn.so)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_02_amd as moe
import synth
from gpu_util import (GpuLayer, assert_routing_equal, assert_y_close, compare_h_codes, run_ffn, run_layer,
                      run_oracle, say, t8, t16, tf)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()
    cfg = synth.CONFIGS["tiny"]
    gl = GpuLayer(synth.make_layer(cfg, threads=4))
    x, mask = synth.activations(cfg)
    return cfg, gl, x, mask


def _rows(cfg, m, seed):
    rng = np.random.default_rng(seed)
    return synth.to_bf16_bits(rng.standard_normal((m, cfg.dims.hidden)).astype(np.float32))


def test_quant_unit_bit_exact():
    """moe_quant_fp8 on fp32 values spanning every e4m3 regime equals the oracle rule."""
    rng = np.random.default_rng(21)
    r, c = 64, 1024
    v = (rng.standard_normal((r, c)) * np.exp(rng.uniform(-20, 20, (r, 1)))).astype(np.float32)
    v[3, :128] = 0.0                      # zero block
    v[4, 128:256] = -0.0
    v[5, :] = np.where(rng.random(c) < 0.5, 0.0, v[5, :])
    # blocks of exact e4m3 values x power-of-two scales, including midpoints
    finite = np.array([x for x in range(256) if x not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(8, c)).astype(np.uint8)
    codes[:, ::128] = 0x7E
    v[8:16] = (oracle.decode_e4m3(codes) * 2.0 ** -7).astype(np.float32)
    mids = (oracle.E4M3_TABLE[1:0x7E] + oracle.E4M3_TABLE[2:0x7F]) / 2
    v[16, :mids.size] = mids.astype(np.float32)
    v[16, 127] = 448.0
    say("quant unit", v.shape)
    gc = torch.empty((r, c), dtype=torch.uint8, device="cuda")
    gs = torch.empty((r, c // 128), dtype=torch.float32, device="cuda")
    moe.quant_fp8(tf(v), gc, gs)
    torch.cuda.synchronize()
    oc, os_ = oracle.quant_1x128(v)
    assert np.array_equal(gs.cpu().numpy(), os_)
    assert np.array_equal(gc.cpu().numpy(), oc)
    # bf16 input path
    xb = synth.to_bf16_bits(v)
    moe.quant_fp8(t16(xb), gc, gs)
    torch.cuda.synchronize()
    oc2, os2 = oracle.quant_1x128(oracle.decode_bf16(xb).astype(np.float32))
    assert np.array_equal(gs.cpu().numpy(), os2)
    assert np.array_equal(gc.cpu().numpy(), oc2)


def test_quant_code_sweep():
    """The fp32 -> e4m3 code step over a dense sweep of the format's domain.

    Every 128-value block holds 448 at its first position, so its scale is
    exactly 1 and the other 127 values are coded as they are.  The values:
    every 61st fp32 bit pattern of magnitude below 448, every pattern within
    4 ulps of each e4m3 value and of each rounding midpoint, each with a
    random sign.  Codes must equal the oracle's round-to-nearest-even rule.
    """
    rng = np.random.default_rng(33)
    top = np.float32(448.0).view(np.uint32)
    sweep = np.arange(0, top, 61, dtype=np.uint32)
    grid = oracle.E4M3_TABLE[:0x7F].astype(np.float32)            # 0 .. 448
    mids = ((oracle.E4M3_TABLE[:0x7E] + oracle.E4M3_TABLE[1:0x7F]) / 2).astype(np.float32)
    near = np.concatenate([grid, mids]).view(np.uint32).astype(np.int64)
    near = (near[:, None] + np.arange(-4, 5)[None, :]).ravel()
    near = near[(near >= 0) & (near < top)].astype(np.uint32)
    mags = np.concatenate([sweep, near]).view(np.float32)
    vals = np.where(rng.random(mags.size) < 0.5, -mags, mags).astype(np.float32)
    per = 127
    nblk = -(-vals.size // per)
    blocks = np.zeros((nblk, 128), np.float32)
    blocks[:, 0] = 448.0
    flat = np.zeros(nblk * per, np.float32)
    flat[:vals.size] = vals
    blocks[:, 1:] = flat.reshape(nblk, per)
    cols = 8192
    nb_row = cols // 128
    nrow = -(-nblk // nb_row)
    v = np.zeros((nrow * nb_row, 128), np.float32)
    v[:, 0] = 448.0
    v[:nblk] = blocks
    v = v.reshape(nrow, cols)
    say("quant sweep", v.shape, "values", vals.size)
    gc = torch.empty((nrow, cols), dtype=torch.uint8, device="cuda")
    gs = torch.empty((nrow, nb_row), dtype=torch.float32, device="cuda")
    moe.quant_fp8(tf(v), gc, gs)
    torch.cuda.synchronize()
    oc, os_ = oracle.quant_1x128(v)
    assert np.all(os_ == 1.0)
    assert np.array_equal(gs.cpu().numpy(), os_)
    got = gc.cpu().numpy()
    bad = np.flatnonzero(got.ravel() != oc.ravel())
    assert bad.size == 0, f"{bad.size} codes differ, first at value {v.ravel()[bad[0]]!r}"


def _packed_reference(a: np.ndarray, is_bf16: bool) -> np.ndarray:
    """The documented tile layout, built index by index from row-major bytes."""
    b = np.ascontiguousarray(a).view(np.uint8).reshape(a.shape[0], -1)
    rows, rb = b.shape
    nst = rb // 128
    out = np.empty(rows * rb, np.uint8)
    for g in range(rows // 16):
        for st in range(nst):
            base = (g * nst + st) * 2048
            for r in range(16):
                for q in range(4):
                    for h in range(2):
                        src = st * 128 + (64 * h + 16 * q if is_bf16 else 32 * q + 16 * h)
                        dst = base + h * 1024 + (r + 16 * q) * 16
                        out[dst:dst + 16] = b[g * 16 + r, src:src + 16]
    return out


@pytest.mark.parametrize("is_bf16", [False, True])
def test_pack_weights_layout(is_bf16):
    """moe_pack_weights writes exactly the documented tile permutation."""
    rng = np.random.default_rng(33)
    a = rng.integers(0, 256, (48, 384), dtype=np.uint8)
    src = t8(a)
    dst = torch.empty_like(src)
    moe.pack_weights(src, dst, is_bf16=is_bf16)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().reshape(-1), _packed_reference(a, is_bf16))


def test_layer_parity(tiny):
    cfg, gl, x, mask = tiny
    say("tiny layer M=8")
    g = run_layer(gl, x, mask)
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    assert np.array_equal(g["x_codes"], o.x_codes)
    assert np.array_equal(g["x_scales"], o.x_scales)
    bad, n = compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    say(f"tiny layer: max row rel err {err:.3e}, h code flips {bad}/{n}")


def test_h_requant_unit_bit_exact(tiny):
    """The GPU requantization fed the oracle's fl32(h) gives the oracle's codes."""
    cfg, gl, x, mask = tiny
    o = run_oracle(gl, x, mask)
    xq, xs = oracle.quant_rows(x, mask)
    ew = gl.expert_fn()
    hs = []
    for u, e in enumerate(o.routing.union_ids):
        lo, hi = o.routing.offs[u], o.routing.offs[u + 1]
        rr = o.routing.rows[lo:hi]
        g = oracle.block_gemm(xq[rr], xs[rr], ew(int(e))["gate"], ew(int(e))["s_gate"])
        uu = oracle.block_gemm(xq[rr], xs[rr], ew(int(e))["up"], ew(int(e))["s_up"])
        hs.append((oracle.silu(g) * uu).astype(np.float32))
    h32 = np.concatenate(hs)
    gc = torch.empty(h32.shape, dtype=torch.uint8, device="cuda")
    gsc = torch.empty((h32.shape[0], h32.shape[1] // 128), dtype=torch.float32, device="cuda")
    moe.quant_fp8(tf(h32), gc, gsc)
    torch.cuda.synchronize()
    oc, os_ = oracle.quant_1x128(h32)
    assert np.array_equal(gc.cpu().numpy(), oc)
    assert np.array_equal(gsc.cpu().numpy(), os_)
    for s in range(h32.shape[0]):
        assert np.array_equal(o.h_codes[s], oc[s])


def test_ffn_fp8_with_oracle_routing(tiny):
    cfg, gl, x, mask = tiny
    o = run_oracle(gl, x, mask, shared=False)
    g = run_ffn(gl, x, mask, o.routing)
    compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    err = assert_y_close(g["y"], o)
    say(f"ffn_fp8 (routed only): max row rel err {err:.3e}")


def test_pads_zero_under_nan_poison(tiny):
    cfg, gl, x, mask = tiny
    m2 = mask.copy()
    m2[[1, 6]] = 0
    xn = x.copy()
    xn[[1, 6]] = 0x7FC0
    xz = x.copy()
    xz[[1, 6]] = 0
    gn = run_layer(gl, xn, m2)
    gz = run_layer(gl, xz, m2)
    assert not gn["y"][[1, 6]].any()
    assert np.array_equal(gn["y"], gz["y"])
    assert (gn["ids"][[1, 6]] == -1).all() and (gn["slot_of"][[1, 6]] == -1).all()
    o = run_oracle(gl, xn, m2)
    assert_routing_equal(gn, o.routing, m2)
    assert_y_close(gn["y"], o)


def test_invariants_slot_permutation_companions_repeat(tiny):
    cfg, gl, x, mask = tiny
    base = run_layer(gl, x, mask)
    again = run_layer(gl, x, mask)
    assert np.array_equal(base["y"], again["y"])                     # repeat
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    p = run_layer(gl, x[perm], mask[perm])
    assert np.array_equal(p["y"], base["y"][perm])                   # slot permutation
    assert np.array_equal(p["ids"], base["ids"][perm])
    x2 = x.copy()
    x2[[0, 2, 5]] = _rows(cfg, 3, 5)
    c = run_layer(gl, x2, mask)
    for r in (1, 3, 4, 6, 7):
        assert np.array_equal(c["y"][r], base["y"][r])               # companion rows


def test_decode_and_generic_paths_give_identical_rows(tiny):
    """The same rows inside an 8-row step (fused decode kernels) and inside a
    40-row step (grouped kernels + combine) give identical bits."""
    cfg, gl, x, mask = tiny
    base = run_layer(gl, x, mask)
    big = _rows(cfg, 40, 9)
    where = np.array([0, 7, 13, 21, 22, 30, 38, 39])
    big[where] = x
    g = run_layer(gl, big, np.ones(40, np.uint8))
    assert np.array_equal(g["y"][where], base["y"])
    assert np.array_equal(g["ids"][where], base["ids"])


@pytest.mark.parametrize("m", [17, 24])
def test_two_row_halves_match_tiled(tiny, m):
    """A split step of 17-24 rows (both row halves in each work item) and the same
    rows inside a 40-row tiled step give identical bits."""
    cfg, gl, _, _ = tiny
    x = _rows(cfg, m, 300 + m)
    mask = np.ones(m, np.uint8)
    mask[m - 2] = 0
    x[m - 2] = 0x7FC0
    half = run_layer(gl, x, mask)
    big = _rows(cfg, 40, 400 + m)
    big[:m] = x
    bmask = np.ones(40, np.uint8)
    bmask[:m] = mask
    g = run_layer(gl, big, bmask)
    assert np.array_equal(g["y"][:m], half["y"])
    assert np.array_equal(g["ids"][:m], half["ids"])


@pytest.mark.parametrize("m", [1, 3, 16, 17, 24, 25, 32, 33, 37, 200])
def test_ragged_row_counts(tiny, m):
    cfg, gl, _, _ = tiny
    x = _rows(cfg, m, 100 + m)
    mask = np.ones(m, np.uint8)
    if m > 2:
        mask[m // 2] = 0
        x[m // 2] = 0x7FC0
    say(f"tiny ragged M={m}")
    g = run_layer(gl, x, mask)
    o = run_oracle(gl, x, mask)
    assert_routing_equal(g, o.routing, mask)
    assert np.array_equal(g["x_codes"][mask != 0], o.x_codes[mask != 0])
    compare_h_codes(g["h_codes"], g["h_scales"], o, gl)
    assert_y_close(g["y"], o)
    assert not g["y"][mask == 0].any()


def test_all_pad_rows(tiny):
    cfg, gl, x, _ = tiny
    mask = np.zeros(8, np.uint8)
    xn = np.full_like(x, 0x7FC0)
    g = run_layer(gl, xn, mask)
    assert g["n_union"] == 0
    assert not g["y"].any()
    assert (g["ids"] == -1).all()


def test_zero_rows_tie_to_lower_ids(tiny):
    """All-zero inputs make every logit 0; with a zero bias every score ties and
    the lowest ids win."""
    cfg, gl, x, mask = tiny
    zb = torch.zeros_like(gl.bias)
    saved = gl.bias
    gl.bias = zb
    try:
        x0 = np.zeros_like(x)
        g = run_layer(gl, x0, mask)
    finally:
        gl.bias = saved
    k = cfg.dims.top_k
    assert (g["ids"] == np.arange(k)).all()
    assert np.allclose(g["w"], cfg.dims.routed_scale / k, rtol=0, atol=1e-7)


@pytest.mark.parametrize("m", [8, 40])            # split and tiled paths
@pytest.mark.parametrize("flaw", ["union_order", "repeated_row", "row_out_of_range", "pad_row", "rows_descending"])
def test_malformed_routing_contributes_nothing(tiny, m, flaw):
    """A caller routing that breaks the layout moe_ffn_fp8 documents is
    detected on the device and schedules no routed work: y is +0.0."""
    cfg, gl, _, _ = tiny
    x = _rows(cfg, m, 77 + m)
    mask = np.ones(m, np.uint8)
    o = run_oracle(gl, x, mask, shared=False).routing
    union_ids, rows, use_mask = o.union_ids.copy(), o.rows.copy(), mask.copy()
    lo, hi = int(o.offs[0]), int(o.offs[1])
    assert hi - lo >= 2
    if flaw == "union_order":
        union_ids = union_ids[::-1].copy()
    elif flaw == "repeated_row":
        rows[lo + 1] = rows[lo]
    elif flaw == "row_out_of_range":
        rows[hi - 1] = m
    elif flaw == "pad_row":
        use_mask[int(rows[lo])] = 0                       # a pad row left in the expert's list
    else:
        rows[lo], rows[lo + 1] = rows[lo + 1], rows[lo]
    bad = oracle.Routing(o.ids, o.w, union_ids, o.offs, rows, o.slot_of)
    say(f"malformed routing ({flaw}), M={m}")
    g = run_ffn(gl, x, use_mask, bad)
    assert not g["y"].any()
    # the well-formed routing on the same call shape does produce output
    good = run_ffn(gl, x, mask, o)
    assert good["y"].any()


def test_workspace_reuse_across_sizes(tiny):
    """One workspace sized for the largest M serves smaller calls."""
    cfg, gl, x, mask = tiny
    a = run_layer(gl, x, mask, ws_rows=300)
    b = run_layer(gl, x, mask)
    assert np.array_equal(a["y"], b["y"])


@pytest.mark.parametrize("m", [16, 17, 25, 32, 33, 48, 64, 65, 66, 128, 129, 200])
def test_forced_routing_tile_fill(tiny, m):
    """Every real row picks the same four experts (correction bias +100 on
    them), so each holds exactly the real-row count of slots: counts of
    16 k and 16 k + 1 put the last 16-slot group of a 128-slot tile just
    full or just started (the tiled kernels compute only the groups that
    hold real rows), 128 and 129 fill one tile and start a second.  Parity
    against the oracle, and the first 8 rows equal the 8-row split step on
    those rows bit for bit."""
    cfg, gl, _, _ = tiny
    bias = gl.host.bias.astype(np.float32).copy()
    bias[[1, 6, 11, 14]] += 100.0
    gf = gl.with_bias(bias)
    x = _rows(cfg, m, 500 + m)
    mask = np.ones(m, np.uint8)
    if m == 66:                               # one pad: 65 slots per expert
        mask[40] = 0
        x[40] = 0x7FC0
    say(f"tiny forced routing M={m}")
    g = run_layer(gf, x, mask)
    o = run_oracle(gf, x, mask)
    assert_routing_equal(g, o.routing, mask)
    assert list(o.routing.union_ids) == [1, 6, 11, 14]
    assert np.all(np.diff(o.routing.offs) == int(mask.sum()))
    real = mask != 0
    assert np.array_equal(g["x_codes"][real], o.x_codes[real])
    compare_h_codes(g["h_codes"], g["h_scales"], o, gf)
    assert_y_close(g["y"], o)
    assert not g["y"][~real].any()
    small = run_layer(gf, x[:8], mask[:8])
    assert np.array_equal(g["y"][:8], small["y"])


def test_logit_kernels_give_identical_routing(tiny):
    """The same 100 rows as a 100-row step (float64 logits one wave per logit)
    and as the first rows of a 200-row step (8-row x 8-expert logit waves):
    the logits take one lane order and butterfly in both, so the ids, the
    float32 combine weights and the y rows are equal bit for bit."""
    cfg, gl, _, _ = tiny
    x = _rows(cfg, 100, 901)
    mask = np.ones(100, np.uint8)
    mask[37] = 0
    x[37] = 0x7FC0
    say("tiny logit kernels: 100 vs 200 rows")
    a = run_layer(gl, x, mask)
    big = _rows(cfg, 200, 902)
    big[:100] = x
    bmask = np.ones(200, np.uint8)
    bmask[:100] = mask
    b = run_layer(gl, big, bmask)
    assert np.array_equal(a["ids"], b["ids"][:100])
    assert np.array_equal(a["w"].view(np.uint32), b["w"][:100].view(np.uint32))
    assert np.array_equal(a["y"], b["y"][:100])
    o = run_oracle(gl, x, mask)
    assert_routing_equal(a, o.routing, mask)


@pytest.mark.parametrize("m", [1, 8, 16])
def test_reused_workspace_with_changing_inputs(tiny, m):
    """One workspace and routing buffers reused by consecutive steps whose
    inputs differ (A, B, A, B): every step equals the same step run alone on a
    fresh workspace, bit for bit.  The small-step launch passes data between
    workgroups through the workspace within one launch, so a value left over
    from the previous step (a stale cache line) would show up here."""
    cfg, gl, _, _ = tiny
    d = gl.dims
    xa = _rows(cfg, m, 3100 + m)
    xb = _rows(cfg, m, 3200 + m)
    mask = np.ones(m, np.uint8)
    if m > 4:
        mask[m // 2] = 0
        xb[m // 2] = 0x7FC0
    fresh = {k: run_layer(gl, x, mask) for k, x in (("a", xa), ("b", xb))}
    ws = moe.workspace(d, m)
    rt = moe.Routing.empty(d, m)
    y = torch.empty((m, d.hidden), dtype=torch.int16, device="cuda")
    mk = t8(mask)
    for k, x in (("a", xa), ("b", xb), ("a", xa), ("b", xb)):
        moe.layer(d, t16(x), mk, gl.router_w, gl.bias, gl.experts, gl.shared, y, rt, ws)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), fresh[k]["y"]), k
        assert np.array_equal(rt.topk_ids.cpu().numpy(), fresh[k]["ids"]), k
