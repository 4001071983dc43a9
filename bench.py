#!/usr/bin/env python3
"""Benchmark of the routed fp8 MoE FFN layer on one MI355X.

Headline workload: the span-8 decode step (8 rows of one request: 1 committed
token + 7 drafts; hidden 6144, 256 routed experts top-8, inter 2048 fp8 e4m3
with 128x128 block scales, one bf16 shared expert of inter 2048).  A step is
one moe_layer call.  Expert weights are rotated over several device replicas
so every step reads its weights from HBM, as the pages time the layer with
every call's weights read from HBM (mstar PR #388, decode table note).

Also measured: the 4096-token prefill over 4 stacked layers with independent
weights (prefill TFLOPS), and the CPU oracle on the decode step (baseline).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "MoE-layer µs and expert-weight HBM GB/s (% peak), 8-row span step; prefill TFLOPS"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- HIP events via the runtime
class HipEvents:
    def __init__(self, n):
        # the runtime torch already loaded (same soname), never a second copy
        self.rt = C.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = []
        for _ in range(n):
            h = C.c_void_p()
            if self.rt.hipEventCreate(C.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h)

    def elapsed_ms(self, a, b) -> float:
        self.rt.hipEventSynchronize(b)
        out = C.c_float()
        if self.rt.hipEventElapsedTime(C.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for h in self.ev:
            self.rt.hipEventDestroy(h)


# ----------------------------------------------------------------------------- device layers
def device_layer(cfg, layer, torch, moe, replicas=1):
    """Stream a seeded layer to the GPU expert by expert; `replicas` copies.
    Every replica holds its own copy of every weight (routed, shared, router),
    so a call on one replica never finds another's weights in a cache."""
    import synth
    d = cfg.dims
    E, I, H = d.n_experts, d.inter, d.hidden
    dev = "cuda"
    reps = []
    for _ in range(replicas):
        reps.append(dict(
            wg=torch.empty((E, I, H), dtype=torch.uint8, device=dev), wu=torch.empty((E, I, H), dtype=torch.uint8, device=dev),
            wd=torch.empty((E, H, I), dtype=torch.uint8, device=dev),
            sg=torch.empty((E, I // 128, H // 128), dtype=torch.float32, device=dev),
            su=torch.empty((E, I // 128, H // 128), dtype=torch.float32, device=dev),
            sd=torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=dev)))
    r0 = reps[0]

    def put(e, t):
        r0["wg"][e].copy_(torch.from_numpy(t["gate"]))
        r0["wu"][e].copy_(torch.from_numpy(t["up"]))
        r0["wd"][e].copy_(torch.from_numpy(t["down"]))
        r0["sg"][e].copy_(torch.from_numpy(t["s_gate"]))
        r0["su"][e].copy_(torch.from_numpy(t["s_up"]))
        r0["sd"][e].copy_(torch.from_numpy(t["s_down"]))

    synth.for_each_expert(cfg, layer, put)
    # weights in the library's packed tile layout (row-major copies freed)
    for k in ("wg", "wu", "wd"):
        packed = torch.empty_like(r0[k])
        moe.pack_weights(r0[k], packed, is_bf16=False)
        r0[k] = packed
    for r in reps[1:]:
        for k in r:
            r[k].copy_(r0[k])
    sh = synth.shared_expert(cfg, layer)
    t16 = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)
    shared0 = moe.pack_shared(moe.Shared(t16(sh["gate"]), t16(sh["up"]), t16(sh["down"])))
    router0 = t16(synth.router_weight(cfg, layer))
    bias0 = torch.from_numpy(synth.router_bias(cfg, layer)).to(dev)
    out = []
    for i, r in enumerate(reps):
        shared = shared0 if i == 0 else moe.Shared(shared0.w_gate.clone(), shared0.w_up.clone(),
                                                   shared0.w_down.clone(), moe.WEIGHTS_PACKED)
        out.append(dict(
            experts=moe.Experts(r["wg"], r["wu"], r["wd"], r["sg"], r["su"], r["sd"], moe.WEIGHTS_PACKED),
            shared=shared,
            router_w=router0 if i == 0 else router0.clone(),
            bias=bias0 if i == 0 else bias0.clone()))
    torch.cuda.synchronize()
    return out


def decode_bytes(nu, d, m):
    """Algorithmic HBM bytes of one layer step: union experts' fp8 weights and
    block scales, the bf16 shared expert, the router, x in and y out."""
    H, I, Is, E = d.hidden, d.inter, d.shared_inter, d.n_experts
    per_expert = 3 * I * H + 4 * (3 * (I // 128) * (H // 128))
    routed = nu * per_expert
    fixed = 3 * Is * H * 2 + E * H * 2 + 4 * E + 2 * m * H * 2
    return routed, fixed


def gateup_bytes(nu, d, m):
    """Algorithmic bytes of the routed gate/up kernel (small steps): gate and up
    codes + scales of the union experts, x codes and scales."""
    H, I = d.hidden, d.inter
    return nu * (2 * I * H + 4 * 2 * (I // 128) * (H // 128)) + m * H + m * (H // 128) * 4


def down_decode_bytes(nu, d, m):
    """Algorithmic bytes of the down kernel (small steps): down codes + scales
    of the union experts, h codes + scales, the shared down weights (bf16)
    and the shared h rows."""
    H, I, K, Is = d.hidden, d.inter, d.top_k, d.shared_inter
    return (nu * (I * H + 4 * (H // 128) * (I // 128)) + m * K * (I + 4 * (I // 128))
            + H * Is * 2 + m * Is * 2)


def front_bytes(d, m):
    """Algorithmic bytes of the fused front kernel (small steps): the router
    weights, the first half of the shared gate/up K range (bf16), x (bf16)
    once, x codes and scales out."""
    H, Is, E = d.hidden, d.shared_inter, d.n_experts
    return E * H * 2 + Is * H * 2 + m * H * 2 + m * H + m * (H // 128) * 4


def select_bytes(d, m):
    """Algorithmic bytes of the select/union launch (small steps): the second
    half of the shared gate/up K range (bf16)."""
    return d.shared_inter * d.hidden * 2


def kernel_bytes(name, nu, d, m):
    """Algorithmic bytes per launch of the kernels that stream weights."""
    return {"gateup": gateup_bytes(nu, d, m),
            "down": down_decode_bytes(nu, d, m),
            "front": front_bytes(d, m),
            "select_union": select_bytes(d, m)}.get(name)


def layer_flops(d, m_real, slots):
    H, I, Is = d.hidden, d.inter, d.shared_inter
    fp8 = 2.0 * slots * (2 * I * H + I * H)
    bf16 = 2.0 * m_real * 3 * Is * H
    router = 2.0 * m_real * d.n_experts * H
    return fp8, bf16, router


COUNTERS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_span8_hbm_counters.md")


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when the kernel sources changed since the counters were taken."""
    from sparse_moe_ffn_02_amd.profile_summary import load_traffic
    tr = load_traffic(COUNTERS)
    if not tr:
        return None
    k = tr["kernels"].get(kernel + "_split") or tr["kernels"].get(kernel)
    return None if k is None else k["read_bytes"] + k["write_bytes"]


def cpu_info():
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    model = platform.processor()
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return threads, model


def graph_replay_us(torch, step, n_graphs, steps, warmup, rt_lib, stream):
    """One captured step per weight replica, replayed in rotation.  Returns the
    mean us per step over `steps` back-to-back replays and the p10/p50/p90 of
    single replays (each bracketed by its own events)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_graphs):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    graphs = []
    for i in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % n_graphs].replay()
    torch.cuda.synchronize()
    ev = HipEvents(2 + 2 * steps)
    rt_lib.hipEventRecord(ev.ev[0], C.c_void_p(stream))
    for i in range(steps):
        graphs[i % n_graphs].replay()
    rt_lib.hipEventRecord(ev.ev[1], C.c_void_p(stream))
    torch.cuda.synchronize()
    mean_us = 1e3 * ev.elapsed_ms(ev.ev[0], ev.ev[1]) / steps
    for i in range(steps):
        rt_lib.hipEventRecord(ev.ev[2 + 2 * i], C.c_void_p(stream))
        graphs[i % n_graphs].replay()
        rt_lib.hipEventRecord(ev.ev[3 + 2 * i], C.c_void_p(stream))
    torch.cuda.synchronize()
    each = np.array([1e3 * ev.elapsed_ms(ev.ev[2 + 2 * i], ev.ev[3 + 2 * i]) for i in range(steps)])
    ev.close()
    del graphs
    p10, p50, p90 = (float(np.percentile(each, q)) for q in (10, 50, 90))
    return mean_us, p10, p50, p90


def graph_chain_us(torch, step, n_calls, steps, warmup, rt_lib, stream):
    """One graph holding n_calls consecutive steps (step(0) .. step(n_calls - 1),
    the weight replicas in rotation), as a decode graph over consecutive
    layers holds them, replayed back to back.  Returns the mean us per step
    over at least `steps` steps, and the p10/p50/p90 over single replays
    (each bracketed by its own events) of the us per step inside one replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_calls):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            step(i)
    for _ in range(max(1, warmup // n_calls)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(10, (steps + n_calls - 1) // n_calls)
    ev = HipEvents(2 + 2 * reps)
    rt_lib.hipEventRecord(ev.ev[0], C.c_void_p(stream))
    for _ in range(reps):
        g.replay()
    rt_lib.hipEventRecord(ev.ev[1], C.c_void_p(stream))
    torch.cuda.synchronize()
    us = 1e3 * ev.elapsed_ms(ev.ev[0], ev.ev[1]) / (reps * n_calls)
    for i in range(reps):
        rt_lib.hipEventRecord(ev.ev[2 + 2 * i], C.c_void_p(stream))
        g.replay()
        rt_lib.hipEventRecord(ev.ev[3 + 2 * i], C.c_void_p(stream))
    torch.cuda.synchronize()
    each = np.array([1e3 * ev.elapsed_ms(ev.ev[2 + 2 * i], ev.ev[3 + 2 * i]) / n_calls for i in range(reps)])
    ev.close()
    del g
    p10, p50, p90 = (float(np.percentile(each, q)) for q in (10, 50, 90))
    return us, p10, p50, p90


def copy_gbs(torch, rt_lib, stream, mib=1024, reps=10):
    """Plain device-to-device copy bandwidth (bytes read + bytes written per
    second) of a MIB MiB buffer: the practical streaming ceiling measured on
    the same GPU in the same run, beside the datasheet peak."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = HipEvents(2)
    rt_lib.hipEventRecord(ev.ev[0], C.c_void_p(stream))
    for _ in range(reps):
        dst.copy_(src)
    rt_lib.hipEventRecord(ev.ev[1], C.c_void_p(stream))
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(ev.ev[0], ev.ev[1]) / reps
    ev.close()
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * n / (ms * 1e-3) / 1e9


def rows_sweep(torch, moe, synth, md, d, reps, rt_lib, stream, steps, warmup):
    """Layer time against the row count on the span-8 layer (one committed row
    plus drafts, the same recipe at every count): the small-step path serves
    up to moe.split_rows(inter) rows, the tiled path above."""
    out = []
    for m in (1, 2, 4, 8, 9, 12, 16, 17, 24, 32, 33, 48, 64, 128, 256):
        cfg = synth.with_rows(synth.CONFIGS["span8"], m)
        x_np, mask_np = synth.activations(cfg)
        x = torch.from_numpy(x_np.view(np.int16)).cuda()
        mask = torch.from_numpy(mask_np).cuda()
        ws = moe.workspace(md, m)
        y = torch.empty((m, d.hidden), dtype=torch.int16, device="cuda")
        rt = moe.Routing.empty(md, m)

        def step(i):
            r = reps[i % len(reps)]
            moe.layer(md, x, mask, r["router_w"], r["bias"], r["experts"], r["shared"], y, rt, ws)

        us, p10, p50, p90 = graph_replay_us(torch, step, len(reps), steps, warmup, rt_lib, stream)
        nu = int(rt.n_union.item())
        rb, fb = decode_bytes(nu, d, m)
        out.append({"rows": m, "path": "split" if m <= moe.split_rows(d.inter) else "tiled", "union_experts": nu,
                    "us": round(us, 2),
                    "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                    "gbs": round((rb + fb) / (us * 1e-6) / 1e9, 1)})
        log(f"[bench] rows sweep M={m}: {us:.1f} us, |U|={nu}, {(rb + fb) / (us * 1e-6) / 1e9:.0f} GB/s")
    return out


def tp8_rank_sweep(torch, moe, synth, rt_lib, stream, steps, warmup, replicas):
    """One TP8 rank's share of the layer on one GPU: every expert's I/8 = 256
    slice (shared expert likewise), span-decode token counts 1..10, no
    collective (the rank's partial outputs are what it would reduce-scatter)."""
    cfg0 = synth.CONFIGS["tp8rank"]
    d = cfg0.dims
    md = moe.Dims(d.hidden, d.n_experts, d.top_k, d.inter, d.shared_inter, d.routed_scale)
    t0 = time.time()
    reps = device_layer(cfg0, 0, torch, moe, replicas=replicas)
    log(f"[bench] tp8-rank layer (I={d.inter}) ready in {time.time() - t0:.1f}s")
    out = []
    for m in (1, 2, 4, 5, 6, 8, 9, 10):
        cfg = synth.with_rows(cfg0, m)
        x_np, mask_np = synth.activations(cfg)
        x = torch.from_numpy(x_np.view(np.int16)).cuda()
        mask = torch.from_numpy(mask_np).cuda()
        ws = moe.workspace(md, m)
        y = torch.empty((m, d.hidden), dtype=torch.int16, device="cuda")
        rt = moe.Routing.empty(md, m)

        def step(i):
            r = reps[i % len(reps)]
            moe.layer(md, x, mask, r["router_w"], r["bias"], r["experts"], r["shared"], y, rt, ws)

        us, p10, p50, p90 = graph_replay_us(torch, step, len(reps), steps, warmup, rt_lib, stream)
        nu = int(rt.n_union.item())
        rb, fb = decode_bytes(nu, d, m)
        out.append({"tokens": m, "union_experts": nu, "us": round(us, 2), "us_p10": round(p10, 2),
                    "us_p90": round(p90, 2), "gbs": round((rb + fb) / (us * 1e-6) / 1e9, 1)})
        log(f"[bench] tp8-rank M={m}: {us:.1f} us, |U|={nu}, {(rb + fb) / (us * 1e-6) / 1e9:.0f} GB/s")
    # the fixed-order sum of the 8 ranks' partial outputs for an 8-row step ([row][src][H] region)
    parts = torch.randint(-2000, 2000, (8, 8, d.hidden), dtype=torch.int16, device="cuda")
    ysum = torch.empty((8, d.hidden), dtype=torch.int16, device="cuda")
    sum_us = graph_replay_us(torch, lambda i: moe.sum_partials(parts, None, ysum), 1, steps, warmup, rt_lib,
                             stream)[0]
    log(f"[bench] tp8 fixed-order sum of 8 partials (8 rows): {sum_us:.1f} us")
    del reps
    torch.cuda.empty_cache()
    return {"sum_partials_8x8_us": round(sum_us, 2),
            "workload": "one TP8 rank's share on one GPU: hidden 6144, 256 experts top-8, expert inter 256 "
                        "(I/8) fp8 e4m3 128x128 scales, shared expert inter 256 bf16, span-decode rows "
                        "(1 committed + drafts), weights rotated over device replicas, no collective",
            "points": out}


def gateup_tiled_bytes(nu, slots, d, m):
    """Algorithmic HBM bytes of the tiled gate/up kernel (one launch): the
    union experts' gate and up codes and block scales, the x codes and scales,
    the shared expert's gate/up weights and its bf16 x rows, and the outputs
    (h codes and scales of every slot, the shared expert's bf16 h)."""
    H, I, Is = d.hidden, d.inter, d.shared_inter
    weights = nu * (2 * I * H + 4 * 2 * (I // 128) * (H // 128)) + 2 * Is * H * 2
    acts_in = m * H + m * (H // 128) * 4 + (m * H * 2 if Is else 0)
    acts_out = slots * I + slots * (I // 128) * 4 + m * Is * 2
    return weights + acts_in + acts_out


def gateup_tiled_flops(slots, d, m):
    """fp8 and bf16 MFMA flops of the tiled gate/up kernel."""
    H, I, Is = d.hidden, d.inter, d.shared_inter
    return 2.0 * slots * 2 * I * H, 2.0 * m * 2 * Is * H


PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill4096_hbm_counters.md")
PREFILL_MFMA = os.path.join(ROOT, "profiles", "prefill4096_mfma_counters.md")


def traced_kernel_us(lib, torch, fn, calls, per_call=16):
    """Mean us per launch of each library kernel over `calls` calls of fn,
    from HIP events the library records around each launch on its stream."""
    tev = HipEvents(2 * per_call * calls)
    pairs = (C.c_void_p * (2 * per_call * calls))(*[h.value for h in tev.ev])
    kid = (C.c_int32 * (per_call * calls))()
    cnt = C.c_int32(0)
    assert lib.moe_trace_set(pairs, per_call * calls, kid, C.byref(cnt)) == 0
    for i in range(calls):
        fn(i)
    torch.cuda.synchronize()
    lib.moe_trace_set(None, 0, None, None)
    per = {}
    for i in range(cnt.value):
        name = lib.moe_kernel_name(kid[i]).decode()
        per.setdefault(name, []).append(tev.elapsed_ms(tev.ev[2 * i], tev.ev[2 * i + 1]))
    tev.close()
    return {k: 1e3 * float(np.mean(v)) for k, v in per.items()}


def prefill_bench(args, torch, moe, synth, md, d, ev, rt_lib, stream, lib):
    """4096-token prefill chunk through `args.prefill_layers` stacked layers:
    layer l + 1 takes layer l's output rescaled per row to unit RMS (moe_add_rmsnorm
    with a zero residual and unit gamma), the rescale timed on its own."""
    pcfg = synth.CONFIGS["prefill4096x4"]
    n_layers = args.prefill_layers
    layers = []
    for l in range(n_layers):
        t0 = time.time()
        layers.append(device_layer(pcfg, l, torch, moe, replicas=1)[0])
        log(f"[bench] prefill layer {l} ready in {time.time() - t0:.1f}s")
    Mp = pcfg.rows
    H = d.hidden
    x0 = torch.from_numpy(synth.activations(pcfg, layer=0)[0].view(np.int16)).cuda()
    xin = [x0] + [torch.empty_like(x0) for _ in range(n_layers - 1)]
    wsp = moe.workspace(md, Mp)
    yp = torch.empty((Mp, H), dtype=torch.int16, device="cuda")
    zero = torch.zeros_like(yp)
    ones = torch.full((H,), 0x3F80, dtype=torch.int16, device="cuda")        # bf16 1.0
    rscr = torch.empty_like(yp)
    xtmp = torch.empty_like(yp)
    rts = [moe.Routing.empty(md, Mp) for _ in layers]

    def pstep():
        for l, L in enumerate(layers):
            moe.layer(md, xin[l], None, L["router_w"], L["bias"], L["experts"], L["shared"], yp, rts[l], wsp)
            if l + 1 < n_layers:
                moe.add_rmsnorm(yp, None, zero, ones, 1e-6, rscr, xin[l + 1])

    def rescales():
        for _ in range(n_layers - 1):
            moe.add_rmsnorm(yp, None, zero, ones, 1e-6, rscr, xtmp)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        rt_lib.hipEventRecord(ev.ev[0], C.c_void_p(stream))
        for _ in range(n):
            fn()
        rt_lib.hipEventRecord(ev.ev[1], C.c_void_p(stream))
        torch.cuda.synchronize()
        return ev.elapsed_ms(ev.ev[0], ev.ev[1]) / n

    ms_chain = timed(pstep, args.prefill_steps)
    ms_resc = timed(rescales, args.prefill_steps) if n_layers > 1 else 0.0
    ms_layers = ms_chain - ms_resc
    f8 = f16 = fr = 0.0
    pbytes = 0
    loads = []
    for l in range(n_layers):
        nu_l = int(rts[l].n_union.item())
        sl = int(rts[l].offs[nu_l].item())
        a, b_, c_ = layer_flops(d, Mp, sl)
        f8 += a; f16 += b_; fr += c_
        rb, fb = decode_bytes(nu_l, d, Mp)
        pbytes += rb + fb
        loads.append(np.diff(rts[l].offs[:nu_l + 1].cpu().numpy()))
    t_s = ms_layers * 1e-3
    out = {
        "workload": f"4096-token prefill chunk through {n_layers} stacked MoE layers (independent seeded weights; "
                    "layer l+1 takes layer l's output rescaled per row to unit RMS), Zipf(1.1) router bias, "
                    "hidden 6144, 256 experts top-8, inter 2048 fp8 e4m3 128x128 scales, bf16 shared expert",
        "layers": n_layers,
        "ms_per_step": round(ms_chain, 4),
        "ms_rescale_total": round(ms_resc, 4),
        "ms_per_layer": round(ms_layers / n_layers, 4),
        "tflops_total": round((f8 + f16 + fr) / t_s / 1e12, 2),
        "tflops_fp8": round(f8 / t_s / 1e12, 2),
        "fp8_mfma_frac": round(f8 / t_s / 1e12 / FP8_PEAK_TFLOPS, 4),
        "mfma_composite_frac": round((f8 / 1e12 / FP8_PEAK_TFLOPS + f16 / 1e12 / BF16_PEAK_TFLOPS) / t_s, 4),
        "hbm_frac": round(pbytes / t_s / 1e9 / HBM_PEAK_GBS, 4),
        "expert_rows_max": int(max(l.max() for l in loads)),
        "expert_rows_mean": round(float(np.mean([l.mean() for l in loads])), 1),
        "timing": "chain of layers and rescales timed with HIP events; the rescales alone timed the same way "
                  "and subtracted for the per-layer figures",
    }
    log(f"[bench] prefill4096 x{n_layers} layers: {ms_chain:.2f} ms/step ({ms_resc:.3f} ms of rescales), "
        f"{out['tflops_total']} TFLOPS")

    # per-kernel live timings of layer 0 (its input as in the chain)
    L0 = layers[0]
    nu0 = int(rts[0].n_union.item())
    sl0 = int(rts[0].offs[nu0].item())

    def call0(i):
        moe.layer(md, xin[0], None, L0["router_w"], L0["bias"], L0["experts"], L0["shared"], yp, rts[0], wsp)
    kus = traced_kernel_us(lib, torch, call0, max(2, args.prefill_steps))
    out["kernel_us"] = {k: round(v, 2) for k, v in kus.items()}
    gb = gateup_tiled_bytes(nu0, sl0, d, Mp)
    g8, g16 = gateup_tiled_flops(sl0, d, Mp)
    gus = kus["gateup"]
    from sparse_moe_ffn_02_amd.profile_summary import load_mfma, load_traffic
    tr = load_traffic(PREFILL_COUNTERS)
    tk = tr["kernels"].get("gateup_tiled") if tr else None
    mf = load_mfma(PREFILL_MFMA)
    mk = mf["kernels"].get("gateup_tiled") if mf else None
    out["roofline"] = {"kernel": "gateup_tiled", "bound": "hbm", "achieved": round(gb / (gus * 1e-6) / 1e9, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gb / (gus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "traffic": (tk["read_bytes"] + tk["write_bytes"]) if tk else None,
                       "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                       "algorithmic_bytes": gb, "kernel_us": round(gus, 2),
                       "flops_fp8": g8, "flops_bf16": g16,
                       "tflops": round((g8 + g16) / (gus * 1e-6) / 1e12, 1),
                       "fp8_mfma_frac": round(g8 / (gus * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
                       "mfma_busy_frac": mk["busy_frac"] if mk else None,
                       "why_hbm": "256 flop per byte at this shape, below the fp8 ridge of 625 (5 PFLOP/s / 8 TB/s)"}
    log(f"[bench] prefill gateup_tiled: {gus:.1f} us, {gb / 1e9:.2f} GB -> {gb / (gus * 1e-6) / 1e9:.0f} GB/s, "
        f"{(g8 + g16) / (gus * 1e-6) / 1e12:.0f} TFLOP/s")

    # layer 0 followed by the next layer's residual add + RMSNorm, unfused and fused
    res_np, gam_np = synth.norm_inputs(pcfg, rows=Mp)
    res = torch.from_numpy(res_np.view(np.int16)).cuda()
    gam = torch.from_numpy(gam_np.view(np.int16)).cuda()
    r_out = torch.empty_like(res)
    n_out = torch.empty_like(res)

    def unfused():
        call0(0)
        moe.add_rmsnorm(yp, None, res, gam, 1e-6, r_out, n_out)

    def fused():
        moe.layer_add_rmsnorm(md, xin[0], None, L0["router_w"], L0["bias"], L0["experts"], L0["shared"], res, gam,
                              1e-6, yp, r_out, n_out, rts[0], wsp)
    # alternate the two so that clock drift does not favour either; medians of 3
    t_unf, t_fus = [], []
    for _ in range(3):
        t_unf.append(timed(unfused, args.prefill_steps))
        t_fus.append(timed(fused, args.prefill_steps))
    ms_unf, ms_fus = float(np.median(t_unf)), float(np.median(t_fus))
    out["add_rmsnorm"] = {"unfused_ms": round(ms_unf, 4), "fused_ms": round(ms_fus, 4),
                          "timing": "median of 3 alternating runs of --prefill-steps calls each",
                          "workload": "layer 0 of the chunk followed by the residual add + RMSNorm "
                                      "(bf16 residual [4096, 6144], gamma [6144], eps 1e-6)"}
    log(f"[bench] prefill layer + add/RMSNorm: unfused {ms_unf:.3f} ms, fused {ms_fus:.3f} ms")
    return out


def route_ahead_bench(torch, moe, synth, cfg, md, d, reps, rt_lib, stream, n_layers=8, reps_timed=30):
    """Route-ahead experiment on a chain of span-8 decode layers.

    Residual stream: h_0 = x_0 (the span rows); layer l maps x_l to y_l and
    h_{l+1} = bf16(h_l + y_l), x_{l+1} = RMSNorm(h_{l+1}) (gamma 1, eps 1e-6),
    moe_add_rmsnorm.  Layer l has its own router (seeded by l) and takes the
    weights of replica l mod 4.  The plan for layer l+1 is the union of
    routing x_l with layer l+1's router (pre-gating, formed on a second
    stream while layer l runs); its experts' gate/up bytes are then read by
    moe_prefetch_experts, either while layer l runs ("during") or once layer
    l is done, beside the residual epilogue and layer l+1's routing chain
    ("next").  A "perfect" plan (the union layer l+1 really uses, recorded
    from an earlier pass) bounds what any predictor could gain.  Reported:
    the plan's coverage / waste / per-row agreement per layer, and the
    chain's us per layer for each variant against the chain without it."""
    from sparse_moe_ffn_02_amd import route_ahead as ra
    M, H = cfg.rows, d.hidden
    i16 = dict(dtype=torch.int16, device="cuda")
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    routers = [(t16(synth.router_weight(cfg, l)), torch.from_numpy(synth.router_bias(cfg, l)).cuda())
               for l in range(n_layers)]
    x0_np, mask_np = synth.activations(cfg)
    mask = torch.from_numpy(mask_np).cuda()
    xs = [torch.empty((M, H), **i16) for _ in range(n_layers + 1)]
    hs = [torch.empty((M, H), **i16) for _ in range(n_layers + 1)]
    ys = [torch.empty((M, H), **i16) for _ in range(n_layers)]
    xs[0].copy_(t16(x0_np))
    hs[0].copy_(xs[0])
    gamma = torch.full((H,), 0x3F80, **i16)
    rt = [moe.Routing.empty(md, M) for _ in range(n_layers)]
    rp = [moe.Routing.empty(md, M) for _ in range(n_layers)]
    ws, ws_side = moe.workspace(md, M), moe.workspace(md, M)
    aux = torch.cuda.Stream()
    exp = lambda l: reps[l % len(reps)]
    perfect = [None] * n_layers

    def chain(plan=None, when="next", cap=1 << 40, wg=0, serial=False):
        main = torch.cuda.current_stream()
        for l in range(n_layers):
            ahead = plan is not None and l + 1 < n_layers
            if ahead and not serial:
                ready = torch.cuda.Event()
                ready.record(main)
                aux.wait_event(ready)
                with torch.cuda.stream(aux):
                    if plan == "pregate":
                        r = rp[l + 1]
                        moe.route(md, xs[l], mask, routers[l + 1][0], routers[l + 1][1], r, ws_side)
                        src = (r.n_union, r.union_ids)
                    else:
                        src = perfect[l + 1]
                    if when == "during":
                        moe.prefetch_experts(md, src[0], src[1], exp(l + 1)["experts"], moe.PREFETCH_GATE_UP, cap, wg)
            moe.layer(md, xs[l], mask, routers[l][0], routers[l][1], exp(l)["experts"], exp(l)["shared"], ys[l],
                      rt[l], ws)
            moe.add_rmsnorm(ys[l], mask, hs[l], gamma, 1e-6, hs[l + 1], xs[l + 1])
            if ahead and serial:
                src = perfect[l + 1]
                moe.prefetch_experts(md, src[0], src[1], exp(l + 1)["experts"], moe.PREFETCH_GATE_UP, cap, wg)
            elif ahead and when == "next":
                done = torch.cuda.Event()
                done.record(main)
                aux.wait_event(done)
                with torch.cuda.stream(aux):
                    moe.prefetch_experts(md, src[0], src[1], exp(l + 1)["experts"], moe.PREFETCH_GATE_UP, cap, wg)
        if plan is not None and not serial:
            joined = torch.cuda.Event()
            joined.record(aux)
            main.wait_event(joined)

    def prefetch_only(cap=1 << 40, wg=0):
        for l in range(1, n_layers):
            moe.prefetch_experts(md, perfect[l][0], perfect[l][1], exp(l)["experts"], moe.PREFETCH_GATE_UP, cap, wg)

    def prefetch_twice(cap):
        for l in range(1, n_layers):
            for _ in range(2):
                moe.prefetch_experts(md, perfect[l][0], perfect[l][1], exp(l)["experts"], moe.PREFETCH_GATE_UP, cap,
                                     0)

    def timed(fn):
        return graph_chain_us(torch, lambda i: fn(), 1, reps_timed, 5, rt_lib, stream)[0]

    def timed_eager(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = HipEvents(2)
        rt_lib.hipEventRecord(ev.ev[0], C.c_void_p(stream))
        for _ in range(reps_timed):
            fn()
        rt_lib.hipEventRecord(ev.ev[1], C.c_void_p(stream))
        torch.cuda.synchronize()
        us = 1e3 * ev.elapsed_ms(ev.ev[0], ev.ev[1]) / reps_timed
        ev.close()
        return us

    chain()
    torch.cuda.synchronize()
    ref_out = xs[n_layers].clone()
    for l in range(n_layers):
        perfect[l] = (rt[l].n_union.clone(), rt[l].union_ids.clone())
    unions = [ra.union_of(rt[l].topk_ids.cpu().numpy(), mask_np) for l in range(n_layers)]
    chain("pregate")
    torch.cuda.synchronize()
    same = bool(torch.equal(xs[n_layers], ref_out))
    per_layer = []
    for l in range(1, n_layers):
        planned = ra.union_of(rp[l].topk_ids.cpu().numpy(), mask_np)
        per_layer.append({"layer": l, "union": len(unions[l]), "planned": len(planned),
                          "coverage": round(ra.coverage(planned, unions[l]), 4),
                          "waste": round(ra.waste(planned, unions[l]), 4),
                          "row_agreement": round(ra.row_agreement(rp[l].topk_ids.cpu().numpy(),
                                                                  rt[l].topk_ids.cpu().numpy(), mask_np), 4)})
    base = timed(chain) / n_layers
    gu_expert = 2 * d.inter * d.hidden
    base_eager = timed_eager(chain) / n_layers
    variants = []
    for mode, tfn, b in (("graph", timed, base), ("eager", timed_eager, base_eager)):
        for plan in ("pregate", "perfect"):
            for when in ("during", "next"):
                for cap_mb in (64, 128, 256):
                    for wg in (256, 1024):
                        us = tfn(lambda: chain(plan, when, cap_mb << 20, wg)) / n_layers
                        variants.append({"launch": mode, "plan": plan, "when": when, "cap_mb": cap_mb,
                                         "workgroups": wg, "us_per_layer": round(us, 2),
                                         "saved_us_per_layer": round(b - us, 2)})
                        log(f"[bench] route-ahead {mode} {plan}/{when} cap {cap_mb} MB wg {wg}: {us:.1f} us/layer "
                            f"(without: {b:.1f})")
    # the cache effect alone: a prefetch serialized right before the layer it serves, against the
    # chain plus the prefetches timed on their own; and a second read of the same bytes right after
    # the first, against the first (per prefetched layer)
    pf_bytes = sum(len(unions[l]) * gu_expert for l in range(1, n_layers)) / (n_layers - 1)
    per_pf = n_layers / (n_layers - 1)
    serial_rows, reread_rows = [], []
    for cap_mb in (32, 64, 128, 192, 1 << 20):
        cap = cap_mb << 20
        serial = timed(lambda: chain("perfect", cap=cap, serial=True)) / n_layers
        alone = timed(lambda: prefetch_only(cap)) / n_layers * per_pf
        twice = timed(lambda: prefetch_twice(cap)) / n_layers * per_pf
        nbytes = float(np.mean([min(len(unions[l]) * gu_expert, cap) for l in range(1, n_layers)]))
        gain = (base * n_layers + alone * (n_layers - 1) - serial * n_layers) / (n_layers - 1)
        label = "all" if cap_mb >= 1 << 20 else cap_mb
        serial_rows.append({"cap_mb": label, "bytes_per_layer": int(nbytes), "prefetch_alone_us": round(alone, 2),
                            "serial_us_per_layer": round(serial, 2), "warm_layer_gain_us": round(gain, 2)})
        reread_rows.append({"cap_mb": label, "first_read_gbs": round(nbytes / (alone * 1e-6) / 1e9, 1),
                            "second_read_gbs": round(nbytes / max(twice - alone, 1e-3) / 1e3, 1)})
        log(f"[bench] route-ahead serial cap {label} MB: prefetch {alone:.1f} us ({nbytes / 1e6:.0f} MB), "
            f"layer gain when warm {gain:.1f} us; re-read {reread_rows[-1]['second_read_gbs']:.0f} GB/s vs first "
            f"{reread_rows[-1]['first_read_gbs']:.0f} GB/s")
    wide = timed(lambda: prefetch_only(1 << 40, 1024)) / n_layers * per_pf
    log(f"[bench] route-ahead: coverage {np.mean([p['coverage'] for p in per_layer]):.3f}")
    del ws, ws_side
    return {"workload": f"{n_layers} chained span-8 decode layers (own router per layer, weights of replica l mod "
                        f"{len(reps)}), residual stream h_(l+1) = h_l + y_l, x_(l+1) = RMSNorm(h_(l+1)); plan for "
                        "layer l+1 = union of x_l routed by layer l+1's router (pre-gating), gate/up bytes prefetched",
            "chain_outputs_identical": same,
            "plan_quality": per_layer,
            "mean_coverage": round(float(np.mean([p["coverage"] for p in per_layer])), 4),
            "mean_waste": round(float(np.mean([p["waste"] for p in per_layer])), 4),
            "us_per_layer_without": round(base, 2),
            "us_per_layer_without_eager": round(base_eager, 2),
            "variants": variants,
            "serial_perfect": serial_rows,
            "reread": reread_rows,
            "union_gate_up_bytes_per_layer": int(pf_bytes),
            "prefetch_all_1024_workgroups_us": round(wide, 2),
            "timing": "us per layer: hipGraph replay of the whole chain (both streams captured), and eager "
                      "launches on two streams (the side stream joined at the end of each chain)"}


def cpu_oracle_baseline(synth, cfg, x_np, mask_np, nu, total_b, M, union):
    """The CPU oracle, as it stands, on the span-8 step (the JSON line's
    baseline, on every host core the process may use), and its wall time on
    the tiny, span-8 and DP8 steps with one thread and with all of them.
    Expert weights come from the seeded generator in their row-major
    checkpoint layout, as the oracle takes them."""
    import oracle
    from threadpoolctl import threadpool_limits
    threads, model = cpu_info()

    def run(c, union_hint=None):
        d = c.dims
        x, mk = synth.activations(c)
        host = {}
        if union_hint is not None:
            synth.for_each_expert(c, 0, lambda e, t: host.__setitem__(e, t), experts=union_hint)

        def expert(e):
            if e not in host:
                host[e] = synth.routed_expert(c, 0, e)
            return host[e]
        wr, b, sh = synth.router_weight(c, 0), synth.router_bias(c, 0), synth.shared_expert(c, 0)
        # the experts a step needs are generated before the timed part
        ids, _, _ = oracle.route(x, mk, wr, b, d.top_k, d.routed_scale)
        for e in sorted(set(int(v) for v in ids[mk != 0].ravel())):
            expert(e)
        t1 = {}
        for label, lim in (("threads_all", threads), ("threads_1", 1)):
            with threadpool_limits(lim):
                c0 = time.time()
                oracle.layer(x, mk, wr, b, d.top_k, d.routed_scale, expert, sh)
                t1[label] = round(time.time() - c0, 3)
        return t1

    log(f"[bench] CPU oracle ({threads} threads and 1 thread): tiny, span8, dp8")
    secs = {"tiny": run(synth.CONFIGS["tiny"]), "span8": run(cfg, union), "dp8": run(synth.CONFIGS["dp8"])}
    cpu_s = secs["span8"]["threads_all"]
    base = {"value": round(total_b / cpu_s / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"one whole span-8 step ({M} rows, |U|={nu}) in {cpu_s:.2f} s on {model}; float64 numpy; "
                      "the same algorithmic bytes as the GPU line over the oracle's wall time",
            "seconds": cpu_s}
    log(f"[bench] oracle seconds: {secs}")
    return base, {"cores_all": threads, "cpu_model": model, **secs}


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4, help="device copies of the decode layer's weights")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="only the prefill part (profiling)")
    ap.add_argument("--prefill-layers", type=int, default=4, help="stacked layers of the prefill step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweeps", action="store_true",
                    help="skip the row-count and TP8-rank sweeps and the DP8 and 512-token legs")
    ap.add_argument("--route-ahead-only", action="store_true", help="only the span-8 step and the route-ahead leg")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs the layer on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path has no inter-GPU sharding)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import sparse_moe_ffn_02_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calib_copy:
        n = args.calib_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x5")
        return
    lib = moe.load()
    if args.prefill_only:
        pd = synth.CONFIGS["prefill4096x4"].dims
        pmd = moe.Dims(pd.hidden, pd.n_experts, pd.top_k, pd.inter, pd.shared_inter, pd.routed_scale)
        pev = HipEvents(2)
        pev.rt.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        out = prefill_bench(args, torch, moe, synth, pmd, pd, pev, pev.rt, torch.cuda.current_stream().cuda_stream,
                            lib)
        pev.close()
        print(json.dumps({"prefill": out}), flush=True)
        return

    # ---------------- decode: span-8 step
    cfg = synth.CONFIGS["span8"]
    d = cfg.dims
    md = moe.Dims(d.hidden, d.n_experts, d.top_k, d.inter, d.shared_inter, d.routed_scale)
    t0 = time.time()
    log(f"[bench] generating span8 layer (seed {cfg.seed}) x{args.replicas} replicas")
    reps = device_layer(cfg, 0, torch, moe, replicas=args.replicas)
    log(f"[bench] layer ready in {time.time() - t0:.1f}s")
    x_np, mask_np = synth.activations(cfg)
    M = cfg.rows
    x = torch.from_numpy(x_np.view(np.int16)).cuda()
    mask = torch.from_numpy(mask_np).cuda()
    ws = moe.workspace(md, M)
    y = torch.empty((M, d.hidden), dtype=torch.int16, device="cuda")
    rt = moe.Routing.empty(md, M)

    def step(i):
        r = reps[i % len(reps)]
        moe.layer(md, x, mask, r["router_w"], r["bias"], r["experts"], r["shared"], y, rt, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nu = int(rt.n_union.item())
    slots = int(rt.offs[nu].item())
    ev = HipEvents(2)
    stream = torch.cuda.current_stream().cuda_stream
    rt_lib = ev.rt
    rt_lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
    torch.cuda.synchronize()
    rt_lib.hipEventRecord(ev.ev[0], C.c_void_p(stream))
    for i in range(args.steps):
        step(i)
    rt_lib.hipEventRecord(ev.ev[1], C.c_void_p(stream))
    torch.cuda.synchronize()
    ms_eager = ev.elapsed_ms(ev.ev[0], ev.ev[1]) / args.steps
    routed_b, fixed_b = decode_bytes(nu, d, M)
    total_b = routed_b + fixed_b
    log(f"[bench] span8 eager: {ms_eager * 1e3:.1f} us/step, |U|={nu}, {total_b / 1e6:.1f} MB -> "
        f"{total_b / (ms_eager * 1e-3) / 1e9:.0f} GB/s")

    # graph replay: one captured step per weight replica, replayed in rotation
    us_step, us_p10, us_p50, us_p90 = graph_replay_us(torch, step, len(reps), args.steps, args.warmup, rt_lib,
                                                      stream)
    log(f"[bench] span8 graph replay, one call per graph: {us_step:.1f} us/step (single replays p10/p50/p90 "
        f"{us_p10:.1f}/{us_p50:.1f}/{us_p90:.1f})")
    # a graph of consecutive layer calls (replicas in rotation), as a decode graph holds them
    n_chain = 4 * len(reps)
    us_chain, ch_p10, ch_p50, ch_p90 = graph_chain_us(torch, step, n_chain, args.steps, args.warmup, rt_lib, stream)
    log(f"[bench] span8 graph replay, {n_chain} consecutive calls per graph: {us_chain:.1f} us/step "
        f"(per replay p10/p50/p90 {ch_p10:.1f}/{ch_p50:.1f}/{ch_p90:.1f})")
    # hot weights: the same chain on one replica only (its weights partly held in the caches between calls)
    us_hot = graph_chain_us(torch, lambda i: step(0), n_chain, args.steps, args.warmup, rt_lib, stream)[0]
    log(f"[bench] span8 hot weights (one replica): {us_hot:.1f} us/step")
    copy_bw = copy_gbs(torch, rt_lib, stream)
    log(f"[bench] device copy: {copy_bw:.0f} GB/s")
    ms_step = min(us_step, us_chain) * 1e-3
    gbs = total_b / (ms_step * 1e-3) / 1e9
    log(f"[bench] span8: {ms_step * 1e3:.1f} us/step -> {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of peak)")

    # traced pass: per-kernel HIP events, same steps, same stream
    kern_us = traced_kernel_us(lib, torch, step, args.steps)
    streaming = {k: v for k, v in kern_us.items() if kernel_bytes(k, nu, d, M) is not None}
    dom = max(streaming, key=lambda k: streaming[k])
    dom_bytes = kernel_bytes(dom, nu, d, M)
    dom_gbs = dom_bytes / (kern_us[dom] * 1e-6) / 1e9
    log(f"[bench] kernels (us): " + ", ".join(f"{k}={v:.1f}" for k, v in kern_us.items()))
    log(f"[bench] kernel GB/s: " + ", ".join(
        f"{k}={kernel_bytes(k, nu, d, M) / (v * 1e-6) / 1e9:.0f}" for k, v in streaming.items()))

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "span-8 decode step: 8 rows of one request (1 committed + 7 drafts), hidden 6144, "
                               "256 routed experts top-8, inter 2048 fp8 e4m3 128x128 block scales, "
                               "1 bf16 shared expert inter 2048; weights rotated over "
                               f"{args.replicas} device replicas (read from HBM every step)",
                   "rows": M, "union_experts": nu, "slots": slots, "seed": cfg.seed},
        "layer_us": round(ms_step * 1e3, 2),
        "layer_us_eager": round(ms_eager * 1e3, 2),
        "layer_us_graph_one_call": round(us_step, 2),
        "layer_us_graph_chain": round(us_chain, 2),
        "layer_us_single_replay_p10_p50_p90": [round(us_p10, 2), round(us_p50, 2), round(us_p90, 2)],
        "layer_us_graph_chain_p10_p50_p90": [round(ch_p10, 2), round(ch_p50, 2), round(ch_p90, 2)],
        "layer_us_hot_weights": round(us_hot, 2),
        "timing": (f"hipGraph replay, the faster of one moe_layer call per graph and {n_chain} consecutive "
                   "calls per graph (weight replicas in rotation, as a decode graph over consecutive layers "
                   "holds them); every call reads its replica's weights from HBM; eager launches also "
                   "reported"),
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "copy_gbs": round(copy_bw, 1),
        "frac_of_copy": round(gbs / copy_bw, 4),
        "copy_note": "torch device-to-device copy of 1 GiB, bytes read + written per second, same GPU, same run",
        "bytes_per_step": total_b,
        "routed_weight_bytes": routed_b,
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dom),
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes": dom_bytes, "kernel_us": round(kern_us[dom], 2),
                     "frac_of_copy": round(dom_gbs / copy_bw, 4)},
    }

    # ---------------- the layer with the next layer's residual add + RMSNorm, unfused and fused
    res_np, gam_np = synth.norm_inputs(cfg, rows=M)
    res = torch.from_numpy(res_np.view(np.int16)).cuda()
    gam = torch.from_numpy(gam_np.view(np.int16)).cuda()
    r_out = torch.empty_like(res)
    n_out = torch.empty_like(res)

    def step_unfused(i):
        step(i)
        moe.add_rmsnorm(y, mask, res, gam, 1e-6, r_out, n_out)

    def step_fused(i):
        r = reps[i % len(reps)]
        moe.layer_add_rmsnorm(md, x, mask, r["router_w"], r["bias"], r["experts"], r["shared"], res, gam, 1e-6,
                              y, r_out, n_out, rt, ws)

    us_unf = graph_replay_us(torch, step_unfused, len(reps), args.steps, args.warmup, rt_lib, stream)[0]
    us_fus = graph_replay_us(torch, step_fused, len(reps), args.steps, args.warmup, rt_lib, stream)[0]
    log(f"[bench] span8 + residual add + RMSNorm: unfused {us_unf:.1f} us, fused {us_fus:.1f} us")
    result["add_rmsnorm"] = {"workload": "span-8 step followed by the next layer's residual add + RMSNorm "
                                         "(bf16 residual [8, 6144], gamma [6144], eps 1e-6)",
                             "unfused_us": round(us_unf, 2), "fused_us": round(us_fus, 2),
                             "layer_only_us": round(us_step, 2),
                             "timing": "hipGraph replay, weights rotated as above"}

    # ---------------- route-ahead prefetch of the next layer's predicted union
    if args.route_ahead_only or not args.no_sweeps:
        result["route_ahead"] = route_ahead_bench(torch, moe, synth, cfg, md, d, reps, rt_lib, stream)
    if args.route_ahead_only:
        ev.close()
        print(json.dumps(result), flush=True)
        return

    # ---------------- the other decode and chunk workloads on the same layer
    if not args.no_sweeps:
        # DP8 step: 8 independent rows, pads at slots 2, 5, 7 (a larger union)
        dcfg = synth.CONFIGS["dp8"]
        xd_np, md_np = synth.activations(dcfg)
        xd = torch.from_numpy(xd_np.view(np.int16)).cuda()
        mkd = torch.from_numpy(md_np).cuda()

        def step_dp8(i):
            r = reps[i % len(reps)]
            moe.layer(md, xd, mkd, r["router_w"], r["bias"], r["experts"], r["shared"], y, rt, ws)

        us_dp8 = graph_replay_us(torch, step_dp8, len(reps), args.steps, args.warmup, rt_lib, stream)[0]
        nu_dp8 = int(rt.n_union.item())
        rb8, fb8 = decode_bytes(nu_dp8, d, M)
        result["dp8"] = {"workload": "DP8-style decode step: 8 independent rows (pads at slots 2, 5, 7), same layer",
                         "us": round(us_dp8, 2), "union_experts": nu_dp8, "bytes": rb8 + fb8,
                         "gbs": round((rb8 + fb8) / (us_dp8 * 1e-6) / 1e9, 1),
                         "hbm_frac": round((rb8 + fb8) / (us_dp8 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] dp8: {us_dp8:.1f} us, |U|={nu_dp8}, {(rb8 + fb8) / (us_dp8 * 1e-6) / 1e9:.0f} GB/s")
        # 512-token chunk with the Zipf-skewed router bias
        pcfg5 = synth.CONFIGS["prefill512"]
        xp_np, mp_np = synth.activations(pcfg5)
        xp5 = torch.from_numpy(xp_np.view(np.int16)).cuda()
        mp5 = torch.from_numpy(mp_np).cuda()
        zb = torch.from_numpy(np.ascontiguousarray(synth.router_bias(pcfg5), dtype=np.float32)).cuda()
        m5 = pcfg5.rows
        ws5 = moe.workspace(md, m5)
        y5 = torch.empty((m5, d.hidden), dtype=torch.int16, device="cuda")
        rt5 = moe.Routing.empty(md, m5)

        def step_p512(i):
            r = reps[i % len(reps)]
            moe.layer(md, xp5, mp5, r["router_w"], zb, r["experts"], r["shared"], y5, rt5, ws5)

        us_p5 = graph_replay_us(torch, step_p512, len(reps), min(args.steps, 50), min(args.warmup, 5), rt_lib, stream)[0]
        nu5 = int(rt5.n_union.item())
        sl5 = int(rt5.offs[nu5].item())
        rb5, fb5 = decode_bytes(nu5, d, m5)
        f8, f16, fr = layer_flops(d, m5, sl5)
        result["prefill512"] = {"workload": "512-token chunk, Zipf(1.1) router bias, same layer",
                                "us": round(us_p5, 2), "union_experts": nu5,
                                "tflops_total": round((f8 + f16 + fr) / (us_p5 * 1e-6) / 1e12, 2),
                                "hbm_frac": round((rb5 + fb5) / (us_p5 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] prefill512: {us_p5:.1f} us, |U|={nu5}, {(rb5 + fb5) / (us_p5 * 1e-6) / 1e9:.0f} GB/s")
        del ws5, y5

    # ---------------- CPU oracle baseline on the same decode step
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["cpu_oracle_seconds"] = cpu_oracle_baseline(
            synth, cfg, x_np, mask_np, nu, total_b, M, [int(e) for e in rt.union_ids[:nu].cpu().numpy()])
    if not args.no_sweeps:
        result["rows_sweep"] = rows_sweep(torch, moe, synth, md, d, reps, rt_lib, stream, min(args.steps, 100),
                                          args.warmup)
    del reps
    torch.cuda.empty_cache()
    if not args.no_sweeps:
        result["tp8_rank_sweep"] = tp8_rank_sweep(torch, moe, synth, rt_lib, stream, min(args.steps, 100),
                                                  args.warmup, args.replicas)

    if not args.no_prefill:
        result["prefill"] = prefill_bench(args, torch, moe, synth, md, d, ev, rt_lib, stream, lib)
    ev.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
