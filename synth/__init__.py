"""Seeded synthetic inputs for the routed fp8 MoE FFN layer.

This module only draws numbers: it holds none of the layer's arithmetic.
Both the CPU oracle (via the tests) and the GPU path consume exactly the
arrays produced here, so a given (config, seed) always yields the same bytes.

Shapes follow the GLM-5.2 MoE block described on the pages (hidden 6144,
256 routed experts, routed experts stored as a [gate_proj, up_proj, down_proj]
fp8 triple with block scales; openinfer PR #610 "What", mstar PR #388 decode
table note, MoE-Infinity PR #140 fp8 store commits).  Distributions:

* activations x ~ N(0, 1), rounded to bf16 (RNE, via torch's bf16 cast);
* router weight Wr ~ N(0, 1)/sqrt(H) -> bf16 [E, H], so logits are ~N(0, 1);
* correction bias fp32 [E]: ~N(0, 0.1), or the Zipf-skewed rule
  b_e = (1 + pi(e))^-1.1 with pi a seeded permutation (prefill workloads);
* routed weights ~N(0, 0.02) fp32, then stored as checkpoint-style e4m3 codes
  with one fp32 scale per 128x128 block: s = amax/448 (fp32), codes are
  torch's float8_e4m3fn cast of w/s (a library conversion; weight preparation
  happens offline, outside the layer);
* shared expert ~N(0, 0.02) -> bf16;
* for the residual add + RMSNorm epilogue: residual stream ~N(0, 4) -> bf16
  [M, H] (larger than a layer output, as a residual stream is) and the norm
  weight gamma ~N(1, 0.1) -> bf16 [H].

Every tensor draws from its own PCG64 stream,
SeedSequence(entropy=seed, spawn_key=(layer, tensor_id, expert)), so experts
can be generated in parallel and in any order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

# tensor ids in the spawn key
T_X, T_WR, T_BIAS, T_WG, T_WU, T_WD, T_SG, T_SU, T_SD, T_PERT, T_ZIPF, T_RES, T_GAMMA = range(13)

BLOCK = 128


@dataclass(frozen=True)
class Dims:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    routed_scale: float = 2.5


@dataclass(frozen=True)
class Config:
    """One workload: layer dims, row count, row recipe and seed."""
    name: str
    dims: Dims
    rows: int
    seed: int
    n_layers: int = 1
    row_kind: str = "iid"          # "iid" | "span"
    pad_slots: tuple = ()          # slots that are pad rows
    bias_kind: str = "normal"      # "normal" | "zipf"


TINY = Dims(hidden=512, n_experts=16, top_k=4, inter=256, shared_inter=256)
GLM = Dims(hidden=6144, n_experts=256, top_k=8, inter=2048, shared_inter=2048)
# edge shapes: H not a multiple of 256 or 512, E not a multiple of 64, odd
# counts of 128-blocks in I and H, a single-block shared expert
ODD = Dims(hidden=640, n_experts=40, top_k=6, inter=384, shared_inter=128)
# one TP8 rank's share of the GLM layer: every expert's (and the shared
# expert's) inter slice of 2048 / 8
TP8R = Dims(hidden=6144, n_experts=256, top_k=8, inter=256, shared_inter=256)

CONFIGS: Dict[str, Config] = {
    # 8 rows, tiny layer, every row real
    "tiny": Config("tiny", TINY, 8, 1000),
    # 8 rows of one request: 1 committed token + 7 drafts (base + 0.1 noise)
    "span8": Config("span8", GLM, 8, 1001, row_kind="span"),
    # 8 independent rows, slots 2, 5, 7 are pads
    "dp8": Config("dp8", GLM, 8, 1001, pad_slots=(2, 5, 7)),
    # prefill chunk, Zipf-skewed router bias
    "prefill512": Config("prefill512", GLM, 512, 1001, bias_kind="zipf"),
    # large prefill over 4 independent layers
    "prefill4096x4": Config("prefill4096x4", GLM, 4096, 1004, n_layers=4, bias_kind="zipf"),
    # edge-shape layer (parity only), 8 rows with one pad
    "odd": Config("odd", ODD, 8, 1005, pad_slots=(3,)),
    # one TP8 rank's share, span-decode rows (token count set per use)
    "tp8rank": Config("tp8rank", TP8R, 10, 1006, row_kind="span"),
}


def _rng(seed: int, layer: int, tensor: int, expert: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(layer, tensor, expert))
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), RNE via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _block_fp8(w: np.ndarray) -> tuple:
    """[N, K] fp32 -> (e4m3 codes uint8 [N, K], fp32 scales [N/128, K/128]).

    Checkpoint-style weight preparation (not part of the layer): one scale per
    128x128 block, s = amax/448 in fp32, codes = torch float8_e4m3fn(w / s).
    An all-zero block gets s = 1.
    """
    n, k = w.shape
    t = torch.from_numpy(w).view(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    amax = t.abs().amax(dim=(1, 3), keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (t / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).reshape(n, k).numpy()
    return np.ascontiguousarray(codes), np.ascontiguousarray(s.reshape(n // BLOCK, k // BLOCK).numpy())


# ----------------------------------------------------------------------------
# per-tensor generators
# ----------------------------------------------------------------------------

def router_weight(cfg: Config, layer: int = 0) -> np.ndarray:
    d = cfg.dims
    w = _rng(cfg.seed, layer, T_WR).standard_normal((d.n_experts, d.hidden), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(d.hidden))
    return to_bf16_bits(w)


def router_bias(cfg: Config, layer: int = 0) -> np.ndarray:
    d = cfg.dims
    if cfg.bias_kind == "zipf":
        perm = _rng(cfg.seed, layer, T_ZIPF).permutation(d.n_experts)
        return np.power(1.0 + perm.astype(np.float64), -1.1).astype(np.float32)
    b = _rng(cfg.seed, layer, T_BIAS).standard_normal(d.n_experts, dtype=np.float32)
    return (b * np.float32(0.1)).astype(np.float32)


def routed_expert(cfg: Config, layer: int, e: int) -> Dict[str, np.ndarray]:
    """Codes and scales of routed expert e: gate/up [I, H], down [H, I]."""
    d = cfg.dims
    out = {}
    for name, tid, shape in (("gate", T_WG, (d.inter, d.hidden)),
                             ("up", T_WU, (d.inter, d.hidden)),
                             ("down", T_WD, (d.hidden, d.inter))):
        w = _rng(cfg.seed, layer, tid, e).standard_normal(shape, dtype=np.float32)
        w *= np.float32(0.02)
        out[name], out["s_" + name] = _block_fp8(w)
    return out


def shared_expert(cfg: Config, layer: int = 0) -> Dict[str, np.ndarray]:
    d = cfg.dims
    if d.shared_inter == 0:
        return {}
    out = {}
    for name, tid, shape in (("gate", T_SG, (d.shared_inter, d.hidden)),
                             ("up", T_SU, (d.shared_inter, d.hidden)),
                             ("down", T_SD, (d.hidden, d.shared_inter))):
        w = _rng(cfg.seed, layer, tid).standard_normal(shape, dtype=np.float32)
        w *= np.float32(0.02)
        out[name] = to_bf16_bits(w)
    return out


def activations(cfg: Config, layer: int = 0, pad_fill: str = "nan") -> tuple:
    """(x bf16 bits [M, H], row_mask uint8 [M]).

    span rows: row 0 = bf16(base), row j = bf16(base + 0.1 eps_j).
    pad rows (cfg.pad_slots) are filled with quiet-NaN bits ("nan") or zeros
    ("zero"); the layer must never read them.
    """
    d = cfg.dims
    m = cfg.rows
    if cfg.row_kind == "span":
        g = _rng(cfg.seed, layer, T_X)
        base = g.standard_normal(d.hidden, dtype=np.float32)
        eps = _rng(cfg.seed, layer, T_PERT).standard_normal((m, d.hidden), dtype=np.float32)
        x = np.repeat(base[None, :], m, axis=0)
        x[1:] += np.float32(0.1) * eps[1:]
    else:
        x = _rng(cfg.seed, layer, T_X).standard_normal((m, d.hidden), dtype=np.float32)
    bits = to_bf16_bits(x)
    mask = np.ones(m, dtype=np.uint8)
    for s in cfg.pad_slots:
        mask[s] = 0
        bits[s, :] = 0x7FC0 if pad_fill == "nan" else 0
    return bits, mask


@dataclass
class Layer:
    """One MoE layer's parameters as numpy arrays (host copies)."""
    dims: Dims
    router_w: np.ndarray
    bias: np.ndarray
    w_gate: np.ndarray   # uint8 [E, I, H]
    w_up: np.ndarray     # uint8 [E, I, H]
    w_down: np.ndarray   # uint8 [E, H, I]
    s_gate: np.ndarray   # f32 [E, I/128, H/128]
    s_up: np.ndarray
    s_down: np.ndarray   # f32 [E, H/128, I/128]
    shared: Dict[str, np.ndarray] = field(default_factory=dict)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def for_each_expert(cfg: Config, layer: int, fn: Callable[[int, Dict[str, np.ndarray]], None],
                    experts: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> None:
    """Generate routed experts in parallel and hand each to fn(e, tensors).

    fn is called from the calling thread, in ascending expert order, so it may
    copy into device memory without locking.
    """
    ids = list(range(cfg.dims.n_experts)) if experts is None else list(experts)
    threads = threads or default_threads()
    with ThreadPoolExecutor(threads) as ex:
        window = threads * 2
        futs = {}
        nxt = 0
        for i, e in enumerate(ids):
            while nxt < len(ids) and nxt < i + window:
                futs[nxt] = ex.submit(routed_expert, cfg, layer, ids[nxt])
                nxt += 1
            fn(e, futs.pop(i).result())


def make_layer(cfg: Config, layer: int = 0, threads: Optional[int] = None) -> Layer:
    """All parameters of one layer on the host (9.7 GB of codes at GLM size)."""
    d = cfg.dims
    E, I, H = d.n_experts, d.inter, d.hidden
    wg = np.empty((E, I, H), np.uint8)
    wu = np.empty((E, I, H), np.uint8)
    wd = np.empty((E, H, I), np.uint8)
    sg = np.empty((E, I // BLOCK, H // BLOCK), np.float32)
    su = np.empty_like(sg)
    sd = np.empty((E, H // BLOCK, I // BLOCK), np.float32)

    def put(e, t):
        wg[e], wu[e], wd[e] = t["gate"], t["up"], t["down"]
        sg[e], su[e], sd[e] = t["s_gate"], t["s_up"], t["s_down"]

    for_each_expert(cfg, layer, put, threads=threads)
    return Layer(d, router_weight(cfg, layer), router_bias(cfg, layer),
                 wg, wu, wd, sg, su, sd, shared_expert(cfg, layer))


def with_rows(cfg: Config, rows: int) -> Config:
    return replace(cfg, rows=rows)


def norm_inputs(cfg: Config, layer: int = 0, rows: Optional[int] = None) -> tuple:
    """(residual bf16 bits [rows, H], gamma bf16 bits [H]) for the residual
    add + RMSNorm epilogue; rows defaults to the config's row count."""
    m = cfg.rows if rows is None else rows
    h = cfg.dims.hidden
    res = _rng(cfg.seed, layer, T_RES).standard_normal((m, h), dtype=np.float32) * np.float32(2.0)
    gamma = np.float32(1.0) + np.float32(0.1) * _rng(cfg.seed, layer, T_GAMMA).standard_normal(h, dtype=np.float32)
    return to_bf16_bits(res), to_bf16_bits(gamma)
