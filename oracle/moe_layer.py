"""Plain, slow CPU oracle of the routed fp8 MoE FFN layer (test infrastructure).

Every step follows the statement of the problem on the pages, written out in
float64 numpy with no blocking, fusion or reordering beyond what the
definition states.  Readings of points the pages leave open are marked
"reading:".

Steps and their sources:

* routing -- noaux-tc router: a score per expert, an e_score_correction_bias
  added for selection only, top-k (mstar PR #388, "Tests"/router notes:
  NoAuxTcRouter._topk_op and the router kernel; MoE-Infinity PR #140, the
  "[256] router bias" of the resident-weight mis-map fix).  Reading: the score
  is the sigmoid of the logit, the selected sigmoids are renormalized to sum
  to 1 and scaled by 2.5; ties go to the lower expert id.
* union and compaction -- the step's rows share one expert union whose order
  is the same under every row mapping (openinfer PR #610, "What" and "Gates").
  Reading: ascending expert id, rows ascending inside each expert.
* activation quantization -- e4m3 per 128 columns (mstar PR #388, FlashInfer
  crossover note).  Reading: s = fl32(amax / 448), codes = RNE-saturating
  e4m3 of fl32(x / s); an all-zero block gets s = 1 and zero codes.
* gate/up and down GEMMs with fp8 weights and 128x128 block scales, weights
  stored as a [gate_proj, up_proj, down_proj] triple (MoE-Infinity PR #140,
  expert-node commit; mstar PR #388, kernel switches note: the reference mode
  is the per-expert dequant loop).
* SiLU(gate) * up (openinfer PR #610, "What": union/GEMM/SiLU phases), then
  the same 1x128 quantization of the result.
* fixed-order weighted combine plus the shared expert; pad rows are written
  as zeros and are never read (openinfer PR #610, description and "Gates").
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from .codec import decode_bf16, decode_e4m3, encode_bf16, encode_e4m3

BLOCK = 128
E4M3_MAX = np.float32(448.0)


def sigmoid(l: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(l, dtype=np.float64)))


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def route(x_bits: np.ndarray, row_mask: np.ndarray, router_w_bits: np.ndarray,
          bias: np.ndarray, top_k: int, routed_scale: float = 2.5):
    """Top-k routing of every real row.

    logits l = x . Wr^T (bf16 operands, exact products, float64 sums);
    selection score c = sigmoid(l) + bias; the k largest c are selected,
    ties to the lower expert id; weights w = scale * sigmoid(l_j) / sum_sel.

    Returns ids int32 [M, k] ascending per row, w float64 [M, k] in the same
    order, and the float64 logits of the real rows.  Pad rows: ids -1, w 0.
    """
    m = x_bits.shape[0]
    e = router_w_bits.shape[0]
    if not (0 < top_k <= e):
        raise ValueError("top_k must be in [1, n_experts]")
    real = np.flatnonzero(np.asarray(row_mask) != 0)
    ids = np.full((m, top_k), -1, dtype=np.int32)
    w = np.zeros((m, top_k), dtype=np.float64)
    logits = np.zeros((m, e), dtype=np.float64)
    if real.size == 0:
        return ids, w, logits
    x = decode_bf16(x_bits[real])
    wr = decode_bf16(router_w_bits)
    l = x @ wr.T
    logits[real] = l
    sig = sigmoid(l)
    c = sig + np.asarray(bias, dtype=np.float64)[None, :]
    for i, r in enumerate(real):
        order = np.argsort(-c[i], kind="stable")      # stable: ties keep the lower id first
        sel = np.sort(order[:top_k])
        tot = 0.0
        for j in sel:                                  # ascending id
            tot += sig[i, j]
        ids[r] = sel
        w[r] = routed_scale * (sig[i, sel] / tot)
    return ids, w, logits


@dataclass
class Routing:
    ids: np.ndarray        # int32 [M, k]
    w: np.ndarray          # float64 [M, k]
    union_ids: np.ndarray  # int32 [n_union], ascending
    offs: np.ndarray       # int32 [n_union + 1]
    rows: np.ndarray       # int32 [slots]: row of each slot
    slot_of: np.ndarray    # int32 [M, k]: slot of (row, j); -1 for pad rows

    @property
    def n_union(self) -> int:
        return int(self.union_ids.size)


def union(ids: np.ndarray, w: np.ndarray, row_mask: np.ndarray) -> Routing:
    """Expert union of the real rows (ascending id) and per-expert row lists.

    Slots are numbered expert by expert in union order; inside an expert its
    rows are ascending.
    """
    m, k = ids.shape
    real = np.asarray(row_mask) != 0
    used = sorted({int(e) for r in range(m) if real[r] for e in ids[r]})
    offs = [0]
    rows: List[int] = []
    slot_of = np.full((m, k), -1, dtype=np.int32)
    for e in used:
        for r in range(m):
            if not real[r]:
                continue
            hit = np.flatnonzero(ids[r] == e)
            if hit.size:
                slot_of[r, hit[0]] = len(rows)
                rows.append(r)
        offs.append(len(rows))
    return Routing(ids=ids, w=w, union_ids=np.array(used, dtype=np.int32),
                   offs=np.array(offs, dtype=np.int32), rows=np.array(rows, dtype=np.int32),
                   slot_of=slot_of)


# ----------------------------------------------------------------------------
# 1x128 quantization
# ----------------------------------------------------------------------------

def quant_1x128(v: np.ndarray):
    """float32 [R, K] -> (e4m3 codes uint8 [R, K], float32 scales [R, K/128]).

    Per row and 128-column block, in float32 arithmetic: a = max |v|;
    a == 0 -> s = 1 and all codes 0; else s = fl32(a / 448) and
    code = e4m3_rne_sat(fl32(v / s)).
    """
    v = np.asarray(v, dtype=np.float32)
    r, k = v.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    b = v.reshape(r, k // BLOCK, BLOCK)
    a = np.abs(b).max(axis=2)
    zero = a == 0
    s = np.where(zero, np.float32(1.0), a / E4M3_MAX).astype(np.float32)
    q = (b / s[:, :, None]).astype(np.float32)
    codes = encode_e4m3(q)
    codes[zero] = 0
    return codes.reshape(r, k), s


# ----------------------------------------------------------------------------
# block-scaled fp8 GEMM
# ----------------------------------------------------------------------------

def block_gemm(a_codes: np.ndarray, a_scales: np.ndarray,
               w_codes: np.ndarray, w_scales: np.ndarray) -> np.ndarray:
    """out[i, n] = sum_kb s_a[i, kb] * s_w[n // 128, kb] * sum_{h in kb} a[i, h] * w[n, h].

    a: codes [m, K] with scales [m, K/128]; w: codes [N, K] with scales
    [N/128, K/128].  Each 128-term inner sum is exact in float64 (every
    product is a multiple of 2^-18 below 2^18, so the sum needs < 44 bits),
    so the library matmul used for it is exact in any order.  K-blocks are
    accumulated in ascending order.
    """
    m, k = a_codes.shape
    n = w_codes.shape[0]
    a = decode_e4m3(a_codes)
    w = decode_e4m3(w_codes)
    out = np.zeros((m, n), dtype=np.float64)
    for kb in range(k // BLOCK):
        sl = slice(kb * BLOCK, (kb + 1) * BLOCK)
        p = a[:, sl] @ w[:, sl].T
        sw = np.repeat(w_scales[:, kb].astype(np.float64), BLOCK)
        out += (a_scales[:, kb].astype(np.float64)[:, None] * sw[None, :]) * p
    return out


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------

@dataclass
class ExpertOut:
    h_codes: np.ndarray    # uint8 [m, I]
    h_scales: np.ndarray   # float32 [m, I/128]
    d: np.ndarray          # float64 [m, H]


def routed_expert(x_codes: np.ndarray, x_scales: np.ndarray, ew: Dict[str, np.ndarray]) -> ExpertOut:
    """One routed expert on its rows: gate/up GEMMs, SiLU(gate)*up,
    1x128 requantization, down GEMM."""
    g = block_gemm(x_codes, x_scales, ew["gate"], ew["s_gate"])
    u = block_gemm(x_codes, x_scales, ew["up"], ew["s_up"])
    h32 = (silu(g) * u).astype(np.float32)
    hq, hs = quant_1x128(h32)
    d = block_gemm(hq, hs, ew["down"], ew["s_down"])
    return ExpertOut(hq, hs, d)


def shared_expert(x_bits: np.ndarray, sw: Dict[str, np.ndarray]) -> np.ndarray:
    """bf16 shared expert on rows x: g, u = x Wg^T, x Wu^T; h = bf16(fl32(silu(g) u));
    S = h Wd^T.  float64 sums."""
    x = decode_bf16(x_bits)
    g = x @ decode_bf16(sw["gate"]).T
    u = x @ decode_bf16(sw["up"]).T
    h = decode_bf16(encode_bf16((silu(g) * u).astype(np.float32)))
    return h @ decode_bf16(sw["down"]).T


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

@dataclass
class LayerOut:
    routing: Routing
    x_codes: np.ndarray          # uint8 [M, H] (pad rows 0)
    x_scales: np.ndarray         # float32 [M, H/128] (pad rows 0)
    h_codes: Dict[int, np.ndarray]   # slot -> uint8 [I]   (evaluated slots)
    h_scales: Dict[int, np.ndarray]  # slot -> float32 [I/128]
    y_ref: np.ndarray            # float64 [M, H] before bf16 rounding (NaN where not evaluated)
    y_bits: np.ndarray           # uint16 [M, H]
    evaluated: np.ndarray        # rows whose outputs were computed


def quant_rows(x_bits: np.ndarray, row_mask: np.ndarray):
    """x codes/scales for real rows; pad rows left zero and never read."""
    m, h = x_bits.shape
    codes = np.zeros((m, h), dtype=np.uint8)
    scales = np.zeros((m, h // BLOCK), dtype=np.float32)
    real = np.flatnonzero(np.asarray(row_mask) != 0)
    if real.size:
        xf = decode_bf16(x_bits[real]).astype(np.float32)
        codes[real], scales[real] = quant_1x128(xf)
    return codes, scales


def ffn(x_bits: np.ndarray, row_mask: np.ndarray, routing: Routing,
        expert: Callable[[int], Dict[str, np.ndarray]],
        shared: Optional[Dict[str, np.ndarray]] = None,
        rows: Optional[Sequence[int]] = None,
        pmap: Callable = map) -> LayerOut:
    """Routed experts (+ shared expert when given) and the fixed-order combine.

    y[r] = bf16( (((0 + w_1 D_1) + w_2 D_2) + ... + w_k D_k) + S[r] ) with
    the row's experts in ascending id.  `rows` restricts the evaluation to a
    subset of rows (each row is independent of the others); pad rows are
    always +0.0.  `pmap` (a map-like callable, e.g. a thread pool's map)
    evaluates the union experts; each expert's output depends on its own rows
    only, so the order in which they are evaluated changes nothing.
    """
    m, hdim = x_bits.shape
    real = np.asarray(row_mask) != 0
    xq, xs = quant_rows(x_bits, row_mask)
    want = np.flatnonzero(real) if rows is None else np.array(sorted(set(int(r) for r in rows if real[r])), dtype=np.int64)
    want_set = set(int(r) for r in want)
    y_ref = np.full((m, hdim), np.nan)
    y_ref[~real] = 0.0
    dslot: Dict[int, np.ndarray] = {}
    hq: Dict[int, np.ndarray] = {}
    hs: Dict[int, np.ndarray] = {}
    work = []
    for u, e in enumerate(routing.union_ids):
        lo, hi = int(routing.offs[u]), int(routing.offs[u + 1])
        slots = [s for s in range(lo, hi) if int(routing.rows[s]) in want_set]
        if slots:
            work.append((int(e), slots))

    def run(item):
        e, slots = item
        r_of = routing.rows[slots]
        return slots, routed_expert(xq[r_of], xs[r_of], expert(e))

    for slots, out in pmap(run, work):
        for i, s in enumerate(slots):
            dslot[s] = out.d[i]
            hq[s] = out.h_codes[i]
            hs[s] = out.h_scales[i]
    s_rows = None
    if shared is not None and len(want):
        s_rows = shared_expert(x_bits[want], shared)
    for i, r in enumerate(want):
        acc = np.zeros(hdim, dtype=np.float64)
        for j in range(routing.ids.shape[1]):          # ids ascending
            acc = acc + routing.w[r, j] * dslot[int(routing.slot_of[r, j])]
        if s_rows is not None:
            acc = acc + s_rows[i]
        y_ref[r] = acc
    y_bits = np.zeros((m, hdim), dtype=np.uint16)
    if len(want):
        y_bits[want] = encode_bf16(y_ref[want])
    return LayerOut(routing, xq, xs, hq, hs, y_ref, y_bits, want)


def layer(x_bits: np.ndarray, row_mask: np.ndarray, router_w_bits: np.ndarray, bias: np.ndarray,
          top_k: int, routed_scale: float, expert: Callable[[int], Dict[str, np.ndarray]],
          shared: Optional[Dict[str, np.ndarray]] = None,
          rows: Optional[Sequence[int]] = None, pmap: Callable = map) -> LayerOut:
    """The whole layer: route, union, routed experts, shared expert, combine."""
    ids, w, _ = route(x_bits, row_mask, router_w_bits, bias, top_k, routed_scale)
    rt = union(ids, w, row_mask)
    return ffn(x_bits, row_mask, rt, expert, shared, rows, pmap)
