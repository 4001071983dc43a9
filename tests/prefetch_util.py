"""Expected checksum of moe_prefetch_experts, computed on the host from the
packed weight bytes copied back from the device (the fetch order and the
16 KiB chunk rounding of the entry point's contract)."""
from __future__ import annotations

import numpy as np
import torch

import sparse_moe_ffn_02_amd as moe

CHUNK = 16384


def expected_checksum(experts: moe.Experts, ids, parts: int, max_bytes: int, n_experts: int) -> int:
    mats = []
    if parts & moe.PREFETCH_GATE_UP:
        mats += [experts.w_gate, experts.w_up]
    if parts & moe.PREFETCH_DOWN:
        mats.append(experts.w_down)
    budget = (max_bytes // CHUNK) * CHUNK
    total = np.uint64(0)
    for e in ids:
        for m in mats:
            per = m[0].numel()
            # chunks are counted over the whole order, skipped experts included
            take = min(per, budget)
            budget -= take
            if 0 <= e < n_experts and take > 0:
                words = m[int(e)].reshape(-1)[:take].cpu().numpy().view(np.uint32)
                total += np.sum(words, dtype=np.uint64)
            if budget <= 0:
                return int(total % np.uint64(1 << 32))
    return int(total % np.uint64(1 << 32))


def prefetch_checksum(dims: moe.Dims, n_union: torch.Tensor, union_ids: torch.Tensor, experts: moe.Experts,
                      parts: int, max_bytes: int, workgroups: int = 0) -> int:
    cs = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.prefetch_experts(dims, n_union, union_ids, experts, parts, max_bytes, workgroups, cs)
    torch.cuda.synchronize()
    return int(cs.cpu().numpy().view(np.uint32)[0])
