"""Set measures of a route-ahead plan (MoE-Infinity PR #140, route-ahead
expert prefetch commit: the per-token union of a block's routed experts is
the prefetch plan, judged by its coverage of the experts the block then uses
and by the waste of fetching experts it does not use).

Host-side bookkeeping only, on numpy arrays copied back from the device; no
part of the layer's arithmetic.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def union_of(topk_ids: np.ndarray, row_mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Ascending ids of the experts picked by any real row of topk_ids [M, k]
    (ids < 0 are pads and ignored)."""
    ids = np.asarray(topk_ids)
    if row_mask is not None:
        ids = ids[np.asarray(row_mask).astype(bool)]
    ids = ids.reshape(-1)
    return np.unique(ids[ids >= 0]).astype(np.int64)


def coverage(planned: Iterable[int], used: Iterable[int]) -> float:
    """Share of the used experts that the plan fetched: |P n U| / |U|
    (1.0 when nothing is used)."""
    p, u = set(int(e) for e in planned), set(int(e) for e in used)
    return 1.0 if not u else len(p & u) / len(u)


def waste(planned: Iterable[int], used: Iterable[int]) -> float:
    """Share of the fetched experts that go unused: |P \\ U| / |P|
    (0.0 for an empty plan)."""
    p, u = set(int(e) for e in planned), set(int(e) for e in used)
    return 0.0 if not p else len(p - u) / len(p)


def row_agreement(planned_ids: np.ndarray, used_ids: np.ndarray, row_mask: Optional[np.ndarray] = None) -> float:
    """Mean over real rows of the share of a row's used top-k that its
    planned top-k holds (both [M, k], pads < 0 ignored)."""
    a, b = np.asarray(planned_ids), np.asarray(used_ids)
    rows = range(a.shape[0]) if row_mask is None else np.nonzero(np.asarray(row_mask))[0]
    shares = []
    for r in rows:
        used = set(int(e) for e in b[r] if e >= 0)
        if used:
            shares.append(len(used & set(int(e) for e in a[r] if e >= 0)) / len(used))
    return float(np.mean(shares)) if shares else 1.0
