"""Oracle for the dispatch pool (test infrastructure only).

Source: DeepGEMM PR #9 "feat(mega): add fused shared side-LoRA kernels",
section "2026-09-21: restore wide-K wgrad safely" -> Implementation (pool rows
of each expert start at the expert's true physical offset; group starts are
not rounded into a neighbour), and "Historical implementation" -> Summary
(expert padding is zeroed before shared contractions).  PR #17 "Align MegaMoE
training with upgraded K-grouped TMA and layouts", Summary: one pool layout
serves forward and backward, and the block size is queried from the library.

Reading taken where the pages are silent: within one expert, rows follow the
ascending flat route index f = t*k + j (the pages' atomic dispatch leaves the
order free); a route id of -1 is a dropped route and gets no row; any other
id outside [0, E) is an error, is dropped and is counted.

Written as a plain sort plus the closed-form offsets, in pure Python.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def capacity(T: int, topk: int, E: int, block_m: int) -> int:
    """Upper bound on pool rows for any routing: every active route gets a row
    and each non-empty expert adds at most block_m - 1 padding rows."""
    routes = T * topk
    return routes + min(E, routes) * (block_m - 1)


def build_pool(topk_idx: np.ndarray, E: int, block_m: int,
               cap: Optional[int] = None) -> Dict[str, np.ndarray]:
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    if cap is None:
        cap = capacity(T, k, E, block_m)
    routes = []          # (expert, flat route index)
    bad = 0
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e == -1:
                continue
            if e < 0 or e >= E:
                bad += 1
                continue
            routes.append((e, t * k + j))
    counts = [0] * E
    for e, _ in routes:
        counts[e] += 1
    padded = [((c + block_m - 1) // block_m) * block_m for c in counts]
    offsets = [0]
    for p in padded:
        offsets.append(offsets[-1] + p)
    route_to_row = [-1] * (T * k)
    row_to_route = [-1] * cap
    nxt = list(offsets[:-1])
    for e, f in sorted(routes):
        row = nxt[e]
        nxt[e] += 1
        route_to_row[f] = row
        row_to_route[row] = f
    return {
        "counts": np.array(counts, dtype=np.int32),
        "offsets": np.array(offsets, dtype=np.int32),
        "route_to_row": np.array(route_to_row, dtype=np.int32),
        "row_to_route": np.array(row_to_route, dtype=np.int32),
        "bad_routes": np.int64(bad),
        "capacity": np.int64(cap),
    }


def gather_pool(x: np.ndarray, pool: Dict[str, np.ndarray], topk: int) -> np.ndarray:
    """The saved expert input: row p holds the token of route row_to_route[p],
    padding rows are zero (PR #9, Historical implementation -> Summary)."""
    r2r = pool["row_to_route"]
    out = np.zeros((len(r2r), x.shape[1]), dtype=x.dtype)
    for p, f in enumerate(r2r):
        if f >= 0:
            out[p] = x[f // topk]
    return out
