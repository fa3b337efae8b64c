"""Static expert placements, the comparator of the shared LRU slot cache (FreeToken linux guide,
performance/compat: global LRU against a static placement).

A static placement fixes the resident (layer, expert) keys before the trace; every access to
another key is a miss and nothing is ever copied in.  `partition` is routing-unaware: the C slots
are split evenly over the layers (the first C mod L layers get one more) and each layer holds its
lowest-numbered experts.  `top_frequency` pins the C keys used most often in the trace (ties:
lower layer, then lower expert): the best any static placement can do on that trace.
"""
from __future__ import annotations

import numpy as np


def _access_counts(trace: np.ndarray, L: int, E: int) -> np.ndarray:
    """Decode accesses per key [L, E]: one per distinct id per (step, layer)."""
    steps, _, k = trace.shape
    hit = np.zeros((steps, L, E), dtype=bool)
    s_idx = np.repeat(np.arange(steps), L * k)
    l_idx = np.tile(np.repeat(np.arange(L), k), steps)
    hit[s_idx, l_idx, trace.reshape(-1)] = True
    return hit.sum(axis=0)


def resident_mask(trace: np.ndarray, L: int, E: int, C: int, placement: str) -> np.ndarray:
    C = int(max(0, min(C, L * E)))
    mask = np.zeros((L, E), dtype=bool)
    if placement == "partition":
        share = C // L + (np.arange(L) < C % L)
        for layer in range(L):
            mask[layer, :min(int(share[layer]), E)] = True
    elif placement == "top_frequency":
        cnt = _access_counts(trace, L, E).reshape(-1)
        order = np.lexsort((np.arange(L * E), -cnt))  # count descending, then key ascending
        order = order[cnt[order] > 0][:C]
        mask.reshape(-1)[order] = True
    else:
        raise ValueError(placement)
    return mask


def miss_rate(trace: np.ndarray, L: int, E: int, C: int, placement: str) -> float:
    cnt = _access_counts(trace, L, E)
    mask = resident_mask(trace, L, E, C, placement)
    total = cnt.sum()
    return float(cnt[~mask].sum() / total) if total else 0.0
