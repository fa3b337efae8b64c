"""ORACLE (test infrastructure only): grouping of (token, choice) pairs by expert.

The pages do not describe this step; the plain reading is a counting sort of
the flattened top-k ids (flat index t*k + j), stable within an expert:

* counts[e]   number of pairs routed to e
* offsets     exclusive prefix sum of counts, length E+1
* perm[p]     flat index of the pair at sorted position p
* inv_perm[i] sorted position of flat index i
"""
import numpy as np


def permute(topk_idx: np.ndarray, E: int):
    ids = np.asarray(topk_idx, dtype=np.int64).ravel().tolist()
    n = len(ids)
    counts = [0] * E
    for e in ids:
        counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E]
    perm = [0] * n
    inv = [0] * n
    for i, e in enumerate(ids):
        p = cursor[e]
        perm[p] = i
        inv[i] = p
        cursor[e] = p + 1
    as32 = lambda v: np.asarray(v, dtype=np.int32)
    return as32(counts), as32(offsets), as32(perm), as32(inv)
