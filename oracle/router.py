"""ORACLE (test infrastructure only): router scores, top-k selection, gates.

The pages state that the router activates a few experts per token: 6 of 256
routed experts per layer for DeepSeek-V4-Flash (FreeToken linux guide, "MoE
memory handling" section; FreeToken RTX 5090 page, introduction).  The router
form is not given there; the plain reading used here:

* logits  l = x W_r^T + b  (binary32, fixed summation order: 64 contiguous
          segments summed in ascending index, joined pairwise neighbours first;
          ``c/router_canon.c``)
* top-k   the k largest logits, largest first; equal logits -> lower expert id
          first (selection on logits equals selection on softmax
          probabilities, since exp is increasing)
* gates   softmax over all E logits, renormalised over the k selected:
          g_j = p_{S_j} / sum_{i in S} p_i    (float64, from the binary32 logits)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_oracle_c.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle's C file with gcc (no fused multiply-add)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(_HERE, "c", "router_canon.c"), "-o", _LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        lib.oracle_router_logits.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, vp]
        lib.oracle_router_logits.restype = ctypes.c_int
        _lib = lib
    return _lib


def router_logits(x: np.ndarray, w_router: np.ndarray, bias, act: str) -> np.ndarray:
    """[T, E] binary32 logits in the canonical order.  x, w_router: float32 or bf16 bits."""
    is_bf16 = act == "bf16"
    dt = np.uint16 if is_bf16 else np.float32
    x = np.ascontiguousarray(x, dtype=dt)
    w = np.ascontiguousarray(w_router, dtype=dt)
    T, d = x.shape
    E = w.shape[0]
    if d > 16384 or d % 64:
        raise ValueError("oracle router needs d a multiple of 64 and at most 16384")
    out = np.empty((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _load().oracle_router_logits(x.ctypes.data, w.ctypes.data, int(is_bf16),
                                 None if b is None else b.ctypes.data, T, d, E, out.ctypes.data)
    return out


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """k rounds of 'take the largest remaining logit, lowest id among equals'. -> int32 [T, k]."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    taken = np.zeros((T, E), dtype=bool)
    out = np.empty((T, k), dtype=np.int32)
    ids = np.arange(E)
    for j in range(k):
        cur = np.where(taken, -np.inf, lg)
        m = cur.max(axis=1, keepdims=True)
        is_max = (cur == m) & ~taken
        pick = np.where(is_max, ids[None, :], E).min(axis=1)
        out[:, j] = pick
        taken[np.arange(T), pick] = True
    return out


def renorm_gates(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over all E logits (float64), renormalised over the selected ids. -> float64 [T, k]."""
    l64 = np.asarray(logits, dtype=np.float64)
    M = l64.max(axis=1, keepdims=True)
    e = np.exp(l64 - M)
    p = e / e.sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    return ps / ps.sum(axis=1, keepdims=True)


def route(x, w_router, bias, act: str, k: int, forced_idx=None):
    """-> (logits f32 [T,E], topk_idx int32 [T,k], gates float64 [T,k])."""
    lg = router_logits(x, w_router, bias, act)
    idx = topk_select(lg, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int32)
    return lg, idx, renorm_gates(lg, idx)
