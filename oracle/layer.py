"""ORACLE (test infrastructure only): the whole routed-expert MoE layer, float64.

For each token t (FreeToken linux guide, "MoE memory handling": a router picks
a few experts per token and only those run; the combine is the plain reading
of a gate-weighted mixture):

    y_t = sum_j g_tj * E_{S_tj}(x_t)  [+ E_shared(x_t), weight 1]

Where the experts' weights live (an HBM slot, a pinned host pool) changes only
speed, not the result: the FreeToken RTX 5090 page, section on reconfiguration
at scheduler safe points, says host memory stays the canonical store, so cache
capacity affects performance and not correctness.  The oracle therefore
ignores slots entirely.
"""
from __future__ import annotations

import numpy as np

from .ffn import swiglu_expert
from .numerics import act_to_f64, expert_to_f64
from .permute import permute
from .router import route


def layer_from_inputs(li):
    """synth.LayerInputs -> dict of the arrays the oracle needs (weights decoded lazily)."""
    return dict(x=li.x, w_router=li.w_router, bias=li.bias, act=li.wl.act, k=li.wl.k, E=li.wl.E,
                experts=li.experts, shared=li.shared)


def _expert_cache(experts):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = expert_to_f64(experts[e])
        return cache[e]

    return get


def moe_layer(x, w_router, bias, act, k, E, experts, shared=None, forced_idx=None):
    """Sparse evaluation: route, group pairs by expert, run each expert once on its rows.

    Returns dict(y float64 [T,d], logits, topk_idx, gates, counts, offsets, perm, inv_perm).
    """
    logits, idx, gates = route(x, w_router, bias, act, k, forced_idx)
    counts, offsets, perm, inv = permute(idx, E)
    xf = act_to_f64(x, act)
    T, d = xf.shape
    get = _expert_cache(experts)
    y_pairs = np.zeros((T * k, d), dtype=np.float64)  # rows in flat (t*k + j) order
    with np.errstate(over="ignore"):
        for e in range(E):
            lo, hi = offsets[e], offsets[e + 1]
            if hi == lo:
                continue
            flat = perm[lo:hi]
            y_pairs[flat] = swiglu_expert(xf[flat // k], *get(e))
        y = (gates[:, :, None] * y_pairs.reshape(T, k, d)).sum(axis=1)
        if shared is not None:
            y = y + swiglu_expert(xf, *expert_to_f64(shared))
    return dict(y=y, logits=logits, topk_idx=idx, gates=gates, counts=counts, offsets=offsets,
                perm=perm, inv_perm=inv)


def moe_layer_dense(x, w_router, bias, act, k, E, experts, shared=None, forced_idx=None):
    """Dense evaluation: every expert on every token, weighted by the gates scattered into [T, E]."""
    logits, idx, gates = route(x, w_router, bias, act, k, forced_idx)
    T = logits.shape[0]
    G = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(G, idx.astype(np.int64), gates, axis=1)
    xf = act_to_f64(x, act)
    y = np.zeros_like(xf)
    with np.errstate(over="ignore"):
        for e in range(E):
            y += G[:, e:e + 1] * swiglu_expert(xf, *expert_to_f64(experts[e]))
        if shared is not None:
            y = y + swiglu_expert(xf, *expert_to_f64(shared))
    return dict(y=y, logits=logits, topk_idx=idx, gates=gates, G=G)


def moe_layer_tokens(tokens, x, w_router, bias, act, k, E, experts, shared=None, forced_idx=None):
    """The layer for a subset of tokens only (each token's result depends on its own row alone).

    Returns dict(y [n,d], logits [n,E], topk_idx [n,k], gates [n,k]) for x[tokens].
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.asarray(x)[tokens]
    fi = None if forced_idx is None else np.asarray(forced_idx)[tokens]
    logits, idx, gates = route(xs, w_router, bias, act, k, fi)
    xf = act_to_f64(xs, act)
    n, d = xf.shape
    get = _expert_cache(experts)
    y = np.zeros((n, d), dtype=np.float64)
    with np.errstate(over="ignore"):
        for t in range(n):
            for j in range(k):
                y[t] += gates[t, j] * swiglu_expert(xf[t:t + 1], *get(int(idx[t, j])))[0]
        if shared is not None:
            y = y + swiglu_expert(xf, *expert_to_f64(shared))
    return dict(y=y, logits=logits, topk_idx=idx, gates=gates)
