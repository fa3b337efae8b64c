"""ORACLE (test infrastructure only): one SwiGLU expert, float64.

The pages do not give the expert form; the plain reading of a "SwiGLU expert":
    h = silu(x W_g^T) * (x W_u^T),   silu(a) = a / (1 + exp(-a)),
    y = h W_d^T,
no biases, W_g, W_u: [f, d], W_d: [d, f] (rows = outputs).
"""
import numpy as np

from .numerics import round_to_bf16


def swiglu_expert(a: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, h_bf16: bool = False,
                  y_bf16: bool = False) -> np.ndarray:
    """a: [n, d] float64 -> [n, d] float64.  h_bf16: h rounded to bfloat16 before the down
    projection, as the bf16 layers may store it (otherwise h stays float64).  y_bf16: the expert's
    output rows rounded to bfloat16, as a bf16 prefill may store them before the gate-weighted
    combine (the intermediate rows of a bf16 layer may be bf16, like h)."""
    g = a @ wg.T
    u = a @ wu.T
    h = (g / (1.0 + np.exp(-g))) * u
    if h_bf16:
        h = round_to_bf16(h)
    y = h @ wd.T
    return round_to_bf16(y) if y_bf16 else y
