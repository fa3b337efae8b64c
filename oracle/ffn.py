"""ORACLE (test infrastructure only): one SwiGLU expert, float64.

The pages do not give the expert form; the plain reading of a "SwiGLU expert":
    h = silu(x W_g^T) * (x W_u^T),   silu(a) = a / (1 + exp(-a)),
    y = h W_d^T,
no biases, W_g, W_u: [f, d], W_d: [d, f] (rows = outputs).
"""
import numpy as np


def swiglu_expert(a: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """a: [n, d] float64 -> [n, d] float64."""
    g = a @ wg.T
    u = a @ wu.T
    h = (g / (1.0 + np.exp(-g))) * u
    return h @ wd.T
