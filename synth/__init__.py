"""Seeded synthetic inputs for the routed-expert MoE layer.

This module produces inputs only: activations, router weights and bias,
expert weights (bf16, fp32, or int4 with bf16 group scales), slot orders and
routing traces.  It computes no step of the layer itself, and both the oracle
and the HIP path read their inputs from here.

The pages describe an offloaded-MoE runtime measured on agent workloads with
trained checkpoints; neither is available, so these generators stand in for
them with the layer shapes of the models the pages name (a Qwen3.6-35B-A3B
shaped decode layer, a DeepSeek-V4-Flash shaped layer with 6 of 256 routed
experts per token; FreeToken linux guide, "MoE memory handling" section).

Bits are defined by ``synth/gen.c`` (counter-based SplitMix64 streams,
Irwin-Hall Gaussian shape, exact IEEE rounding), so every tensor can be
regenerated independently of the others.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_synth.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile gen.c into _synth.so with gcc (OpenMP)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(_HERE, "gen.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
    vp = ctypes.c_void_p
    lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, f32, vp]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, f32, vp]
    lib.synth_raw_u64.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_quant_int4.argtypes = [vp, u64, u64, f32, i64, i64, vp, vp]
    for fn in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_raw_u64, lib.synth_quant_int4):
        fn.restype = None
    _lib = lib
    return lib


# ----------------------------------------------------------------------------------------------
# stream identifiers: one independent stream per (tensor kind, layer, expert)
# ----------------------------------------------------------------------------------------------
KIND_ROUTER, KIND_WG, KIND_WU, KIND_WD, KIND_X, KIND_SH_WG, KIND_SH_WU, KIND_SH_WD = range(1, 9)


def stream_id(kind: int, layer: int = 0, expert: int = 0) -> int:
    return (kind << 40) | (layer << 20) | expert


def raw_u64(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_raw_u64(seed, stream, start, n, out.ctypes.data)
    return out


def normal_f32(seed: int, stream: int, shape, sigma: float, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, stream, start, n, sigma, out.ctypes.data)
    return out.reshape(shape)


def normal_bf16(seed: int, stream: int, shape, sigma: float, start: int = 0) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of fl32(z * sigma), rounded to nearest even."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(seed, stream, start, n, sigma, out.ctypes.data)
    return out.reshape(shape)


def quant_int4(seed: int, stream: int, rows: int, K: int, sigma: float, w: Optional[np.ndarray] = None):
    """Symmetric int4 (offset-binary nibbles, element 2i low) with bf16 scales per 128 inputs.

    Returns (packed uint8 [rows, K//2], scales uint16 [rows, K//128]).  The
    float matrix is generated from (seed, stream, sigma) unless ``w`` is given.
    """
    if K % 128:
        raise ValueError("int4 groups need K % 128 == 0")
    packed = np.empty((rows, K // 2), dtype=np.uint8)
    scales = np.empty((rows, K // 128), dtype=np.uint16)
    wp = None
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        assert w.shape == (rows, K)
        wp = w.ctypes.data
    _load().synth_quant_int4(wp, seed, stream, sigma, rows, K, packed.ctypes.data, scales.ctypes.data)
    return packed, scales


# ----------------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one MoE layer workload."""

    name: str
    d: int
    E: int
    k: int
    f: int
    act: str  # "f32" | "bf16"
    wdt: str  # "f32" | "bf16" | "int4"
    T_list: tuple
    shared: bool = False
    zipf_bias: Optional[float] = None  # Zipf exponent s of the router bias, None = no bias
    identity_slots: bool = False
    w_sigma: float = 0.02
    x_sigma: float = 1.0
    layers: int = 1


WORKLOADS = {
    # tiny fp32 layer: T=16, d=64, E=8, top-2, d_ff=128, no bias, identity slot table
    "tiny_fp32": Workload("tiny_fp32", d=64, E=8, k=2, f=128, act="f32", wdt="f32",
                          T_list=(16,), identity_slots=True),
    # Qwen3.6-35B-A3B shaped decode layer: d=2048, E=128, top-8, d_ff=768, bf16
    "qwen_a3b_decode_bf16": Workload("qwen_a3b_decode_bf16", d=2048, E=128, k=8, f=768, act="bf16",
                                     wdt="bf16", T_list=(1, 4, 16, 64), zipf_bias=1.1),
    # DeepSeek-V4-Flash shaped prefill layer: d=4096, E=256, top-6, d_ff=2048, +1 shared, bf16
    "dsv4_prefill_bf16": Workload("dsv4_prefill_bf16", d=4096, E=256, k=6, f=2048, act="bf16",
                                  wdt="bf16", T_list=(512, 2048, 8192), shared=True, zipf_bias=1.1),
    # same layer in decode with int4 g128 experts (shared expert int4 too)
    "dsv4_decode_int4": Workload("dsv4_decode_int4", d=4096, E=256, k=6, f=2048, act="bf16",
                                 wdt="int4", T_list=(1, 2, 8), shared=True, zipf_bias=1.1),
    # 24 stacked int4 layers held in a pinned host pool behind an LRU slot cache
    "dsv4_offload_int4": Workload("dsv4_offload_int4", d=4096, E=256, k=6, f=2048, act="bf16",
                                  wdt="int4", T_list=(1,), shared=True, zipf_bias=1.1, layers=24),
}


def router_bias(seed: int, E: int, s: float, layer: int = 0) -> np.ndarray:
    """b_e = -s * ln(r_e), r = 1 + a seeded permutation of 0..E-1 (softmax(b) is the Zipf(s) pmf)."""
    rng = np.random.default_rng([seed, 0xB1A5, layer])
    r = 1.0 + rng.permutation(E).astype(np.float64)
    return (-s * np.log(r)).astype(np.float32)


def slot_order(seed: int, E: int, layer: int = 0) -> np.ndarray:
    """Seeded permutation: expert e lives in slot order[e]."""
    rng = np.random.default_rng([seed, 0x5107, layer])
    return rng.permutation(E).astype(np.int32)


def _dense(seed, stream, shape, sigma, dt):
    if dt == "f32":
        return normal_f32(seed, stream, shape, sigma)
    if dt == "bf16":
        return normal_bf16(seed, stream, shape, sigma)
    raise ValueError(dt)


@dataclass
class ExpertWeights:
    """Canonical (row-major, out x in) weights of one SwiGLU expert.

    dense dtypes: wg, wu [f, d], wd [d, f] as float32 or bf16 bits (uint16).
    int4: wg, wu, wd are packed nibbles [rows, K//2] and sg, su, sd their
    bf16 scales [rows, K//128].
    """

    wdt: str
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    sg: Optional[np.ndarray] = None
    su: Optional[np.ndarray] = None
    sd: Optional[np.ndarray] = None


def expert_weights(wl: Workload, seed: int, layer: int, expert: int, shared: bool = False) -> ExpertWeights:
    kinds = (KIND_SH_WG, KIND_SH_WU, KIND_SH_WD) if shared else (KIND_WG, KIND_WU, KIND_WD)
    e = 0 if shared else expert
    sg_, su_, sd_ = (stream_id(kd, layer, e) for kd in kinds)
    d, f, s = wl.d, wl.f, wl.w_sigma
    if wl.wdt == "int4":
        pg, sg = quant_int4(seed, sg_, f, d, s)
        pu, su = quant_int4(seed, su_, f, d, s)
        pd, sd = quant_int4(seed, sd_, d, f, s)
        return ExpertWeights("int4", pg, pu, pd, sg, su, sd)
    return ExpertWeights(wl.wdt, _dense(seed, sg_, (f, d), s, wl.wdt), _dense(seed, su_, (f, d), s, wl.wdt),
                         _dense(seed, sd_, (d, f), s, wl.wdt))


@dataclass
class LayerInputs:
    wl: Workload
    seed: int
    layer: int
    T: int
    x: np.ndarray  # [T, d] float32 or bf16 bits
    w_router: np.ndarray  # [E, d] same dtype as x
    bias: Optional[np.ndarray]  # [E] float32 or None
    slot_of_expert: np.ndarray  # [E] int32
    experts: list = field(default_factory=list)  # list[ExpertWeights] (may be lazily empty)
    shared: Optional[ExpertWeights] = None


def layer_inputs(wl: Workload, T: int, seed: int = 0, layer: int = 0, batch: int = 0,
                 with_experts: bool = True) -> LayerInputs:
    """All inputs of one layer call.  ``batch`` selects an independent activation batch."""
    x = _dense(seed, stream_id(KIND_X, layer, batch), (T, wl.d), wl.x_sigma, wl.act)
    wr = _dense(seed, stream_id(KIND_ROUTER, layer, 0), (wl.E, wl.d), wl.w_sigma, wl.act)
    bias = router_bias(seed, wl.E, wl.zipf_bias, layer) if wl.zipf_bias is not None else None
    slots = np.arange(wl.E, dtype=np.int32) if wl.identity_slots else slot_order(seed, wl.E, layer)
    li = LayerInputs(wl, seed, layer, T, x, wr, bias, slots)
    if with_experts:
        li.experts = [expert_weights(wl, seed, layer, e) for e in range(wl.E)]
        if wl.shared:
            li.shared = expert_weights(wl, seed, layer, 0, shared=True)
    return li


def forced_topk(seed: int, T: int, E: int, k: int, batch: int = 0) -> np.ndarray:
    """Random distinct top-k sets [T, k] (int32), for permutation tests and trace replay."""
    rng = np.random.default_rng([seed, 0x7013, batch])
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False)
    return out


# ----------------------------------------------------------------------------------------------
# decode routing trace with temporal reuse (stand-in for the pages' replayed agent traces)
# ----------------------------------------------------------------------------------------------
def routing_trace(seed: int, steps: int, L: int, E: int, k: int, s: float = 1.1, p_reuse: float = 0.6) -> np.ndarray:
    """Trace [steps, L, k] of distinct expert ids per (step, layer), ascending within a row.

    Each layer ranks its experts by a seeded permutation; popularity of rank r
    is proportional to r^-s.  Step 0 draws k distinct experts (draws with
    replacement, duplicates rejected).  Each later step keeps every expert of
    the previous step independently with probability p_reuse (coins flipped in
    ascending expert order), then fills up to k with Zipf draws that reject
    experts already chosen.  Random numbers are consumed layer-major within a
    step, coins before draws.
    """
    rng = np.random.default_rng([seed, 0x7ACE])
    ranks = [np.random.default_rng([seed, 0x2A4C, l]).permutation(E) for l in range(L)]
    pmf = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(pmf / pmf.sum())
    cdf[-1] = 1.0
    out = np.empty((steps, L, k), dtype=np.int32)
    prev = [None] * L
    for t in range(steps):
        for l in range(L):
            chosen = []
            if prev[l] is not None:
                for e in prev[l]:  # ascending
                    if rng.random() < p_reuse:
                        chosen.append(int(e))
            cs = set(chosen)
            while len(chosen) < k:
                r = int(np.searchsorted(cdf, rng.random(), side="right"))
                e = int(ranks[l][min(r, E - 1)])
                if e not in cs:
                    cs.add(e)
                    chosen.append(e)
            row = np.sort(np.array(chosen, dtype=np.int32))
            out[t, l] = row
            prev[l] = row
    return out
