"""Pins of the oracle router: summation order, top-k selection and gates."""
import json
import os

import numpy as np
import pytest

import synth
from oracle.numerics import bf16_to_f64
from oracle.router import renorm_gates, router_logits, topk_select


def _f32_to_bf16_bits(a):
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_golden_summation_order(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "router_order_cases.json")))
    for case in g["cases"]:
        d = case["d"]
        x = np.zeros((1, d), np.float32)
        for i, v in case["x"].items():
            x[0, int(i)] = v
        w = np.ones((1, d), np.float32)
        if case["act"] == "bf16":
            x, w = _f32_to_bf16_bits(x), _f32_to_bf16_bits(w)
        lg = router_logits(x, w, None, case["act"])
        assert lg[0, 0] == np.float32(case["logit"]), case["name"]


def test_exact_when_every_partial_sum_is_exact():
    # small integers: every product and partial sum is exact, so any order gives the exact dot product
    rng = np.random.default_rng(0)
    for act, d in (("f32", 64), ("f32", 256), ("bf16", 512), ("bf16", 2048), ("bf16", 128)):
        x = rng.integers(-8, 9, size=(5, d)).astype(np.float32)
        w = rng.integers(-8, 9, size=(7, d)).astype(np.float32)
        b = rng.integers(-4, 5, size=7).astype(np.float32)
        exact = x.astype(np.int64) @ w.astype(np.int64).T + b.astype(np.int64)
        if act == "bf16":
            x, w = _f32_to_bf16_bits(x), _f32_to_bf16_bits(w)
        lg = router_logits(x, w, b, act)
        assert np.array_equal(lg.astype(np.int64), exact)


@pytest.mark.parametrize("act,d", [("bf16", 2048), ("bf16", 4096), ("f32", 64)])
def test_binary32_error_within_the_summation_bound(act, d):
    T, E = 8, 32
    x = (synth.normal_bf16 if act == "bf16" else synth.normal_f32)(0, 1, (T, d), 1.0)
    w = (synth.normal_bf16 if act == "bf16" else synth.normal_f32)(0, 2, (E, d), 0.02)
    b = synth.router_bias(0, E, 1.1)
    lg = router_logits(x, w, b, act).astype(np.float64)
    xf = bf16_to_f64(x) if act == "bf16" else x.astype(np.float64)
    wf = bf16_to_f64(w) if act == "bf16" else w.astype(np.float64)
    exact = xf @ wf.T + b.astype(np.float64)
    # each sum passes through at most d/64 + 6 + 1 roundings (plus one per product for fp32)
    u = 2.0 ** -24
    n = d // 64 + 7 + (1 if act == "f32" else 0)
    bound = n * u * (np.abs(xf) @ np.abs(wf).T + np.abs(b)) * 1.01
    assert np.all(np.abs(lg - exact) <= bound)


def test_topk_equals_stable_argsort():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((200, 64)).astype(np.float32)
    ties = np.round(rng.standard_normal((200, 64)) * 2).astype(np.float32)  # many equal values
    for arr in (lg, ties):
        for k in (1, 2, 6, 8, 64):
            want = np.argsort(-arr, axis=1, kind="stable")[:, :k]
            assert np.array_equal(topk_select(arr, k), want)


def test_gates_are_softmax_over_the_selected_logits():
    rng = np.random.default_rng(2)
    lg = (rng.standard_normal((100, 128)) * 3).astype(np.float32)
    idx = topk_select(lg, 8)
    g = renorm_gates(lg, idx)
    sel = np.take_along_axis(lg.astype(np.float64), idx.astype(np.int64), axis=1)
    direct = np.exp(sel - sel[:, :1])
    direct /= direct.sum(axis=1, keepdims=True)
    assert np.allclose(g, direct, rtol=1e-13, atol=0)
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 0)  # gate order follows logit order


def test_golden_gates(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_gates_closed_form.json")))
    for c in g["cases"]:
        lg = np.array([c["logits"]], np.float32)
        idx = topk_select(lg, c["k"])
        assert idx[0].tolist() == c["idx"]
        assert np.allclose(renorm_gates(lg, idx)[0], c["gates"], rtol=1e-14, atol=1e-16)
