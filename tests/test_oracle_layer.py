"""Pins of the oracle MoE layer: expert form, sparse vs dense, k = E mixture, int4 reduction."""
import numpy as np
import torch

import synth
from oracle.layer import moe_layer, moe_layer_dense, moe_layer_tokens
from oracle.numerics import bf16_to_f64, dequant_int4, expert_to_f64
from oracle.router import router_logits


def _small(wdt="f32", act="f32", E=8, k=2, d=64, f=128, T=16, shared=False, bias=None, seed=0):
    wl = synth.Workload("t", d=d, E=E, k=k, f=f, act=act, wdt=wdt, T_list=(T,), shared=shared, zipf_bias=bias)
    return wl, synth.layer_inputs(wl, T, seed=seed)


def _args(li, **kw):
    return dict(x=li.x, w_router=li.w_router, bias=li.bias, act=li.wl.act, k=li.wl.k, E=li.wl.E,
                experts=li.experts, shared=li.shared, **kw)


def test_single_expert_is_the_textbook_swiglu_ffn():
    # E = 1, k = 1: the gate is 1 and y = W_d (silu(W_g x) * (W_u x))
    wl, li = _small(E=1, k=1)
    out = moe_layer(**_args(li))
    assert np.all(out["gates"] == 1.0)
    wg, wu, wd = (torch.from_numpy(a) for a in expert_to_f64(li.experts[0]))
    x = torch.from_numpy(li.x.astype(np.float64))
    want = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(x, wg))
                                      * torch.nn.functional.linear(x, wu), wd)
    assert np.allclose(out["y"], want.numpy(), rtol=1e-12, atol=1e-14)


def test_sparse_equals_dense_masked_by_gates():
    for kw in (dict(), dict(act="bf16", wdt="bf16", bias=1.1, E=16, k=4, T=33),
               dict(act="bf16", wdt="int4", d=128, f=256, E=8, k=3, T=9, shared=True, bias=1.1)):
        wl, li = _small(**kw)
        s = moe_layer(**_args(li))
        dd = moe_layer_dense(**_args(li))
        assert np.allclose(s["y"], dd["y"], rtol=1e-12, atol=1e-13)
        # each row of the dense gate matrix has exactly k nonzeros summing to one
        assert np.all((dd["G"] > 0).sum(axis=1) == wl.k)
        assert np.allclose(dd["G"].sum(axis=1), 1.0, atol=1e-14)


def test_k_equals_E_is_the_dense_softmax_mixture():
    wl, li = _small(E=6, k=6, T=10, bias=1.1)
    out = moe_layer(**_args(li))
    lg = router_logits(li.x, li.w_router, li.bias, "f32").astype(np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    x = li.x.astype(np.float64)
    want = np.zeros_like(x)
    for e in range(6):
        wg, wu, wd = expert_to_f64(li.experts[e])
        g = x @ wg.T
        want += p[:, e:e + 1] * (((g / (1 + np.exp(-g))) * (x @ wu.T)) @ wd.T)
    assert np.allclose(out["y"], want, rtol=1e-12, atol=1e-14)


def test_shared_expert_is_added_with_weight_one():
    wl, li = _small(act="bf16", wdt="bf16", shared=True, T=5)
    with_sh = moe_layer(**_args(li))
    li.shared = None
    without = moe_layer(**_args(li))
    li2 = synth.layer_inputs(wl, 5)
    wg, wu, wd = expert_to_f64(li2.shared)
    x = bf16_to_f64(li2.x)
    g = x @ wg.T
    sh = ((g / (1 + np.exp(-g))) * (x @ wu.T)) @ wd.T
    assert np.allclose(with_sh["y"] - without["y"], sh, rtol=1e-10, atol=1e-12)


def test_int4_layer_equals_dense_layer_on_dequantised_weights():
    wl, li = _small(act="bf16", wdt="int4", d=256, f=128, E=4, k=2, T=7, bias=1.1)
    out = moe_layer(**_args(li))
    as_f32 = []
    for ew in li.experts:
        as_f32.append(synth.ExpertWeights("f32", dequant_int4(ew.wg, ew.sg).astype(np.float32),
                                          dequant_int4(ew.wu, ew.su).astype(np.float32),
                                          dequant_int4(ew.wd, ew.sd).astype(np.float32)))
    # q*s is exact in binary32, so the float layer on those weights is the same computation
    ref = moe_layer(li.x, li.w_router, li.bias, "bf16", 2, 4, as_f32)
    assert np.array_equal(out["topk_idx"], ref["topk_idx"])
    assert np.allclose(out["y"], ref["y"], rtol=1e-14, atol=1e-15)


def test_token_subset_matches_full_layer():
    wl, li = _small(act="bf16", wdt="bf16", E=16, k=4, T=40, bias=1.1, shared=True)
    full = moe_layer(**_args(li))
    toks = [0, 7, 39, 13]
    sub = moe_layer_tokens(toks, **_args(li))
    assert np.array_equal(sub["topk_idx"], full["topk_idx"][toks])
    assert np.allclose(sub["y"], full["y"][toks], rtol=1e-12, atol=1e-14)


def test_forced_routing_uses_renormalised_softmax_at_the_given_ids():
    wl, li = _small(E=8, k=2, T=6, bias=None)
    forced = synth.forced_topk(5, 6, 8, 2)
    out = moe_layer(**_args(li, forced_idx=forced))
    assert np.array_equal(out["topk_idx"], forced)
    lg = out["logits"].astype(np.float64)
    sel = np.take_along_axis(lg, forced.astype(np.int64), axis=1)
    want = np.exp(sel - sel.max(axis=1, keepdims=True))
    want /= want.sum(axis=1, keepdims=True)
    assert np.allclose(out["gates"], want, rtol=1e-13)
