"""End-to-end MoE layer on the GPU (route -> permute -> slot-indirected grouped SwiGLU -> combine)
against the float64 oracle.  Integers bit-exact; outputs within the per-token normwise relative
tolerance: 1e-4 for fp32 layers, 2e-2 for bf16 / int4 layers (the GPU rounds the SwiGLU output to
bf16 before the down projection, as the bf16 layers allow)."""
import gc

import numpy as np
import pytest

import synth
from gpu_util import need_gpu, rel_err_per_token, small_workload, to_dev, tol_for, y_to_f64
from oracle.layer import moe_layer, moe_layer_tokens

pytestmark = pytest.mark.gpu


def _run(layer, li, forced=None):
    import torch

    x = layer.x_to_device(li.x)
    out = layer.forward(x, forced_idx=None if forced is None else to_dev(forced, "i32"))
    torch.cuda.synchronize()
    return out


def _check_ints(out, ref):
    assert np.array_equal(out["topk_idx"].cpu().numpy(), ref["topk_idx"])
    for key in ("counts", "offsets", "perm", "inv_perm"):
        assert np.array_equal(out[key].cpu().numpy(), ref[key]), key


def _check_experts_whole(out, x, wl, experts, shared, T, tight=None, int4_bf16=False):
    """Every token of the 3 heaviest and 3 lightest touched experts (and of the shared expert):
    their rows of y_perm (the expert's own output, before the gates) against the oracle's expert on
    the same tokens, per-row normwise relative error <= 2e-2 against exact weights.  With `tight`,
    also against the oracle with the GPU's roundings (h rounded to bf16; bf16 y_perm rows rounded to
    bf16; with int4_bf16, int4 weights seen as bf16(q*s)): every row within `tight`, and the mean row error at most half of the mean
    against the plain oracle (the roundings the oracle now models were most of the difference; what
    is left is binary32 accumulation and the h elements whose bf16 rounding flips between a binary32
    and a binary64 h)."""
    from oracle.ffn import swiglu_expert
    from oracle.numerics import act_to_f64, expert_to_f64

    counts = out["counts"].cpu().numpy()
    off = out["offsets"].cpu().numpy()
    perm = out["perm"].cpu().numpy()
    touched = np.flatnonzero(counts)
    order = touched[np.argsort(counts[touched], kind="stable")]
    pick = sorted(set(order[:3].tolist() + order[-3:].tolist()))
    xf = act_to_f64(x, "bf16")
    yp_all = out["y_perm"]
    y_bf16 = str(yp_all.dtype) == "torch.bfloat16"  # prefill rows rounded once to bf16
    groups = [(int(e), perm[off[e]:off[e + 1]] // wl.k, yp_all[off[e]:off[e + 1]], experts[int(e)]) for e in pick]
    if shared is not None:
        groups.append((-1, np.arange(T), yp_all[T * wl.k:T * wl.k + T], shared))
    # experts the library runs on the decode kernels (few tokens) take exact q*s products
    from expert_offload_cache_amd._lib import lib, MOE_INT4_G128

    gemv_max = lib().moe_prefill_gemv_tokens(MOE_INT4_G128) if int4_bf16 else 0
    worst, worst_t, errs, errs_t = 0.0, 0.0, [], []
    for e, toks, yp, ew in groups:
        y = y_to_f64(yp)
        err = rel_err_per_token(y, swiglu_expert(xf[toks], *expert_to_f64(ew)))
        worst = max(worst, float(err.max()))
        errs.append(err)
        assert err.max() <= 2e-2, (e, len(toks), err.max())
        if tight is not None:
            on_gemm = int4_bf16 and (e == -1 or len(toks) > gemv_max)
            ref = swiglu_expert(xf[toks], *expert_to_f64(ew, int4_bf16=on_gemm), h_bf16=True, y_bf16=y_bf16)
            et = rel_err_per_token(y, ref)
            worst_t = max(worst_t, float(et.max()))
            errs_t.append(et)
            assert et.max() <= tight, (e, len(toks), et.max(), err.max())
    mean = float(np.concatenate(errs).mean())
    mean_t = float(np.concatenate(errs_t).mean()) if errs_t else float("nan")
    print(f"whole experts {pick} (+shared {shared is not None}), n_e {[int(counts[e]) for e in pick]}: "
          f"row rel err max {worst:.3g} mean {mean:.3g}; with the GPU's roundings max {worst_t:.3g} mean {mean_t:.3g}")
    if tight is not None:
        assert mean_t <= 0.5 * mean, (mean_t, mean)
    return worst, worst_t


SMALL = [
    # (act, wdt, d, f, E, k, T, shared)
    ("f32", "f32", 64, 128, 8, 2, 16, False),
    ("f32", "f32", 128, 64, 5, 3, 70, False),
    ("bf16", "bf16", 256, 96, 16, 4, 9, False),
    ("bf16", "bf16", 512, 160, 12, 3, 130, True),
    ("bf16", "bf16", 128, 64, 4, 4, 1, True),
    # decode path on the matrix cores: several 16-token groups per workgroup (shared expert: 3)
    ("bf16", "bf16", 384, 64, 4, 2, 40, True),
    # router logits in 4 x 4 token-expert tiles (32-64 tokens): a partial last token tile (33)
    # and a partial last expert tile (6 experts)
    ("bf16", "bf16", 512, 128, 6, 2, 33, True),
    # gate/up K = 4096 inputs: the K-streaming kernel (beyond the split-input kernel's shapes)
    ("bf16", "bf16", 4096, 64, 4, 2, 3, False),
    # gate/up K = 4096 inputs with more than 16 tokens: the K-streaming kernel's 32-token plan
    ("bf16", "bf16", 4096, 64, 4, 2, 20, False),
    # 66 input fragments: neither matrix-core gate/up plan divides them, the VALU kernel runs it;
    # 132 down row blocks: the split-input down kernel
    ("bf16", "bf16", 2112, 64, 4, 2, 20, False),
    # 10 gate/up input fragments and 20 down row blocks: the streaming plans do not divide them,
    # the split-input kernel runs both projections
    ("bf16", "bf16", 320, 96, 8, 2, 9, True),
    # int4 decode: K-streaming for both projections, experts spanning several 16-token items
    ("bf16", "int4", 512, 512, 8, 2, 20, True),
    # int4, one token: the VALU kernel
    ("bf16", "int4", 512, 256, 8, 3, 1, True),
    # int4, f = 128: the down projection's input split does not apply, the VALU kernel runs it
    ("bf16", "int4", 256, 128, 8, 2, 5, True),
    ("bf16", "int4", 512, 256, 16, 4, 67, False),
    # int4 at the DeepSeek-shaped d and d_ff with few tokens: the deep-issue decode kernel (every
    # weight load of a wave in flight at once), both of its gate/up plans and its down plan
    ("bf16", "int4", 4096, 2048, 8, 2, 1, True),
    ("bf16", "int4", 4096, 2048, 8, 3, 2, False),
    ("bf16", "int4", 4096, 2048, 16, 4, 7, True),
    # int4 with many tokens per expert: the int4 MFMA grouped GEMM (down: an odd number of groups)
    ("bf16", "int4", 512, 256, 6, 2, 300, True),
    ("bf16", "int4", 1024, 384, 16, 4, 257, False),
    # many tokens per expert: the MFMA grouped GEMM (several 128-token tiles, ragged tails)
    ("bf16", "bf16", 256, 128, 6, 2, 300, True),
    ("bf16", "bf16", 512, 384, 16, 4, 257, False),
    ("bf16", "bf16", 256, 256, 3, 1, 1000, True),
    ("bf16", "bf16", 512, 256, 6, 2, 300, True),
    ("bf16", "bf16", 1024, 768, 16, 4, 257, False),
    ("bf16", "bf16", 512, 512, 3, 1, 1000, True),
]


@pytest.mark.parametrize("act,wdt,d,f,E,k,T,shared", SMALL)
def test_small_layers(act, wdt, d, f, E, k, T, shared):
    need_gpu()
    from expert_offload_cache_amd.layer import DeviceLayer

    print(f"layer {act}/{wdt} d={d} f={f} E={E} k={k} T={T} shared={shared}", flush=True)
    wl = small_workload(act, wdt, d, f, E, k, shared=shared, bias=None if act == "f32" else 1.1)
    li = synth.layer_inputs(wl, T, seed=5)
    layer = DeviceLayer.from_inputs(li)
    out = _run(layer, li)
    ref = moe_layer(li.x, li.w_router, li.bias, act, k, E, li.experts, li.shared)
    _check_ints(out, ref)
    err = rel_err_per_token(y_to_f64(out["y"]), ref["y"])
    print(f"max per-token rel err {err.max():.3g}")
    assert err.max() <= tol_for(wl)
    assert int(out["ws"][:4].view(dtype=__import__("torch").int32).item()) == 0


@pytest.fixture(scope="module")
def qwen_layer():
    need_gpu()
    from expert_offload_cache_amd.layer import DeviceLayer

    wl = synth.WORKLOADS["qwen_a3b_decode_bf16"]
    li = synth.layer_inputs(wl, 64, seed=0)
    layer = DeviceLayer.from_inputs(li)
    yield wl, li, layer
    del layer
    gc.collect()


@pytest.mark.parametrize("T", [1, 4, 16, 32, 64, 256])
def test_qwen_a3b_decode_layer(qwen_layer, T):
    wl, li64, layer = qwen_layer
    print(f"qwen-a3b decode bf16 T={T}", flush=True)
    li = synth.layer_inputs(wl, T, seed=0, with_experts=False)
    out = _run(layer, li)
    ref = moe_layer(li.x, li64.w_router, li64.bias, "bf16", wl.k, wl.E, li64.experts)
    _check_ints(out, ref)
    err = rel_err_per_token(y_to_f64(out["y"]), ref["y"])
    print(f"U={int((ref['counts'] > 0).sum())} max per-token rel err {err.max():.3g}")
    assert err.max() <= 2e-2


@pytest.mark.parametrize("T", [1, 64])
def test_forward_into_preallocated_buffers(qwen_layer, T):
    """forward(..., bufs=layer.buffers(T)) writes bitwise what a forward with fresh outputs
    returns, call after call with different inputs."""
    import torch

    wl, _, layer = qwen_layer
    print(f"preallocated buffers T={T}", flush=True)
    bufs = layer.buffers(T)
    keys = ("y", "topk_idx", "topk_w", "logits", "counts", "offsets", "perm", "inv_perm", "y_perm")
    for b in (1, 2, 1):
        x = layer.x_to_device(synth.layer_inputs(wl, T, seed=0, batch=b, with_experts=False).x)
        fresh = layer.forward(x)
        got = layer.forward(x, bufs=bufs)
        torch.cuda.synchronize()
        assert got["y"].data_ptr() == bufs["y"].data_ptr()
        for key in keys:
            a, r = got[key], fresh[key]
            if a.dtype == torch.bfloat16:
                a, r = a.view(torch.int16), r.view(torch.int16)
            assert torch.equal(a, r), f"batch {b}: {key}"


def test_determinism_and_slot_order_invariance(qwen_layer):
    """Two runs are bitwise identical; a different slot order gives bitwise identical outputs."""
    import torch
    from expert_offload_cache_amd.layer import DeviceLayer

    wl, li, layer = qwen_layer
    a = _run(layer, li)["y"].clone()
    b = _run(layer, li)["y"].clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    other = np.random.default_rng(99).permutation(wl.E).astype(np.int32)
    layer2 = DeviceLayer(wl.d, wl.f, wl.E, wl.k, wl.act, wl.wdt, li.w_router, li.bias, li.experts, None,
                         slot_of_expert=other)
    c = _run(layer2, li)["y"]
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    del layer2


@pytest.mark.parametrize("T", [16, 256])
def test_absent_slot_is_flagged_not_read(qwen_layer, T):
    import torch
    import expert_offload_cache_amd as moe

    wl, li, layer = qwen_layer
    lt = synth.layer_inputs(wl, T, seed=0, with_experts=False)
    x = layer.x_to_device(lt.x)
    out = layer.forward(x)
    counts = out["counts"].cpu().numpy()
    e_bad = int(np.argmax(counts))
    soe = layer.slot_of_expert.clone()
    soe[e_bad] = -1
    ws = layer.workspace(T)
    y_perm, ws = moe.expert_ffn_grouped(x, out["perm"], out["offsets"], out["counts"], soe, layer.pool,
                                        layer.n_slots, layer.stride, "bf16", wl.f, wl.k, ws=ws,
                                        y_dtype=out["y_perm"].dtype)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 1
    off = out["offsets"].cpu().numpy()
    yp = y_to_f64(y_perm)
    assert np.all(yp[off[e_bad]:off[e_bad + 1]] == 0)
    ref = y_to_f64(out["y_perm"])
    keep = np.ones(len(yp), bool)
    keep[off[e_bad]:off[e_bad + 1]] = False
    assert np.array_equal(yp[keep], ref[keep])


@pytest.mark.parametrize("T", [1, 2, 8])
def test_int4_absent_slot_is_flagged_not_read(dsv4_int4_layer, T):
    """The few-token int4 kernels: an absent slot sets the status word and gives that expert zero
    rows; every other row is bitwise the full call's."""
    import torch
    import expert_offload_cache_amd as moe

    wl, _, layer = dsv4_int4_layer
    lt = synth.layer_inputs(wl, T, seed=0, with_experts=False)
    x = layer.x_to_device(lt.x)
    out = layer.forward(x)
    counts = out["counts"].cpu().numpy()
    e_bad = int(np.argmax(counts))
    soe = layer.slot_of_expert.clone()
    soe[e_bad] = -1
    ws = layer.workspace(T)
    y_perm, ws = moe.expert_ffn_grouped(x, out["perm"], out["offsets"], out["counts"], soe, layer.pool,
                                        layer.n_slots, layer.stride, "int4", wl.f, wl.k, shared_w=layer.shared, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 1
    off = out["offsets"].cpu().numpy()
    yp = y_to_f64(y_perm)
    assert np.all(yp[off[e_bad]:off[e_bad + 1]] == 0)
    keep = np.ones(len(yp), bool)
    keep[off[e_bad]:off[e_bad + 1]] = False
    assert np.array_equal(yp[keep], y_to_f64(out["y_perm"])[keep])


@pytest.fixture(scope="module")
def dsv4_int4_layer():
    need_gpu()
    from expert_offload_cache_amd.layer import DeviceLayer

    wl = synth.WORKLOADS["dsv4_decode_int4"]
    li = synth.layer_inputs(wl, 8, seed=0)
    layer = DeviceLayer.from_inputs(li)
    yield wl, li, layer
    del layer
    gc.collect()


@pytest.mark.parametrize("T", [1, 2, 8])
def test_dsv4_int4_decode_layer(dsv4_int4_layer, T):
    wl, li8, layer = dsv4_int4_layer
    print(f"dsv4 decode int4 T={T}", flush=True)
    li = synth.layer_inputs(wl, T, seed=0, with_experts=False)
    out = _run(layer, li)
    ref = moe_layer(li.x, li8.w_router, li8.bias, "bf16", wl.k, wl.E, li8.experts, li8.shared)
    _check_ints(out, ref)
    err = rel_err_per_token(y_to_f64(out["y"]), ref["y"])
    print(f"max per-token rel err {err.max():.3g}")
    assert err.max() <= 2e-2


@pytest.mark.parametrize("T", [512, 2048, 8192])
def test_dsv4_int4_prefill_layer_sampled(dsv4_int4_layer, T):
    """Full-size int4 prefill (the int4 MFMA GEMM): routing integers bit-exact, outputs on sampled
    tokens against the oracle's exactly dequantised weights; every token of the heaviest and lightest
    experts against exact weights (2e-2) and, tightly, against the oracle that rounds q*s and h to
    bf16 as the GEMM does."""
    wl, li8, layer = dsv4_int4_layer
    print(f"dsv4 prefill int4 T={T}", flush=True)
    li = synth.layer_inputs(wl, T, seed=0, with_experts=False)
    out = _run(layer, li)
    from oracle.permute import permute as o_permute
    from oracle.router import route as o_route

    _, idx, _ = o_route(li.x, li8.w_router, li8.bias, "bf16", wl.k)
    assert np.array_equal(out["topk_idx"].cpu().numpy(), idx)
    c, o, p, ip = o_permute(idx, wl.E)
    for key, v in (("counts", c), ("offsets", o), ("perm", p), ("inv_perm", ip)):
        assert np.array_equal(out[key].cpu().numpy(), v), key
    toks = sorted({0, T // 3, T - 1, *np.random.default_rng(T).choice(T, 3, replace=False).tolist()})
    ref = moe_layer_tokens(toks, li.x, li8.w_router, li8.bias, "bf16", wl.k, wl.E, li8.experts, li8.shared)
    err = rel_err_per_token(y_to_f64(out["y"])[toks], ref["y"])
    print(f"max n_e {int(c.max())} sampled max rel err {err.max():.3g}")
    assert err.max() <= 2e-2
    assert int(out["ws"][:4].view(dtype=__import__("torch").int32).item()) == 0
    _check_experts_whole(out, li.x, wl, li8.experts, li8.shared, T, tight=TIGHT, int4_bf16=True)


# Row tolerance against the oracle that rounds like the GPU (h to bf16; int4 weights to bf16(q*s)),
# 8x below the plain bound: what is left is binary32 accumulation order and the h elements whose
# bf16 rounding flips (a flip moves a row by about 1e-4, a few flips in the worst of 8192 rows).
TIGHT = 2.5e-3


def test_tiny_fp32_layer():
    need_gpu()
    from expert_offload_cache_amd.layer import DeviceLayer

    wl = synth.WORKLOADS["tiny_fp32"]
    li = synth.layer_inputs(wl, 16, seed=0)
    layer = DeviceLayer.from_inputs(li)
    out = _run(layer, li)
    ref = moe_layer(li.x, li.w_router, li.bias, "f32", wl.k, wl.E, li.experts)
    _check_ints(out, ref)
    assert np.array_equal(out["logits"].cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32))
    g = out["topk_w"].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g - ref["gates"]) / ref["gates"]) <= 1e-6
    err = rel_err_per_token(y_to_f64(out["y"]), ref["y"])
    print(f"max per-token rel err {err.max():.3g}")
    assert err.max() <= 1e-4


@pytest.fixture(scope="module")
def dsv4_bf16_layer():
    need_gpu()
    from expert_offload_cache_amd.layer import DeviceLayer

    wl = synth.WORKLOADS["dsv4_prefill_bf16"]
    li = synth.layer_inputs(wl, 8192, seed=0)
    layer = DeviceLayer.from_inputs(li)
    yield wl, li, layer
    del layer
    gc.collect()


@pytest.mark.parametrize("T", [512, 2048, 8192])
def test_dsv4_prefill_layer_sampled(dsv4_bf16_layer, T):
    """Full-size prefill: every routing integer bit-exact; outputs checked on sampled tokens."""
    wl, li_full, layer = dsv4_bf16_layer
    print(f"dsv4 prefill bf16 T={T}", flush=True)
    li = synth.layer_inputs(wl, T, seed=0, with_experts=False)
    out = _run(layer, li)
    from oracle.permute import permute as o_permute
    from oracle.router import route as o_route

    _, idx, gates = o_route(li.x, li_full.w_router, li_full.bias, "bf16", wl.k)
    assert np.array_equal(out["topk_idx"].cpu().numpy(), idx)
    c, o, p, ip = o_permute(idx, wl.E)
    for key, v in (("counts", c), ("offsets", o), ("perm", p), ("inv_perm", ip)):
        assert np.array_equal(out[key].cpu().numpy(), v), key
    toks = sorted({0, 1, T // 2, T - 1, *np.random.default_rng(T).choice(T, 4, replace=False).tolist()})
    ref = moe_layer_tokens(toks, li.x, li_full.w_router, li_full.bias, "bf16", wl.k, wl.E, li_full.experts,
                           li_full.shared)
    y = y_to_f64(out["y"])[toks]
    err = rel_err_per_token(y, ref["y"])
    print(f"max n_e {int(c.max())} sampled max rel err {err.max():.3g}")
    assert err.max() <= 2e-2
    if T >= 2048:
        _check_experts_whole(out, li.x, wl, li_full.experts, li_full.shared, T, tight=TIGHT)


EDGE = [
    # (name, act, wdt, d, f, E, k, T, shared, forced expert or None)
    ("one expert, decode", "bf16", "bf16", 256, 128, 1, 1, 5, False, None),
    ("one expert, prefill", "bf16", "bf16", 512, 256, 1, 1, 300, True, None),
    ("all tokens on expert 2, bf16 prefill", "bf16", "bf16", 512, 256, 8, 1, 700, False, 2),
    ("all tokens on expert 5, int4 prefill", "bf16", "int4", 512, 256, 8, 1, 700, True, 5),
    ("k = E, decode (every expert holds every token)", "bf16", "bf16", 256, 96, 8, 8, 20, True, None),
    ("1024 experts, most empty", "bf16", "bf16", 256, 64, 1024, 8, 16, False, None),
    ("int4, k = E", "bf16", "int4", 256, 128, 4, 4, 33, False, None),
]


@pytest.mark.parametrize("name,act,wdt,d,f,E,k,T,shared,forced", EDGE, ids=[c[0] for c in EDGE])
def test_degenerate_layers(name, act, wdt, d, f, E, k, T, shared, forced):
    """Degenerate routings against the oracle: a single expert, every token on one expert (one
    expert's chunks fill the launch, the others are empty), k = E, and a thousand mostly empty
    experts."""
    need_gpu()
    from expert_offload_cache_amd.layer import DeviceLayer

    print(f"edge layer: {name}", flush=True)
    wl = small_workload(act, wdt, d, f, E, k, shared=shared, bias=1.1)
    li = synth.layer_inputs(wl, T, seed=9)
    layer = DeviceLayer.from_inputs(li)
    fidx = None if forced is None else np.full((T, k), forced, dtype=np.int32)
    out = _run(layer, li, forced=fidx)
    ref = moe_layer(li.x, li.w_router, li.bias, act, k, E, li.experts, li.shared, forced_idx=fidx)
    _check_ints(out, ref)
    err = rel_err_per_token(y_to_f64(out["y"]), ref["y"])
    print(f"max per-token rel err {err.max():.3g}")
    assert err.max() <= tol_for(wl)
    assert int(out["ws"][:4].view(dtype=__import__("torch").int32).item()) == 0


def test_empty_batch_is_a_no_op():
    """T = 0: every hot-path call returns OK; the permutation of an empty batch has zero counts and
    offsets and writes nothing else."""
    need_gpu()
    import torch
    from expert_offload_cache_amd._lib import lib, MOE_BF16

    E, k, d = 8, 2, 256
    counts = torch.full((E,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), 7, dtype=torch.int32, device="cuda")
    assert lib().moe_route(None, MOE_BF16, 0, d, None, None, E, k, None, None, None, None, None) == 0
    assert lib().moe_permute(None, 0, k, E, counts.data_ptr(), offsets.data_ptr(), None, None, None, 0, None) == 0
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * E and offsets.cpu().tolist() == [0] * (E + 1)
    assert lib().moe_combine(None, 0, None, None, 0, k, d, 0, None, MOE_BF16, None) == 0


# every kernel path that writes y_perm: decode GEMVs (deep int4, K-streaming bf16 and int4, the
# split-input and vector-ALU kernels), the bf16 and int4 GEMMs and their light-expert launches
Y16 = [
    # (act, wdt, d, f, E, k, T, shared)
    ("bf16", "bf16", 512, 256, 8, 2, 3, True),       # K-streaming bf16, few tokens
    ("bf16", "bf16", 4096, 64, 4, 2, 20, False),     # K-streaming bf16, 32-token items
    ("bf16", "bf16", 2112, 64, 4, 2, 20, False),     # split-input down (132 row blocks)
    ("bf16", "bf16", 320, 96, 8, 2, 9, True),        # split-input kernel, both projections
    ("bf16", "int4", 4096, 2048, 8, 2, 1, True),     # deep int4 decode kernel
    ("bf16", "int4", 512, 512, 8, 2, 20, True),      # K-streaming int4
    ("bf16", "int4", 256, 128, 8, 2, 5, True),       # vector-ALU int4 down
    ("bf16", "bf16", 512, 256, 64, 2, 300, True),    # bf16 GEMM + its light-expert launch
    ("bf16", "int4", 512, 256, 32, 2, 300, True),    # int4 GEMM + light experts
    ("bf16", "bf16", 256, 256, 3, 1, 1000, True),    # GEMM tiles with ragged tails
]


@pytest.mark.parametrize("act,wdt,d,f,E,k,T,shared", Y16)
def test_bf16_rows_are_the_binary32_rows_rounded(act, wdt, d, f, E, k, T, shared):
    """y_perm as bf16 rows is the binary32 y_perm of the same call rounded to nearest even, bit for
    bit (the kernels round their binary32 sums once at the store), and the combine over bf16 rows
    equals the combine over binary32 rows holding the same values, bit for bit (widening is exact)."""
    need_gpu()
    import torch
    import expert_offload_cache_amd as moe
    from expert_offload_cache_amd.layer import DeviceLayer

    print(f"bf16 rows {wdt} d={d} f={f} E={E} k={k} T={T}", flush=True)
    wl = small_workload(act, wdt, d, f, E, k, shared=shared, bias=1.1)
    li = synth.layer_inputs(wl, T, seed=11)
    layer = DeviceLayer.from_inputs(li)
    x = layer.x_to_device(li.x)
    out = layer.forward(x)
    args = (x, out["perm"], out["offsets"], out["counts"], layer.slot_of_expert, layer.pool, layer.n_slots,
            layer.stride, layer.wdt, layer.f, layer.k)
    y32, _ = moe.expert_ffn_grouped(*args, shared_w=layer.shared, y_dtype=torch.float32)
    y16, _ = moe.expert_ffn_grouped(*args, shared_w=layer.shared, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    # combine: bf16 rows against the same values held as binary32
    w, inv = out["topk_w"], out["inv_perm"]
    a = moe.combine(y16, w, inv, k, shared, torch.bfloat16)
    b = moe.combine(y16.float(), w, inv, k, shared, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
