"""GPU router and permutation against the oracle: bit-exact logits, ids, counts, offsets,
permutation; gates within 1e-6 relative.  Sizes span several tiles with ragged tails, up to the
full prefill batch (8192 tokens x 256 experts x d 4096)."""
import numpy as np
import pytest

import synth
from gpu_util import need_gpu, to_dev
from oracle.permute import permute as o_permute
from oracle.router import renorm_gates, router_logits, topk_select

pytestmark = pytest.mark.gpu

ROUTE_CASES = [
    # (act, d, E, k, T, bias)
    ("f32", 64, 8, 2, 16, None),          # tiny fp32 layer
    ("f32", 256, 40, 3, 77, 1.1),         # fp32, ragged T on the tiled path
    ("bf16", 2048, 128, 8, 1, 1.1),       # Qwen-A3B shaped decode
    ("bf16", 2048, 128, 8, 4, 1.1),
    ("bf16", 2048, 128, 8, 16, 1.1),
    ("bf16", 2048, 128, 8, 64, 1.1),
    ("bf16", 4096, 256, 6, 1, 1.1),       # DeepSeek-V4-Flash shaped decode
    ("bf16", 4096, 256, 6, 2, 1.1),
    ("bf16", 4096, 256, 6, 8, 1.1),
    ("bf16", 4096, 256, 6, 65, 1.1),      # just past the decode kernel
    ("bf16", 4096, 256, 6, 333, 1.1),     # ragged tiles
    ("bf16", 4096, 256, 6, 512, 1.1),     # prefill batches
    ("bf16", 4096, 256, 6, 2048, 1.1),
    ("bf16", 4096, 256, 6, 8192, 1.1),
    ("bf16", 1024, 1024, 8, 70, None),    # maximum expert count
    ("bf16", 512, 100, 100, 9, 1.1),      # k = E, ragged E
    ("bf16", 2048, 128, 8, 100, 1.1),     # subtree-split prefill kernel, ragged tokens
    ("bf16", 2048, 100, 4, 97, None),     # ... ragged experts, no bias
    ("bf16", 6144, 96, 4, 130, 1.1),      # ... three chunks per segment
    ("bf16", 1024, 256, 8, 33, 1.1),      # tiled decode logits, 2 chunks of 8 a lane
    ("bf16", 1024, 512, 8, 5, None),      # one wave a pair, 512 experts
    ("bf16", 2048, 100, 4, 3, None),      # ragged experts
    ("bf16", 2048, 256, 8, 2, 1.1),
]


@pytest.mark.parametrize("act,d,E,k,T,bias", ROUTE_CASES)
def test_route_bit_exact(act, d, E, k, T, bias):
    need_gpu()
    import expert_offload_cache_amd as moe

    print(f"route act={act} d={d} E={E} k={k} T={T}", flush=True)
    gen = synth.normal_bf16 if act == "bf16" else synth.normal_f32
    x = gen(11, synth.stream_id(synth.KIND_X, 0, T), (T, d), 1.0)
    w = gen(11, synth.stream_id(synth.KIND_ROUTER, 0, E), (E, d), 0.02)
    b = synth.router_bias(11, E, bias) if bias else None
    lg = router_logits(x, w, b, act)
    idx = topk_select(lg, k)
    g = renorm_gates(lg, idx)
    xd, wd = to_dev(x, act), to_dev(w, act)
    bd = None if b is None else to_dev(b, "f32")
    gi, gw, gl = moe.route(xd, wd, bd, k)
    gl = gl.cpu().numpy()
    assert np.array_equal(gl.view(np.uint32), lg.view(np.uint32)), "logits differ"
    assert np.array_equal(gi.cpu().numpy(), idx)
    gw = gw.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gw - g) / g) <= 1e-6
    # near-ties: report the smallest k-th / (k+1)-th gap the case exercised
    if k < E:
        s = -np.sort(-lg, axis=1)
        print(f"min top-k gap {np.min(s[:, k - 1] - s[:, k]):.3g}")


def test_route_forced_ids():
    need_gpu()
    import expert_offload_cache_amd as moe

    T, d, E, k = 37, 4096, 256, 6
    x = synth.normal_bf16(2, 5, (T, d), 1.0)
    w = synth.normal_bf16(2, 6, (E, d), 0.02)
    b = synth.router_bias(2, E, 1.1)
    forced = synth.forced_topk(2, T, E, k)
    lg = router_logits(x, w, b, "bf16")
    g = renorm_gates(lg, forced)
    gi, gw, _ = moe.route(to_dev(x, "bf16"), to_dev(w, "bf16"), to_dev(b, "f32"), k, forced_idx=to_dev(forced, "i32"))
    assert np.array_equal(gi.cpu().numpy(), forced)
    assert np.max(np.abs(gw.cpu().numpy() - g) / g) <= 1e-6


PERM_CASES = [
    # (T, E, k, kind)
    (1, 8, 2, "rand"), (16, 8, 2, "rand"), (64, 128, 8, "rand"), (1, 256, 6, "rand"), (333, 256, 6, "rand"),
    (8192, 256, 6, "rand"), (1000, 1024, 8, "rand"), (4096, 64, 1, "one"), (700, 5, 5, "all"),
    (8192, 256, 6, "zipf"),
    # beyond 8192 pairs with a workspace: the sort split over workgroups (ragged last workgroup,
    # one expert holding every pair, every expert in every token, a thousand experts)
    (2048, 256, 6, "zipf"), (3001, 7, 3, "rand"), (12000, 64, 1, "one"), (700, 16, 16, "all"),
    (1500, 1024, 8, "rand"), (40000, 256, 6, "zipf"),
]


@pytest.mark.parametrize("T,E,k,kind", PERM_CASES)
def test_permute_bit_exact(T, E, k, kind):
    need_gpu()
    import expert_offload_cache_amd as moe

    print(f"permute T={T} E={E} k={k} {kind}", flush=True)
    ws = moe.permute_workspace(T, k, E, "cuda")
    if kind == "rand":
        idx = synth.forced_topk(T, T, E, k)
    elif kind == "one":
        idx = np.full((T, k), 3, dtype=np.int32)  # every pair on one expert
    elif kind == "all":
        idx = np.tile(np.arange(E, dtype=np.int32)[::-1], (T, 1))
    else:
        tr = synth.routing_trace(0, T, 1, E, k, p_reuse=0.0)  # independent Zipf draws per token
        idx = np.ascontiguousarray(tr[:, 0, :])
    c, o, p, ip = o_permute(idx, E)
    for w in ([None] if ws is None else [None, ws]):  # one workgroup, and the split sort
        gc, go, gp, gip = moe.permute(to_dev(idx, "i32"), E, ws=w)
        assert np.array_equal(gc.cpu().numpy(), c)
        assert np.array_equal(go.cpu().numpy(), o)
        assert np.array_equal(gp.cpu().numpy(), p)
        assert np.array_equal(gip.cpu().numpy(), ip)
    assert (ws is not None) == (T * k > 8192)


RP_CASES = [
    # (act, d, E, k, T, bias, kind): moe_route_permute; for T = 1 one block selects and sorts
    # (when its LDS holds E and the ids), other shapes run the two calls' kernels
    ("f32", 64, 8, 2, 1, None, "rand"),        # one wave
    ("f32", 64, 8, 2, 2, 1.1, "rand"),
    ("f32", 64, 8, 2, 16, None, "rand"),
    ("bf16", 2048, 128, 8, 1, 1.1, "rand"),    # Qwen-A3B shaped decode, 8 waves
    ("bf16", 2048, 128, 8, 2, 1.1, "rand"),
    ("bf16", 2048, 128, 8, 4, 1.1, "rand"),
    ("bf16", 2048, 128, 8, 64, 1.1, "rand"),
    ("bf16", 4096, 256, 6, 1, 1.1, "rand"),    # DeepSeek-V4-Flash shaped decode, 16 waves
    ("bf16", 4096, 256, 6, 2, 1.1, "rand"),
    ("bf16", 4096, 256, 6, 8, 1.1, "rand"),
    ("bf16", 512, 100, 16, 2, None, "rand"),   # ragged E
    ("bf16", 256, 16, 16, 2, 1.1, "rand"),     # k = E
    ("bf16", 512, 40, 3, 1, 1.1, "rand"),      # 3 waves rounded to 4
    ("bf16", 512, 100, 16, 1, None, "rand"),
    ("bf16", 256, 16, 16, 1, 1.1, "rand"),
    ("bf16", 256, 64, 8, 1, None, "ties"),
    ("bf16", 256, 64, 8, 1, None, "flat"),
    ("bf16", 4096, 256, 6, 1, 1.1, "forced"),
    ("bf16", 256, 64, 8, 2, None, "ties"),     # pairs of equal logits: lower id first
    ("bf16", 256, 64, 8, 40, None, "ties"),
    ("bf16", 256, 64, 8, 2, None, "flat"),     # every logit +0: experts 0..k-1, equal gates
    ("bf16", 4096, 256, 6, 2, 1.1, "forced"),  # replayed ids
    ("bf16", 4096, 256, 6, 37, 1.1, "forced"),
    ("bf16", 512, 512, 64, 1, 1.1, "rand"),    # largest E the one block holds, k = 64
    ("bf16", 512, 512, 64, 2, 1.1, "rand"),
    ("bf16", 512, 513, 8, 1, 1.1, "rand"),     # past it: two launches
    ("bf16", 1024, 1024, 8, 2, None, "rand"),
    ("bf16", 2048, 128, 8, 65, 1.1, "rand"),
    ("bf16", 4096, 256, 6, 512, 1.1, "rand"),  # prefill batch
    # more ties, equal logits and replayed ids on both paths
    ("bf16", 1024, 64, 8, 1, None, "ties"),
    ("bf16", 1024, 64, 8, 1, None, "flat"),
    ("bf16", 1024, 64, 8, 9, None, "ties"),
    ("bf16", 2048, 128, 8, 1, 1.1, "forced"),
    ("bf16", 2048, 128, 8, 5, 1.1, "forced"),
    ("bf16", 1024, 512, 16, 1, 1.1, "rand"),
    ("bf16", 2048, 100, 4, 1, None, "rand"),
    ("bf16", 1024, 256, 8, 64, 1.1, "rand"),
    # more than 64 tokens: a wave per token selects (ties, equal logits, replayed ids, k = 64 of
    # 1024, ragged E), and beyond 8192 pairs the sort is split over workgroups
    ("bf16", 256, 64, 8, 100, None, "ties"),
    ("bf16", 256, 64, 8, 100, None, "flat"),
    ("bf16", 4096, 256, 6, 300, 1.1, "forced"),
    ("bf16", 512, 1024, 64, 70, 1.1, "rand"),
    ("bf16", 512, 1000, 16, 80, None, "rand"),
    ("bf16", 512, 40, 40, 66, 1.1, "rand"),
    ("bf16", 4096, 256, 6, 2048, 1.1, "rand"),
    ("f32", 128, 8, 2, 4500, None, "rand"),
    ("f32", 128, 8, 2, 1, None, "rand"),       # one token, binary32 activations
    ("f32", 192, 100, 7, 1, 1.1, "forced"),
]


@pytest.mark.parametrize("act,d,E,k,T,bias,kind", RP_CASES)
def test_route_permute_matches_the_two_calls_and_the_oracle(act, d, E, k, T, bias, kind):
    need_gpu()
    import expert_offload_cache_amd as moe

    print(f"route_permute act={act} d={d} E={E} k={k} T={T} {kind}", flush=True)
    gen = synth.normal_bf16 if act == "bf16" else synth.normal_f32
    x = gen(13, synth.stream_id(synth.KIND_X, 1, T), (T, d), 1.0)
    if kind == "ties":
        w = np.repeat(gen(13, synth.stream_id(synth.KIND_ROUTER, 1, E), (E // 2, d), 0.02), 2, axis=0)
    elif kind == "flat":
        w = np.zeros_like(gen(13, synth.stream_id(synth.KIND_ROUTER, 1, E), (E, d), 0.02))
    else:
        w = gen(13, synth.stream_id(synth.KIND_ROUTER, 1, E), (E, d), 0.02)
    b = synth.router_bias(13, E, bias) if bias else None
    forced = synth.forced_topk(13, T, E, k) if kind == "forced" else None
    lg = router_logits(x, w, b, act)
    idx = forced if forced is not None else topk_select(lg, k)
    g = renorm_gates(lg, idx)
    c, o, p, ip = o_permute(idx, E)

    xd, wd = to_dev(x, act), to_dev(w, act)
    bd = None if b is None else to_dev(b, "f32")
    fd = None if forced is None else to_dev(forced, "i32")
    pws = moe.permute_workspace(T, k, E, "cuda")
    out = moe.route_permute(xd, wd, bd, k, forced_idx=fd, ws=pws)
    moe.route_permute(xd, wd, bd, k, forced_idx=fd, out=out, ws=pws)  # again into the same buffers
    got = [a.cpu().numpy() for a in out]
    gi, gw, gl = moe.route(xd, wd, bd, k, forced_idx=fd)
    two = [gi, gw, gl] + list(moe.permute(gi, E))
    two = [a.cpu().numpy() for a in two]
    for name, a, r in zip(["topk_idx", "topk_w", "logits", "counts", "offsets", "perm", "inv_perm"], got, two):
        assert a.shape == r.shape and np.array_equal(a.view(np.uint32), r.view(np.uint32)), name
    assert np.array_equal(got[2].view(np.uint32), lg.view(np.uint32)), "logits differ from the oracle"
    assert np.array_equal(got[0], idx)
    assert np.max(np.abs(got[1].astype(np.float64) - g) / g) <= 1e-6
    for a, r in zip(got[3:], (c, o, p, ip)):
        assert np.array_equal(a, r)
    if kind == "ties":
        assert np.all(got[0][:, 0] % 2 == 0)  # of an equal pair the even (lower) id comes first
    if kind == "flat":
        assert np.array_equal(got[0], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
        assert np.all(got[1] == np.float32(1.0 / k))


def test_route_permute_empty_batch():
    need_gpu()
    import torch

    import expert_offload_cache_amd as moe

    E, k, d = 128, 8, 2048
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    w = to_dev(synth.normal_bf16(1, 1, (E, d), 0.02), "bf16")
    out = moe.route_permute(x, w, None, k)
    torch.cuda.synchronize()
    assert out[0].shape == (0, k) and out[5].numel() == 0
    assert np.array_equal(out[3].cpu().numpy(), np.zeros(E, np.int32))
    assert np.array_equal(out[4].cpu().numpy(), np.zeros(E + 1, np.int32))
