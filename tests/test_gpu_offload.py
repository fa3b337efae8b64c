"""Offloaded stack on the GPU: pinned host pool -> LRU slot cache -> layer kernels, against the
oracle (layer outputs) and the oracle's LRU simulator (hit/miss sequence, miss counts).

Small int4 stack: 4 layers of E=8 experts (top-2, d=256, d_ff=128, shared expert), 16 distinct
expert images; a 40-token prefill that prefetches each next layer, then a 25-step decode trace.
"""
import gc

import numpy as np
import pytest

import synth
from gpu_util import need_gpu, rel_err_per_token, small_workload, y_to_f64
from oracle.layer import moe_layer, moe_layer_tokens
from oracle.lru import LRUSim

pytestmark = pytest.mark.gpu

L, E, K, D, F = 4, 8, 2, 256, 128
T_PRE, STEPS, IMAGES = 40, 25, 16


def _wl():
    return small_workload("bf16", "int4", D, F, E, K, shared=True, bias=1.1)


def _trace():
    return synth.routing_trace(seed=3, steps=STEPS, L=L, E=E, k=K)


def _layer_weights(stack, wl, l):
    experts = []
    for e in range(E):
        i = stack.image_of(l, e)
        experts.append(synth.expert_weights(wl, 0, i // E, i % E))
    shared = synth.expert_weights(wl, 0, stack.shared_layer_of(l), 0, shared=True)
    return experts, shared


def _expected(trace, C):
    """Simulator replay of the same request sequence -> (hit flags, [(slot, key)] of every copy)."""
    sim = LRUSim(C)
    flags, copies = [], []
    reqs = [(l, list(range(E)), "prefill") for l in range(L)]
    reqs += [(l, np.unique(trace[s, l]).tolist(), "decode") for s in range(STEPS) for l in range(L)]
    for l, ids, phase in reqs:
        slots, fl, _ = sim.request(l, ids, phase=phase)
        flags += fl
        copies += [(sl, l * E + e) for e, sl, h in zip(sorted(ids), slots, fl) if not h]
    return np.array(flags, dtype=np.uint8), copies


def _run(C):
    from expert_offload_cache_amd.offload import OffloadStack

    wl = _wl()
    stack = OffloadStack(wl, L, C, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
    _, pre = stack.prefill(keep_outputs=True)
    _, dec = stack.decode(_trace(), keep_outputs=True)
    res = dict(pre=[(i.cpu().numpy(), y_to_f64(y)) for i, y in pre], dec=[(s, l, y_to_f64(y)) for s, l, y in dec],
               trace=stack.cache.trace(), stats=stack.cache.stats(), stack=stack)
    return wl, res


@pytest.fixture(scope="module")
def runs():
    need_gpu()
    out = {}
    for C in (16, 20, 32):
        print(f"offload stack L={L} E={E} C={C}", flush=True)
        out[C] = _run(C)
    yield out
    for _, r in out.values():
        r["stack"].close()
    gc.collect()


@pytest.mark.parametrize("C", [16, 20, 32])
def test_hit_miss_sequence_matches_simulator(runs, C):
    _, r = runs[C]
    want, copies = _expected(_trace(), C)
    assert np.array_equal(r["trace"], want)
    log = r["stack"].cache.copy_log()
    assert [(int(a), int(b)) for a, b in log[:, :2]] == copies
    st = r["stats"]
    n_dec = STEPS * L * K
    assert st["dec_acc"] == n_dec and st["pre_acc"] == L * E
    assert st["dec_miss"] == int((want[L * E:] == 0).sum())
    assert st["bytes_h2d"] == int((want == 0).sum()) * r["stack"].stride


def test_decode_outputs_match_oracle(runs):
    wl, r = runs[20]
    stack, trace = r["stack"], _trace()
    per_layer = {l: _layer_weights(stack, wl, l) for l in range(L)}
    worst = 0.0
    for s, l, y in r["dec"]:
        li = synth.layer_inputs(wl, 8, 0, layer=l, batch=1, with_experts=False)
        x = li.x[s % 8:s % 8 + 1]
        experts, shared = per_layer[l]
        ref = moe_layer(x, li.w_router, li.bias, "bf16", K, E, experts, shared, forced_idx=trace[s, l:l + 1])
        worst = max(worst, float(rel_err_per_token(y, ref["y"]).max()))
    print(f"decode max per-token rel err {worst:.3g}")
    assert worst <= 2e-2


def test_prefill_outputs_match_oracle(runs):
    wl, r = runs[20]
    stack = r["stack"]
    for l, (idx, y) in enumerate(r["pre"]):
        li = synth.layer_inputs(wl, T_PRE, 0, layer=l, batch=0, with_experts=False)
        experts, shared = _layer_weights(stack, wl, l)
        toks = [0, 7, T_PRE // 2, T_PRE - 1]
        ref = moe_layer_tokens(toks, li.x, li.w_router, li.bias, "bf16", K, E, experts, shared)
        assert np.array_equal(idx[toks], ref["topk_idx"])
        err = rel_err_per_token(y[toks], ref["y"])
        assert err.max() <= 2e-2, (l, err)


def test_outputs_do_not_depend_on_capacity(runs):
    """Cache capacity changes which copies happen, never the layer outputs (bitwise)."""
    ref = runs[32][1]
    for C in (16, 20):
        r = runs[C][1]
        for (s0, l0, y0), (s1, l1, y1) in zip(ref["dec"], r["dec"]):
            assert (s0, l0) == (s1, l1) and np.array_equal(y0, y1)
        for (i0, y0), (i1, y1) in zip(ref["pre"], r["pre"]):
            assert np.array_equal(i0, i1) and np.array_equal(y0, y1)


def test_native_decode_step_matches_the_call_by_call_loop(runs):
    """moe_decode_step (one call per step) makes the same calls as the Python loop over layers:
    outputs, the cache's hit/miss sequence, copy plan and statistics are bitwise the same."""
    from expert_offload_cache_amd.offload import OffloadStack

    _, ref = runs[16]  # the fixture's decode runs through moe_decode_step
    stack = OffloadStack(_wl(), L, 16, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
    try:
        stack.prefill()
        _, dec = stack.decode(_trace(), keep_outputs=True, native=False)
        assert np.array_equal(stack.cache.trace(), ref["trace"])
        assert stack.cache.stats() == ref["stats"]
        log = stack.cache.copy_log()
        assert np.array_equal(log, ref["stack"].cache.copy_log())
    finally:
        stack.close()
    assert len(dec) == len(ref["dec"]) == STEPS * L
    for (s0, l0, y0), (s1, l1, y1) in zip(ref["dec"], dec):
        assert (s0, l0) == (s1, l1) and np.array_equal(y0, y_to_f64(y1))


def test_split_launch_matches_plain_decode(runs):
    """Split launches (resident experts before the copies' wait, missed ones after) change when the
    experts run, not what they compute: outputs and the cache's decisions are bitwise those of the
    plain decode at the same capacity."""
    from expert_offload_cache_amd.offload import OffloadStack

    _, ref = runs[16]
    stack = OffloadStack(_wl(), L, 16, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
    try:
        stack.prefill()
        _, dec = stack.decode(_trace(), keep_outputs=True, split_launch=True)
        assert np.array_equal(stack.cache.trace(), ref["trace"])
        st = stack.cache.stats()
        assert st["dec_miss"] == ref["stats"]["dec_miss"] > 0
    finally:
        stack.close()
    for (s0, l0, y0), (s1, l1, y1) in zip(ref["dec"], dec):
        assert (s0, l0) == (s1, l1) and np.array_equal(y0, y_to_f64(y1))


def test_native_split_matches_the_call_by_call_loop(runs):
    """moe_decode_step_split makes the split-launch loop's calls: outputs, the hit/miss sequence
    and copy plan are bitwise those of the Python loop (and of the plain decode)."""
    from expert_offload_cache_amd.offload import OffloadStack

    _, ref = runs[16]
    got = []
    for native in (True, False):
        stack = OffloadStack(_wl(), L, 16, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
        try:
            stack.prefill()
            _, dec = stack.decode(_trace(), keep_outputs=True, split_launch=True, native=native)
            got.append((stack.cache.trace(), stack.cache.copy_log(), stack.cache.stats(),
                        [(s, l, y_to_f64(y)) for s, l, y in dec]))
        finally:
            stack.close()
    (t0, c0, st0, d0), (t1, c1, st1, d1) = got
    assert np.array_equal(t0, t1) and np.array_equal(c0, c1) and st0 == st1
    assert np.array_equal(t0, ref["trace"]) and st0["dec_miss"] > 0
    assert len(d0) == len(d1) == len(ref["dec"])
    for (s0, l0, y0), (s1, l1, y1), (s2, l2, y2) in zip(d0, d1, ref["dec"]):
        assert (s0, l0) == (s1, l1) == (s2, l2) and np.array_equal(y0, y1) and np.array_equal(y0, y2)


def test_resize_mid_trace():
    """Shrink then grow between decode steps: outputs bitwise equal to a fixed-capacity run, and
    hits, slots and moves equal to the simulator's."""
    need_gpu()
    from expert_offload_cache_amd.offload import OffloadStack

    wl, trace = _wl(), _trace()
    stack = OffloadStack(wl, L, 32, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
    try:
        stack.new_cache(20)
        stack.prefill()
        outs = []
        plan = [(0, 9, None), (9, 17, 12), (17, STEPS, 28)]
        for a, b, cap in plan:
            if cap is not None:
                stack.resize(cap)
            _, o = stack.decode(trace[a:b], keep_outputs=True, first_step=a)
            outs += [(s, l, y_to_f64(y)) for s, l, y in o]
        sim = LRUSim(20)
        flags, copies = [], []
        for l in range(L):
            slots, fl, _ = sim.request(l, list(range(E)), phase="prefill")
            flags += fl
            copies += [(sl, l * E + e, None) for e, sl, h in zip(range(E), slots, fl) if not h]
        for a, b, cap in plan:
            if cap is not None:
                copies += [(new, key[0] * E + key[1], -2 - old) for old, new, key in sim.resize(cap)]
            for s in range(a, b):
                for l in range(L):
                    ids = np.unique(trace[s, l]).tolist()
                    slots, fl, _ = sim.request(l, ids)
                    flags += fl
                    copies += [(sl, l * E + e, None) for e, sl, h in zip(ids, slots, fl) if not h]
        assert np.array_equal(stack.cache.trace(), np.array(flags, dtype=np.uint8))
        log = stack.cache.copy_log()
        got = [(int(a), int(b), int(m) if m <= -2 else None) for a, b, m in log]
        assert got == copies
    finally:
        stack.close()
    ref = _run(32)[1]
    for (s0, l0, y0), (s1, l1, y1) in zip(ref["dec"], outs):
        assert (s0, l0) == (s1, l1) and np.array_equal(y0, y1)
    ref["stack"].close()


@pytest.mark.parametrize("copy_too", [True, False])
def test_hybrid_miss_split(copy_too):
    """Hybrid miss handling: the host runs its share of each layer's misses from the pinned images
    while the rest is copied.  With copy_too the host's misses are still inserted (deferred copies)
    and the cache sees every request in full; without it the cache sees only the GPU share (as the
    simulator fed the same split).  Outputs match the oracle."""
    need_gpu()
    from expert_offload_cache_amd.offload import OffloadStack
    from oracle.hybrid import host_misses, hybrid_split

    wl, trace = _wl(), _trace()
    # equal host and PCIe rates with a fixed host cost of 0.3 expert-times: a layer with one miss
    # keeps it on the GPU, two misses put one on the host
    rates = (1.0, 1.0, copy_too, 0.3)
    stack = OffloadStack(wl, L, 16, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
    try:
        stack.prefill()
        _, dec = stack.decode(trace, keep_outputs=True, hybrid=rates)
        outs = [(s, l, y_to_f64(y)) for s, l, y in dec]
        sim = LRUSim(16)
        flags = []
        for l in range(L):
            flags += sim.request(l, list(range(E)), phase="prefill")[1]
        n_cpu_total = 0
        for s in range(STEPS):
            for l in range(L):
                ids = np.unique(trace[s, l]).tolist()
                miss = [e for e in ids if (l, e) not in sim.od]
                on_cpu = host_misses(miss, hybrid_split(len(miss), rates[0], rates[1], rates[3]))
                n_cpu_total += len(on_cpu)
                flags += sim.request(l, [e for e in ids if copy_too or e not in on_cpu])[1]
        assert np.array_equal(stack.cache.trace(), np.array(flags, dtype=np.uint8))
        assert stack.cpu_experts == n_cpu_total > 0
    finally:
        stack.close()
    per_layer = {}
    worst = 0.0
    for s, l, y in outs:
        if l not in per_layer:
            per_layer[l] = _layer_weights(stack, wl, l)
        li = synth.layer_inputs(wl, 8, 0, layer=l, batch=1, with_experts=False)
        experts, shared = per_layer[l]
        ref = moe_layer(li.x[s % 8:s % 8 + 1], li.w_router, li.bias, "bf16", K, E, experts, shared,
                        forced_idx=trace[s, l:l + 1])
        worst = max(worst, float(rel_err_per_token(y, ref["y"]).max()))
    assert worst <= 2e-2


@pytest.mark.parametrize("copy_too", [True, False])
def test_native_hybrid_matches_the_call_by_call_loop(copy_too):
    """moe_decode_step_hybrid makes the hybrid loop's calls: outputs, the cache's hit/miss
    sequence, copy plan and the number of host-run experts are bitwise those of the Python loop."""
    need_gpu()
    from expert_offload_cache_amd.offload import OffloadStack

    wl, trace = _wl(), _trace()
    rates = (1.0, 1.0, copy_too, 0.3)
    got = []
    for native in (True, False):
        stack = OffloadStack(wl, L, 16, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
        try:
            stack.prefill()
            _, dec = stack.decode(trace, keep_outputs=True, hybrid=rates, native=native)
            got.append((stack.cache.trace(), stack.cache.copy_log(), stack.cache.stats(), stack.cpu_experts,
                        [(s, l, y_to_f64(y)) for s, l, y in dec]))
        finally:
            stack.close()
    (t0, c0, st0, n0, d0), (t1, c1, st1, n1, d1) = got
    assert np.array_equal(t0, t1) and np.array_equal(c0, c1) and st0 == st1
    assert n0 == n1 > 0
    assert len(d0) == len(d1) == STEPS * L
    for (s0, l0, y0), (s1, l1, y1) in zip(d0, d1):
        assert (s0, l0) == (s1, l1) and np.array_equal(y0, y1)


def test_resize_right_after_mark_read_without_a_sync():
    """A shrink enqueued straight after the last layer's mark_read (no host synchronisation, the
    layer's kernels possibly still queued) must not let those kernels read evicted table entries:
    outputs stay bitwise those of a fixed-capacity run and no absent slot is flagged."""
    need_gpu()
    import torch
    from expert_offload_cache_amd.offload import OffloadStack

    wl, trace = _wl(), _trace()
    stack = OffloadStack(wl, L, 32, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
    try:
        stack.prefill()
        _, o = stack.decode(trace[:6], keep_outputs=True)
        outs = [(s, l, y_to_f64(y)) for s, l, y in o]
        # step 6 by hand, so that the shrink follows the last mark_read with work still queued
        s = 6
        forced = stack._forced(trace[s:s + 1])
        ys = []
        with torch.cuda.stream(stack.compute):
            for l in range(L):
                xl = stack.x_dec[l][s % 8:s % 8 + 1]
                idx, w, perm = stack._layer(l, xl, forced[0, l:l + 1])
                # the ids are forced from the trace, so the host needs no read-back before the lookup
                stack.cache.lookup(l, np.unique(trace[s, l]))
                stack.cache.fill(stack.copy, stack.compute)
                ys.append(stack._experts(l, xl, w, perm).clone())
                stack.cache.mark_read(l, stack.compute)
            stack.resize(12)  # evicts entries the last layer's kernels may not have read yet
        torch.cuda.synchronize()
        outs += [(s, l, y_to_f64(y)) for l, y in enumerate(ys)]
        status = int(stack._workspace(1)[:4].view(torch.int32).item())
        _, o = stack.decode(trace[7:], keep_outputs=True, first_step=7)
        outs += [(st, l, y_to_f64(y)) for st, l, y in o]
    finally:
        stack.close()
    assert status == 0
    ref = _run(32)[1]
    ref_dec = {(st, l): y for st, l, y in ref["dec"]}
    assert len(outs) == STEPS * L
    for st, l, y in outs:
        assert np.array_equal(y, ref_dec[(st, l)]), (st, l)
    ref["stack"].close()


def test_native_decode_step_several_tokens():
    """moe_decode_step at T=4 (ids read back by a copy and an event rather than the published word,
    experts launched ahead of the cache's decision through the slot table as it stands, misses run
    again after their copies) against the same calls made one by one: outputs bitwise equal, and
    the same hit/miss sequence, copy plan and statistics, at a capacity that forces misses."""
    need_gpu()
    import torch
    from expert_offload_cache_amd import DECODE_LAYER, decode_step
    from expert_offload_cache_amd.offload import OffloadStack

    T, C, steps = 4, 16, 12
    rng = np.random.default_rng(11)
    # skewed expert popularity, so that the 16 slots see both hits and misses
    pop = 1.0 / np.arange(1, E + 1) ** 1.5
    ids = np.stack([rng.choice(E, K, replace=False, p=pop / pop.sum()) for _ in range(steps * L * T)])
    ids = ids.astype(np.int32).reshape(steps, L, T, K)
    got = []
    for native in (True, False):
        stack = OffloadStack(_wl(), L, C, seed=0, n_images=IMAGES, prefill_tokens=T_PRE)
        try:
            stack.prefill()
            dev = stack.device
            forced = torch.from_numpy(ids).to(dev)
            b, ws = stack._buffers(T), stack._workspace(T)
            xs = [stack.x_dec[l][0:T] for l in range(L)]
            assert all(x.shape[0] == T for x in xs)
            ys = [torch.empty_like(b["y"]) for _ in range(L)]
            host_idx = torch.empty((T, K), dtype=torch.int32, pin_memory=True)
            outs = []
            if native:
                arr = np.zeros(L, dtype=DECODE_LAYER)
                arr["x"] = [x.data_ptr() for x in xs]
                arr["w_router"] = [w.data_ptr() for w in stack.w_router]
                arr["bias"] = [0 if bb is None else bb.data_ptr() for bb in stack.bias]
                arr["shared_w"] = [0 if sw is None else sw.data_ptr() for sw in stack.shared]
                arr["y"] = [y.data_ptr() for y in ys]
                arr["layer"] = np.arange(L)
            with torch.cuda.stream(stack.compute):
                for s in range(steps):
                    if native:
                        arr["forced"] = [forced[s, l].data_ptr() for l in range(L)]
                        decode_step(stack.cache, arr, T, D, F, E, K, stack.act_code, stack.wl.wdt, stack.slot_pool,
                                    stack.n_slots, stack.stride, stack.slot_table, b["route"], b["perm"],
                                    b["y_perm"], ws, host_idx, stack.compute, stack.copy)
                    else:
                        for l in range(L):
                            _, w, perm = stack._layer(l, xs[l], forced[s, l])
                            stack.cache.lookup(l, np.unique(ids[s, l]))
                            stack.cache.fill(stack.copy, stack.compute)
                            ys[l].copy_(stack._experts(l, xs[l], w, perm))
                            stack.cache.mark_read(l, stack.compute)
                    outs += [y_to_f64(y.clone()) for y in ys]
            stack.compute.synchronize()
            status = int(ws[:4].view(torch.int32).item())
            got.append((stack.cache.trace(), stack.cache.copy_log(), stack.cache.stats(), outs, status))
        finally:
            stack.close()
    (t0, c0, st0, o0, s0), (t1, c1, st1, o1, s1) = got
    assert s0 == s1 == 0
    assert np.array_equal(t0, t1) and np.array_equal(c0, c1) and st0 == st1
    assert st0["dec_miss"] > 0 and st0["dec_hit"] > 0
    assert len(o0) == len(o1) == steps * L
    for i, (y0, y1) in enumerate(zip(o0, o1)):
        assert np.array_equal(y0, y1), divmod(i, L)
