"""Pins of the LRU slot-cache simulator: brute force, stack distances, special cases, a hand trace."""
import itertools
import json
import os

import numpy as np
import pytest

import synth
from oracle.lru import BruteLRU, CapacityError, LRUSim, stack_distance_hits


def _random_requests(rng, L, E, steps, kmax):
    reqs = []
    for _ in range(steps):
        for l in range(L):
            n = int(rng.integers(1, kmax + 1))
            reqs.append((l, rng.choice(E, size=n, replace=False).tolist()))
    return reqs


def test_golden_hand_trace(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "lru_hand_trace.json")))
    sim = LRUSim(g["capacity"])
    slots = []
    for layer, ids in g["requests"]:
        s, _, _ = sim.request(layer, ids)
        slots.append(s)
    assert sim.log == g["hitmiss"]
    assert slots == g["slots"]
    assert [list(k) for k in sim.resident().keys()] == g["final_oldest_to_newest"]


def test_simulator_equals_brute_force_on_tiny_traces():
    rng = np.random.default_rng(0)
    for L, E, C in itertools.product((1, 2, 3), (2, 4, 6), (1, 2, 3, 5)):
        kmax = min(E, C)
        for seed in range(3):
            reqs = _random_requests(np.random.default_rng([seed, L, E, C]), L, E, 30, kmax)
            a, b = LRUSim(C), BruteLRU(C)
            for layer, ids in reqs:
                sa, fa, _ = a.request(layer, ids)
                sb, fb = b.request(layer, ids)
                assert sa == sb and fa == fb
            assert a.log == b.log


def test_simulator_equals_stack_distance_recomputation():
    for L, E, C, seed in ((1, 6, 3, 0), (2, 8, 5, 1), (3, 6, 4, 2), (2, 16, 7, 3), (4, 32, 20, 4)):
        reqs = _random_requests(np.random.default_rng(seed), L, E, 40, min(E, C, 6))
        sim = LRUSim(C)
        for layer, ids in reqs:
            sim.request(layer, ids)
        assert sim.log == stack_distance_hits(reqs, C)


def test_special_cases():
    L, E, k, steps = 3, 8, 2, 25
    tr = synth.routing_trace(0, steps, L, E, k)
    reqs = [(l, tr[t, l].tolist()) for t in range(steps) for l in range(L)]
    # capacity covers every key: only compulsory misses
    sim = LRUSim(L * E)
    for r in reqs:
        sim.request(*r)
    assert len(sim.log) - sum(sim.log) == len({(l, e) for l, ids in reqs for e in ids})
    # reuse probability 1 and C >= L*k: no misses after the first step
    tr1 = synth.routing_trace(0, steps, L, E, k, p_reuse=1.0)
    sim = LRUSim(L * k)
    for t in range(steps):
        for l in range(L):
            sim.request(l, tr1[t, l].tolist())
    assert sum(sim.log[L * k:]) == len(sim.log) - L * k
    # C = k with L >= 2 layers: every access misses (the other layer's k keys evict everything)
    sim = LRUSim(k)
    for r in reqs:
        sim.request(*r)
    assert sum(sim.log) == 0


def test_capacity_error_and_stats():
    sim = LRUSim(3)
    with pytest.raises(CapacityError):
        sim.request(0, [0, 1, 2, 3])
    sim.request(0, [0, 1], phase="prefill")
    sim.request(0, [1, 2])
    assert sim.stats == dict(dec_acc=2, dec_hit=1, dec_miss=1, pre_acc=2, pre_miss=2)


def test_resize_simulator_equals_brute_force():
    """Resizes between requests: same hits, slots and moves as the linear-scan reading."""
    rng = np.random.default_rng(11)
    for trial in range(200):
        L, E = 3, 6
        C = int(rng.integers(3, 12))
        a, b = LRUSim(C), BruteLRU(C)
        for step in range(40):
            if rng.random() < 0.15:
                C2 = int(rng.integers(3, 14))
                assert a.resize(C2) == b.resize(C2)
            layer = int(rng.integers(0, L))
            ids = rng.choice(E, size=int(rng.integers(1, 3)), replace=False)
            sa, fa, _ = a.request(layer, ids)
            sb, fb = b.request(layer, ids)
            assert (sa, fa) == (sb, fb)


def test_resize_keeps_the_most_recent_keys():
    """Closed form: a shrink keeps, among the residents just before it, the C' with the latest use
    in the access history (a grow keeps them all); every slot is then below C' and used once."""
    rng = np.random.default_rng(12)
    for trial in range(100):
        C = int(rng.integers(4, 12))
        sim = LRUSim(C)
        last_use = {}
        t = 0
        for step in range(50):
            if rng.random() < 0.2:
                C = int(rng.integers(2, 14))
                before = set(sim.od)
                sim.resize(C)
                expect = set(sorted(before, key=lambda key: -last_use[key])[:C])
                assert set(sim.od) == expect
                slots = list(sim.od.values())
                assert len(set(slots)) == len(slots) and all(0 <= s < C for s in slots)
            layer = int(rng.integers(0, 3))
            ids = sorted(set(int(e) for e in rng.choice(6, size=min(C, int(rng.integers(1, 3))), replace=False)))
            _, flags, _ = sim.request(layer, ids)
            # use order inside a request: hits ascending, then misses ascending
            for e in [e for e, f in zip(ids, flags) if f] + [e for e, f in zip(ids, flags) if not f]:
                last_use[(layer, e)] = t
                t += 1
