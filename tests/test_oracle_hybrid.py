"""Pins of the oracle's hybrid miss split (oracle/hybrid.py) and the library's copy of the rule.

The oracle enumerates every n; the pins below fix it by other means: the crossing point of the two
linear cost lines (the cost is the max of a decreasing and an increasing line, so the integer
optimum sits next to where they cross), hand cases, and limits."""
import math
import random

import pytest

from oracle.hybrid import host_misses, hybrid_split, miss_time


def _crossing_answer(m, c, p, F):
    """Integer argmin of t(n) from the crossing of (m - n)/p and F + n/c, ties to the smaller n."""
    if m <= 0 or c <= 0:
        return 0
    x = (m / p - F) / (1.0 / p + 1.0 / c)  # where the PCIe line meets the host line
    cand = {0}
    for n in (math.floor(x), math.ceil(x)):
        cand.add(min(max(n, 1), m))
    def t(n):
        return m / p if n == 0 else max((m - n) / p, F + n / c)
    return min(sorted(cand), key=lambda n: (t(n), n))


def test_equal_rates_no_fixed_cost_halves_the_misses():
    # with equal rates the host takes the smaller half: (m - n) = n, or one fewer on the host
    for m in range(0, 20):
        assert hybrid_split(m, 1.0, 1.0) == m // 2


def test_one_miss_goes_to_the_host_only_if_it_is_faster_there():
    p = 4.0  # PCIe: 0.25 s an expert
    assert hybrid_split(1, 8.0, p, 0.0) == 1           # host 0.125 s
    assert hybrid_split(1, 8.0, p, 0.2) == 0           # host 0.2 + 0.125 > 0.25
    assert hybrid_split(1, 8.0, p, 0.1) == 1           # 0.225 < 0.25
    assert hybrid_split(1, 4.0, p, 0.0) == 0           # a tie stays on the GPU


def test_fixed_cost_above_the_copy_time_keeps_everything_on_the_gpu():
    for m in range(1, 12):
        assert hybrid_split(m, 100.0, 1.0, host_fixed_s=m / 1.0) == 0


def test_hand_cases():
    # m=6, host twice as fast as PCIe: crossing at n = 6*2/3 = 4 -> t = max(2/1, 4/2) = 2
    assert hybrid_split(6, 2.0, 1.0) == 4
    # the same with a 0.5 s fixed host cost: t(3) = max(3, 0.5 + 1.5) = 3, t(4) = max(2, 2.5) = 2.5
    assert hybrid_split(6, 2.0, 1.0, 0.5) == 4
    # and with 1.5 s: t(3) = max(3, 3) = 3, t(4) = max(2, 3.5) = 3.5 -> 3
    assert hybrid_split(6, 2.0, 1.0, 1.5) == 3
    assert miss_time(6, 3, 2.0, 1.0, 1.5) == 3.0 and miss_time(6, 0, 2.0, 1.0, 1.5) == 6.0
    # no host path
    assert hybrid_split(5, 0.0, 1.0, 0.0) == 0
    # a very fast host with no fixed cost takes every miss
    assert hybrid_split(7, 1e9, 1.0) == 7


def test_enumeration_equals_the_crossing_point():
    rng = random.Random(7)
    for _ in range(4000):
        m = rng.randint(0, 24)
        p = rng.uniform(0.5, 100.0)
        c = rng.choice([0.0, rng.uniform(0.1, 200.0)])
        F = rng.choice([0.0, rng.uniform(0.0, 3.0 * m / p + 1e-9)])
        assert hybrid_split(m, c, p, F) == _crossing_answer(m, c, p, F), (m, c, p, F)


def test_host_takes_the_highest_numbered_misses():
    assert host_misses([9, 3, 17, 5], 2) == [9, 17]
    assert host_misses([9, 3], 0) == []
    assert host_misses([4], 1) == [4]


def test_bad_rate():
    with pytest.raises(ValueError):
        hybrid_split(3, 1.0, 0.0)


def test_library_rule_equals_the_oracle():
    """The library's split (moe_hybrid_split, the rule moe_decode_step_hybrid applies) against the
    oracle on random cases, bit for bit (same double arithmetic, no tolerance)."""
    import expert_offload_cache_amd as moe

    rng = random.Random(11)
    for _ in range(3000):
        m = rng.randint(0, 24)
        p = rng.uniform(0.5, 100.0)
        c = rng.choice([0.0, rng.uniform(0.1, 200.0)])
        F = rng.choice([0.0, rng.uniform(0.0, 3.0 * m / p + 1e-9)])
        assert moe.hybrid_split(m, c, p, F) == hybrid_split(m, c, p, F), (m, c, p, F)
