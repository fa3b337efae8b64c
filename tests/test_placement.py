"""Static-placement comparator: the library's vectorised version against the oracle's loops, and
the oracle against closed forms (no GPU)."""
import numpy as np
import pytest

import synth
from oracle.lru import LRUSim, static_miss_rate, static_resident


def test_oracle_special_cases():
    tr = synth.routing_trace(5, 40, 3, 8, 2)
    for pl in ("partition", "top_frequency"):
        assert static_miss_rate(tr, 3, 8, 0, pl) == 1.0
        assert static_miss_rate(tr, 3, 8, 24, pl) == 0.0
        assert len(static_resident(tr, 3, 8, 7, pl)) == 7
    # partition: 7 slots over 3 layers -> 3, 2, 2 lowest-numbered experts
    assert static_resident(tr, 3, 8, 7, "partition") == {(0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (2, 0), (2, 1)}


def test_top_frequency_is_the_best_static_placement():
    """Brute force on a tiny trace: no C-key set has fewer misses than the top-frequency set."""
    import itertools

    tr = synth.routing_trace(6, 25, 2, 4, 2)
    keys = [(l, e) for l in range(2) for e in range(4)]
    accesses = [(l, int(e)) for t in range(25) for l in range(2) for e in set(tr[t, l])]
    for C in range(0, 9):
        best = min(sum(a not in set(s) for a in accesses) for s in itertools.combinations(keys, C))
        assert round(static_miss_rate(tr, 2, 4, C, "top_frequency") * len(accesses)) == best


@pytest.mark.parametrize("L,E,k,C,seed", [(3, 8, 2, 7, 0), (6, 32, 4, 70, 1), (24, 256, 6, 2458, 2)])
def test_library_equals_oracle(L, E, k, C, seed):
    from expert_offload_cache_amd import placement

    tr = synth.routing_trace(seed, 30, L, E, k)
    for pl in ("partition", "top_frequency"):
        mask = placement.resident_mask(tr, L, E, C, pl)
        assert {(l, e) for l, e in zip(*np.nonzero(mask))} == static_resident(tr, L, E, C, pl)
        assert placement.miss_rate(tr, L, E, C, pl) == pytest.approx(static_miss_rate(tr, L, E, C, pl), abs=1e-12)


def test_lru_beats_static_partition_on_a_reuse_trace():
    """The comparison's shape on the offload trace generator (reuse p = 0.6): the shared LRU
    misses less than the routing-unaware partition at the same capacity."""
    from expert_offload_cache_amd import placement

    L, E, k, C = 8, 64, 4, 200
    tr = synth.routing_trace(3, 200, L, E, k)
    sim = LRUSim(C)
    for t in range(200):
        for l in range(L):
            sim.request(l, tr[t, l])
    lru = sim.stats["dec_miss"] / sim.stats["dec_acc"]
    assert lru < placement.miss_rate(tr, L, E, C, "partition")
