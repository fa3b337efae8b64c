"""The C++ slot cache in policy-only mode (no HIP calls) against the oracle's LRU simulator:
hit/miss sequence, slot assignment, statistics, write-after-read guards, pinned slots,
capacity errors and the failure path."""
import numpy as np
import pytest

import synth
from oracle.lru import LRUSim


@pytest.fixture(scope="module")
def moe():
    import expert_offload_cache_amd as m

    return m


def _replay(moe, L, E, C, reqs):
    """reqs: list of (kind, layer, ids); kind 'dec' = lookup+fill+mark_read, 'pre' = prefetch+mark_read."""
    c = moe.SlotCache(L, E, C)
    sim = LRUSim(C)
    for kind, layer, ids in reqs:
        if kind == "dec":
            slots, nm = c.lookup(layer, ids)
            ss, fl, _ = sim.request(layer, ids, "decode")
            order = np.argsort(ids, kind="stable")
            assert list(slots[order]) == ss
            assert nm == len(fl) - sum(fl)
            c.policy_fill()
        else:
            c.policy_prefetch(layer)
            sim.request(layer, range(E), "prefill")
        c.policy_mark_read(layer)
    return c, sim


def test_decode_trace_matches_simulator(moe):
    for L, E, C, k, seed in ((1, 8, 3, 2, 0), (3, 16, 10, 4, 1), (4, 32, 40, 6, 2), (24, 256, 2458, 6, 3)):
        steps = 30 if L < 24 else 60
        tr = synth.routing_trace(seed, steps, L, E, k)
        reqs = [("dec", l, list(tr[t, l][::-1])) for t in range(steps) for l in range(L)]  # unsorted ids
        c, sim = _replay(moe, L, E, C, reqs)
        assert np.array_equal(c.trace(), np.array(sim.log, dtype=np.uint8))
        st = c.stats()
        assert (st["dec_acc"], st["dec_hit"], st["dec_miss"]) == (sim.stats["dec_acc"], sim.stats["dec_hit"],
                                                                   sim.stats["dec_miss"])
        for l in range(L):
            for e in range(E):
                assert c.slot_of(l, e) == sim.od.get((l, e), -1)


def test_prefill_then_decode_matches_simulator(moe):
    L, E, C, k = 6, 16, 40, 3  # C >= 2E: prefetch(l+1) never touches the two newest layers
    tr = synth.routing_trace(7, 20, L, E, k)
    reqs = [("pre", l, None) for l in range(L)] + [("dec", l, list(tr[t, l])) for t in range(20) for l in range(L)]
    c, sim = _replay(moe, L, E, C, reqs)
    assert np.array_equal(c.trace(), np.array(sim.log, dtype=np.uint8))
    st = c.stats()
    assert st["pre_acc"] == L * E and st["pre_miss"] == sim.stats["pre_miss"]


def test_copies_wait_for_the_last_read_of_the_slot(moe):
    # every copy into a slot must wait for the most recent mark_read that covered the slot
    L, E, C, k = 3, 12, 7, 3
    tr = synth.routing_trace(1, 40, L, E, k)
    c = moe.SlotCache(L, E, C)
    last_read = {}  # slot -> seq
    seq = 0
    expect = []
    for t in range(40):
        for l in range(L):
            before = {s: last_read.get(s, -1) for s in range(C)}
            slots, nm = c.lookup(l, tr[t, l])
            log_before = len(c.copy_log())
            c.policy_fill()
            new = c.copy_log()[log_before:]
            for slot, key, wait in new:
                expect.append((slot, before[slot], wait))
            seq += 1
            c.policy_mark_read(l)
            for s in slots:
                last_read[int(s)] = seq
    assert expect and all(b == w for _, b, w in expect)
    assert any(w > 0 for _, _, w in expect)


def test_evicting_an_unread_slot_is_refused(moe):
    L, E = 3, 8
    c = moe.SlotCache(L, E, 2 * E - 1)  # one slot short of double buffering
    c.policy_prefetch(0)
    with pytest.raises(moe.MoeError) as ei:
        c.policy_prefetch(1)  # would evict a slot of layer 0, still unread
    assert ei.value.status == -7
    before = c.trace().copy()
    c.policy_mark_read(0)
    c.policy_prefetch(1)  # allowed once layer 0 is marked read
    assert len(c.trace()) == len(before) + E


def test_capacity_and_argument_errors(moe):
    c = moe.SlotCache(2, 8, 3)
    with pytest.raises(moe.MoeError) as ei:
        c.lookup(0, [0, 1, 2, 3])
    assert ei.value.status == -6
    with pytest.raises(moe.MoeError):
        c.lookup(0, [1, 1])  # duplicate
    with pytest.raises(moe.MoeError):
        c.lookup(2, [1])  # layer out of range
    with pytest.raises(moe.MoeError):
        c.lookup(0, [8])  # expert out of range
    assert len(c.trace()) == 0  # refused requests leave no trace
    with pytest.raises(moe.MoeError):
        moe.SlotCache(2, 8, 0)


def test_failed_copy_leaves_the_entry_non_resident(moe):
    c = moe.SlotCache(1, 8, 4)
    c.lookup(0, [1, 2, 3])
    c.inject_copy_failures(1)
    with pytest.raises(moe.MoeError) as ei:
        c.policy_fill()
    assert ei.value.status == -5
    assert c.slot_of(0, 1) == -1  # the first copy (expert 1) failed
    assert c.slot_of(0, 2) >= 0 and c.slot_of(0, 3) >= 0
    c.policy_mark_read(0)
    slots, nm = c.lookup(0, [1, 2])
    assert nm == 1  # expert 1 misses again; it can take the freed slot
    c.policy_fill()
    assert c.slot_of(0, 1) >= 0


def test_resize_matches_simulator(moe):
    """Shrinks and grows at safe points: the C++ cache's hits, slots and moves equal the simulator's."""
    L, E, k = 4, 16, 3
    tr = synth.routing_trace(21, 60, L, E, k)
    caps = {10: 20, 20: 9, 30: 14, 40: 6, 50: 25}
    c = moe.SlotCache(L, E, 16)
    sim = LRUSim(16)
    for t in range(60):
        if t in caps:
            n0 = len(c.copy_log())
            c.policy_resize(caps[t])
            moves = sim.resize(caps[t])
            log = c.copy_log()[n0:]
            assert [(int(a), int(b), int(m)) for a, b, m in log] == \
                [(new, key[0] * E + key[1], -2 - old) for old, new, key in moves]
        for l in range(L):
            slots, nm = c.lookup(l, tr[t, l])
            ss, fl, _ = sim.request(l, tr[t, l])
            assert list(slots) == ss and nm == len(fl) - sum(fl)
            c.policy_fill()
            c.policy_mark_read(l)
    assert np.array_equal(c.trace(), np.array(sim.log, dtype=np.uint8))
    for l in range(L):
        for e in range(E):
            assert c.slot_of(l, e) == sim.od.get((l, e), -1)


def test_resize_only_at_a_safe_point(moe):
    c = moe.SlotCache(2, 8, 6)
    c.lookup(0, [1, 2])
    with pytest.raises(moe.MoeError) as ei:
        c.policy_resize(4)  # misses not filled yet
    assert ei.value.status == -7
    c.policy_fill()
    with pytest.raises(moe.MoeError) as ei:
        c.policy_resize(4)  # layer 0 not marked read
    assert ei.value.status == -7
    c.policy_mark_read(0)
    c.policy_resize(4)
    assert c.slot_of(0, 1) >= 0 and c.slot_of(0, 2) >= 0
    with pytest.raises(moe.MoeError):
        c.policy_resize(0)


def test_fill_split_defers_the_listed_copies(moe):
    """The deferred experts are still requested (same hits and slots as the plain LRU); their
    copies are enqueued after the others."""
    L, E, k = 3, 16, 4
    tr = synth.routing_trace(31, 30, L, E, k)
    c = moe.SlotCache(L, E, 10)
    sim = LRUSim(10)
    for t in range(30):
        for l in range(L):
            slots, nm = c.lookup(l, tr[t, l])
            ss, fl, _ = sim.request(l, tr[t, l])
            assert list(slots) == ss
            miss = [int(e) for e, h in zip(sorted(tr[t, l]), fl) if not h]
            later = miss[len(miss) // 2:]
            n0 = len(c.copy_log())
            c.policy_fill_split(later)
            keys = [int(kk) % E for kk in c.copy_log()[n0:, 1]]
            assert keys == [e for e in miss if e not in later] + later
            c.policy_mark_read(l)
    assert np.array_equal(c.trace(), np.array(sim.log, dtype=np.uint8))


def test_failed_copy_releases_its_pin(moe):
    """A copy that fails frees its slot; when another layer takes that slot, marking the first layer
    read must not unpin it (the other layer's kernels may still read it)."""
    c = moe.SlotCache(3, 4, 2)
    try:
        c.lookup(0, [0])                  # (0,0) -> slot 0, pinned by layer 0
        c.inject_copy_failures(1)
        with pytest.raises(moe.MoeError):
            c.policy_fill()               # the copy fails: (0,0) is dropped, slot 0 is free again
        assert c.slot_of(0, 0) == -1
        slots, _ = c.lookup(1, [2])       # (1,2) takes slot 0, pinned by layer 1
        assert list(slots) == [0]
        c.policy_fill()
        c.policy_mark_read(0)             # layer 0 no longer holds slot 0
        with pytest.raises(moe.MoeError) as err:
            c.lookup(2, [0, 1])           # needs both slots: slot 0 is still pinned by layer 1
        assert err.value.status == moe._lib.MOE_ESTATE
        c.policy_mark_read(1)
        slots, nm = c.lookup(2, [0, 1])
        assert nm == 2 and sorted(slots) == [0, 1]
    finally:
        c.close()
