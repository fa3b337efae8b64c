"""ORACLE (test infrastructure only): the expert-slot cache shared by all MoE layers.

What the pages fix (FreeToken linux guide, "MoE memory handling" section and its
mechanism table; FreeToken GGUF page, "MoE backends" section, offload backend;
FreeToken RTX 5090 page, memory-hierarchy and evaluation sections):
  * GPU memory holds a set of expert slots; the full routed pool stays in host RAM;
  * one LRU policy is shared across all MoE layers, so the key is (layer, expert);
  * a missed expert is copied to the GPU and kept there for reuse;
  * prefill streams the next layer's experts while the current layer runs;
  * the reported quantity is the fraction of expert reads that missed.

Readings where the pages are silent (all three implementations below follow them):
  * a request is the set S of distinct experts one layer needs at one step;
  * the members of S that are resident are hits and become most recent, in
    ascending expert id; then each other member, in ascending id, is a miss: it
    takes the lowest-numbered free slot if there is one, otherwise the least
    recently used resident entry is evicted and its slot reused;
  * |S| must not exceed the capacity C (then no member of S evicts another);
  * a prefill prefetch of layer l is the request S = all E experts of l;
  * the hit/miss log lists the members of each request in ascending id.
"""
from __future__ import annotations

import heapq
from collections import OrderedDict


class CapacityError(ValueError):
    pass


class LRUSim:
    """O(1) LRU over (layer, expert) keys with slot assignment."""

    def __init__(self, capacity: int):
        if capacity < 1:
            raise CapacityError("capacity must be >= 1")
        self.C = capacity
        self.od = OrderedDict()  # key -> slot, oldest first
        self.free = list(range(capacity))
        heapq.heapify(self.free)
        self.log = []  # 1 = hit, 0 = miss, per access
        self.stats = dict(dec_acc=0, dec_hit=0, dec_miss=0, pre_acc=0, pre_miss=0)

    def request(self, layer: int, ids, phase: str = "decode"):
        """-> (slots in ascending id order, hit flags, evicted keys)."""
        ids = sorted(set(int(e) for e in ids))
        if len(ids) > self.C:
            raise CapacityError(f"request of {len(ids)} experts exceeds capacity {self.C}")
        hit = {e: (layer, e) in self.od for e in ids}
        for e in ids:
            if hit[e]:
                self.od.move_to_end((layer, e))
        evicted = []
        for e in ids:
            if hit[e]:
                continue
            if self.free:
                slot = heapq.heappop(self.free)
            else:
                key, slot = self.od.popitem(last=False)
                evicted.append(key)
            self.od[(layer, e)] = slot
        flags = [1 if hit[e] else 0 for e in ids]
        self.log.extend(flags)
        nh = sum(flags)
        if phase == "decode":
            self.stats["dec_acc"] += len(ids)
            self.stats["dec_hit"] += nh
            self.stats["dec_miss"] += len(ids) - nh
        else:
            self.stats["pre_acc"] += len(ids)
            self.stats["pre_miss"] += len(ids) - nh
        return [self.od[(layer, e)] for e in ids], flags, evicted

    def resize(self, capacity: int):
        """Change the capacity between requests (a safe point).

        Growing adds free slots C..C'-1.  Shrinking keeps the C' most recently used entries
        (the LRU ones are evicted, oldest first); each kept entry whose slot is >= C' moves to
        the lowest free slot below C', taking the kept entries in ascending old-slot order.
        Returns the moves as [(old_slot, new_slot, key)] in that order.
        """
        if capacity < 1:
            raise CapacityError("capacity must be >= 1")
        moves = []
        if capacity < self.C:
            while len(self.od) > capacity:
                self.od.popitem(last=False)
            used = set(self.od.values())
            free = sorted(s for s in range(capacity) if s not in used)
            for key, slot in sorted(self.od.items(), key=lambda kv: kv[1]):
                if slot >= capacity:
                    new = free.pop(0)
                    self.od[key] = new  # assignment keeps the key's LRU position
                    moves.append((slot, new, key))
            used = set(self.od.values())
            self.free = [s for s in range(capacity) if s not in used]
        else:
            self.free = list(self.free) + list(range(self.C, capacity))
        heapq.heapify(self.free)
        self.C = capacity
        return moves

    def resident(self):
        return dict(self.od)


class BruteLRU:
    """Timestamp per resident key; the victim is found by a linear scan (argmin time, not in S)."""

    def __init__(self, capacity: int):
        self.C = capacity
        self.time = 0
        self.stamp = {}  # key -> last use time
        self.slot = {}  # key -> slot
        self.log = []

    def request(self, layer: int, ids, phase: str = "decode"):
        ids = sorted(set(int(e) for e in ids))
        if len(ids) > self.C:
            raise CapacityError("request exceeds capacity")
        S = {(layer, e) for e in ids}
        was = {e: (layer, e) in self.stamp for e in ids}
        for e in ids:
            if was[e]:
                self.time += 1
                self.stamp[(layer, e)] = self.time
        for e in ids:
            if was[e]:
                continue
            used = set(self.slot.values())
            free = [s for s in range(self.C) if s not in used]
            if free:
                s = min(free)
            else:
                victim, best = None, None
                for key, ts in self.stamp.items():
                    if key in S:
                        continue
                    if best is None or ts < best:
                        victim, best = key, ts
                s = self.slot.pop(victim)
                del self.stamp[victim]
            self.time += 1
            self.stamp[(layer, e)] = self.time
            self.slot[(layer, e)] = s
        flags = [1 if was[e] else 0 for e in ids]
        self.log.extend(flags)
        return [self.slot[(layer, e)] for e in ids], flags

    def resize(self, capacity: int):
        """Same reading as LRUSim.resize, by linear scans."""
        moves = []
        if capacity < self.C:
            while len(self.stamp) > capacity:
                victim = min(self.stamp, key=lambda kk: self.stamp[kk])
                del self.stamp[victim]
                del self.slot[victim]
            for key in sorted(self.slot, key=lambda kk: self.slot[kk]):
                old = self.slot[key]
                if old >= capacity:
                    used = set(self.slot.values())
                    new = min(s for s in range(capacity) if s not in used)
                    self.slot[key] = new
                    moves.append((old, new, key))
        self.C = capacity
        return moves


def stack_distance_hits(requests, capacity: int):
    """Hit flags recomputed from stack distances alone (Mattson et al., 1970).

    An LRU cache of C entries holds exactly the C most recently used distinct
    keys, so a member of a request is a hit iff it was used before and fewer
    than C distinct other keys were used since its last use.  The use order
    within a request is: hits ascending, then misses ascending.
    ``requests`` is a sequence of (layer, ids).
    """
    history = []  # keys in use order
    last = {}  # key -> index of last use in history
    flags = []
    for layer, ids in requests:
        ids = sorted(set(int(e) for e in ids))
        h = []
        for e in ids:
            key = (layer, e)
            if key not in last:
                h.append(0)
                continue
            distinct = set(history[last[key] + 1:])
            distinct.discard(key)
            h.append(1 if len(distinct) < capacity else 0)
        flags.extend(h)
        order = [e for e, f in zip(ids, h) if f] + [e for e, f in zip(ids, h) if not f]
        for e in order:
            last[(layer, e)] = len(history)
            history.append((layer, e))
    return flags


# ----------------------------------------------------------------------------------------------
# Static placements (FreeToken linux guide, performance/compat: global LRU against a static expert
# placement; Codex page, results).  A static placement fixes the resident keys before the trace and
# never changes them: every access to another key is a miss.  Two readings:
#   * "partition"      routing-unaware: the C slots are split evenly over the layers (the first
#                      C mod L layers get one more) and layer l holds its lowest-numbered experts;
#   * "top_frequency"  the C keys accessed most often in the trace (ties: lower layer, then lower
#                      expert) -- the best any static placement can do on that trace.
# ----------------------------------------------------------------------------------------------
def static_resident(trace, L: int, E: int, C: int, placement: str):
    """Set of resident (layer, expert) keys of a static placement over trace [steps, L, k]."""
    C = max(0, min(C, L * E))
    if placement == "partition":
        keys = set()
        for layer in range(L):
            share = C // L + (1 if layer < C % L else 0)
            for e in range(min(share, E)):
                keys.add((layer, e))
        return keys
    if placement == "top_frequency":
        count = {}
        steps = len(trace)
        for t in range(steps):
            for layer in range(L):
                for e in set(int(v) for v in trace[t][layer]):
                    count[(layer, e)] = count.get((layer, e), 0) + 1
        order = sorted(count, key=lambda key: (-count[key], key[0], key[1]))
        return set(order[:C])
    raise ValueError(placement)


def static_miss_rate(trace, L: int, E: int, C: int, placement: str) -> float:
    """Decode misses / decode accesses of a static placement (one access per distinct id per
    (step, layer), as for the LRU)."""
    res = static_resident(trace, L, E, C, placement)
    acc = miss = 0
    for t in range(len(trace)):
        for layer in range(L):
            for e in set(int(v) for v in trace[t][layer]):
                acc += 1
                miss += (layer, e) not in res
    return miss / acc if acc else 0.0
