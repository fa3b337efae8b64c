"""ORACLE (test infrastructure only): how many of a layer's cache misses the host runs.

What the pages fix (FreeToken RTX 5090 page, the miss-split paragraph; stork.ai article, the
miss-policy paragraph; FreeToken linux guide, mechanism table): a miss is served by a PCIe copy
into a GPU slot, by the CPU running the expert where its weights already live, or by both at once,
and the runtime estimates the split from host and PCIe bandwidths measured on the machine.

Reading (the pages give no formula): one layer has m missed experts.  Sending n of them to the host
and copying the other m - n, the layer's miss work ends when the slower side ends:

    t(0) = m / pcie_rate
    t(n) = max((m - n) / pcie_rate,  host_fixed_s + n / cpu_rate)      for 1 <= n <= m

with both rates in expert images per second, measured on the box, and host_fixed_s the host path's
cost that does not scale with n (the activation row to the host, waking the host threads, the
output rows back), paid once a layer as soon as the host takes any expert.  The host takes the n
with the smallest t(n); ties go to the smaller n (fewer experts off the GPU).  The host takes the
highest-numbered misses (the choice of which does not change t).
"""
from __future__ import annotations


def miss_time(m: int, n: int, cpu_rate: float, pcie_rate: float, host_fixed_s: float = 0.0) -> float:
    """t(n) above: seconds until a layer's m misses are served with n of them on the host."""
    if not 0 <= n <= m:
        raise ValueError("need 0 <= n <= m")
    pcie = (m - n) / pcie_rate
    if n == 0:
        return pcie
    return max(pcie, host_fixed_s + n / cpu_rate)


def hybrid_split(m: int, cpu_rate: float, pcie_rate: float, host_fixed_s: float = 0.0) -> int:
    """The number of a layer's m misses run on the host: argmin over n of t(n), ties to the smaller n.
    A host rate of zero (no host path) gives 0."""
    if pcie_rate <= 0:
        raise ValueError("pcie_rate must be > 0")
    if m <= 0 or cpu_rate <= 0:
        return 0
    best, best_t = 0, miss_time(m, 0, cpu_rate, pcie_rate, host_fixed_s)
    for n in range(1, m + 1):
        t = miss_time(m, n, cpu_rate, pcie_rate, host_fixed_s)
        if t < best_t:
            best, best_t = n, t
    return best


def host_misses(miss_ids, n_host: int):
    """The misses the host takes: the n_host highest-numbered of a layer's missed expert ids."""
    ids = sorted(int(e) for e in miss_ids)
    return ids[len(ids) - n_host:] if n_host > 0 else []
