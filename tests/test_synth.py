"""The seeded input generator: its definition, distribution and the int4 format."""
import numpy as np

import synth
from oracle.numerics import bf16_to_f32, dequant_int4

M64 = (1 << 64) - 1


def _splitmix_next(state):
    # SplitMix64 as published by Steele, Lea and Flood (OOPSLA 2014)
    state = (state + 0x9E3779B97F4A7C15) & M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return state, z ^ (z >> 31)


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_stream_is_the_splitmix64_sequence():
    seed, stream = 7, synth.stream_id(synth.KIND_WG, 3, 11)
    state = _mix(seed ^ _mix((stream + 0x632BE59BD9B4E019) & M64))
    ref = []
    for _ in range(10):
        state, out = _splitmix_next(state)
        ref.append(out)
    got = synth.raw_u64(seed, stream, 0, 10)
    assert [int(v) for v in got] == ref
    # counter access: output c on its own equals the c-th element of the sequence
    assert int(synth.raw_u64(seed, stream, 6, 1)[0]) == ref[6]


def test_irwin_hall_values_and_moments():
    seed, stream = 3, 12345
    raw = synth.raw_u64(seed, stream, 0, 30)
    ref = []
    for i in range(10):
        s = 0
        for j in range(3):
            r = int(raw[3 * i + j])
            s += (r & 0xFFFF) + ((r >> 16) & 0xFFFF) + ((r >> 32) & 0xFFFF) + (r >> 48)
        ref.append((s - 393210) / 65536.0)
    got = synth.normal_f32(seed, stream, (10,), 1.0)
    assert np.array_equal(got, np.array(ref, dtype=np.float32))
    z = synth.normal_f32(0, 99, (1_000_000,), 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.var() - 1.0) < 1e-2
    assert z.min() >= -6.0 and z.max() <= 6.0
    # Irwin-Hall(12) mass within one unit of the mean, from its closed-form CDF
    # F(x) = 1/12! sum_k (-1)^k C(12,k) (x-k)^12  (the normal value, 0.6827, differs by ~0.005)
    from math import comb, factorial

    F = lambda x: sum((-1) ** j * comb(12, j) * (x - j) ** 12 for j in range(int(x) + 1)) / factorial(12)
    assert abs(np.mean(np.abs(z) < 1.0) - (F(7.0) - F(5.0))) < 2e-3


def _rne_bits(f32):
    u = f32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_is_round_to_nearest_even_of_the_f32_value():
    f = synth.normal_f32(1, 5, (4096,), 0.02)
    b = synth.normal_bf16(1, 5, (4096,), 0.02)
    assert np.array_equal(b, _rne_bits(f))
    # decoded value is the nearest bf16: error at most half an ulp (2^-8 relative)
    back = bf16_to_f32(b).astype(np.float64)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2.0 ** -8 + 1e-45)


def test_int4_quantiser_roundtrip_bound():
    rows, K, sigma = 64, 512, 0.02
    w = synth.normal_f32(4, 77, (rows, K), sigma).astype(np.float64)
    packed, scales = synth.quant_int4(4, 77, rows, K, sigma)
    wt = dequant_int4(packed, scales)
    s = np.repeat(bf16_to_f32(scales).astype(np.float64), 128, axis=1)
    q = np.where(s > 0, wt / np.where(s > 0, s, 1), 0)
    assert np.all(np.abs(q) <= 7) and np.all(q == np.round(q))
    # |w~ - w| <= s/2, except where |w| exceeds 7s (clamped): there |w~ - w| <= |w| - 7s
    err = np.abs(wt - w)
    clamp = np.abs(w) > 7 * s
    assert np.all(err[~clamp] <= s[~clamp] * 0.5 * (1 + 2.0 ** -20))
    assert np.all(err[clamp] <= (np.abs(w) - 7 * s)[clamp] + 1e-12)
    # scale is the bf16 rounding of max|w|/7 in each group
    g = np.abs(w).reshape(rows, K // 128, 128).max(axis=2)
    want = _rne_bits((g.astype(np.float32) / np.float32(7.0)).astype(np.float32))
    assert np.array_equal(scales, want)
    # nibble order: element 2i low nibble, 2i+1 high nibble of byte i
    packed2, _ = synth.quant_int4(0, 0, 1, 128, 1.0, w=np.array([[7 * 1.0] + [-7.0] + [0.0] * 126]))
    assert packed2[0, 0] == (7 + 8) | ((-7 + 8) << 4)


def test_router_bias_is_zipf_prior():
    E, s = 128, 1.1
    b = synth.router_bias(0, E, s).astype(np.float64)
    p = np.exp(b - b.max())
    p /= p.sum()
    ranks = np.argsort(-p, kind="stable")
    pmf = np.arange(1, E + 1) ** (-s)
    pmf /= pmf.sum()
    assert np.allclose(p[ranks], pmf, rtol=1e-6)


def test_routing_trace_structure_and_reuse():
    steps, L, E, k = 400, 3, 64, 6
    tr = synth.routing_trace(0, steps, L, E, k)
    assert tr.shape == (steps, L, k)
    assert np.all(np.diff(tr, axis=2) > 0)  # ascending and distinct
    assert tr.min() >= 0 and tr.max() < E
    overlap = np.mean([len(set(tr[t, l]) & set(tr[t - 1, l])) / k for t in range(1, steps) for l in range(L)])
    assert 0.6 <= overlap <= 0.8
    assert np.array_equal(tr, synth.routing_trace(0, steps, L, E, k))
