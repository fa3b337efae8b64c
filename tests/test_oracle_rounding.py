"""Pins of the oracle's bfloat16 rounding modes (oracle/numerics.py round_to_bf16, the int4
weights seen as bf16(q * s), SwiGLU with h and with the output rows rounded to bf16): hand cases, then the bit-level
round-to-nearest-even of binary32 patterns as an independent method."""
import numpy as np

import synth
from oracle.ffn import swiglu_expert
from oracle.numerics import dequant_int4, expert_to_f64, round_to_bf16


def _bits_rne(x32: np.ndarray) -> np.ndarray:
    """bf16 rounding of binary32 values on their bit patterns: add 0x7FFF plus the kept lowest bit,
    drop the low 16 bits (finite values)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def test_hand_cases():
    s = 1.0 + 2.0 ** -7  # a bf16 scale with its last fraction bit set
    got = round_to_bf16(np.array([3 * s, -5 * s, 1 * s, 7 * s, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 0.0]))
    # 3s = 1.10000011b x 2: the dropped bit is exactly a half -> even (up); -5s: below half -> down;
    # s itself is exact; 7s: above half -> up; 1 + 2^-8: tie -> 1 (even); 1 + 3*2^-8: tie -> up to even
    assert got.tolist() == [3.03125, -5.03125, 1.0078125, 7.0625, 1.0, 1.015625, 0.0]


def test_matches_the_bit_level_rounding():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000), rng.standard_normal(20000) * 1e-20,
                        rng.standard_normal(20000) * 1e20]).astype(np.float32)
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), _bits_rne(x))


def test_int4_weights_as_bf16():
    wl = synth.Workload("r", d=256, E=2, k=1, f=128, act="bf16", wdt="int4", T_list=(1,))
    ew = synth.expert_weights(wl, 0, 0, 1)
    exact = dequant_int4(ew.wg, ew.sg)
    rounded = dequant_int4(ew.wg, ew.sg, round_bf16=True)
    # q * s is exact in binary32, so the bit-level rounding of its binary32 value is the reference
    assert np.array_equal(rounded, _bits_rne(exact.astype(np.float32)))
    assert np.all(np.abs(rounded - exact) <= np.abs(exact) * 2.0 ** -8)
    assert np.any(rounded != exact)  # |q| in {3, 5, 6, 7} times an 8-bit scale needs more bits
    wg, wu, wd = expert_to_f64(ew, int4_bf16=True)
    assert np.array_equal(wg, rounded) and np.array_equal(wd, dequant_int4(ew.wd, ew.sd, True))


def test_swiglu_with_h_rounded():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((5, 64))
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((32, 64), (32, 64), (64, 32)))
    g, u = a @ wg.T, a @ wu.T
    h = g / (1.0 + np.exp(-g)) * u
    want = _bits_rne(h.astype(np.float32)) @ wd.T  # h is rounded once; f32 first is exact enough here
    got = swiglu_expert(a, wg, wu, wd, h_bf16=True)
    # the two roundings can differ only where h's float64 value lies within a binary32 ulp of a tie
    assert np.max(np.abs(got - want)) <= 1e-6 * np.max(np.abs(want))
    assert not np.array_equal(got, swiglu_expert(a, wg, wu, wd))


def test_swiglu_with_y_rounded_hand_cases():
    # one input, one hidden unit: silu(64) is 64 in binary64 (exp(-64) is far below half an ulp of
    # 1), u = 1, so y = 64 wd exactly; wd = (1 + 2^-8)/64 and (1 + 3*2^-8)/64 put y on the two ties
    # of the rounding hand cases above (to 1.0 and up to 1.015625), and (1 + 2^-7)/64 on a bf16 value
    a = np.array([[1.0]])
    wg, wu = np.array([[64.0]]), np.array([[1.0]])
    wd = np.array([[(1 + 2.0 ** -8) / 64], [(1 + 3 * 2.0 ** -8) / 64], [(1 + 2.0 ** -7) / 64], [-(1 + 2.0 ** -8) / 64]])
    assert swiglu_expert(a, wg, wu, wd).tolist() == [[1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -7, -(1 + 2.0 ** -8)]]
    assert swiglu_expert(a, wg, wu, wd, y_bf16=True).tolist() == [[1.0, 1.015625, 1.0078125, -1.0]]


def test_swiglu_with_y_rounded_is_a_bf16_value_within_half_an_ulp():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((7, 96))
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((48, 96), (48, 96), (96, 48)))
    y = swiglu_expert(a, wg, wu, wd, h_bf16=True)
    yr = swiglu_expert(a, wg, wu, wd, h_bf16=True, y_bf16=True)
    bits = yr.astype(np.float32).view(np.uint32)
    assert np.array_equal(yr.astype(np.float32).astype(np.float64), yr)  # binary32-exact
    assert np.all(bits & 0xFFFF == 0)  # and a bf16 value
    assert np.all(np.abs(yr - y) <= np.abs(y) * 2.0 ** -8)  # unit roundoff of 8 significant bits
    assert not np.array_equal(yr, y)
