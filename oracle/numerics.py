"""ORACLE (test infrastructure only): exact decoding of the stored number formats.

bfloat16 -> wider float is exact (the 16 stored bits are the top half of the
binary32 pattern).  int4 weights follow the symmetric per-row, 128-wide-group
format with bfloat16 scales: stored nibble u, integer q = u - 8, weight
q * s; element 2i sits in the low nibble of byte i and element 2i+1 in the
high nibble.  q * s is exact in binary64 (and in binary32).
"""
import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Each value rounded to the nearest bfloat16 value (8 significant bits, ties to even), returned
    as float64.  Written from the definition: a = m * 2^e with 0.5 <= |m| < 1; keep m to 8 bits,
    rounding half to even (numpy's rint), and scale back.  Finite normal values only."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def dequant_int4(packed: np.ndarray, scales: np.ndarray, round_bf16: bool = False) -> np.ndarray:
    """packed uint8 [rows, K/2], scales bf16 bits [rows, K/128] -> float64 [rows, K].

    round_bf16: the weight each matrix-core product sees when q * s is rounded to bfloat16 before a
    bf16 product (the int4 prefill reading: the weights are dequantised to bf16, then multiplied);
    off, the exact q * s."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    K = 2 * half
    q = np.empty((rows, K), dtype=np.int64)
    q[:, 0::2] = (packed & 0x0F).astype(np.int64) - 8
    q[:, 1::2] = (packed >> 4).astype(np.int64) - 8
    s = bf16_to_f64(scales)  # [rows, K/128]
    w = q.astype(np.float64) * np.repeat(s, 128, axis=1)
    return round_to_bf16(w) if round_bf16 else w


def expert_to_f64(ew, int4_bf16: bool = False):
    """synth.ExpertWeights -> (Wg [f,d], Wu [f,d], Wd [d,f]) as float64, exactly (with int4_bf16,
    int4 weights as bf16(q * s), see dequant_int4)."""
    if ew.wdt == "int4":
        return (dequant_int4(ew.wg, ew.sg, int4_bf16), dequant_int4(ew.wu, ew.su, int4_bf16),
                dequant_int4(ew.wd, ew.sd, int4_bf16))
    if ew.wdt == "bf16":
        return bf16_to_f64(ew.wg), bf16_to_f64(ew.wu), bf16_to_f64(ew.wd)
    return (np.asarray(ew.wg, np.float64), np.asarray(ew.wu, np.float64), np.asarray(ew.wd, np.float64))


def act_to_f64(x: np.ndarray, act: str) -> np.ndarray:
    return bf16_to_f64(x) if act == "bf16" else np.asarray(x, dtype=np.float64)
