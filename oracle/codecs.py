"""Exact decoders of the stored number formats to float64 (test infrastructure).

bf16 is the upper 16 bits of an IEEE-754 binary32 value. The fp8 format is
OCP E4M3 ("fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
no infinities, and S.1111.111 as NaN. The pages only say "FP8 KV Cache"
("vLLM长序列推理优化：DCP切分KV Cache原理与实战", section 7); the format
choice is a reading of that passage. Both decoders are written from the
format definitions with integer bit arithmetic.
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    with np.errstate(invalid="ignore"):  # NaN payloads widen without trapping
        return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64, exactly.

    exponent field e, mantissa field m:
      e == 0            -> (-1)^s * 2^(1-7) * (m / 8)        (subnormal)
      e in 1..15        -> (-1)^s * 2^(e-7) * (1 + m / 8)
      e == 15, m == 7   -> NaN
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


E4M3_MAX = 448.0


def f64_to_e4m3(values) -> np.ndarray:
    """float64 -> OCP E4M3 codes (uint8): the nearest code, ties to the code
    with an even mantissa, magnitudes above 448 saturated to 448.

    Written from the format definition: a magnitude a in [2^e, 2^(e+1)) with
    e >= -6 is a multiple of 2^(e-3) when it is representable (3 mantissa
    bits); below 2^-6 the spacing stays 2^-9 (subnormals). Round a / 2^(e-3)
    to an integer n in [0, 16] with ties to even; the code is then
    ((e + 7) << 3) + n - 8, which also covers n == 16 (the next exponent)
    and the subnormals (e == -6, exponent field 0, mantissa n). The sign bit
    is kept for zeros as well.
    """
    y = np.asarray(values, dtype=np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E4M3_MAX)
    _, k = np.frexp(a)  # a = f * 2^k with f in [0.5, 1), so floor(log2 a) = k - 1
    e = np.maximum(k.astype(np.int64) - 1, -6)
    n = np.rint(np.ldexp(a, -(e - 3))).astype(np.int64)  # rint rounds ties to even
    code = np.where(n == 0, 0, ((e + 7) << 3) + n - 8)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)
