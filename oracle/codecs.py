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
