"""Element-format decoders, written from the format definitions (test infrastructure).

* bf16: the upper 16 bits of an IEEE binary32 pattern.
* E2M1 (OCP MX v1.0 FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit;
  exponent field 0 is subnormal: 0.5 * m.  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
* E8M0 (OCP MX v1.0 scale): 2^(v - 127), v = 255 is NaN.
* E4M3 (OCP "FN" variant): bias 7, no infinities, S.1111.111 is NaN, max 448;
  exponent field 0 is subnormal: m/8 * 2^-6.
Formats enter the method through the weight formats the pages name (MXFP4,
NVFP4, BF16: explainer page, "what happened" section and results table).
"""
import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return s * mag


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    v = np.asarray(codes, dtype=np.int64)
    out = np.exp2(v - 127.0)
    return np.where(v == 255, np.nan, out)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def unpack_nibbles(packed: np.ndarray, n: int) -> np.ndarray:
    """Bytes -> n 4-bit codes; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8).ravel()
    out = np.empty(2 * p.size, dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out[:n]


def e2m1_scalar(code: int) -> float:
    """One code by the textbook reading (used for hand-checked examples)."""
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    if e == 0:
        return sign * 0.5 * m
    return sign * math.ldexp(1.0 + 0.5 * m, e - 1)
