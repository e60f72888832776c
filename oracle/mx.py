"""MXFP8 (E4M3 elements, E8M0 scale per 32) quantisation, in one term or
as two terms (the value and its residual, each quantised), and the bf16
rounding of the expert outputs y, both mirrored for the prefill path (test
infrastructure).

Written from the OCP Microscaling Formats (MX) v1.0 conversion rule: for each
block of 32 consecutive values, shared exponent X = floor(log2(max|V|)) - 8
(8 = exponent of E4M3's largest normal, 448 = 1.75 * 2^8), clamped to the
E8M0 range; each element is V / 2^X rounded to the nearest E4M3 value (ties to
the even code), magnitudes beyond 448 saturate to 448.  A block of zeros gets
the smallest scale.  The element rounding here searches the full table of
E4M3 values instead of manipulating bits.
"""
import numpy as np

from .formats import e4m3_to_f64

# all finite non-negative E4M3 values, in code order (codes 0x00..0x7E)
_E4M3_POS = e4m3_to_f64(np.arange(0x7F))
_E4M3_MIDS = 0.5 * (_E4M3_POS[:-1] + _E4M3_POS[1:])


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value (ties to even code), saturating at +-448; returns fp64."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    lo = np.searchsorted(_E4M3_MIDS, a, side="left")
    hi = np.searchsorted(_E4M3_MIDS, a, side="right")
    code = np.where(lo != hi, lo + (lo & 1), lo)      # tie -> even of (lo, lo+1)
    code = np.minimum(code, 0x7E)
    return np.copysign(_E4M3_POS[code], v)


def mx_scale_exponent(block: np.ndarray) -> int:
    amax = float(np.max(np.abs(block)))
    if amax == 0.0:
        return -127
    m, e = np.frexp(amax)           # amax = m * 2^e, m in [0.5, 1)
    return int(np.clip((e - 1) - 8, -127, 127))


def mxfp8_quantize(v: np.ndarray) -> np.ndarray:
    """Quantise a 1-D vector (length a multiple of 32) block by block and return
    the dequantised fp64 values."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    for b in range(0, v.size, 32):
        blk = v[b: b + 32]
        X = mx_scale_exponent(blk)
        out[b: b + 32] = e4m3_round(blk / np.ldexp(1.0, X)) * np.ldexp(1.0, X)
    return out


def mxfp8_quantize_f32(v: np.ndarray) -> np.ndarray:
    """As mxfp8_quantize, applied to the fp32-rounded values: the kernels hold
    h in fp32 when they quantise it, so the oracle takes the same decision on
    the same precision."""
    return mxfp8_quantize(np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64))


def mxfp8_two_term(v: np.ndarray) -> np.ndarray:
    """Two MXFP8 terms: q1 = mxfp8_quantize(v), then the residual v - q1 (exact
    in fp64, and exact in fp32 too for bf16 or fp32 inputs) quantised the
    same way with its own block scales; returns q1 + q2.  This is the
    matrix cores' operand when a bf16 activation is carried as two E4M3
    terms instead of one."""
    v = np.asarray(v, dtype=np.float64)
    q1 = mxfp8_quantize(v)
    return q1 + mxfp8_quantize(v - q1)


def mxfp8_two_term_f32(v: np.ndarray) -> np.ndarray:
    """mxfp8_two_term of the fp32-rounded values (h is held in fp32 when the
    kernels quantise it)."""
    return mxfp8_two_term(np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64))


def bf16_round_f32(v: np.ndarray) -> np.ndarray:
    """The prefill path stores each expert output y in bf16: the kernel holds
    y in fp32 and rounds it to the nearest bf16 value (8 significant bits,
    ties to even).  Written from that definition: round to fp32 first, then
    keep 8 significant bits of the mantissa with round-half-even (np.rint),
    on the fixed 2^-133 grid below the smallest normal 2^-126; beyond the
    largest bf16 value (just under 2^128) the result is infinite.  Returns fp64."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    out = np.empty_like(f)
    fin = np.isfinite(f)
    out[~fin] = f[~fin]
    a = f[fin]
    m, e = np.frexp(a)                                  # a = m * 2^e, |m| in [0.5, 1)
    normal = np.abs(a) >= np.ldexp(1.0, -126)
    r = np.where(normal, np.ldexp(np.rint(np.ldexp(m, 8)), e - 8), np.ldexp(np.rint(np.ldexp(a, 133)), -133))
    r = np.where(np.abs(r) >= np.ldexp(1.0, 128), np.copysign(np.inf, r), r)   # rounded past the largest bf16
    out[fin] = r
    return out
