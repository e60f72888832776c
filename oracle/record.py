"""Parse one packed expert record into fp64 matrices (test infrastructure).

Record = gate [I, H], up [I, H], down [H, I], each row-major with the reduction
dimension contiguous.  For f32 / bf16 the elements follow one another.  For
MXFP4 the three E2M1 code blocks (two codes per byte, low nibble first) come
first, then the three E8M0 scale blocks, one scale per 32 consecutive
elements of a row.  For the NVFP4-like format the code blocks are followed by
three E4M3 scale blocks (one per 16 elements) and three little-endian fp32
per-tensor scales: w = e2m1 * e4m3 * tensor_scale.
Every weight is reproduced exactly in fp64 (the dequantised values have at
most 3 + 4 + 24 significant bits), so the oracle and the kernels see the
same weights.
"""
import numpy as np

from .formats import bf16_bits_to_f64, e2m1_to_f64, e4m3_to_f64, e8m0_to_f64, unpack_nibbles

F32, BF16, MXFP4, NVFP4 = 0, 1, 2, 3

# per-code values from the format decoders, looked up per element
_E2M1 = e2m1_to_f64(np.arange(16))
_E8M0 = e8m0_to_f64(np.arange(256))
_E4M3 = e4m3_to_f64(np.arange(256))


def _shapes(H, I):
    return ((I, H), (I, H), (H, I))


def decode_record(rec: np.ndarray, H: int, I: int, w_dtype: int):
    """-> (G [I,H], U [I,H], D [H,I]) as float64 arrays."""
    rec = np.asarray(rec, dtype=np.uint8)
    shapes = _shapes(H, I)
    mats = []
    if w_dtype in (F32, BF16):
        esz = 4 if w_dtype == F32 else 2
        off = 0
        for r, c in shapes:
            n = r * c
            raw = rec[off: off + n * esz]
            if w_dtype == F32:
                m = raw.view(np.float32).astype(np.float64)
            else:
                m = bf16_bits_to_f64(raw.view(np.uint16))
            mats.append(m.reshape(r, c))
            off += n * esz
        return tuple(mats)

    blk = 32 if w_dtype == MXFP4 else 16
    code_off, off = [], 0
    for r, c in shapes:
        code_off.append(off)
        off += r * c // 2
    scale_off = []
    for r, c in shapes:
        scale_off.append(off)
        off += r * c // blk
    tscale = None
    if w_dtype == NVFP4:
        tscale = rec[off: off + 12].view("<f4").astype(np.float64)
    for i, (r, c) in enumerate(shapes):
        n = r * c
        codes = unpack_nibbles(rec[code_off[i]: code_off[i] + n // 2], n).reshape(r, c // blk, blk)
        sc = rec[scale_off[i]: scale_off[i] + n // blk].reshape(r, c // blk)
        vals = _E2M1[codes]
        if w_dtype == MXFP4:
            s = _E8M0[sc]
        else:
            s = _E4M3[sc] * tscale[i]
        mats.append((vals * s[..., None]).reshape(r, c))
    return tuple(mats)
