"""MXFP4 codec of the oracle: FP4 E2M1 element codes with E8M0 block scales.

Test infrastructure only (see the package docstring).  The decode page runs
"a8w4" MoE GEMVs: fp4 weights times MXFP8 activations on the f8f6f4 scaled
MFMA (its ``mfma_f4f8``: format 4 for the fp4 operand, 32 fp4 values per
lane, one E8M0 scale per 32 along k).  The pages do not print the fp4 format
or its quantiser, so this module writes out the OCP MX definitions they rely
on, in fp64:

* An E2M1 code is 4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit,
  subnormals at exponent field 0, no NaN or infinity.  Magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; code | 8 is the negative.
* Two codes per byte along the contiguous axis, element 2i in the low
  nibble and element 2i+1 in the high nibble (the order the gfx950 MFMA
  reads an fp4 operand in: nibble p of a lane's operand is k = p within its
  32-element group, low nibble first).
* The MXFP4 quantiser takes blocks of 32 consecutive elements.  Scale
  exponent floor(log2(block max)) - 2 (2 is E2M1's largest exponent, as 8 is
  E4M3's in the MXFP8 rule the 8192^3 workload states), biased by 127 and
  clamped to [1, 254]; an all-zero block gets byte 1.  Elements are divided by
  the scale (an exact power of two) and rounded to the nearest E2M1 value,
  ties to the even code, saturating at +-6; the sign of zero is kept.
"""
from __future__ import annotations

import numpy as np

from .mx import MX_BLOCK, e8m0_value

__all__ = ["e2m1_value", "E2M1_VALUES", "E2M1_MAX", "round_to_e2m1", "mx4_scale_bytes",
           "mx4_quantize", "mx4_dequantize", "pack_fp4", "unpack_fp4"]

E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of one E2M1 code (low 4 bits of ``code``), exact."""
    code = int(code) & 0xF
    sign = -1.0 if code >> 3 else 1.0
    exp_field = (code >> 1) & 0x3
    mant = code & 0x1
    if exp_field == 0:                       # subnormal: (m/2) * 2^(1-1)
        mag = mant / 2.0
    else:                                    # normal: (1 + m/2) * 2^(e-1)
        mag = (1.0 + mant / 2.0) * 2.0 ** (exp_field - 1)
    return sign * mag


#: fp64 value of each of the 16 codes.
E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)

# The non-negative values are the codes 0..7, strictly increasing.
_POS4 = E2M1_VALUES[:8]


def round_to_e2m1(y) -> np.ndarray:
    """E2M1 codes (uint8, 0..15) of fp64 values y: nearest, ties to the even code, saturating at +-6.

    Written as a search over the 8 magnitudes: the two neighbours of |y| and
    the nearer one, the even code on a tie; the sign bit follows y's sign
    (so -0.0 and negatives that round to zero give code 8).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS4, a, side="left"), 1, 7)    # _POS4[hi-1] < a <= _POS4[hi]
    lo = hi - 1
    d_lo = a - _POS4[lo]
    d_hi = _POS4[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E2M1_MAX, 7, code)                       # saturate
    code = code.astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(8), code).astype(np.uint8)


def mx4_scale_bytes(block_max) -> np.ndarray:
    """E8M0 byte of blocks with largest magnitude ``block_max``: floor(log2 max) - 2 + 127 in [1, 254].

    floor(log2 max) is read exactly from ``frexp`` (max = f * 2^ex, f in
    [0.5, 1), floor = ex - 1); a zero block gets 1.
    """
    amax = np.asarray(block_max, dtype=np.float64)
    _, ex = np.frexp(amax)
    byte = np.clip((ex.astype(np.int64) - 1) - 2 + 127, 1, 254)
    return np.where(amax == 0.0, 1, byte).astype(np.uint8)


def pack_fp4(codes) -> np.ndarray:
    """[R, L] codes (0..15) -> [R, L/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.ndim != 2 or c.shape[1] % 2:
        raise ValueError("pack_fp4 wants [R, L] with L even")
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_fp4(packed) -> np.ndarray:
    """[R, L/2] bytes -> [R, L] codes (0..15)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def mx4_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4-quantise a [R, L] array along L: (packed codes uint8 [R, L/2], scales uint8 [R, L/32])."""
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("mx4_quantize wants [R, L] with L a multiple of 32")
    R, L = x.shape
    xb = x.astype(np.float64).reshape(R, L // MX_BLOCK, MX_BLOCK)
    if not np.all(np.isfinite(xb)):
        raise ValueError("non-finite input to mx4_quantize")
    scales = mx4_scale_bytes(np.abs(xb).max(axis=2))
    y = xb * np.ldexp(1.0, 127 - scales.astype(np.int64))[..., None]
    codes = round_to_e2m1(y).reshape(R, L)
    return pack_fp4(codes), scales


def mx4_dequantize(packed, scales) -> np.ndarray:
    """fp64 values of MXFP4 data: E2M1(code) * 2^(scale-127), blocks of 32 along L."""
    codes = unpack_fp4(packed)
    scales = np.asarray(scales, dtype=np.uint8)
    R, L = codes.shape
    if scales.shape != (R, L // MX_BLOCK) or L % MX_BLOCK:
        raise ValueError("scales must be [R, L/32]")
    vals = E2M1_VALUES[codes]
    mult = e8m0_value(scales)
    return (vals.reshape(R, L // MX_BLOCK, MX_BLOCK) * mult[..., None]).reshape(R, L)
