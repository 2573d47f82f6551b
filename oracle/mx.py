"""MX codec of the oracle: FP8 E4M3 element codes and E8M0 block scales.

Test infrastructure only (see the package docstring).  Everything here is
written from the definitions, in fp64, with no blocking or bit tricks:

* An E4M3 byte is decoded by the closed form of the OCP E4M3 ("FN") format:
  sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
  exponent field 0, a single NaN pattern (S.1111.111) and no infinities.
  The grouped wgrad page types its operands ``fp8e4m3`` and its scales
  ``fp8e8m0`` (kernel signature); the decode page divides block maxima by
  448, the largest finite E4M3 value (``mx8_scale``), and uses the scale byte
  127 as the unit scale (its o_proj stage).  The bit layout itself is the
  OCP one, which is what gfx950's fp8 MFMAs consume.
* An E8M0 byte s is the power of two 2^(s-127); 255 is NaN and never produced.
* The MX quantiser takes blocks of 32 consecutive elements along the
  contiguous axis.  Scale exponent: floor(log2(block max)) - 8, i.e. the
  block max lands in [256, 512) after scaling (the 8192^3 workload's
  statement of the rule), the byte clamped to [1, 254] as the decode page's
  ``mx8_scale`` clamps it; an all-zero block gets byte 1.  Elements are
  divided by the scale (exact: a power of two) and rounded to the nearest
  E4M3 value, ties to the even code, saturating at +-448 (the decode page's
  ``mx8_q`` clamps to +-FP8_MAX before converting); the sign of zero is kept.
* The round-up scale rule (the decode page's ``mx8_scale``, "aiter's MXFP8
  RoundUp rule"): the scale is the smallest power of two not below
  block_max / 448, where that quotient is the f32 product of the block max
  and the f32 nearest to 1/448 (the page computes it in f32, and that f32
  value decides the integer byte, so the oracle takes the same f32 product);
  the byte is clamped to [1, 254].  The elements are then rounded exactly as
  under the default rule.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["e4m3_value", "E4M3_VALUES", "E4M3_MAX", "e8m0_value",
           "round_to_e4m3", "mx_scale_bytes", "mx_scale_bytes_roundup", "mx_quantize", "mx_dequantize",
           "MX_BLOCK"]

MX_BLOCK = 32          # elements per E8M0 scale along the contiguous axis
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte (OCP E4M3FN), as a Python float (exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code >> 7 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:                       # subnormal: (m/8) * 2^(1-7)
        mag = (mant / 8.0) * 2.0 ** -6
    else:                                    # normal: (1 + m/8) * 2^(e-7)
        mag = (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return sign * mag


#: fp64 value of each of the 256 codes (NaN for 0x7F and 0xFF).
E4M3_VALUES = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)

# The non-negative finite values are the codes 0x00..0x7E, strictly increasing.
_POS = E4M3_VALUES[:0x7F]


def e8m0_value(byte) -> np.ndarray:
    """2^(s-127) for E8M0 byte(s) s in 0..254 (fp64); 255 raises."""
    s = np.asarray(byte, dtype=np.int64)
    if np.any(s == 255) or np.any(s < 0) or np.any(s > 255):
        raise ValueError("E8M0 byte 255 (NaN) or out of range")
    return np.ldexp(1.0, s - 127)


def round_to_e4m3(y) -> np.ndarray:
    """Nearest E4M3 code to each fp64 value ``y`` (already divided by its scale).

    Round to nearest; a value half-way between two neighbours takes the even
    code (even mantissa); magnitudes above 448 saturate to 448; the sign of
    the input is kept, also when the magnitude rounds to zero.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("non-finite input to the E4M3 rounding")
    a = np.abs(y)
    hi = np.searchsorted(_POS, a, side="left")     # first table value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    above = a > _POS[-1]                           # saturate
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)        # exact hit
    code = np.where(above, len(_POS) - 1, code)
    code = code.astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def mx_scale_bytes(block_max) -> np.ndarray:
    """E8M0 byte of blocks whose largest magnitude is ``block_max`` (fp64).

    floor(log2(block_max)) is read exactly from ``frexp`` (block_max = f*2^ex
    with f in [0.5, 1), so the floor is ex-1); the scale exponent is that
    minus 8, biased by 127 and clamped to [1, 254]; a zero block gets 1.
    """
    amax = np.asarray(block_max, dtype=np.float64)
    _, ex = np.frexp(amax)
    byte = np.clip((ex.astype(np.int64) - 1) - 8 + 127, 1, 254)
    return np.where(amax == 0.0, 1, byte).astype(np.uint8)


def mx_scale_bytes_roundup(block_max) -> np.ndarray:
    """E8M0 byte of blocks by the round-up rule: the smallest power of two 2^e
    with 2^e >= t, t = f32(block_max) * f32(1/448) rounded to f32; byte e + 127
    clamped to [1, 254] (a zero block gets 1).

    The power of two is read from ``frexp`` in fp64 (exact for an f32 t):
    t = f * 2^ex with f in [0.5, 1); t is itself a power of two when f = 0.5
    (then e = ex - 1), otherwise the next one up is 2^ex.
    """
    amax = np.asarray(block_max, dtype=np.float64)
    t = np.asarray(amax.astype(np.float32) * np.float32(1.0 / E4M3_MAX), dtype=np.float32)
    f, ex = np.frexp(t.astype(np.float64))
    e = np.where(f == 0.5, ex.astype(np.int64) - 1, ex.astype(np.int64))
    byte = np.clip(e + 127, 1, 254)
    return np.where(t == 0.0, 1, byte).astype(np.uint8)


def mx_quantize(x, rule: str = "floor") -> tuple[np.ndarray, np.ndarray]:
    """MX-quantise a [R, L] array along its last (contiguous) axis.

    Returns ``(codes uint8 [R, L], scales uint8 [R, L/32])``; block j of row r
    holds elements 32j..32j+31, aligned to the start of the row.  ``rule``:
    "floor" (2^(floor(log2 max) - 8), the default) or "roundup" (the smallest
    power of two not below max / 448, computed in f32 as the decode page does).
    """
    if rule not in ("floor", "roundup"):
        raise ValueError("rule must be 'floor' or 'roundup'")
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("mx_quantize wants [R, L] with L a multiple of 32")
    R, L = x.shape
    xb = x.astype(np.float64).reshape(R, L // MX_BLOCK, MX_BLOCK)
    if not np.all(np.isfinite(xb)):
        raise ValueError("non-finite input to mx_quantize")
    amax = np.abs(xb).max(axis=2)
    scales = mx_scale_bytes(amax) if rule == "floor" else mx_scale_bytes_roundup(amax)
    y = xb * np.ldexp(1.0, 127 - scales.astype(np.int64))[..., None]
    codes = round_to_e4m3(y).reshape(R, L)
    return codes, scales


def mx_dequantize(codes, scales) -> np.ndarray:
    """fp64 values of MX data: E4M3(code) * 2^(scale-127), block of 32 along L."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, L = codes.shape
    if scales.shape != (R, L // MX_BLOCK) or L % MX_BLOCK:
        raise ValueError("scales must be [R, L/32]")
    vals = E4M3_VALUES[codes]
    if np.any(np.isnan(vals)):
        raise ValueError("E4M3 NaN code in MX data")
    mult = e8m0_value(scales)
    return (vals.reshape(R, L // MX_BLOCK, MX_BLOCK) * mult[..., None]).reshape(R, L)
