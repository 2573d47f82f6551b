"""Acceptance bounds for comparing a computed result with the oracle.

Test infrastructure only (see the package docstring).

* bf16 weight gradient: every element must satisfy
      |out - ref| <= 2^-7 * |ref| + 2^-12 * rms(ref)
  with rms over the whole reference.  The relative term is twice bf16's
  round-to-nearest half-ulp (2^-8 relative at worst); the absolute term
  absorbs f32 accumulation error in elements that cancel to near zero.
* f32 data gradient:  max |out - ref| <= 1e-5 * sqrt(N) * max |ref|, N the
  contraction length (f32 accumulation error grows like sqrt(N) * 2^-24 per
  unit magnitude, so 1e-5 * sqrt(N) leaves roughly two orders of margin).
"""
from __future__ import annotations

import numpy as np

__all__ = ["wgrad_excess", "wgrad_ok", "dgrad_bound", "dgrad_ok", "rms"]


def rms(ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def wgrad_excess(out, ref, ref_rms: float | None = None) -> float:
    """max over elements of |out-ref| - (2^-7|ref| + 2^-12 rms); <= 0 passes.

    ``ref_rms`` overrides the rms when only a sample of the reference is at
    hand (pass an estimate of the rms over the whole output).
    """
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if out.size == 0:
        return -np.inf
    if not np.all(np.isfinite(out)):
        return np.inf
    r = rms(ref) if ref_rms is None else float(ref_rms)
    bound = 2.0 ** -7 * np.abs(ref) + 2.0 ** -12 * r
    return float(np.max(np.abs(out - ref) - bound))


def wgrad_ok(out, ref, ref_rms: float | None = None) -> bool:
    return wgrad_excess(out, ref, ref_rms) <= 0.0


def dgrad_bound(ref, N: int, ref_absmax: float | None = None) -> float:
    m = float(np.max(np.abs(ref))) if ref_absmax is None else float(ref_absmax)
    return 1e-5 * np.sqrt(N) * m


def dgrad_ok(out, ref, N: int, ref_absmax: float | None = None) -> bool:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape or not np.all(np.isfinite(out)):
        return False
    if out.size == 0:
        return True
    return float(np.max(np.abs(out - ref))) <= dgrad_bound(ref, N, ref_absmax)
