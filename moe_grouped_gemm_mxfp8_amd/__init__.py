"""MI355X (gfx950) MoE grouped GEMMs: MXFP8 weight gradient, f32 data gradient,
expert-grouped MXFP8 / a8w4 GEMM (forward, MXFP8 data gradient) and the MX
quantisers, as hand-written HIP kernels behind a C ABI (include/moe_gg.h).

Python entry points (thin wrappers over the C ABI; torch supplies device
memory and the current stream, nothing else):

  wgrad_mxfp8(a, b, scale_a, scale_b, expert_off, out=None, fast=False) -> bf16 [E*N, K]
  grouped_mxfp8(a, b, scale_a, scale_b, expert_off, out=None, fast=False, b_fp4=False) -> bf16 [M, N]
  dgrad_f32(g, w, expert_off, out=None)                     -> f32 [M, K]
  mx_quantize(x, q=None, s=None, rule="floor")              -> (uint8 [R, L], uint8 [R, L/32])
  mx_quantize_t(x, q=None, s=None, rule="floor")            -> (uint8 [L, R], uint8 [L, R/32])
  mx4_quantize(x, q=None, s=None)                           -> (uint8 [R, L/2], uint8 [R, L/32])
  mx4_quantize_t(x, q=None, s=None)                         -> (uint8 [L, R/2], uint8 [L, R/32])
  row_experts(expert_off, M, out=None)                      -> int32 [M]

There is no CPU fallback: calling any of them without the built library or
without a GPU raises.
"""
from __future__ import annotations

from ._lib import EINVAL, ELAUNCH, EUNSUPPORTED, OK, MoeGGError, status_string
from .ops import (dgrad_f32, grouped_mxfp8, mx4_quantize, mx4_quantize_t, mx_quantize, mx_quantize_t,
                  row_experts, wgrad_mxfp8)

__all__ = ["wgrad_mxfp8", "grouped_mxfp8", "dgrad_f32", "mx_quantize", "mx_quantize_t", "mx4_quantize", "mx4_quantize_t",
           "row_experts", "status_string",
           "MoeGGError", "OK", "EINVAL", "EUNSUPPORTED", "ELAUNCH"]
