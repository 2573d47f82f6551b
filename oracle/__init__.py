"""Plain CPU oracle for the MoE grouped-GEMM backward (MXFP8 wgrad, f32 dgrad).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke
check of ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it.  It shares no code, tables or constants with the HIP library in
``moe_grouped_gemm_mxfp8_amd`` and imports nothing from it (nor the other way
round).  Everything is numpy in fp64 and follows the definitions on the
pages, in their order; no blocking, fusion or reordering beyond a library
matmul per expert segment.

Modules:
  mx         E4M3 / E8M0 codec and the MX quantiser (32-element blocks).
  mx4        E2M1 codec and the MXFP4 quantiser (packed two codes per byte).
  grouped    expert lookup, grouped wgrad (MX inputs), grouped dgrad (f32) and
             the expert-grouped MX GEMM (forward / MXFP8 data gradient).
  tolerance  the acceptance bounds used to compare a result with the oracle.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force on tiny inputs, invariants and independent library routines;
none is "parity unpinned".
"""
from .mx import (E4M3_MAX, E4M3_VALUES, MX_BLOCK, e4m3_value, e8m0_value,
                 mx_dequantize, mx_quantize, mx_scale_bytes, mx_scale_bytes_roundup,
                 round_to_e4m3)
from .mx4 import (E2M1_MAX, E2M1_VALUES, e2m1_value, mx4_dequantize, mx4_quantize, mx4_scale_bytes,
                  pack_fp4, round_to_e2m1, unpack_fp4)
from .grouped import (check_offsets, dgrad, dgrad_rows, grouped_gemm, grouped_gemm_rows,
                      row_experts, wgrad, wgrad_from_dequantized, wgrad_rows)
from .tolerance import dgrad_bound, dgrad_ok, rms, wgrad_excess, wgrad_ok

__all__ = [
    "E2M1_MAX", "E2M1_VALUES", "e2m1_value", "mx4_dequantize", "mx4_quantize", "mx4_scale_bytes",
    "pack_fp4", "round_to_e2m1", "unpack_fp4",
    "E4M3_MAX", "E4M3_VALUES", "MX_BLOCK", "e4m3_value", "e8m0_value",
    "mx_dequantize", "mx_quantize", "mx_scale_bytes", "mx_scale_bytes_roundup", "round_to_e4m3",
    "check_offsets", "dgrad", "dgrad_rows", "grouped_gemm", "grouped_gemm_rows", "row_experts", "wgrad",
    "wgrad_from_dequantized", "wgrad_rows",
    "dgrad_bound", "dgrad_ok", "rms", "wgrad_excess", "wgrad_ok",
]
