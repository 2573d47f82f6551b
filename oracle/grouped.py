"""Grouped (expert-segmented) GEMM backward of the oracle, in fp64.

Test infrastructure only (see the package docstring).

Notation.  Tokens are bucketed by expert through ``off`` (int [E+1],
off[0] = 0, nondecreasing, off[E] = M): expert e owns tokens
off[e] <= m < off[e+1] (half-open, so an empty expert owns nothing).

* Row -> expert (the Slang "grouped_gemm_m_data_backward" page,
  ``expert_for_row``): the expert of token row r is the unique e with
  off[e] <= r < off[e+1]; empty experts are skipped.
* Weight gradient (the tinygrad "grouped_mxfp8_wgrad.cpp" page: global
  layouts A = g^T [N, M], B = x^T [K, M], C = grad_w [E*N, K] experts
  stacked; the contraction runs over the expert's token segment; the
  zero-initialised accumulators are stored as they are for an empty expert):
      grad_w[e] = sum over m in expert e of  A[:, m] (outer) B[:, m]
  with A and B the MX-dequantised operands.  Written as one fp64 matmul per
  expert of the sliced operands.
* Data gradient (the Slang page, its per-element path for tiles whose rows
  span several experts, which is the plain definition):
      dx[r, k] = sum_n g[r, n] * W[e(r), n, k]
  in fp64 from the f32 inputs, one matmul per expert segment.
* Expert-grouped MX GEMM (the MoE forward y = x W_e^T and, with the weights
  transposed, an MXFP8 data gradient): token rows bucketed by ``off`` as
  above, both operands MX-quantised along the contraction (the vLLM page's
  mfma_f8f8: fp8 weights with one E8M0 scale per 32 along k, times fp8
  activations):
      C[r, j] = sum_c A[r, c] * B[e(r), j, c]
  with A and B dequantised, one fp64 matmul per expert segment.  B may
  also be MXFP4 (``b_format="e2m1"``, the decode page's a8w4: fp4 weights
  times MXFP8 activations); it is then dequantised by the MXFP4 codec.
"""
from __future__ import annotations

import numpy as np

from .mx import mx_dequantize
from .mx4 import mx4_dequantize

__all__ = ["check_offsets", "row_experts", "wgrad", "wgrad_rows",
           "wgrad_from_dequantized", "dgrad", "dgrad_rows",
           "grouped_gemm", "grouped_gemm_rows"]


def check_offsets(off, M: int, align: int = 1) -> np.ndarray:
    """Validate an expert offset array and return it as int64 [E+1]."""
    off = np.asarray(off).astype(np.int64)
    if off.ndim != 1 or off.size < 2:
        raise ValueError("expert offsets must be [E+1] with E >= 1")
    if off[0] != 0 or off[-1] != M:
        raise ValueError(f"expert offsets must start at 0 and end at M={M}")
    if np.any(np.diff(off) < 0):
        raise ValueError("expert offsets must be nondecreasing")
    if np.any(off % align):
        raise ValueError(f"expert offsets must be multiples of {align}")
    return off


def row_experts(off, M: int) -> np.ndarray:
    """e(r) for every token row r in [0, M): the e with off[e] <= r < off[e+1].

    ``searchsorted(off, r, 'right') - 1`` is the last e whose start is <= r;
    with several experts starting at r (empty ones before a non-empty one),
    that is the non-empty one, which is the expert that owns r.
    """
    off = check_offsets(off, M)
    rows = np.arange(M, dtype=np.int64)
    return (np.searchsorted(off, rows, side="right") - 1).astype(np.int32)


def wgrad_from_dequantized(a, b, off) -> np.ndarray:
    """grad_w [E*N, K] fp64 from dequantised a = g^T [N, M], b = x^T [K, M]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    N, M = a.shape
    K = b.shape[0]
    if b.shape[1] != M:
        raise ValueError("g^T and x^T must share the token axis")
    off = check_offsets(off, M)
    E = off.size - 1
    out = np.zeros((E, N, K), dtype=np.float64)
    for e in range(E):
        o0, o1 = int(off[e]), int(off[e + 1])
        if o1 > o0:
            out[e] = a[:, o0:o1] @ b[:, o0:o1].T
    return out.reshape(E * N, K)


def wgrad(codes_a, scales_a, codes_b, scales_b, off) -> np.ndarray:
    """Grouped MXFP8 weight gradient, fp64 [E*N, K].

    codes_a/scales_a: g^T as E4M3 [N, M] and E8M0 [N, M/32];
    codes_b/scales_b: x^T as E4M3 [K, M] and E8M0 [K, M/32].
    """
    a = mx_dequantize(codes_a, scales_a)
    b = mx_dequantize(codes_b, scales_b)
    return wgrad_from_dequantized(a, b, off)


def wgrad_rows(codes_a, scales_a, codes_b, scales_b, off, e: int, rows) -> np.ndarray:
    """Rows ``rows`` (indices n into [0, N)) of grad_w[e], fp64 [len(rows), K].

    The same definition restricted to a few output rows, for checks at sizes
    where the whole product is too large for the CPU.
    """
    M = codes_a.shape[1]
    off = check_offsets(off, M)
    rows = np.asarray(rows, dtype=np.int64)
    K = codes_b.shape[0]
    o0, o1 = int(off[e]), int(off[e + 1])
    if o1 == o0:
        return np.zeros((rows.size, K), dtype=np.float64)
    b0, b1 = o0 // 32, -(-o1 // 32)
    a = mx_dequantize(codes_a[rows][:, 32 * b0:32 * b1], scales_a[rows][:, b0:b1])
    b = mx_dequantize(codes_b[:, 32 * b0:32 * b1], scales_b[:, b0:b1])
    lo, hi = o0 - 32 * b0, o1 - 32 * b0
    return a[:, lo:hi] @ b[:, lo:hi].T


def dgrad(g, W, off) -> np.ndarray:
    """Grouped data gradient dx [M, K] fp64 from g [M, N] and W [E, N, K]."""
    g = np.asarray(g)
    W = np.asarray(W)
    M, N = g.shape
    E = W.shape[0]
    if W.shape[1] != N:
        raise ValueError("W must be [E, N, K] with N = g.shape[1]")
    off = check_offsets(off, M)
    if off.size != E + 1:
        raise ValueError("offsets must have E+1 entries")
    if not (np.all(np.isfinite(g)) and np.all(np.isfinite(W))):
        raise ValueError("non-finite dgrad input")
    K = W.shape[2]
    out = np.zeros((M, K), dtype=np.float64)
    for e in range(E):
        o0, o1 = int(off[e]), int(off[e + 1])
        if o1 > o0:
            out[o0:o1] = g[o0:o1].astype(np.float64) @ W[e].astype(np.float64)
    return out


def dgrad_rows(g, W, off, rows) -> np.ndarray:
    """Rows ``rows`` of dx, fp64 [len(rows), K]; each row uses its own expert."""
    M = g.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    experts = row_experts(off, M)[rows]
    out = np.empty((rows.size, W.shape[2]), dtype=np.float64)
    for i, (r, e) in enumerate(zip(rows, experts)):
        out[i] = g[r].astype(np.float64) @ W[e].astype(np.float64)
    return out


def _deq_b(codes_b, scales_b, b_format):
    if b_format == "e4m3":
        return mx_dequantize(codes_b, scales_b)
    if b_format == "e2m1":
        return mx4_dequantize(codes_b, scales_b)
    raise ValueError("b_format must be 'e4m3' or 'e2m1'")


def grouped_gemm(codes_a, scales_a, codes_b, scales_b, off, b_format: str = "e4m3") -> np.ndarray:
    """Expert-grouped MX GEMM, fp64 [M, N].

    codes_a/scales_a: A as E4M3 [M, K] and E8M0 [M, K/32] (token rows);
    codes_b/scales_b: B as E4M3 [E, N, K] (or, b_format "e2m1", packed E2M1
    [E, N, K/2]) and E8M0 [E, N, K/32].
    C[r] = deq(A)[r] @ deq(B[e(r)]).T for the expert e(r) that owns row r.
    """
    codes_a = np.asarray(codes_a)
    codes_b = np.asarray(codes_b)
    M, K = codes_a.shape
    E, N, Kb = codes_b.shape
    if b_format == "e2m1":
        Kb *= 2
    if Kb != K:
        raise ValueError("A and B must share the contraction axis")
    off = check_offsets(off, M)
    if off.size != E + 1:
        raise ValueError("offsets must have E+1 entries")
    a = mx_dequantize(codes_a, scales_a)
    out = np.zeros((M, N), dtype=np.float64)
    for e in range(E):
        o0, o1 = int(off[e]), int(off[e + 1])
        if o1 > o0:
            out[o0:o1] = a[o0:o1] @ _deq_b(codes_b[e], scales_b[e], b_format).T
    return out


def grouped_gemm_rows(codes_a, scales_a, codes_b, scales_b, off, rows, b_format: str = "e4m3") -> np.ndarray:
    """Rows ``rows`` of the grouped MX GEMM, fp64 [len(rows), N]; each row uses its own expert."""
    M = np.asarray(codes_a).shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    experts = row_experts(off, M)[rows]
    a = mx_dequantize(np.asarray(codes_a)[rows], np.asarray(scales_a)[rows])
    out = np.empty((rows.size, np.asarray(codes_b).shape[1]), dtype=np.float64)
    for e in np.unique(experts):
        sel = experts == e
        out[sel] = a[sel] @ _deq_b(codes_b[e], scales_b[e], b_format).T
    return out
