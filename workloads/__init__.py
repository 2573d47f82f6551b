"""Seeded synthetic inputs for the MoE grouped-GEMM backward workloads.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no quantisation, no products, no expert lookup), so
both the oracle's tests and the HIP path's tests and benchmark can take their
inputs from it without sharing any computation.

Five workloads are defined.  The problem is the backward pass of an MoE
grouped GEMM whose tokens are bucketed by expert through an offset array
(the grouped wgrad kernel of the tinygrad "grouped_mxfp8_wgrad.cpp" page, its
kernel signature and global layouts; the Slang "grouped_gemm_m_data_backward"
page, its push constants):

  1. ``tiny``       E=2, M=256 tokens split 128/128, N=K=256; g[M,N], x[M,K],
                    W[E,N,K] ~ normal(0,1) f32.
  2. ``dgrad_ragged`` E=8, M=4096, N=1024 (output features), K=2048 (input
                    features); offsets from a multinomial over 7 experts with
                    one expert forced empty; g ~ normal(0,1), W ~ normal(0,1/32).
  3. ``wgrad_aligned`` E=8, M=N=K=2048, 256 tokens per expert; g^T[N,M] and
                    x^T[K,M] ~ normal(0,1).
  4. ``wgrad_zipf``  E=8, M=N=K=8192; per-expert token counts from Zipf(1.1)
                    proportions in 128-token units; g^T, x^T ~ normal(0,1) with
                    1% of entries multiplied by 64.
  5. ``many_small``  E=64, M=16384, N=1536, K=7168; 0..5 units of 128 tokens per
                    expert; wgrad inputs normal(0,1); dgrad g and W ~ normal(0,0.02).

Random numbers come from ``numpy.random.default_rng(seed)`` (PCG64) with the
workload number as the default seed, drawn in the order offsets, g (or g^T),
x (or x^T), W, outlier masks.  f32 normals are drawn with
``standard_normal(dtype=float32)`` and then scaled by the standard deviation.
"""
from __future__ import annotations

import numpy as np

__all__ = ["WORKLOADS", "Workload", "offsets_from_counts", "zipf_units",
           "make_offsets", "make_wgrad_inputs", "make_dgrad_inputs"]


class Workload:
    """Shape and offset recipe of one workload (no tensors)."""

    def __init__(self, idx, name, E, M, N, K, passes):
        self.idx, self.name = idx, name
        self.E, self.M, self.N, self.K = E, M, N, K
        self.passes = passes

    def __repr__(self):
        return (f"Workload({self.idx}, {self.name!r}, E={self.E}, M={self.M}, "
                f"N={self.N}, K={self.K}, passes={self.passes})")


WORKLOADS = {
    1: Workload(1, "tiny", E=2, M=256, N=256, K=256, passes=("wgrad", "dgrad")),
    2: Workload(2, "dgrad_ragged", E=8, M=4096, N=1024, K=2048, passes=("dgrad",)),
    3: Workload(3, "wgrad_aligned", E=8, M=2048, N=2048, K=2048, passes=("wgrad",)),
    4: Workload(4, "wgrad_zipf", E=8, M=8192, N=8192, K=8192, passes=("wgrad",)),
    5: Workload(5, "many_small", E=64, M=16384, N=1536, K=7168, passes=("wgrad", "dgrad")),
}


def offsets_from_counts(counts) -> np.ndarray:
    """Exclusive prefix sum of per-expert token counts: int32 [E+1]."""
    counts = np.asarray(counts, dtype=np.int64)
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off.astype(np.int32)


def zipf_units(total_units: int, E: int, s: float) -> np.ndarray:
    """Split ``total_units`` over E experts in proportion to (e+1)^-s.

    Largest-remainder apportionment; equal remainders go to the lower expert.
    For 64 units, E=8, s=1.1 this gives [25, 12, 8, 5, 4, 4, 3, 3].
    """
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    ideal = total_units * p / p.sum()
    units = np.floor(ideal).astype(np.int64)
    left = total_units - int(units.sum())
    order = sorted(range(E), key=lambda e: (-(ideal[e] - units[e]), e))
    for e in order[:left]:
        units[e] += 1
    return units


def _offsets_multinomial_one_empty(rng, E, M):
    empty = int(rng.integers(E))
    counts = rng.multinomial(M, np.full(E - 1, 1.0 / (E - 1)))
    counts = np.insert(counts, empty, 0)
    return offsets_from_counts(counts)


def _offsets_ragged_units(rng, E, M, unit, max_units):
    total = M // unit
    pinned = rng.choice(E, 2, replace=False)
    units = rng.integers(0, max_units + 1, size=E)
    units[pinned[0]] = 0
    units[pinned[1]] = max_units
    free = np.array([e for e in range(E) if e not in set(int(p) for p in pinned)])
    while int(units.sum()) != total:
        i = int(free[rng.integers(len(free))])
        if units.sum() > total and units[i] > 0:
            units[i] -= 1
        elif units.sum() < total and units[i] < max_units:
            units[i] += 1
    return offsets_from_counts(units * unit)


def make_offsets(idx: int, rng) -> np.ndarray:
    """expert_off int32 [E+1] for workload ``idx`` (draws from ``rng`` where the recipe is random)."""
    w = WORKLOADS[idx]
    if idx == 1:
        return offsets_from_counts([128, 128])
    if idx == 2:
        return _offsets_multinomial_one_empty(rng, w.E, w.M)
    if idx == 3:
        return offsets_from_counts([w.M // w.E] * w.E)
    if idx == 4:
        return offsets_from_counts(zipf_units(w.M // 128, w.E, 1.1) * 128)
    if idx == 5:
        return _offsets_ragged_units(rng, w.E, w.M, 128, 5)
    raise KeyError(idx)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_wgrad_inputs(idx: int, seed: int | None = None) -> dict:
    """f32 wgrad inputs before MX quantisation.

    Returns ``{"gT": [N,M] f32, "xT": [K,M] f32, "off": [E+1] int32}``, the
    token axis contiguous in both operands.  Workload 1 draws g[M,N] and
    x[M,K] and returns their transposes (copied contiguous).
    """
    w = WORKLOADS[idx]
    assert "wgrad" in w.passes, f"workload {idx} has no wgrad pass"
    rng = np.random.default_rng(idx if seed is None else seed)
    off = make_offsets(idx, rng)
    if idx == 1:
        g = _normal(rng, (w.M, w.N))
        x = _normal(rng, (w.M, w.K))
        gT, xT = np.ascontiguousarray(g.T), np.ascontiguousarray(x.T)
    else:
        gT = _normal(rng, (w.N, w.M))
        xT = _normal(rng, (w.K, w.M))
    if idx == 4:
        for arr in (gT, xT):
            mask = rng.random(size=arr.shape) < 0.01
            arr[mask] *= np.float32(64.0)
    return {"gT": gT, "xT": xT, "off": off}


def make_dgrad_inputs(idx: int, seed: int | None = None) -> dict:
    """f32 dgrad inputs: ``{"g": [M,N], "W": [E,N,K], "off": [E+1] int32}``."""
    w = WORKLOADS[idx]
    assert "dgrad" in w.passes, f"workload {idx} has no dgrad pass"
    rng = np.random.default_rng(idx if seed is None else seed)
    off = make_offsets(idx, rng)
    if idx == 1:
        g = _normal(rng, (w.M, w.N))
        _normal(rng, (w.M, w.K))          # x: drawn to keep the shared draw order
        W = _normal(rng, (w.E, w.N, w.K))
    elif idx == 2:
        g = _normal(rng, (w.M, w.N))
        W = _normal(rng, (w.E, w.N, w.K), std=1.0 / 32.0)
    elif idx == 5:
        # the wgrad pass of this workload shares the offsets; its tensors are
        # separate draws (make_wgrad_inputs), so the dgrad stream continues here
        g = _normal(rng, (w.M, w.N), std=0.02)
        W = _normal(rng, (w.E, w.N, w.K), std=0.02)
    else:
        raise KeyError(idx)
    return {"g": g, "W": W, "off": off}


def make_forward_inputs(idx: int, seed: int | None = None) -> dict:
    """f32 MoE forward inputs ``{"x": [M,K], "W": [E,N,K], "off": [E+1] int32}`` for y = x W_e^T.

    The workload's offsets (same draw as its other passes), then x ~ N(0,1) and
    W ~ N(0, 0.02), both from the continuing stream.
    """
    w = WORKLOADS[idx]
    assert "dgrad" in w.passes, f"workload {idx} has no expert weights"
    rng = np.random.default_rng(idx if seed is None else seed)
    off = make_offsets(idx, rng)
    x = _normal(rng, (w.M, w.K))
    W = _normal(rng, (w.E, w.N, w.K), std=0.02)
    return {"x": x, "W": W, "off": off}
