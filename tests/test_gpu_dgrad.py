"""GPU parity of the grouped f32 data gradient against the oracle.

Bar: max |out - ref| <= 1e-5 sqrt(N) max |ref|; exact equality for one-hot
rows and constant weights, which also pins the row -> expert mapping.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _run(torch, mg, g, W, off):
    out = mg.dgrad_f32(dev(torch, g), dev(torch, W), dev(torch, np.asarray(off, np.int32)))
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


CASES = {
    # name: (N, K, per-expert row counts)
    "aligned": (256, 256, [128, 128]),
    "straddle": (64, 256, [100, 156]),
    "ragged_tail": (96, 132, [37, 0, 90, 7]),
    "empty_ends": (128, 128, [0, 60, 200, 0]),
    "many_in_tile": (32, 128, [3, 1, 0, 5, 40, 2, 77, 0, 1]),
    "one_expert_odd": (36, 260, [300]),
    "long_n": (1000, 128, [129, 127]),
    # passes over 32-row blocks (0,3), (2,4), (0,2), (1,3), (2,3) of their tiles; a partial column tile
    "row_blocks": (160, 192, [70, 58, 40, 50, 38, 70, 20, 38]),
    # boundaries 15, 16 and 17 rows into a 32-row block: leading and trailing 16-row half blocks,
    # passes of a half block alone, a partial column tile
    "half_blocks": (96, 160, [16, 31, 34, 31, 38, 20, 30]),
    # the LDS-DMA pass at its edges: one row (127 of the tile's g rows past M), the fewest
    # chunks (N = 32); several experts inside the first two 32-row blocks of a partial tile
    "one_row": (32, 128, [1]),
    "dma_edge_rows": (64, 256, [3, 0, 30, 2]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_dgrad_small(name):
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M = int(off[-1])
    rng = np.random.default_rng(len(name) + 13 * N)
    g = rng.standard_normal((M, N)).astype(np.float32)
    W = (rng.standard_normal((len(counts), N, K)) / np.sqrt(N)).astype(np.float32)
    say("dgrad", name, M, N, K, counts)
    got = _run(torch, mg, g, W, off)
    ref = oracle.dgrad(g, W, off)
    assert oracle.dgrad_ok(got, ref, N), np.max(np.abs(got - ref))


def test_dgrad_one_hot_rows_exact():
    torch, mg = require_gpu()
    counts = [0, 70, 1, 130, 0, 55]
    off = wl.offsets_from_counts(counts)
    M, N, K, E = int(off[-1]), 96, 160, len(counts)
    rng = np.random.default_rng(8)
    W = rng.standard_normal((E, N, K)).astype(np.float32)
    g = np.zeros((M, N), np.float32)
    n_of_r = rng.integers(0, N, size=M)
    g[np.arange(M), n_of_r] = 1.0
    say("dgrad one-hot")
    got = _run(torch, mg, g, W, off)
    e_of_r = oracle.row_experts(off, M)
    assert np.array_equal(got, W[e_of_r, n_of_r].astype(np.float64))


def test_dgrad_constant_weights_exact():
    torch, mg = require_gpu()
    counts = [50, 0, 200, 6]
    off = wl.offsets_from_counts(counts)
    M, N, K = int(off[-1]), 64, 128
    W = np.stack([np.full((N, K), e + 1, np.float32) for e in range(len(counts))])
    say("dgrad constant W")
    got = _run(torch, mg, np.ones((M, N), np.float32), W, off)
    want = N * (oracle.row_experts(off, M).astype(np.float64) + 1)
    assert np.array_equal(got, np.repeat(want[:, None], K, axis=1))


@pytest.mark.parametrize("idx", [1, 2])
def test_dgrad_workloads_full(idx):
    torch, mg = require_gpu()
    inp = wl.make_dgrad_inputs(idx)
    say("dgrad workload", idx)
    got = _run(torch, mg, inp["g"], inp["W"], inp["off"])
    ref = oracle.dgrad(inp["g"], inp["W"], inp["off"])
    N = inp["g"].shape[1]
    assert oracle.dgrad_ok(got, ref, N), (np.max(np.abs(got - ref)), oracle.dgrad_bound(ref, N))


def test_dgrad_many_small_full():
    """The 64-expert workload at full size (the bench's shapes and launch), the whole dx against the
    oracle's whole dx."""
    torch, mg = require_gpu()
    inp = wl.make_dgrad_inputs(5)
    off = inp["off"]
    M, N = inp["g"].shape
    say("dgrad workload 5 full size, whole output")
    out = mg.dgrad_f32(dev(torch, inp["g"]), dev(torch, inp["W"]), dev(torch, off))
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    del out
    ref = oracle.dgrad(inp["g"], inp["W"], off)
    err = float(np.max(np.abs(got - ref)))
    say(f"dgrad workload 5: max err {err:.4g}, bound {oracle.dgrad_bound(ref, N):.4g}")
    assert oracle.dgrad_ok(got, ref, N), err
