"""Seeded random shapes and expert offsets (empty experts, unaligned bounds,
rows of several experts per tile) for the weight gradient, the data gradient,
the grouped GEMM and the row map, each against the oracle at the usual bar."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

SEEDS = list(range(8))


def _counts(rng, E, M):
    """M tokens over E experts, some of them empty, bounds anywhere."""
    p = rng.random(E) * (rng.random(E) > 0.25)
    if p.sum() == 0:
        p[rng.integers(E)] = 1.0
    return rng.multinomial(M, p / p.sum())


@pytest.mark.parametrize("seed", SEEDS)
def test_random_wgrad(seed):
    torch, mg = require_gpu()
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.integers(1, 7))
    M = 128 * int(rng.integers(1, 9))
    N, K = 256 * int(rng.integers(1, 3)), 256 * int(rng.integers(1, 3))
    off = wl.offsets_from_counts(_counts(rng, E, M))
    gT = rng.standard_normal((N, M)).astype(np.float32)
    xT = rng.standard_normal((K, M)).astype(np.float32)
    gT[rng.random(gT.shape) < 0.01] *= 64
    xT[rng.random(xT.shape) < 0.01] *= 64
    ca, sa = oracle.mx_quantize(gT)
    cb, sb = oracle.mx_quantize(xT)
    say("random wgrad", seed, E, M, N, K, off.tolist())
    out = mg.wgrad_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    ref = oracle.wgrad(ca, sa, cb, sb, off)
    got = host(out).astype(np.float64)
    assert oracle.wgrad_excess(got, ref) <= 0
    for e in np.flatnonzero(np.diff(off) == 0):
        assert not np.any(got[e * N:(e + 1) * N])


@pytest.mark.parametrize("seed", SEEDS)
def test_random_dgrad_and_row_map(seed):
    torch, mg = require_gpu()
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.integers(1, 12))
    M = int(rng.integers(1, 700))
    N, K = 4 * int(rng.integers(1, 100)), 4 * int(rng.integers(1, 100))
    off = wl.offsets_from_counts(_counts(rng, E, M))
    g = rng.standard_normal((M, N)).astype(np.float32)
    W = (rng.standard_normal((E, N, K)) / np.sqrt(N)).astype(np.float32)
    say("random dgrad", seed, E, M, N, K, off.tolist())
    off_d = dev(torch, off)
    out = mg.dgrad_f32(dev(torch, g), dev(torch, W), off_d)
    rows = mg.row_experts(off_d, M)
    torch.cuda.synchronize()
    ref = oracle.dgrad(g, W, off)
    assert oracle.dgrad_ok(host(out).astype(np.float64), ref, N)
    assert np.array_equal(host(rows), oracle.row_experts(off, M))


@pytest.mark.parametrize("seed", range(4))
def test_random_dgrad_many_tiles(seed):
    """Hundreds of 128 x 128 tiles, so the XCD-aware tile order is exercised:
    even seeds give a tile count divisible by 8 (the reordered path), odd ones
    not (the plain order); partial row and column tiles and unaligned bounds."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(2500 + seed)
    while True:
        E = int(rng.integers(2, 12))
        M = int(rng.integers(1500, 4200))
        N, K = 4 * int(rng.integers(30, 200)), 4 * int(rng.integers(150, 420))
        tiles = ((M + 127) // 128) * ((K + 127) // 128)
        if (tiles % 8 == 0) == (seed % 2 == 0):
            break
    off = wl.offsets_from_counts(_counts(rng, E, M))
    g = rng.standard_normal((M, N)).astype(np.float32)
    W = (rng.standard_normal((E, N, K)) / np.sqrt(N)).astype(np.float32)
    say("random dgrad, many tiles", seed, E, M, N, K, tiles, off.tolist())
    out = mg.dgrad_f32(dev(torch, g), dev(torch, W), dev(torch, off))
    torch.cuda.synchronize()
    ref = oracle.dgrad(g, W, off)
    assert oracle.dgrad_ok(host(out).astype(np.float64), ref, N)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_grouped(seed):
    torch, mg = require_gpu()
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.integers(1, 10))
    M = int(rng.integers(1, 900))
    N, K = 256 * int(rng.integers(1, 3)), 128 * int(rng.integers(1, 4))
    off = wl.offsets_from_counts(_counts(rng, E, M))
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    b = rng.standard_normal((E * N, K)).astype(np.float32)
    ca, sa = oracle.mx_quantize(a)
    cb, sb = oracle.mx_quantize(b)
    cb, sb = cb.reshape(E, N, K), sb.reshape(E, N, K // 32)
    say("random grouped", seed, E, M, N, K, off.tolist())
    out = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(host(out).astype(np.float64), ref) <= 0


@pytest.mark.parametrize("seed", SEEDS)
def test_random_quantisers(seed):
    """Row and transposing quantisers (both MXFP8 rules, MXFP4) on random shapes
    with a wide dynamic range: codes and scales bit-exact against the oracle."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(4000 + seed)
    R, L = int(rng.integers(1, 300)), 32 * int(rng.integers(1, 20))
    x = (rng.standard_normal((R, L)) * np.exp2(rng.integers(-20, 20, size=(R, L)))).astype(np.float32)
    x[rng.random(x.shape) < 0.05] = 0.0
    say("random quantisers", seed, R, L)
    xd = dev(torch, x)
    for rule in ("floor", "roundup"):
        q, s = mg.mx_quantize(xd, rule=rule)
        cq, cs = oracle.mx_quantize(x, rule=rule)
        assert np.array_equal(host(q), cq) and np.array_equal(host(s), cs), rule
    q, s = mg.mx4_quantize(xd)
    cq, cs = oracle.mx4_quantize(x)
    assert np.array_equal(host(q), cq) and np.array_equal(host(s), cs), "mx4"
    # the transposing forms quantise x^T along R: R a multiple of 32, L of 4
    Rt, Lt = 32 * int(rng.integers(1, 12)), 4 * int(rng.integers(1, 80))
    y = (rng.standard_normal((Rt, Lt)) * np.exp2(rng.integers(-20, 20, size=(Rt, Lt)))).astype(np.float32)
    yd = dev(torch, y)
    yt = np.ascontiguousarray(y.T)
    for rule in ("floor", "roundup"):
        q, s = mg.mx_quantize_t(yd, rule=rule)
        cq, cs = oracle.mx_quantize(yt, rule=rule)
        assert np.array_equal(host(q), cq) and np.array_equal(host(s), cs), ("t", rule)
    q, s = mg.mx4_quantize_t(yd)
    cq, cs = oracle.mx4_quantize(yt)
    assert np.array_equal(host(q), cq) and np.array_equal(host(s), cs), "mx4_t"
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", SEEDS)
def test_random_a8w4(seed):
    torch, mg = require_gpu()
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.integers(1, 10))
    M = int(rng.integers(1, 900))
    N, K = 256 * int(rng.integers(1, 3)), 128 * int(rng.integers(1, 4))
    off = wl.offsets_from_counts(_counts(rng, E, M))
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    b = rng.standard_normal((E * N, K)).astype(np.float32)
    ca, sa = oracle.mx_quantize(a)
    cb, sb = oracle.mx4_quantize(b)
    cb, sb = cb.reshape(E, N, K // 2), sb.reshape(E, N, K // 32)
    say("random a8w4", seed, E, M, N, K, off.tolist())
    out = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off),
                           b_fp4=True)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert oracle.wgrad_excess(host(out).astype(np.float64), ref) <= 0
