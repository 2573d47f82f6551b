"""Pins of the oracle's grouped wgrad / dgrad and its row -> expert mapping.

The oracle is checked against brute-force loops in exact rational arithmetic
on tiny inputs, the invariant that the expert sum equals the ungrouped
product, closed-form special cases (all-ones, one-hot, constant weights,
scale-only), and the expert scan of the Slang data-gradient page.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import mx


def _rand_mx(rng, rows, M, zero_frac=0.1):
    codes = rng.integers(0, 256, size=(rows, M)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3F          # no NaN codes
    codes[rng.random(codes.shape) < zero_frac] = 0
    scales = rng.integers(118, 137, size=(rows, M // 32)).astype(np.uint8)
    return codes, scales


def _exact(code, scale):
    v = Fraction(mx.e4m3_value(int(code)))
    s = int(scale) - 127
    return v * (Fraction(2) ** s)


def _brute_wgrad(ca, sa, cb, sb, off):
    """grad_w[e][n][k] = sum over the expert's tokens of a[n,m] * b[k,m], exactly."""
    N, M = ca.shape
    K = cb.shape[0]
    E = len(off) - 1
    out = np.zeros((E * N, K), dtype=np.float64)
    for e in range(E):
        for n in range(N):
            for k in range(K):
                acc = Fraction(0)
                for m in range(int(off[e]), int(off[e + 1])):
                    acc += _exact(ca[n, m], sa[n, m // 32]) * _exact(cb[k, m], sb[k, m // 32])
                out[e * N + n, k] = float(acc)
    return out


@pytest.mark.parametrize("off", [[0, 32, 32, 96], [0, 0, 64, 96], [0, 96, 96, 96], [0, 40, 41, 96]])
def test_wgrad_brute_force_exact(off):
    rng = np.random.default_rng(sum(off))
    N, K, M = 5, 7, 96
    ca, sa = _rand_mx(rng, N, M)
    cb, sb = _rand_mx(rng, K, M)
    got = oracle.wgrad(ca, sa, cb, sb, off)
    want = _brute_wgrad(ca, sa, cb, sb, off)
    assert got.shape == (3 * N, K)
    scale = np.abs(want).max() + 1e-300
    assert np.max(np.abs(got - want)) <= 1e-13 * scale


def test_wgrad_expert_sum_is_ungrouped_product():
    rng = np.random.default_rng(3)
    N, K, M = 24, 40, 512
    ca, sa = _rand_mx(rng, N, M)
    cb, sb = _rand_mx(rng, K, M)
    off = [0, 128, 128, 200, 352, 512]
    g = oracle.wgrad(ca, sa, cb, sb, off).reshape(5, N, K)
    # ungrouped product computed column by column, independent of the slicing
    a = oracle.mx_dequantize(ca, sa)
    b = oracle.mx_dequantize(cb, sb)
    full = sum(np.outer(a[:, m], b[:, m]) for m in range(M))
    assert np.allclose(g.sum(axis=0), full, rtol=0, atol=1e-11 * np.abs(full).max())
    # E = 1 is the ungrouped product itself
    one = oracle.wgrad(ca, sa, cb, sb, [0, M])
    assert np.allclose(one, full, rtol=0, atol=1e-11 * np.abs(full).max())
    # the empty expert is exactly zero
    assert np.all(g[1] == 0.0)


def test_wgrad_all_ones_counts_tokens():
    # code 0x78 = 256 with scale byte 119 = 2^-8 is exactly 1.0
    N, K, M = 16, 8, 1024
    off = [0, 384, 384, 896, 1024]
    ca = np.full((N, M), 0x78, np.uint8)
    sa = np.full((N, M // 32), 119, np.uint8)
    cb = np.full((K, M), 0x78, np.uint8)
    sb = np.full((K, M // 32), 119, np.uint8)
    g = oracle.wgrad(ca, sa, cb, sb, off).reshape(4, N, K)
    for e, cnt in enumerate(np.diff(off)):
        assert np.all(g[e] == float(cnt))


def test_wgrad_scale_only_probe():
    # unit codes (0x38 = 1.0); each 32-token block of row n carries scale 2^(n+b) in A
    # and 2^(-k) in B, so grad_w[e][n][k] = 32 * sum over the expert's blocks b of 2^(n+b-k)
    N, K, M = 3, 4, 256
    off = [0, 64, 192, 256]
    ca = np.full((N, M), 0x38, np.uint8)
    cb = np.full((K, M), 0x38, np.uint8)
    sa = np.array([[127 + n + b for b in range(M // 32)] for n in range(N)], np.uint8)
    sb = np.array([[127 - k for _ in range(M // 32)] for k in range(K)], np.uint8)
    g = oracle.wgrad(ca, sa, cb, sb, off).reshape(3, N, K)
    for e in range(3):
        blocks = range(off[e] // 32, off[e + 1] // 32)
        for n in range(N):
            for k in range(K):
                assert g[e, n, k] == 32 * sum(2.0 ** (n + b - k) for b in blocks)


def test_wgrad_operand_roles():
    # one nonzero token: grad_w[e][n][k] = a[n,m] * b[k,m] with a from g^T rows, b from x^T rows
    N, K, M = 3, 5, 64
    ca = np.zeros((N, M), np.uint8)
    cb = np.zeros((K, M), np.uint8)
    s_a = np.full((N, 2), 127, np.uint8)
    s_b = np.full((K, 2), 127, np.uint8)
    ca[2, 40] = 0x40           # 2.0
    cb[4, 40] = 0xB8           # -1.0
    g = oracle.wgrad(ca, s_a, cb, s_b, [0, 32, 64]).reshape(2, N, K)
    assert np.count_nonzero(g) == 1 and g[1, 2, 4] == -2.0


def test_wgrad_rows_match_definition_with_unaligned_offsets():
    rng = np.random.default_rng(4)
    N, K, M = 6, 9, 192
    ca, sa = _rand_mx(rng, N, M)
    cb, sb = _rand_mx(rng, K, M)
    off = [0, 45, 45, 130, 192]
    want = _brute_wgrad(ca, sa, cb, sb, off).reshape(4, N, K)
    for e in range(4):
        got = oracle.wgrad_rows(ca, sa, cb, sb, off, e, [5, 0, 3])
        assert np.allclose(got, want[e][[5, 0, 3]], rtol=0, atol=1e-13 * (np.abs(want).max() + 1))


def _brute_dgrad(g, W, off):
    M, N = g.shape
    K = W.shape[2]
    out = np.zeros((M, K))
    for r in range(M):
        e = 0                                    # the data-gradient page's linear expert scan
        while e + 1 < len(off) - 1 and r >= off[e + 1]:
            e += 1
        for k in range(K):
            out[r, k] = float(sum(Fraction(float(g[r, n])) * Fraction(float(W[e, n, k])) for n in range(N)))
    return out


@pytest.mark.parametrize("off", [[0, 3, 3, 10], [0, 0, 4, 10], [0, 10, 10, 10], [0, 1, 2, 10]])
def test_dgrad_brute_force_exact(off):
    rng = np.random.default_rng(len(off) + off[1])
    M, N, K = 10, 6, 5
    g = rng.standard_normal((M, N)).astype(np.float32)
    W = rng.standard_normal((3, N, K)).astype(np.float32)
    got = oracle.dgrad(g, W, off)
    want = _brute_dgrad(g, W, off)
    assert np.max(np.abs(got - want)) <= 1e-14 * np.abs(want).max()
    rows = [9, 0, 4]
    assert np.max(np.abs(oracle.dgrad_rows(g, W, off, rows) - want[rows])) <= 1e-14 * np.abs(want).max()


def test_dgrad_one_hot_rows_pick_weight_rows():
    rng = np.random.default_rng(5)
    M, N, K, E = 64, 12, 9, 5
    off = [0, 0, 20, 20, 50, 64]
    W = rng.standard_normal((E, N, K)).astype(np.float32)
    n_of_r = rng.integers(0, N, size=M)
    g = np.zeros((M, N), np.float32)
    g[np.arange(M), n_of_r] = 1.0
    dx = oracle.dgrad(g, W, off)
    e_of_r = oracle.row_experts(off, M)
    for r in range(M):
        assert np.array_equal(dx[r], W[e_of_r[r], n_of_r[r]].astype(np.float64))


def test_dgrad_constant_weights():
    M, N, K = 40, 7, 3
    off = [0, 10, 10, 33, 40]
    W = np.stack([np.full((N, K), e + 1, np.float32) for e in range(4)])
    dx = oracle.dgrad(np.ones((M, N), np.float32), W, off)
    e_of_r = [0] * 10 + [2] * 23 + [3] * 7
    assert np.array_equal(dx, np.array([[N * (e + 1)] * K for e in e_of_r], np.float64))


def test_dgrad_single_expert_is_plain_product():
    rng = np.random.default_rng(6)
    g = rng.integers(-4, 5, size=(8, 6)).astype(np.float32)
    W = rng.integers(-4, 5, size=(1, 6, 5)).astype(np.float32)
    want = [[sum(int(g[r, n]) * int(W[0, n, k]) for n in range(6)) for k in range(5)] for r in range(8)]
    assert np.array_equal(oracle.dgrad(g, W, [0, 8]), np.array(want, np.float64))


def _scan_expert(off, r):
    E = len(off) - 1
    e = 0
    while e + 1 < E and r >= off[e + 1]:
        e += 1
    return e


@pytest.mark.parametrize("off", [[0, 5, 5, 9, 12], [0, 0, 0, 12], [0, 12, 12, 12], [0, 4, 8, 12], [0, 12]])
def test_row_experts(off):
    M = off[-1]
    got = oracle.row_experts(off, M)
    for r in range(M):
        e = int(got[r])
        assert off[e] <= r < off[e + 1]                 # defining property
        assert e == _scan_expert(off, r)                 # the page's linear scan
    assert got.dtype == np.int32


def test_offsets_validation():
    with pytest.raises(ValueError):
        oracle.check_offsets([1, 4], 4)
    with pytest.raises(ValueError):
        oracle.check_offsets([0, 3], 4)
    with pytest.raises(ValueError):
        oracle.check_offsets([0, 3, 2, 4], 4)
    with pytest.raises(ValueError):
        oracle.check_offsets([0, 100, 256], 256, align=128)
    oracle.check_offsets([0, 128, 256], 256, align=128)


def test_tolerances():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal(10000) * 10
    bf16 = np.asarray(ref, np.float32).view(np.uint32)
    rounded = ((bf16 + 0x7FFF + ((bf16 >> 16) & 1)) & 0xFFFF0000).view(np.float32).astype(np.float64)
    assert oracle.wgrad_ok(rounded, ref)                     # bf16 rounding passes
    assert not oracle.wgrad_ok(ref * (1 + 2.0 ** -6), ref)   # a 2^-6 relative error fails
    bad = ref.copy()
    bad[17] = np.nan
    assert not oracle.wgrad_ok(bad, ref)
    assert oracle.dgrad_ok(ref * (1 + 1e-6), ref, 1024)
    assert not oracle.dgrad_ok(ref + 1e-3 * np.abs(ref).max(), ref, 1024)


# ---- expert-grouped MX GEMM ------------------------------------------------

def _brute_grouped(ca, sa, cb, sb, off):
    """C[m][j] = sum over c of a[m,c] * b[e(m)][j,c], exactly; e(m) by a linear scan."""
    M, K = ca.shape
    E, N, _ = cb.shape
    out = np.zeros((M, N), dtype=np.float64)
    for m in range(M):
        e = max(i for i in range(E) if off[i] <= m)      # last expert starting at or before m
        while off[e + 1] <= m:                           # (never taken for valid offsets)
            e += 1
        for j in range(N):
            acc = Fraction(0)
            for c in range(K):
                acc += _exact(ca[m, c], sa[m, c // 32]) * _exact(cb[e, j, c], sb[e, j, c // 32])
            out[m, j] = float(acc)
    return out


@pytest.mark.parametrize("off", [[0, 3, 3, 7], [0, 0, 5, 7], [0, 7, 7, 7], [0, 1, 2, 7]])
def test_grouped_gemm_brute_force_exact(off):
    rng = np.random.default_rng(sum(off) + 50)
    M, K, N, E = 7, 64, 3, 3
    ca, sa = _rand_mx(rng, M, K)
    cb, sb = _rand_mx(rng, E * N, K)
    cb, sb = cb.reshape(E, N, K), sb.reshape(E, N, K // 32)
    got = oracle.grouped_gemm(ca, sa, cb, sb, off)
    want = _brute_grouped(ca, sa, cb, sb, off)
    # exact products; the oracle's fp64 sums round, the brute force rounds once
    assert np.max(np.abs(got - want)) <= 1e-13 * (np.abs(want).max() + 1e-300)


def test_grouped_gemm_is_the_data_gradient_of_the_dequantised_weights():
    """With B[e] = W_e^T the grouped GEMM is the grouped data gradient g @ W_e."""
    rng = np.random.default_rng(61)
    M, K, N, E = 96, 128, 40, 4
    off = [0, 10, 10, 70, 96]
    ca, sa = _rand_mx(rng, M, K)
    cb, sb = _rand_mx(rng, E * N, K)
    cb, sb = cb.reshape(E, N, K), sb.reshape(E, N, K // 32)
    g = mx.mx_dequantize(ca, sa)                                        # [M, K]
    W = np.stack([mx.mx_dequantize(cb[e], sb[e]).T for e in range(E)])  # [E, K, N]
    np.testing.assert_allclose(oracle.grouped_gemm(ca, sa, cb, sb, off), oracle.dgrad(g, W, off),
                               rtol=1e-12, atol=1e-12)


def test_grouped_gemm_all_ones_counts_the_contraction():
    M, K, N, E = 64, 96, 8, 2
    ca = np.full((M, K), 0x38, np.uint8)                 # 1.0
    sa = np.full((M, K // 32), 127, np.uint8)
    cb = np.full((E, N, K), 0x38, np.uint8)
    sb = np.full((E, N, K // 32), 127, np.uint8)
    assert np.array_equal(oracle.grouped_gemm(ca, sa, cb, sb, [0, 20, 64]), np.full((M, N), float(K)))


def test_grouped_gemm_scale_only_probe():
    """Codes 1.0 and varied scales: each block adds 32 * 2^(sa + sb - 254)."""
    M, K, N, E = 4, 128, 2, 2
    ca = np.full((M, K), 0x38, np.uint8)
    cb = np.full((E, N, K), 0x38, np.uint8)
    sa = np.array([[127, 128, 126, 130]] * M, np.uint8)
    sb = np.zeros((E, N, K // 32), np.uint8)
    sb[0] = [[127, 127, 127, 127], [120, 121, 122, 123]]
    sb[1] = [[130, 127, 127, 127], [127, 127, 127, 100]]
    off = [0, 1, 4]
    got = oracle.grouped_gemm(ca, sa, cb, sb, off)
    for m in range(M):
        e = 0 if m < 1 else 1
        for j in range(N):
            want = sum(32 * 2.0 ** (int(sa[m, b]) + int(sb[e, j, b]) - 254) for b in range(K // 32))
            assert got[m, j] == want


def test_grouped_gemm_rows_match_the_whole_product():
    rng = np.random.default_rng(62)
    M, K, N, E = 80, 64, 24, 3
    off = [0, 33, 33, 80]
    ca, sa = _rand_mx(rng, M, K)
    cb, sb = _rand_mx(rng, E * N, K)
    cb, sb = cb.reshape(E, N, K), sb.reshape(E, N, K // 32)
    whole = oracle.grouped_gemm(ca, sa, cb, sb, off)
    rows = [0, 32, 33, 34, 79]
    assert np.array_equal(oracle.grouped_gemm_rows(ca, sa, cb, sb, off, rows), whole[rows])


def test_oracle_empty_contractions_are_zero():
    """The empty sum: no tokens (weight gradient), N = 0 (data gradient) and
    K = 0 (grouped GEMM) give exact zeros of the output's shape."""
    E, N, K = 3, 8, 16
    z = np.zeros
    got = oracle.wgrad(z((N, 0), np.uint8), z((N, 0), np.uint8), z((K, 0), np.uint8), z((K, 0), np.uint8),
                       z(E + 1, np.int64))
    assert got.shape == (E * N, K) and not np.any(got)
    off = np.array([0, 2, 2, 5])
    got = oracle.dgrad(z((5, 0), np.float32), z((3, 0, K), np.float32), off)
    assert got.shape == (5, K) and not np.any(got)
    got = oracle.grouped_gemm(z((5, 0), np.uint8), z((5, 0), np.uint8), z((3, 256, 0), np.uint8),
                              z((3, 256, 0), np.uint8), off)
    assert got.shape == (5, 256) and not np.any(got)
