"""Pins of the oracle's MXFP4 codec (E2M1 codes, the MXFP4 quantiser) and the a8w4 grouped GEMM.

Each test checks the oracle against something other than itself: the E2M1
value table of the OCP MX specification (tests/golden/e2m1_values.txt), an
exhaustive nearest-value search, closed forms of the scale rule, the packing
order, and exact rational brute force for the grouped GEMM with fp4 weights.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")


def test_e2m1_values_match_the_spec_table():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                code, value = line.split()[:2]
                rows.append((int(code, 16), float(value)))
    assert len(rows) == 16
    for code, value in rows:
        got = oracle.e2m1_value(code)
        assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value), code
    assert np.array_equal(oracle.E2M1_VALUES, np.array([v for _, v in rows]))


def _nearest_search(y):
    """Brute force: the E2M1 code nearest to y; ties to the even code; |y| > 6 saturates; sign kept."""
    a = abs(y)
    best, best_d = None, None
    for c in range(8):
        d = abs(a - oracle.e2m1_value(c))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    if a > 6.0:
        best = 7
    return best | (8 if math.copysign(1.0, y) < 0 else 0)


def test_rounding_against_exhaustive_search():
    rng = np.random.default_rng(3)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = (mags[:-1] + mags[1:]) / 2
    ys = np.concatenate([mags, mids, mids + 1e-9, mids - 1e-9, rng.random(3000) * 9, [6.0, 6.5, 7.9, 100.0, 1e-30]])
    ys = np.concatenate([ys, -ys])
    got = oracle.round_to_e2m1(ys)
    for y, c in zip(ys, got):
        assert c == _nearest_search(float(y)), (y, c)
    assert oracle.round_to_e2m1(np.array([-0.0]))[0] == 8


def test_pack_order_and_round_trip():
    codes = np.array([[1, 2, 3, 4, 15, 0, 8, 7]], np.uint8)
    packed = oracle.pack_fp4(codes)
    assert list(packed[0]) == [0x21, 0x43, 0x0F, 0x78]          # element 2i in the low nibble
    assert np.array_equal(oracle.unpack_fp4(packed), codes)


@pytest.mark.parametrize("J", [-100, -7, 0, 3, 90])
def test_scale_rule_power_of_two(J):
    # a block whose max is 2^J gets byte J-2+127 and the max maps to 4.0 (code 6); elements
    # 2^j for J-3 <= j <= J are exact; 2^(J-4) is a tie 0 / 0.5 and rounds to 0
    blk = np.zeros(32)
    js = np.arange(J - 3, J + 1)
    blk[: js.size] = np.exp2(js.astype(np.float64))
    blk[10] = -(2.0 ** J)
    blk[11] = 2.0 ** (J - 4)
    blk[12] = 3.0 * 2.0 ** (J - 4)                            # 0.75 units: tie 0.5 / 1.0 -> 1.0
    packed, scales = oracle.mx4_quantize(blk[None, :].astype(np.float32))
    assert scales[0, 0] == J - 2 + 127
    codes = oracle.unpack_fp4(packed)[0]
    assert codes[js.size - 1] == 6 and codes[10] == 0xE and codes[11] == 0 and codes[12] == 2
    back = oracle.mx4_dequantize(packed, scales)[0]
    assert np.array_equal(back[: js.size], blk[: js.size]) and back[10] == blk[10]


def test_scale_rule_saturation_and_clamps():
    J = 5
    blk = np.zeros((1, 32))
    blk[0, 0] = 1.9 * 2.0 ** J            # 7.6 units: saturates to 6
    blk[0, 1] = -1.6 * 2.0 ** J           # 6.4 units -> -6
    blk[0, 2] = 1.3 * 2.0 ** J            # 5.2 units -> 6 (nearer than 4)
    blk[0, 3] = 1.25 * 2.0 ** J           # 5.0 units: tie 4 / 6 -> 4 (even code 6)
    packed, scales = oracle.mx4_quantize(blk.astype(np.float32))
    back = oracle.mx4_dequantize(packed, scales)[0] / 2.0 ** (J - 2)
    assert list(back[:4]) == [6.0, -6.0, 6.0, 4.0]
    assert list(oracle.mx4_scale_bytes([0.0, 2.0 ** -130, 2.0 ** -124, 1.0, 3.0e38])) == [1, 1, 1, 125, 127 + 127 - 2]


def test_quantiser_error_bound_random():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    packed, scales = oracle.mx4_quantize(x)
    back = oracle.mx4_dequantize(packed, scales)
    unit = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)
    y = x / unit
    # every block max lands in [4, 8) units; saturation only above 6; otherwise within half a step
    bmax = np.abs(y).reshape(32, 8, 32).max(axis=2)
    assert np.all(bmax >= 4) and np.all(bmax < 8)
    step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    ok = np.abs(back / unit - y) <= step / 2
    sat = np.abs(y) > 6
    assert np.all(ok | sat) and np.all(np.abs(back[sat] / unit[sat]) == 6.0)


def _exact_e4m3(code, scale):
    return Fraction(mx.e4m3_value(int(code))) * Fraction(2) ** (int(scale) - 127)


def _exact_e2m1(code, scale):
    return Fraction(oracle.e2m1_value(int(code))) * Fraction(2) ** (int(scale) - 127)


@pytest.mark.parametrize("off", [[0, 3, 3, 7], [0, 0, 7, 7], [0, 1, 2, 7]])
def test_a8w4_grouped_brute_force_exact(off):
    rng = np.random.default_rng(sum(off) + 40)
    M, N, K, E = 7, 5, 64, 3
    ca = rng.integers(0, 256, (M, K)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x38
    sa = rng.integers(120, 134, (M, K // 32)).astype(np.uint8)
    codes_b = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    cb = np.stack([oracle.pack_fp4(codes_b[e]) for e in range(E)])
    sb = rng.integers(120, 134, (E, N, K // 32)).astype(np.uint8)
    got = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    want = np.zeros((M, N))
    for r in range(M):
        e = max(i for i in range(E) if off[i] <= r < off[i + 1]) if any(off[i] <= r < off[i + 1] for i in range(E)) else None
        for j in range(N):
            acc = Fraction(0)
            for c in range(K):
                acc += _exact_e4m3(ca[r, c], sa[r, c // 32]) * _exact_e2m1(codes_b[e, j, c], sb[e, j, c // 32])
            want[r, j] = float(acc)
    assert np.max(np.abs(got - want)) <= 1e-13 * (np.abs(want).max() + 1e-300)
    rows = np.array([0, 6, 3])
    np.testing.assert_array_equal(oracle.grouped_gemm_rows(ca, sa, cb, sb, off, rows, b_format="e2m1"), got[rows])


def test_a8w4_all_ones_and_scales():
    M, N, K, E = 6, 4, 96, 2
    off = [0, 2, 6]
    ca = np.full((M, K), 0x38, np.uint8)                     # 1.0
    sa = np.full((M, K // 32), 127, np.uint8)
    cb = np.full((E, N, K // 2), 0x22, np.uint8)             # two 1.0 codes per byte
    sb = np.stack([np.full((N, K // 32), 127 + e, np.uint8) for e in range(E)])
    got = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert np.array_equal(got, np.array([[K * 2.0 ** (0 if r < 2 else 1)] * N for r in range(M)]))
    with pytest.raises(ValueError):
        oracle.grouped_gemm(ca, sa, cb, sb, off)                 # packed B read as e4m3: shape mismatch
