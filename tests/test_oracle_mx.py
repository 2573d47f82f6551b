"""Pins of the oracle's MX codec (E4M3 codes, E8M0 scales, the MX quantiser).

Each test checks the oracle against something other than itself: the anchor
values of the formats (tests/golden/e4m3_anchors.txt, with sources), torch's
independent float8_e4m3fn conversion, closed forms of the scale rule, and an
exhaustive nearest-value search on small inputs.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_anchors.txt")


def _anchors():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, byte, value = line.split()[:3]
            rows.append((kind, int(byte, 16), float(value)))
    return rows


def test_anchor_values():
    anchors = _anchors()
    assert len(anchors) >= 15
    for kind, byte, value in anchors:
        got = mx.e4m3_value(byte) if kind == "e4m3" else float(mx.e8m0_value(byte))
        if math.isnan(value):
            assert math.isnan(got), (kind, hex(byte))
        else:
            assert got == value and math.copysign(1, got) == math.copysign(1, value), (kind, hex(byte), got)


def test_e4m3_table_matches_torch_decode():
    # torch's float8_e4m3fn decode is an independent implementation of the format
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_VALUES
    nan = np.isnan(ours)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(t[nan]))
    assert np.array_equal(t[~nan], ours[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ours[~nan]))


def test_e4m3_structure():
    v = oracle.E4M3_VALUES
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 increase
    assert pos.size == 127 and pos[-1] == 448.0
    assert np.array_equal(v[0x80:0xFF], -pos)            # sign bit mirrors
    # the binade [256, 512) has 8 values 256, 288, ..., 448 (3 mantissa bits) minus NaN slot
    assert list(pos[pos >= 256]) == [256, 288, 320, 352, 384, 416, 448]
    # subnormal step is 2^-9
    assert np.array_equal(pos[:8], np.arange(8) * 2.0 ** -9)


def test_e8m0():
    assert mx.e8m0_value(127) == 1.0
    assert np.array_equal(mx.e8m0_value(np.arange(255)), 2.0 ** (np.arange(255) - 127.0))
    with pytest.raises(ValueError):
        mx.e8m0_value(255)


def _torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_rounding_matches_torch_in_range():
    rng = np.random.default_rng(0)
    # values spread over every binade of the format and below it, exactly f32
    mags = np.exp2(rng.uniform(-14, np.log2(460), size=200_000)).astype(np.float32)
    sgn = np.where(rng.random(mags.size) < 0.5, -1, 1).astype(np.float32)
    y = (mags * sgn).astype(np.float64)
    assert np.array_equal(oracle.round_to_e4m3(y), _torch_e4m3(y))


def test_rounding_ties_and_neighbours_match_torch():
    pos = oracle.E4M3_VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                         # exact halfway points
    eps = np.float64(2.0 ** -16)
    cases = np.concatenate([pos, mids, mids * (1 - eps), mids * (1 + eps)])
    cases = np.concatenate([cases, -cases])
    cases32 = cases.astype(np.float32).astype(np.float64)
    assert np.array_equal(cases32, cases)                   # all exact in f32
    ours = oracle.round_to_e4m3(cases)
    assert np.array_equal(ours, _torch_e4m3(cases))
    # ties go to the even code: a few by hand
    assert oracle.round_to_e4m3([272.0])[0] == 0x78          # 272 between 256 and 288 -> 256
    assert oracle.round_to_e4m3([304.0])[0] == 0x7A          # 304 between 288 and 320 -> 320
    assert oracle.round_to_e4m3([2.0 ** -10])[0] == 0x00     # half the smallest subnormal -> 0


def test_rounding_saturates_and_keeps_sign_of_zero():
    got = oracle.round_to_e4m3([448.0, 463.9, 464.0, 470.0, 511.0, 1e30, -470.0, -1e30])
    assert list(got) == [0x7E] * 6 + [0xFE] * 2
    got = oracle.round_to_e4m3([0.0, -0.0, -1e-30, 1e-30])
    assert list(got) == [0x00, 0x80, 0x80, 0x00]


def _exhaustive_nearest(y):
    """Nearest finite E4M3 code by scanning all 254 finite codes (tiny inputs)."""
    best = None
    for code in range(256):
        v = mx.e4m3_value(code)
        if math.isnan(v):
            continue
        if math.copysign(1, v) != math.copysign(1, y):
            continue
        d = abs(v - y)
        key = (d, code & 1)                       # nearer first, then even code
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def test_quantiser_against_exhaustive_search():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((4, 64)) * np.exp2(rng.integers(-20, 20, (4, 1)))).astype(np.float32)
    x[1, 5] = 0.0
    x[2, :32] = 0.0                             # an all-zero block
    codes, scales = oracle.mx_quantize(x)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = float(np.max(np.abs(blk)))
            if amax == 0:
                want_s = 1
            else:
                E = math.floor(math.log2(amax))
                assert 2.0 ** E <= amax < 2.0 ** (E + 1)
                want_s = min(max(E - 8 + 127, 1), 254)
            assert scales[r, b] == want_s
            for i in range(32):
                y = blk[i] * 2.0 ** (127 - want_s)
                want = _exhaustive_nearest(y) if abs(y) <= 448 else (0x7E | (0x80 if y < 0 else 0))
                assert codes[r, 32 * b + i] == want, (r, b, i, y)


@pytest.mark.parametrize("J", [-100, -20, -3, 0, 1, 7, 30, 100])
def test_power_of_two_round_trip(J):
    # a block whose max is 2^J gets scale byte J-8+127 and the max maps to 256 (code 0x78);
    # any element 2^j with j >= J-17 (down to the smallest subnormal) is exact
    js = np.arange(J - 17, J + 1)
    blk = np.zeros(32)
    blk[: js.size] = np.exp2(js.astype(np.float64))
    blk[20] = -(2.0 ** J)
    codes, scales = oracle.mx_quantize(blk[None, :].astype(np.float32))
    assert scales[0, 0] == J - 8 + 127
    assert codes[0, js.size - 1] == 0x78
    assert codes[0, 20] == 0xF8
    back = oracle.mx_dequantize(codes, scales)[0]
    assert np.array_equal(back, blk)
    # one step lower than the smallest subnormal is a tie with 0 and rounds to 0
    low = np.array([[2.0 ** J] + [2.0 ** (J - 18)] + [0.0] * 30], dtype=np.float32)
    c2, _ = oracle.mx_quantize(low)
    assert c2[0, 1] == 0x00


@pytest.mark.parametrize("J", [-5, 0, 12])
def test_scale_rule_ties_and_saturation_closed_form(J):
    u = 2.0 ** (J - 8)                      # the block's quantum at code value 1
    blk = np.zeros(32)
    blk[0] = 2.0 ** J                        # sets the scale: max in [2^J, 2^(J+1))
    blk[1] = 272 * u                         # tie 256/288 -> 256
    blk[2] = 304 * u                         # tie 288/320 -> 320
    blk[3] = 1.9375 * 2.0 ** J               # 496 * u: saturates to 448
    blk[4] = 1.75 * 2.0 ** J                 # 448 * u exactly
    blk[5] = -1.8 * 2.0 ** J                 # 460.8 * u -> -448
    codes, scales = oracle.mx_quantize(blk[None, :].astype(np.float32))
    assert scales[0, 0] == J - 8 + 127
    back = oracle.mx_dequantize(codes, scales)[0]
    assert back[1] == 256 * u and back[2] == 320 * u
    assert back[3] == 448 * u and back[4] == 448 * u and back[5] == -448 * u


def test_scale_byte_clamps():
    assert list(oracle.mx_scale_bytes([0.0, 2.0 ** -120, 2.0 ** -117, 1.0, 3.0e38])) == [1, 1, 2, 119, 127 + 127 - 8]
    # a tiny block clamped to byte 1 still quantises relative to 2^-126
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, 0] = 2.0 ** -120
    codes, scales = oracle.mx_quantize(blk)
    assert scales[0, 0] == 1 and mx.e4m3_value(codes[0, 0]) == 64.0


def test_quantiser_error_bound_random():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[rng.random(x.shape) < 0.02] *= 64
    codes, scales = oracle.mx_quantize(x)
    back = oracle.mx_dequantize(codes, scales)
    unit = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)   # value of code 1.0
    y = x / unit
    err = np.abs(back - x)
    sat = np.abs(y) > 448
    # saturated elements land on +-448 units; the rest are within half a quantum
    assert np.array_equal(back[sat], np.sign(x[sat]) * 448 * unit[sat])
    half_q = np.where(np.abs(y) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 1e-300))) - 4), 2.0 ** -10)
    assert np.all(err[~sat] <= half_q[~sat] * unit[~sat])
    # only values within [448, 512) units can saturate with this scale rule
    assert np.all(np.abs(y[sat]) < 512)


def test_quantiser_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.mx_quantize(np.zeros((2, 33), np.float32))
    with pytest.raises(ValueError):
        oracle.mx_quantize(np.array([[np.inf] + [0.0] * 31], np.float32))


# ---- the round-up scale rule (the decode page's mx8_scale) -----------------

def _exact_roundup_byte(amax):
    """127 + the exponent of the smallest power of two >= amax / 448, in exact rational arithmetic."""
    from fractions import Fraction
    q = Fraction(amax) / 448
    e = 0
    while Fraction(2) ** e < q:
        e += 1
    while Fraction(2) ** (e - 1) >= q:
        e -= 1
    return min(max(e + 127, 1), 254)


@pytest.mark.parametrize("k", [-100, -20, -1, 0, 1, 9, 60, 110])
def test_roundup_exact_multiples_of_448(k):
    # amax = 448 * 2^k is itself 2^k units of 448: the scale is 2^k whichever way f32(1/448)
    # rounds (its relative error is below half an ulp of the product), and the max maps to 448
    amax = 448.0 * 2.0 ** k
    assert oracle.mx_scale_bytes_roundup([amax])[0] == 127 + k
    blk = np.zeros((1, 32), np.float32)
    blk[0, 3] = -amax
    codes, scales = oracle.mx_quantize(blk, rule="roundup")
    assert scales[0, 0] == 127 + k and codes[0, 3] == 0xFE          # -448


def test_roundup_worked_values():
    # hand-evaluated: 449/448 > 1 -> 2^1; 447/448 -> 2^0; 1/448 in (2^-9, 2^-8) -> 2^-8;
    # 3e38/448 = 6.70e35 in (2^119, 2^120) -> 2^120; zero and tiny blocks clamp to 1
    got = oracle.mx_scale_bytes_roundup([449.0, 447.0, 1.0, 3.0e38, 0.0, 1e-40, 2.0 ** -120])
    assert list(got) == [128, 127, 119, 247, 1, 1, 1]


def test_roundup_against_exact_rule_and_floor_rule():
    """Away from the f32 edge (block max within 2^-20 of 448 * 2^k) the byte is the exact smallest
    power of two >= max/448; it is the floor rule's byte, plus one when the max's mantissa exceeds
    1.75 (448 = 1.75 * 2^8).  At the edge it is the exact byte or one less."""
    rng = np.random.default_rng(11)
    amax = (rng.random(4000) * 2 + 0.5) * np.exp2(rng.integers(-60, 60, 4000).astype(np.float64))
    amax = amax.astype(np.float32).astype(np.float64)
    up = oracle.mx_scale_bytes_roundup(amax).astype(int)
    fl = oracle.mx_scale_bytes(amax).astype(int)
    F = np.floor(np.log2(amax))
    m = amax / np.exp2(F)
    for a, u, f, mm in zip(amax, up, fl, m):
        exact = _exact_roundup_byte(a)
        if abs(mm - 1.75) > 2.0 ** -20:
            assert u == exact, (a, u, exact)
            assert u == f + (1 if mm > 1.75 else 0), (a, u, f)
        else:
            assert u in (exact, exact - 1)
    # the edge itself: one f32 ulp either side of 448 * 2^k
    for k in (-3, 0, 5):
        base = np.float32(448.0 * 2.0 ** k)
        for a in (np.nextafter(base, np.float32(0)), base, np.nextafter(base, np.float32(np.inf))):
            u = int(oracle.mx_scale_bytes_roundup([float(a)])[0])
            assert u in (_exact_roundup_byte(float(a)), _exact_roundup_byte(float(a)) - 1)


def test_roundup_quantiser_never_clips_beyond_rounding():
    """With the round-up rule the block max lands in (224, 448] units (448 (1 + 2^-22) at the f32
    edge, saturated to 448), so no element is clipped; codes round as under the default rule."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.02] *= 64
    codes, scales = oracle.mx_quantize(x, rule="roundup")
    unit = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)
    y = x.astype(np.float64) / unit
    bmax = np.abs(y).reshape(64, 8, 32).max(axis=2)
    assert np.all(bmax > 224) and np.all(bmax <= 448 * (1 + 2.0 ** -22))
    # the codes are the default rule's rounding of x / scale
    for r in range(0, 64, 9):
        for b in range(8):
            blk = y[r, 32 * b:32 * b + 32]
            for i in range(0, 32, 5):
                want = _exhaustive_nearest(blk[i]) if abs(blk[i]) <= 448 else (0x7E | (0x80 if blk[i] < 0 else 0))
                assert codes[r, 32 * b + i] == want
    with pytest.raises(ValueError):
        oracle.mx_quantize(x, rule="nearest")
