"""GPU parity of the MX quantiser and the row -> expert map: bit-exact vs the oracle."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _edge_input():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((12, 128)).astype(np.float32)
    x[0] = 0.0                                               # all-zero blocks
    x[1, :32] = np.float32(2.0 ** -120) * rng.standard_normal(32).astype(np.float32)   # clamped scale byte 1
    x[1, 32:64] = np.float32(1e-40)                          # f32 subnormals
    x[1, 64:96] = (rng.standard_normal(32) * 1e-39).astype(np.float32)
    x[2, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    pos = oracle.E4M3_VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    x[3, :32] = 256.0                                        # max sets the scale to 2^0
    x[3, 1:32] = mids[np.linspace(0, len(mids) - 1, 31).astype(int)]   # exact ties
    x[4, :32] = np.linspace(-511, 511, 32)                   # saturation
    x[4, 0] = 300.0
    x[5, :32] = -0.0
    x[5, 5] = -1.0
    x[5, 6] = -2.0 ** -30                                    # rounds to -0
    x[6] *= 64.0
    x[7, ::7] *= 1e6
    return x


@pytest.mark.parametrize("case", ["edge", "row32", "odd_rows", "long_rows"])
def test_quantize_bit_exact(case):
    torch, mg = require_gpu()
    rng = np.random.default_rng({"edge": 1, "row32": 2, "odd_rows": 3, "long_rows": 4}[case])
    if case == "edge":
        x = _edge_input()
    elif case == "row32":
        x = rng.standard_normal((7, 32)).astype(np.float32)
    elif case == "odd_rows":
        x = (rng.standard_normal((37, 96)) * np.exp2(rng.integers(-60, 60, (37, 1)))).astype(np.float32)
    else:
        x = rng.standard_normal((19, 4096 + 32)).astype(np.float32)
    say("quantize", case, x.shape)
    q, s = mg.mx_quantize(dev(torch, x))
    torch.cuda.synchronize()
    want_q, want_s = oracle.mx_quantize(x)
    assert np.array_equal(host(s), want_s)
    got_q = host(q)
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, (bad[:5], x[tuple(bad[0])], got_q[tuple(bad[0])], want_q[tuple(bad[0])])


@pytest.mark.parametrize("idx", [3, 4])
def test_quantize_workload_inputs(idx):
    torch, mg = require_gpu()
    inp = wl.make_wgrad_inputs(idx)
    for name in ("gT", "xT"):
        say("quantize workload", idx, name, inp[name].shape)
        q, s = mg.mx_quantize(dev(torch, inp[name]))
        torch.cuda.synchronize()
        want_q, want_s = oracle.mx_quantize(inp[name])
        assert np.array_equal(host(s), want_s)
        assert np.array_equal(host(q), want_q)


@pytest.mark.parametrize("case", ["edge", "tile", "ragged", "tall", "wide"])
def test_quantize_transposed_bit_exact(case):
    """moe_gg_mx_quantize_t(x) equals the oracle's quantisation of x^T, code for code."""
    torch, mg = require_gpu()
    rng = np.random.default_rng({"edge": 11, "tile": 12, "ragged": 13, "tall": 14, "wide": 15}[case])
    if case == "edge":
        x = np.ascontiguousarray(_edge_input().T)            # [128 tokens, 12 features]
    elif case == "tile":
        x = rng.standard_normal((256, 128)).astype(np.float32)
    elif case == "ragged":                                    # partial tiles in both directions
        x = (rng.standard_normal((160, 100)) * np.exp2(rng.integers(-40, 40, (1, 100)))).astype(np.float32)
    elif case == "tall":
        x = rng.standard_normal((4096 + 32, 36)).astype(np.float32)
        x[rng.random(x.shape) < 0.01] *= 64
    else:   # 3 x 3 tiles, both partial: a pair of feature tiles, then a single one in the tile order
        x = (rng.standard_normal((288, 600)) * np.exp2(rng.integers(-30, 30, (1, 600)))).astype(np.float32)
    say("quantize_t", case, x.shape)
    q, s = mg.mx_quantize_t(dev(torch, x))
    torch.cuda.synchronize()
    want_q, want_s = oracle.mx_quantize(np.ascontiguousarray(x.T))
    assert np.array_equal(host(s), want_s)
    got_q = host(q)
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, (bad[:5], got_q[tuple(bad[0])], want_q[tuple(bad[0])])


def test_quantize_transposed_workload_operand():
    """g [M, N] of the 8192^3 workload -> g^T codes, as the weight gradient's A operand."""
    torch, mg = require_gpu()
    inp = wl.make_wgrad_inputs(4)
    g = np.ascontiguousarray(inp["gT"].T)                     # [M = 8192 tokens, N = 8192]
    say("quantize_t workload 4 g", g.shape)
    q, s = mg.mx_quantize_t(dev(torch, g))
    torch.cuda.synchronize()
    want_q, want_s = oracle.mx_quantize(inp["gT"])
    assert np.array_equal(host(s), want_s)
    assert np.array_equal(host(q), want_q)


def _roundup_edges():
    """Blocks whose max sits on or one f32 ulp either side of 448 * 2^k (where the f32 product
    decides the byte), plus the default edge blocks."""
    x = _edge_input()
    rng = np.random.default_rng(31)
    rows = []
    for k in (-20, -1, 0, 3, 40):
        base = np.float32(448.0 * 2.0 ** k)
        for m in (np.nextafter(base, np.float32(0)), base, np.nextafter(base, np.float32(np.inf))):
            blk = (rng.standard_normal(128) * float(base) / 8).astype(np.float32)
            blk[::32] = -m
            rows.append(blk)
    rows.append(np.zeros(128, np.float32))                   # 28 rows: the transposing quantiser wants L % 4 == 0
    return np.concatenate([x, np.stack(rows)])


@pytest.mark.parametrize("case", ["edges", "random"])
def test_quantize_roundup_bit_exact(case):
    """Both quantisers with the round-up scale rule equal the oracle's round-up quantisation."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(41)
    if case == "edges":
        x = _roundup_edges()
    else:
        x = (rng.standard_normal((160, 96)) * np.exp2(rng.integers(-60, 60, (160, 1)))).astype(np.float32)
        x[rng.random(x.shape) < 0.02] *= 64
    say("quantize roundup", case, x.shape)
    want_q, want_s = oracle.mx_quantize(x, rule="roundup")
    q, s = mg.mx_quantize(dev(torch, x), rule="roundup")
    torch.cuda.synchronize()
    assert np.array_equal(host(s), want_s)
    assert np.array_equal(host(q), want_q)
    xt = np.ascontiguousarray(x.T)                          # quantise_t of x^T is along x's rows
    q, s = mg.mx_quantize_t(dev(torch, xt), rule="roundup")
    torch.cuda.synchronize()
    assert np.array_equal(host(s), want_s)
    assert np.array_equal(host(q), want_q)
    # the default rule is unchanged by the variant's existence, and differs from it here
    fq, fs = oracle.mx_quantize(x)
    assert not np.array_equal(fs, want_s)


OFFSETS = [
    [0, 256],
    [0, 0, 0, 100, 100, 256],
    [0, 100, 256, 256, 256],
    [0, 1, 2, 3, 256],
    list(range(0, 257, 4)),
]


@pytest.mark.parametrize("off", OFFSETS + ["workload2", "workload5"])
def test_row_experts_bit_exact(off):
    torch, mg = require_gpu()
    if off == "workload2":
        off = wl.make_offsets(2, np.random.default_rng(2))
    elif off == "workload5":
        off = wl.make_offsets(5, np.random.default_rng(5))
    off = np.asarray(off, np.int32)
    M = int(off[-1])
    say("row_experts", off[:6], M)
    got = host(mg.row_experts(dev(torch, off), M))
    assert np.array_equal(got, oracle.row_experts(off, M))
