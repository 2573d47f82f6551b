"""GPU parity of the MXFP4 quantiser (bit-exact) and the expert-grouped GEMM with MXFP4
weights (a8w4) against the oracle.

The a8w4 operands are produced by the oracle's quantisers on the CPU and fed,
the same bytes, to both sides.  Bar: the grouped GEMM's (2^-7 |ref| +
2^-12 rms(ref) per element), exact equality where the result is exactly
representable.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _mx4_edges():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((10, 128)).astype(np.float32)
    x[0] = 0.0                                                # zero blocks
    x[1, :32] = np.float32(1e-40)                             # f32 subnormals (scale byte clamps to 1)
    x[1, 32:64] = np.float32(2.0 ** -128) * np.sign(rng.standard_normal(32)).astype(np.float32)
    x[2, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    row = np.zeros(32)
    row[0] = 4.0                                              # max 4.0: scale 2^0, values in units
    row[1:8] = mids                                           # exact ties
    m32 = mids.astype(np.float32)
    row[8:15] = np.nextafter(m32, np.float32(10))             # one f32 ulp above
    row[15:22] = np.nextafter(m32, np.float32(0))             # one f32 ulp below
    row[22:25] = [6.0, 5.9, 3.9]
    row[25:28] = [-0.0, -2.0 ** -30, -0.25]                   # signed zeros
    x[3, :32] = row
    x[3, 32:64] = -row
    x[4, :32] = [7.9 if i == 0 else 6.5 if i == 1 else 0.1 * i for i in range(32)]   # saturation
    x[5] *= 64.0
    x[6, ::5] *= 1e6
    return x


@pytest.mark.parametrize("case", ["edges", "odd_rows", "long_rows"])
def test_mx4_quantize_bit_exact(case):
    torch, mg = require_gpu()
    rng = np.random.default_rng({"edges": 1, "odd_rows": 2, "long_rows": 3}[case])
    if case == "edges":
        x = _mx4_edges()
    elif case == "odd_rows":
        x = (rng.standard_normal((37, 96)) * np.exp2(rng.integers(-60, 60, (37, 1)))).astype(np.float32)
    else:
        x = rng.standard_normal((19, 4096 + 32)).astype(np.float32)
    say("mx4_quantize", case, x.shape)
    q, s = mg.mx4_quantize(dev(torch, x))
    torch.cuda.synchronize()
    want_q, want_s = oracle.mx4_quantize(x)
    assert np.array_equal(host(s), want_s)
    got_q = host(q)
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, (bad[:5], got_q[tuple(bad[0])], want_q[tuple(bad[0])])


def _quant_b4(W):
    E, N, K = W.shape
    q, s = oracle.mx4_quantize(W.reshape(E * N, K))
    return q.reshape(E, N, K // 2), s.reshape(E, N, K // 32)


def _run(torch, mg, ca, sa, cb, sb, off, fast=False):
    out = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb),
                           dev(torch, np.asarray(off, np.int32)), fast=fast, b_fp4=True)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


CASES = {
    # name: (N, K, per-expert token counts)
    "one_expert": (256, 256, [256]),
    "aligned": (512, 256, [256, 0, 512, 256]),
    "straddle": (256, 384, [100, 300, 0, 112]),
    "ragged_m": (256, 256, [37, 0, 200, 63]),
    "many_experts": (256, 128, [16] * 10 + [0] * 3 + [96]),
    "deep_k": (256, 1024, [300, 212]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_a8w4_small(name):
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    rng = np.random.default_rng(len(name) * 17 + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    ca, sa = oracle.mx_quantize(a)
    cb, sb = _quant_b4(rng.standard_normal((E, N, K)).astype(np.float32))
    say("a8w4", name, M, N, K, counts)
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert oracle.wgrad_excess(got, ref) <= 0, oracle.wgrad_excess(got, ref)


@pytest.mark.parametrize("name", ["straddle", "ragged_m", "deep_k"])
def test_a8w4_outliers_in_both_operands(name):
    """1% x64 outliers in the tokens and in the fp4 weights."""
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    rng = np.random.default_rng(len(name) * 23 + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    w = rng.standard_normal((E, N, K)).astype(np.float32)
    w[rng.random(w.shape) < 0.01] *= 64
    ca, sa = oracle.mx_quantize(a)
    cb, sb = _quant_b4(w)
    say("a8w4, outliers in both operands", name, M, N, K, counts)
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert oracle.wgrad_excess(got, ref) <= 0, oracle.wgrad_excess(got, ref)


def test_a8w4_nibble_order():
    """Weights with 1.0 in the low nibble and 0 in the high one (byte 0x02) against token
    codes that differ between even and odd elements: only the even elements may count."""
    torch, mg = require_gpu()
    counts = [256]
    off = wl.offsets_from_counts(counts)
    M, N, K, E = 256, 256, 256, 1
    ca = np.tile(np.array([0x38, 0x40], np.uint8), (M, K // 2))    # 1.0 at even, 2.0 at odd elements
    sa = np.full((M, K // 32), 127, np.uint8)
    cb = np.full((E, N, K // 2), 0x02, np.uint8)
    sb = np.full((E, N, K // 32), 127, np.uint8)
    say("a8w4 nibble order")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    assert np.all(got == float(K // 2))
    got_fast = _run(torch, mg, ca, sa, cb, sb, off, fast=True)
    assert np.all(got_fast == float(K // 2))


def test_a8w4_all_ones_and_expert_scales_exact():
    """A codes 1.0, B codes 1.0 with expert e's scales 2^e: row m gets K * 2^e(m), exactly."""
    torch, mg = require_gpu()
    counts = [50, 0, 150, 100, 12]
    off = wl.offsets_from_counts(counts)
    M, N, K, E = int(off[-1]), 256, 384, len(counts)
    ca = np.full((M, K), 0x38, np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    cb = np.full((E, N, K // 2), 0x22, np.uint8)
    sb = np.broadcast_to((127 + np.arange(E))[:, None, None], (E, N, K // 32)).astype(np.uint8).copy()
    say("a8w4 all-ones, expert scales")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    want = (K * np.exp2(oracle.row_experts(off, M).astype(np.float64)))[:, None] * np.ones((1, N))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["aligned", "straddle", "deep_k"])
def test_a8w4_fast_without_outliers(name):
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    rng = np.random.default_rng(len(name) * 19 + K)
    ca, sa = oracle.mx_quantize(rng.standard_normal((M, K)).astype(np.float32))
    cb, sb = _quant_b4(rng.standard_normal((E, N, K)).astype(np.float32))
    say("a8w4 fast", name)
    got = _run(torch, mg, ca, sa, cb, sb, off, fast=True)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert oracle.wgrad_excess(got, ref) <= 0


def test_a8w4_forward_full_size():
    """The MoE forward y = x W_e^T at the 64-expert workload's full size (M=16384, K=7168 in,
    1536 out, its offsets): every element against the oracle, the rms over the whole output.
    W_e is one of four MXFP4-quantised draws rolled along its rows per expert, so experts differ."""
    torch, mg = require_gpu()
    w = wl.WORKLOADS[5]
    rng = np.random.default_rng(5)
    off = wl.make_offsets(5, rng)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    ca, sa = oracle.mx_quantize(x)
    del x
    wrng = np.random.default_rng(56)
    base = [oracle.mx4_quantize(wrng.standard_normal((w.N, w.K), dtype=np.float32) * np.float32(0.02))
            for _ in range(4)]
    cb = np.empty((w.E, w.N, w.K // 2), np.uint8)
    sb = np.empty((w.E, w.N, w.K // 32), np.uint8)
    for e in range(w.E):
        q, s = base[e % 4]
        cb[e] = np.roll(q, 29 * e, axis=0)
        sb[e] = np.roll(s, 29 * e, axis=0)
    say("a8w4 full-size forward, workload 5", w)
    got = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off),
                           b_fp4=True)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (w.M, w.N)
    out = host(got).astype(np.float64)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert oracle.wgrad_excess(out, ref) <= 0


@pytest.mark.parametrize("case", ["edges", "tile", "ragged", "wide"])
def test_mx4_quantize_transposed_bit_exact(case):
    """moe_gg_mx4_quantize_t(x) equals the oracle's MXFP4 quantisation of x^T, code for code."""
    torch, mg = require_gpu()
    rng = np.random.default_rng({"edges": 21, "tile": 22, "ragged": 23, "wide": 24}[case])
    if case == "edges":
        x = np.ascontiguousarray(np.concatenate([_mx4_edges(), np.zeros((2, 128), np.float32)]).T)   # [128, 12]
    elif case == "tile":
        x = rng.standard_normal((256, 512)).astype(np.float32)
    elif case == "ragged":                                    # partial tiles in both directions
        x = (rng.standard_normal((160, 300)) * np.exp2(rng.integers(-40, 40, (1, 300)))).astype(np.float32)
    else:                                                     # 3 x 3 tiles, both partial
        x = (rng.standard_normal((288, 600)) * np.exp2(rng.integers(-30, 30, (1, 600)))).astype(np.float32)
    say("mx4_quantize_t", case, x.shape)
    q, s = mg.mx4_quantize_t(dev(torch, x))
    torch.cuda.synchronize()
    want_q, want_s = oracle.mx4_quantize(np.ascontiguousarray(x.T))
    assert np.array_equal(host(s), want_s)
    assert np.array_equal(host(q), want_q)


def test_a8w4_as_data_gradient():
    """dx = g W_e with MXFP4 weights: A = MX(g) along N, B[e] = MXFP4(W_e^T) along N from the transposing
    MXFP4 quantiser (workload 2: E=8, M=4096, N=1024, K=2048, one empty expert)."""
    torch, mg = require_gpu()
    inp = wl.make_dgrad_inputs(2)
    g, W, off = inp["g"], inp["W"], inp["off"]
    E, N, K = W.shape
    ca, sa = oracle.mx_quantize(g)
    Wt = np.ascontiguousarray(np.transpose(W, (0, 2, 1)))    # [E, K, N]
    cb, sb = _quant_b4(Wt)                                     # the oracle's codes of W_e^T
    tq = torch.empty((E, K, N // 2), dtype=torch.uint8, device="cuda")
    ts = torch.empty((E, K, N // 32), dtype=torch.uint8, device="cuda")
    for e in range(E):
        mg.mx4_quantize_t(dev(torch, W[e]), tq[e], ts[e])     # the GPU's, from W_e [N, K]
    torch.cuda.synchronize()
    assert np.array_equal(host(tq), cb) and np.array_equal(host(ts), sb)
    say("a8w4 data gradient, workload 2")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off, b_format="e2m1")
    assert oracle.wgrad_excess(got, ref) <= 0
