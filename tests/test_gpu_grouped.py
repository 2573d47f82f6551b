"""GPU parity of the expert-grouped MXFP8 GEMM (forward / MXFP8 data gradient) against the oracle.

The MX operands are produced by the oracle's quantiser on the CPU and fed,
the same bytes, to both sides.  Bar: every element within
2^-7 |ref| + 2^-12 rms(ref) (the weight gradient's tolerance); exact equality
where the result is exactly representable.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _quant_b(Wt):
    """Per-expert MX codes of B [E, N, K] along K."""
    E, N, K = Wt.shape
    q, s = oracle.mx_quantize(Wt.reshape(E * N, K))
    return q.reshape(E, N, K), s.reshape(E, N, K // 32)


def _run(torch, mg, ca, sa, cb, sb, off, fast=False):
    out = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb),
                           dev(torch, np.asarray(off, np.int32)), fast=fast)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


CASES = {
    # name: (N, K, per-expert token counts)
    "one_expert": (256, 256, [256]),
    "aligned": (512, 256, [256, 0, 512, 256]),
    "straddle": (256, 384, [100, 300, 0, 112]),
    "ragged_m": (256, 256, [37, 0, 200, 63]),              # M = 300: a partial row tile
    "many_per_tile": (256, 128, [16] * 10 + [0] * 3 + [96]),
    "empty_ends": (512, 512, [0, 0, 260, 0]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_small(name):
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    rng = np.random.default_rng(len(name) * 11 + N)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    w = rng.standard_normal((E, N, K)).astype(np.float32)
    ca, sa = oracle.mx_quantize(a)
    cb, sb = _quant_b(w)
    say("grouped", name, M, N, K, counts)
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert got.shape == ref.shape
    assert oracle.wgrad_excess(got, ref) <= 0, oracle.wgrad_excess(got, ref)


@pytest.mark.parametrize("name", ["aligned", "straddle", "ragged_m", "many_per_tile"])
def test_grouped_outliers_in_both_operands(name):
    """1% x64 outliers in the tokens and in the weights: where two outliers meet, the
    block-scaled fp8 MFMA's truncation of an 8-element run would lose the run's other
    products; the default entry point multiplies exactly converted bf16 operands."""
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    rng = np.random.default_rng(len(name) * 19 + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    w = rng.standard_normal((E, N, K)).astype(np.float32)
    w[rng.random(w.shape) < 0.01] *= 64
    ca, sa = oracle.mx_quantize(a)
    cb, sb = _quant_b(w)
    say("grouped, outliers in both operands", name, M, N, K, counts)
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(got, ref) <= 0, oracle.wgrad_excess(got, ref)


def test_grouped_all_ones_is_exact():
    torch, mg = require_gpu()
    counts = [100, 0, 400, 12]
    off = wl.offsets_from_counts(counts)
    M, N, K, E = int(off[-1]), 256, 384, len(counts)
    ca = np.full((M, K), 0x38, np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    cb = np.full((E, N, K), 0x38, np.uint8)
    sb = np.full((E, N, K // 32), 127, np.uint8)
    say("grouped all-ones")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    assert np.all(got == float(K))


def test_grouped_expert_scales_pick_each_rows_weights():
    """Codes 1.0 everywhere; expert e's weight scales are 2^e: row m gets K * 2^e(m), exactly."""
    torch, mg = require_gpu()
    counts = [50, 0, 150, 100, 12]
    off = wl.offsets_from_counts(counts)
    M, N, K, E = int(off[-1]), 256, 128, len(counts)
    ca = np.full((M, K), 0x38, np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    cb = np.full((E, N, K), 0x38, np.uint8)
    sb = np.broadcast_to((127 + np.arange(E))[:, None, None], (E, N, K // 32)).astype(np.uint8).copy()
    say("grouped expert scales")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    experts = oracle.row_experts(off, M)
    want = (K * np.exp2(experts.astype(np.float64)))[:, None] * np.ones((1, N))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["aligned", "straddle", "ragged_m"])
def test_grouped_fast_without_outliers(name):
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M, E = int(off[-1]), len(counts)
    rng = np.random.default_rng(len(name) * 13 + K)
    ca, sa = oracle.mx_quantize(rng.standard_normal((M, K)).astype(np.float32))
    cb, sb = _quant_b(rng.standard_normal((E, N, K)).astype(np.float32))
    say("grouped fast", name)
    got = _run(torch, mg, ca, sa, cb, sb, off, fast=True)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(got, ref) <= 0


def test_grouped_as_mxfp8_data_gradient():
    """dx = g W_e: A = MX(g) along N, B[e] = MX(W_e^T) along N (the transposing quantiser's layout)."""
    torch, mg = require_gpu()
    inp = wl.make_dgrad_inputs(2)                            # E=8, M=4096, N=1024, K=2048, one empty expert
    g, W, off = inp["g"], inp["W"], inp["off"]
    E, N, K = W.shape
    ca, sa = oracle.mx_quantize(g)                           # [M, N] along N
    Wt = np.ascontiguousarray(np.transpose(W, (0, 2, 1)))    # [E, K, N]
    cb, sb = _quant_b(Wt)
    say("grouped as MXFP8 dgrad, workload 2")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert got.shape == (g.shape[0], K)
    assert oracle.wgrad_excess(got, ref) <= 0
    # and it is the data gradient of the dequantised operands
    deq_g = oracle.mx_dequantize(ca, sa)
    deq_W = np.stack([oracle.mx_dequantize(cb[e], sb[e]).T for e in range(E)])
    np.testing.assert_allclose(ref, oracle.dgrad(deq_g, deq_W, off), rtol=1e-9, atol=1e-9)


def test_grouped_larger_unaligned():
    """E=8, M=4096, N=K=2048 with unaligned offsets: every element against the oracle."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(77)
    counts = np.array([700, 13, 0, 1200, 555, 900, 0, 728])
    off = wl.offsets_from_counts(counts)
    M, N, K, E = int(off[-1]), 2048, 2048, len(counts)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 64
    ca, sa = oracle.mx_quantize(a)
    del a
    cb, sb = _quant_b(rng.standard_normal((E, N, K)).astype(np.float32))
    say("grouped larger", M, N, K, E)
    got = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(host(got).astype(np.float64), ref) <= 0


def test_grouped_rows_of_no_expert_are_zero():
    """off[0] > 0 and off[E] < M: the rows before and after every expert are +0.0, the rest unchanged."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(5)
    off = np.array([64, 300, 300, 555], np.int32)
    M, N, K, E = 900, 512, 256, 3
    ca, sa = oracle.mx_quantize(rng.standard_normal((M, K)).astype(np.float32))
    cb, sb = _quant_b(rng.standard_normal((E, N, K)).astype(np.float32))
    say("grouped rows of no expert", list(off), M)
    out = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    bits = host(out.view(torch.int16))
    assert np.all(bits[:64] == 0) and np.all(bits[555:] == 0)       # +0.0, not -0.0
    inner = oracle.grouped_gemm(ca[64:555], sa[64:555], cb, sb, off - 64)
    assert oracle.wgrad_excess(got[64:555], inner) <= 0


def test_grouped_most_experts():
    """E = 2048 (the limit of the on-chip offset tables), 0..6 tokens each."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(2048)
    E, N, K = 2048, 256, 128
    counts = rng.integers(0, 7, size=E)
    counts[:5] = 0
    counts[-3:] = 0
    off = wl.offsets_from_counts(counts)
    M = int(off[-1])
    ca, sa = oracle.mx_quantize(rng.standard_normal((M, K)).astype(np.float32))
    cb, sb = _quant_b(rng.standard_normal((E, N, K)).astype(np.float32))
    say("grouped E=2048", M)
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(got, ref) <= 0


def test_grouped_full_size_data_gradient():
    """The 64-expert data gradient at full size (M=16384, contraction 1536, 7168 outputs, the offsets
    and g of that workload): every element against the oracle, the rms over the whole output.
    B[e] is one of four MX-quantised W_e^T draws, rolled along its rows by a per-expert amount, so
    experts differ."""
    torch, mg = require_gpu()
    w = wl.WORKLOADS[5]
    rng = np.random.default_rng(5)
    off = wl.make_offsets(5, rng)
    g = rng.standard_normal((w.M, w.N), dtype=np.float32) * np.float32(0.02)
    ca, sa = oracle.mx_quantize(g)                                   # along the contraction N
    del g
    wrng = np.random.default_rng(55)
    base = [oracle.mx_quantize(wrng.standard_normal((w.K, w.N), dtype=np.float32) * np.float32(0.02))
            for _ in range(4)]
    cb = np.empty((w.E, w.K, w.N), np.uint8)
    sb = np.empty((w.E, w.K, w.N // 32), np.uint8)
    for e in range(w.E):
        q, s = base[e % 4]
        cb[e] = np.roll(q, 37 * e, axis=0)
        sb[e] = np.roll(s, 37 * e, axis=0)
    say("grouped full-size data gradient, workload 5", w)
    got = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    assert tuple(got.shape) == (w.M, w.K)
    out = host(got).astype(np.float64)
    del got
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(out, ref) <= 0


def test_grouped_full_size_forward():
    """The MoE forward y = x W_e^T with MXFP8 weights at the 64-expert workload's full size
    (M=16384, K=7168 in, 1536 out, its offsets): every element against the oracle, the rms over
    the whole output.  W_e is one of four MX-quantised draws rolled along its rows per expert."""
    torch, mg = require_gpu()
    w = wl.WORKLOADS[5]
    rng = np.random.default_rng(5)
    off = wl.make_offsets(5, rng)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    x[rng.random(x.shape) < 0.01] *= 64
    ca, sa = oracle.mx_quantize(x)
    del x
    wrng = np.random.default_rng(57)
    base = [oracle.mx_quantize(wrng.standard_normal((w.N, w.K), dtype=np.float32) * np.float32(0.02))
            for _ in range(4)]
    cb = np.empty((w.E, w.N, w.K), np.uint8)
    sb = np.empty((w.E, w.N, w.K // 32), np.uint8)
    for e in range(w.E):
        q, s = base[e % 4]
        cb[e] = np.roll(q, 29 * e, axis=0)
        sb[e] = np.roll(s, 29 * e, axis=0)
    say("grouped full-size forward, workload 5", w)
    got = mg.grouped_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    assert tuple(got.shape) == (w.M, w.N)
    out = host(got).astype(np.float64)
    ref = oracle.grouped_gemm(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(out, ref) <= 0
