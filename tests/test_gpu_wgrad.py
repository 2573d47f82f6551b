"""GPU parity of the grouped MXFP8 weight gradient against the oracle.

The MX inputs are produced by the oracle's quantiser on the CPU and fed, the
same bytes, to both sides.  Bar: every element within
2^-7 |ref| + 2^-12 rms(ref); exact equality where the result is exactly
representable (all-ones, scale-only, empty experts).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _mx_inputs(gT, xT):
    ca, sa = oracle.mx_quantize(gT)
    cb, sb = oracle.mx_quantize(xT)
    return ca, sa, cb, sb


def _run(torch, mg, ca, sa, cb, sb, off):
    out = mg.wgrad_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb),
                         dev(torch, np.asarray(off, np.int32)))
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


CASES = {
    # name: (N, K, per-expert token counts)
    "one_expert": (256, 256, [256]),
    "two_tiles_each": (512, 512, [128, 384]),
    "empty_first": (256, 512, [0, 256, 128]),
    "empty_middle": (512, 256, [128, 0, 0, 384]),
    "empty_last": (256, 256, [384, 128, 0]),
    "all_empty_but_one": (256, 256, [0, 0, 0, 128, 0]),
    "many_experts": (256, 256, [128] * 3 + [0] * 2 + [256] * 2 + [128] * 5),
    "deep_k": (256, 256, [1024, 128]),
    # expert bounds that are not multiples of 128 (nor of 32): masked edge steps
    "unaligned": (256, 256, [100, 0, 37, 300, 75]),
    "unaligned_tiny": (256, 512, [1, 126, 1, 0, 128]),
    "unaligned_many": (512, 256, [33, 95, 200, 56, 0, 128, 40, 88]),
    "unaligned_shared_step": (256, 256, [60, 4, 64, 0, 128]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_wgrad_small(name):
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M = int(off[-1])
    rng = np.random.default_rng(len(name) * 7 + N)
    gT = rng.standard_normal((N, M)).astype(np.float32)
    xT = rng.standard_normal((K, M)).astype(np.float32)
    gT[rng.random(gT.shape) < 0.01] *= 64
    ca, sa, cb, sb = _mx_inputs(gT, xT)
    say("wgrad", name, N, K, counts)
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.wgrad(ca, sa, cb, sb, off)
    assert got.shape == ref.shape
    assert oracle.wgrad_excess(got, ref) <= 0, oracle.wgrad_excess(got, ref)
    E = len(counts)
    for e in range(E):
        if counts[e] == 0:
            blk = got.reshape(E, N, K)[e]
            assert np.all(blk == 0) and not np.any(np.signbit(blk))


BOUNDS = [1, 2, 3, 4, 5, 31, 32, 33, 63, 64, 65, 95, 96, 97, 126, 127, 129, 191, 255]


@pytest.mark.parametrize("fast", [False, True])
def test_wgrad_every_bound_position(fast):
    """Two experts over 384 tokens, split at token b for b at every byte position
    of a dword and on both sides of the 32-, 64- and 128-token lines: the partial
    steps zero the other expert's codes in the staged tile before the MFMAs.
    Default entry point against the oracle, fast one against the hardware model."""
    import hw_mfma_model as hw
    torch, mg = require_gpu()
    N, K, M = 256, 256, 384
    rng = np.random.default_rng(23)
    gT = rng.standard_normal((N, M)).astype(np.float32)
    xT = rng.standard_normal((K, M)).astype(np.float32)
    gT[rng.random(gT.shape) < 0.01] *= 64
    ca, sa, cb, sb = _mx_inputs(gT, xT)
    say("wgrad every bound position", "fast" if fast else "exact")
    for b in BOUNDS:
        off = np.array([0, b, M], np.int32)
        got = (_run_fast if fast else _run)(torch, mg, ca, sa, cb, sb, off)
        ref = hw.wgrad_one_pass(ca, sa, cb, sb, off) if fast else oracle.wgrad(ca, sa, cb, sb, off)
        assert oracle.wgrad_excess(got, ref) <= 0, (b, oracle.wgrad_excess(got, ref))


def test_wgrad_all_ones_is_exact():
    torch, mg = require_gpu()
    counts = [384, 0, 1152, 128]
    off = wl.offsets_from_counts(counts)
    M, N, K = int(off[-1]), 256, 512
    ca = np.full((N, M), 0x78, np.uint8)            # 256 * 2^-8 = 1.0
    sa = np.full((N, M // 32), 119, np.uint8)
    cb = np.full((K, M), 0x78, np.uint8)
    sb = np.full((K, M // 32), 119, np.uint8)
    say("wgrad all-ones")
    got = _run(torch, mg, ca, sa, cb, sb, off).reshape(4, N, K)
    for e, c in enumerate(counts):
        assert np.all(got[e] == float(c)), (e, np.unique(got[e])[:5])


def test_wgrad_scale_only_is_exact():
    # codes 1.0; row n of g^T carries 2^(n%5 - 2) on even blocks and 2^(n%3) on odd ones,
    # row k of x^T 2^(-(k%4)): each element is a sum of a few powers of two (exact in bf16)
    torch, mg = require_gpu()
    counts = [256, 128]
    off = wl.offsets_from_counts(counts)
    M, N, K = 384, 256, 256
    ca = np.full((N, M), 0x38, np.uint8)
    cb = np.full((K, M), 0x38, np.uint8)
    nb = np.arange(N)[:, None]
    b = np.arange(M // 32)[None, :]
    sa = np.where(b % 2 == 0, 127 + nb % 5 - 2, 127 + nb % 3).astype(np.uint8)
    sb = np.broadcast_to(127 - (np.arange(K) % 4)[:, None], (K, M // 32)).astype(np.uint8).copy()
    say("wgrad scale-only")
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.wgrad(ca, sa, cb, sb, off)
    assert np.array_equal(got, ref)


def _e4m3_times_scale(code, s):
    e, m = (code >> 3) & 15, code & 7
    v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return v * 2.0 ** (s - 127)


def test_wgrad_extreme_scale_bytes():
    """Element values at both ends of bf16's range.  The exact entry point converts
    each code times its scale to bf16, which holds every such value from scale
    bytes 3 to 246 (and larger scale bytes with codes below 2^8) exactly: here
    2^-127 .. 2^-133 at the bottom and up to 1.875 * 2^127 at the top, against
    products brought back to ordinary magnitudes by the other operand's scale.
    Beyond that (2^-136, 1.75 * 2^128) the conversion rounds to bf16: to zero
    and to infinity; the fast entry point's scaled MFMA has neither limit."""
    torch, mg = require_gpu()
    N, K, M = 256, 256, 128
    off = [0, M]

    def call(pairs, g_scale):
        ca = np.full((N, M), 0x38, np.uint8)
        sa = np.full((N, M // 32), g_scale, np.uint8)
        cb = np.empty((K, M), np.uint8)
        sb = np.empty((K, M // 32), np.uint8)
        for k in range(K):
            code, s = pairs[k % len(pairs)]
            cb[k] = code
            sb[k] = s
        ref = oracle.wgrad(ca, sa, cb, sb, off)
        got = {}
        for fast in (False, True):
            out = mg.wgrad_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb),
                                 dev(torch, np.asarray(off, np.int32)), fast=fast)
            torch.cuda.synchronize()
            got[fast] = host(out).astype(np.float64)
        return ref, got

    say("wgrad extreme scale bytes: bottom of bf16's range")
    bottom = [(0x38, 0), (0x08, 0), (0x01, 3), (0x02, 2), (0x08, 1), (0x01, 5)]
    ref, got = call(bottom, 227)                       # g = 2^100
    for k, (code, s) in enumerate(bottom):
        assert ref[0, k] == M * 2.0 ** 100 * _e4m3_times_scale(code, s)
    assert np.array_equal(got[False], ref) and np.array_equal(got[True], ref)

    say("wgrad extreme scale bytes: top of bf16's range")
    top = [(0x77, 247), (0x70, 247), (0x38, 254), (0x7E, 246), (0x7E, 240)]
    ref, got = call(top, 27)                           # g = 2^-100
    assert np.array_equal(got[False], ref) and np.array_equal(got[True], ref)

    say("wgrad extreme scale bytes: beyond bf16's range")
    beyond = [(0x01, 0), (0x7E, 247)]                  # 2^-136 (with g = 2^100) and 1.75 * 2^128 (g = 2^-100)
    ref, got = call(beyond[:1], 227)
    assert np.array_equal(got[True], ref) and np.all(got[False] == 0.0)
    ref, got = call(beyond[1:], 27)
    assert np.array_equal(got[True], ref) and np.all(np.isposinf(got[False]))


def test_wgrad_tiny_workload():
    # the tiny workload's wgrad on MX-quantised g^T and x^T (the ABI has no f32 wgrad)
    torch, mg = require_gpu()
    inp = wl.make_wgrad_inputs(1)
    ca, sa, cb, sb = _mx_inputs(inp["gT"], inp["xT"])
    say("wgrad workload 1")
    got = _run(torch, mg, ca, sa, cb, sb, inp["off"])
    ref = oracle.wgrad(ca, sa, cb, sb, inp["off"])
    assert oracle.wgrad_excess(got, ref) <= 0


def test_wgrad_aligned_workload_full():
    torch, mg = require_gpu()
    inp = wl.make_wgrad_inputs(3)
    ca, sa, cb, sb = _mx_inputs(inp["gT"], inp["xT"])
    say("wgrad workload 3 (E=8, 2048^3)")
    got = _run(torch, mg, ca, sa, cb, sb, inp["off"])
    ref = oracle.wgrad(ca, sa, cb, sb, inp["off"])
    assert oracle.wgrad_excess(got, ref) <= 0


def _full_excess(got, ca, sa, cb, sb, off, N):
    """wgrad_excess of the whole GPU output (bf16 torch tensor [E*N, K]) against the whole oracle
    output, the rms taken over every element (empty experts included); empty experts must be +0.0.

    The oracle's result is built expert by expert (one fp64 matmul each) into one fp64 array; the
    comparison runs expert by expert to bound the temporaries."""
    E = len(off) - 1
    K = cb.shape[0]
    a = oracle.mx_dequantize(ca, sa)
    b = oracle.mx_dequantize(cb, sb)
    ref = np.zeros((E, N, K))
    for e in range(E):
        o0, o1 = int(off[e]), int(off[e + 1])
        if o1 > o0:
            ref[e] = a[:, o0:o1] @ b[:, o0:o1].T
    del a, b
    rms = oracle.rms(ref)
    worst = -np.inf
    for e in range(E):
        blk = host(got[e * N:(e + 1) * N]).astype(np.float64)
        if off[e + 1] == off[e]:
            assert np.all(blk == 0) and not np.any(np.signbit(blk)), f"expert {e} is empty"
        worst = max(worst, oracle.wgrad_excess(blk, ref[e], ref_rms=rms))
    return worst, rms


@pytest.mark.parametrize("idx", [4, 5])
def test_wgrad_full_size(idx):
    """Full-size workloads, the whole output against the whole oracle output."""
    torch, mg = require_gpu()
    w = wl.WORKLOADS[idx]
    inp = wl.make_wgrad_inputs(idx)
    ca, sa, cb, sb = _mx_inputs(inp["gT"], inp["xT"])
    del inp["gT"], inp["xT"]
    off = inp["off"]
    say(f"wgrad workload {idx} full size, whole output", w)
    got = mg.wgrad_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    worst, rms = _full_excess(got, ca, sa, cb, sb, off, w.N)
    say(f"wgrad workload {idx}: worst excess {worst:.4g} (rms {rms:.4g})")
    assert worst <= 0, worst


def test_wgrad_full_size_unaligned_offsets():
    """The 8192^3 workload with expert bounds moved off the 128 (and 32) grid, whole output."""
    torch, mg = require_gpu()
    w = wl.WORKLOADS[4]
    inp = wl.make_wgrad_inputs(4)
    counts = np.array([3200 - 37, 1536 + 42, 1024 - 5, 640, 512, 512 - 7, 384 + 7, 384])
    off = wl.offsets_from_counts(counts)
    assert int(off[-1]) == w.M
    ca, sa, cb, sb = _mx_inputs(inp["gT"], inp["xT"])
    del inp
    say("wgrad workload 4 full size, unaligned offsets, whole output", list(off))
    got = mg.wgrad_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb), dev(torch, off))
    torch.cuda.synchronize()
    worst, rms = _full_excess(got, ca, sa, cb, sb, off, w.N)
    say(f"wgrad workload 4 unaligned: worst excess {worst:.4g} (rms {rms:.4g})")
    assert worst <= 0, worst


def test_wgrad_most_experts():
    """E = 1024 (the limit of the kernel's on-chip expert ranking), most experts empty, the others
    with 1..300 tokens at unaligned bounds; the whole output against the oracle with the stated
    bound (rms over every element), and the empty experts' blocks exactly +0.0."""
    torch, mg = require_gpu()
    rng = np.random.default_rng(1024)
    E, N, K = 1024, 256, 256
    counts = np.zeros(E, np.int64)
    live = rng.choice(E, 12, replace=False)
    counts[live] = rng.integers(1, 300, size=12)
    M = int(np.ceil(counts.sum() / 128) * 128)
    counts[live[-1]] += M - counts.sum()                    # M a multiple of 128
    off = wl.offsets_from_counts(counts)
    gT = rng.standard_normal((N, M)).astype(np.float32)
    xT = rng.standard_normal((K, M)).astype(np.float32)
    ca, sa, cb, sb = _mx_inputs(gT, xT)
    say("wgrad E=1024", M, sorted(int(c) for c in counts[live]))
    got = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.wgrad(ca, sa, cb, sb, off)
    empty = np.repeat(counts == 0, N)
    assert np.all(got[empty] == 0.0) and not np.any(np.signbit(got[empty]))
    excess = oracle.wgrad_excess(got, ref)
    say(f"wgrad E=1024: whole-output excess {excess:.4g}")
    assert excess <= 0, excess


# ---- the single-pass entry point (moe_gg_wgrad_mxfp8_fast) -------------------

def _run_fast(torch, mg, ca, sa, cb, sb, off):
    out = mg.wgrad_mxfp8(dev(torch, ca), dev(torch, cb), dev(torch, sa), dev(torch, sb),
                         dev(torch, np.asarray(off, np.int32)), fast=True)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


@pytest.mark.parametrize("name", ["two_tiles_each", "empty_middle", "many_experts", "deep_k", "unaligned",
                                  "unaligned_many"])
def test_wgrad_fast_follows_hardware_rounding(name):
    """With 64x outliers the single pass follows the measured run-of-8 rounding model."""
    import hw_mfma_model as hw
    torch, mg = require_gpu()
    N, K, counts = CASES[name]
    off = wl.offsets_from_counts(counts)
    M = int(off[-1])
    rng = np.random.default_rng(len(name) * 7 + N)
    gT = rng.standard_normal((N, M)).astype(np.float32)
    xT = rng.standard_normal((K, M)).astype(np.float32)
    gT[rng.random(gT.shape) < 0.01] *= 64
    ca, sa, cb, sb = _mx_inputs(gT, xT)
    say("wgrad fast", name)
    got = _run_fast(torch, mg, ca, sa, cb, sb, off)
    model = hw.wgrad_one_pass(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(got, model) <= 0
    empties = [e for e, c in enumerate(counts) if c == 0]
    for e in empties:
        assert np.all(got.reshape(len(counts), N, K)[e] == 0)


@pytest.mark.parametrize("idx", [1, 3])
def test_wgrad_fast_exact_tolerance_without_outliers(idx):
    """Without outliers the single pass meets the exact-sum tolerance as well."""
    torch, mg = require_gpu()
    inp = wl.make_wgrad_inputs(idx)
    ca, sa, cb, sb = _mx_inputs(inp["gT"], inp["xT"])
    say("wgrad fast workload", idx)
    got = _run_fast(torch, mg, ca, sa, cb, sb, inp["off"])
    ref = oracle.wgrad(ca, sa, cb, sb, inp["off"])
    assert oracle.wgrad_excess(got, ref) <= 0


def test_wgrad_fast_and_precise_agree_exactly_on_narrow_range():
    """Codes within 2^6 of each other: both entry points give the exact bf16 result."""
    torch, mg = require_gpu()
    counts = [256, 128, 0, 384]
    off = wl.offsets_from_counts(counts)
    M, N, K = int(off[-1]), 256, 512
    rng = np.random.default_rng(31)
    ca = rng.choice(np.array([0x40, 0x48, 0x50, 0xC0, 0xC8, 0x58], np.uint8), size=(N, M))
    cb = rng.choice(np.array([0x38, 0x3C, 0xB8, 0x44], np.uint8), size=(K, M))
    sa = rng.integers(120, 124, size=(N, M // 32)).astype(np.uint8)
    sb = rng.integers(120, 124, size=(K, M // 32)).astype(np.uint8)
    say("wgrad fast vs precise, narrow range")
    fast = _run_fast(torch, mg, ca, sa, cb, sb, off)
    prec = _run(torch, mg, ca, sa, cb, sb, off)
    ref = oracle.wgrad(ca, sa, cb, sb, off)
    assert oracle.wgrad_excess(fast, ref) <= 0 and oracle.wgrad_excess(prec, ref) <= 0
    assert np.max(np.abs(fast - prec)) <= 2.0 ** -7 * np.max(np.abs(ref))
