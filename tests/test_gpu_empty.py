"""Empty sizes on the GPU: a contraction of length zero writes the empty sum
(+0.0 everywhere, against the oracle's zeros); a call with no output element
returns without touching anything.  Zero-size operands are passed as empty
tensors."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _u8(torch, *shape):
    return torch.empty(shape, dtype=torch.uint8, device="cuda:0")


@pytest.mark.parametrize("fast", [False, True])
def test_wgrad_without_tokens_writes_zeros(fast):
    torch, mg = require_gpu()
    E, N, K = 3, 256, 512
    say("wgrad M=0", E, N, K, fast)
    off = dev(torch, np.zeros(E + 1, np.int32))
    out = torch.full((E * N, K), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    mg.wgrad_mxfp8(_u8(torch, N, 0), _u8(torch, K, 0), _u8(torch, N, 0), _u8(torch, K, 0), off, out=out, fast=fast)
    torch.cuda.synchronize()
    ref = oracle.wgrad(np.zeros((N, 0), np.uint8), np.zeros((N, 0), np.uint8), np.zeros((K, 0), np.uint8),
                       np.zeros((K, 0), np.uint8), np.zeros(E + 1, np.int64))
    assert np.array_equal(host(out), ref)
    assert int((out.view(torch.int16) != 0).sum()) == 0          # +0.0, not -0.0


def test_dgrad_empty_contraction_writes_zeros():
    torch, mg = require_gpu()
    counts = [100, 0, 156, 20]
    off = wl.offsets_from_counts(counts)
    M, K, E = int(off[-1]), 260, len(counts)
    say("dgrad N=0", M, K, counts)
    out = torch.full((M, K), float("nan"), dtype=torch.float32, device="cuda:0")
    mg.dgrad_f32(torch.empty((M, 0), dtype=torch.float32, device="cuda:0"),
                 torch.empty((E, 0, K), dtype=torch.float32, device="cuda:0"),
                 dev(torch, off.astype(np.int32)), out=out)
    torch.cuda.synchronize()
    ref = oracle.dgrad(np.zeros((M, 0), np.float32), np.zeros((E, 0, K), np.float32), off)
    assert np.array_equal(host(out), ref)
    assert int((out.view(torch.int32) != 0).sum()) == 0


@pytest.mark.parametrize("b_fp4", [False, True])
@pytest.mark.parametrize("fast", [False, True])
def test_grouped_empty_contraction_writes_zeros(fast, b_fp4):
    torch, mg = require_gpu()
    counts = [0, 200, 57, 0]
    off = wl.offsets_from_counts(counts)
    M, N, E = int(off[-1]), 512, len(counts)
    off_dev = dev(torch, off.astype(np.int32))
    say("grouped K=0", M, N, counts, fast, b_fp4)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    mg.grouped_mxfp8(_u8(torch, M, 0), _u8(torch, E, N, 0), _u8(torch, M, 0), _u8(torch, E, N, 0), off_dev,
                     out=out, fast=fast, b_fp4=b_fp4)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(np.zeros((M, 0), np.uint8), np.zeros((M, 0), np.uint8),
                              np.zeros((E, N, 0), np.uint8), np.zeros((E, N, 0), np.uint8), off)
    assert np.array_equal(host(out), ref)
    assert int((out.view(torch.int16) != 0).sum()) == 0


def test_empty_outputs_are_no_ops():
    torch, mg = require_gpu()
    say("empty outputs")
    off = dev(torch, np.zeros(4, np.int32))
    out = mg.dgrad_f32(torch.empty((0, 64), dtype=torch.float32, device="cuda:0"),
                       torch.zeros((3, 64, 128), dtype=torch.float32, device="cuda:0"), off)
    assert out.shape == (0, 128)
    out = mg.grouped_mxfp8(_u8(torch, 0, 256), _u8(torch, 3, 256, 256), _u8(torch, 0, 8), _u8(torch, 3, 256, 8), off)
    assert out.shape == (0, 256)
    for fn in (mg.mx_quantize, mg.mx4_quantize):
        q, s = fn(torch.empty((0, 64), dtype=torch.float32, device="cuda:0"))
        assert q.shape[0] == 0 and s.shape[0] == 0
    q, s = mg.mx_quantize_t(torch.empty((0, 64), dtype=torch.float32, device="cuda:0"))
    assert q.numel() == 0
    assert mg.row_experts(off, 0).shape == (0,)
    torch.cuda.synchronize()
