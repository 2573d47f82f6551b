"""The entry points under HIP graph capture: the library allocates nothing and
enqueues only its kernels on the caller's stream, so a captured sequence
(quantise g^T and x^T, weight gradient, data gradient, grouped GEMM) replays
to the same bytes as the eager calls.  Each replay follows eager work that
rewrites the inputs in place, and every replay is checked."""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


def test_captured_sequence_replays_like_eager_calls():
    torch, mg = require_gpu()
    d = torch.device("cuda:0")
    counts = [384, 0, 256, 128]
    off = torch.from_numpy(wl.offsets_from_counts(counts)).to(d)
    M, N, K, E = 768, 512, 256, len(counts)
    gT = torch.empty((N, M), device=d)
    xT = torch.empty((K, M), device=d)
    g = torch.empty((M, N), device=d)
    W = torch.empty((E, N, K), device=d)
    qa = torch.empty((N, M), dtype=torch.uint8, device=d); sa = torch.empty((N, M // 32), dtype=torch.uint8, device=d)
    qb = torch.empty((K, M), dtype=torch.uint8, device=d); sb = torch.empty((K, M // 32), dtype=torch.uint8, device=d)
    gw = torch.empty((E * N, K), dtype=torch.bfloat16, device=d)
    dx = torch.empty((M, K), dtype=torch.float32, device=d)
    ga = torch.empty((M, N), dtype=torch.uint8, device=d); gs = torch.empty((M, N // 32), dtype=torch.uint8, device=d)
    wq = torch.empty((E * K, N), dtype=torch.uint8, device=d); wsc = torch.empty((E * K, N // 32), dtype=torch.uint8, device=d)
    gy = torch.empty((M, K), dtype=torch.bfloat16, device=d)

    def fill(seed):
        gen = torch.Generator(device=d).manual_seed(seed)
        for t in (gT, xT, g, W):
            t.copy_(torch.randn(t.shape, generator=gen, device=d))
        gT[torch.rand(gT.shape, generator=gen, device=d) < 0.01] *= 64

    def step():
        mg.mx_quantize(gT, qa, sa)
        mg.mx_quantize(xT, qb, sb)
        mg.wgrad_mxfp8(qa, qb, sa, sb, off, out=gw)
        mg.dgrad_f32(g, W, off, out=dx)
        mg.mx_quantize(g, ga, gs)
        mg.mx_quantize_t(W[0], wq[:K], wsc[:K])        # B[0] = MX(W_0^T) along N; experts 1.. stay zero
        mg.grouped_mxfp8(ga, wq.view(E, K, N), gs, wsc.view(E, K, N // 32), off, out=gy)

    outs = (qa, sa, qb, sb, gw, dx, ga, gs, gy)
    fill(1)
    wq.zero_(); wsc.zero_()
    say("graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (2, 3, 4):
        fill(seed)
        say("eager then replay", seed)
        step()
        torch.cuda.synchronize()
        eager = [t.clone() for t in outs]
        for t in outs:
            t.fill_(0x7F) if t.dtype == torch.uint8 else t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip("qa sa qb sb gw dx ga gs gy".split(), eager, outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (seed, name)
