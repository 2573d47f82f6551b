"""Concurrent calls: the library keeps no mutable global state, so calls
enqueued on two streams at once, or made from two host threads each with its
own stream, give the same bytes as the same calls made one after another.
Streams keep the default priority."""
import threading

import numpy as np
import pytest

import workloads as wl
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


def _setup(torch, mg, d):
    gen = torch.Generator(device=d).manual_seed(7)
    counts = [100, 0, 290, 122, 256]                       # unaligned bounds and an empty expert
    off = torch.from_numpy(wl.offsets_from_counts(counts)).to(d)
    M, N, K, E = 768, 512, 256, len(counts)
    gT = torch.randn((N, M), generator=gen, device=d)
    gT[torch.rand(gT.shape, generator=gen, device=d) < 0.01] *= 64
    xT = torch.randn((K, M), generator=gen, device=d)
    g = torch.randn((M, N), generator=gen, device=d)
    W = torch.randn((E, N, K), generator=gen, device=d) * 0.05
    qa, sa = mg.mx_quantize(gT)
    qb, sb = mg.mx_quantize(xT)
    ga, gs = mg.mx_quantize(g)
    wq = torch.empty((E, K, N), dtype=torch.uint8, device=d)
    wsc = torch.empty((E, K, N // 32), dtype=torch.uint8, device=d)
    for e in range(E):
        mg.mx_quantize_t(W[e], wq[e], wsc[e])
    torch.cuda.synchronize()
    return dict(off=off, gT=gT, g=g, W=W, qa=qa, sa=sa, qb=qb, sb=sb, ga=ga, gs=gs, wq=wq, wsc=wsc)


def _ops(mg, t):
    """The calls under test; each returns its output tensor."""
    return [
        lambda: mg.wgrad_mxfp8(t["qa"], t["qb"], t["sa"], t["sb"], t["off"]),
        lambda: mg.dgrad_f32(t["g"], t["W"], t["off"]),
        lambda: mg.grouped_mxfp8(t["ga"], t["wq"], t["gs"], t["wsc"], t["off"]),
        lambda: mg.mx_quantize(t["gT"])[0],
        lambda: mg.wgrad_mxfp8(t["qa"], t["qb"], t["sa"], t["sb"], t["off"], fast=True),
    ]


def _same(a, b):
    return a.dtype == b.dtype and a.shape == b.shape and bool(torch_equal(a, b))


def torch_equal(a, b):
    import torch
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def test_two_streams_match_sequential_calls():
    torch, mg = require_gpu()
    d = torch.device("cuda:0")
    t = _setup(torch, mg, d)
    ops = _ops(mg, t)
    say("streams: sequential reference")
    ref = [op().clone() for op in ops]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (s1, s2):
        s.wait_stream(torch.cuda.current_stream())
    say("streams: interleaved on two streams")
    outs = []
    for rep in range(3):
        for i, op in enumerate(ops):
            with torch.cuda.stream(s1 if (i + rep) % 2 == 0 else s2):
                outs.append((i, op()))
    torch.cuda.synchronize()
    for i, out in outs:
        assert _same(out, ref[i]), f"call {i} on a second stream differs"


def test_two_host_threads_match_sequential_calls():
    torch, mg = require_gpu()
    d = torch.device("cuda:0")
    t = _setup(torch, mg, d)
    ops = _ops(mg, t)
    say("threads: sequential reference")
    ref = [op().clone() for op in ops]
    torch.cuda.synchronize()
    results = {0: [], 1: []}
    errors = []

    def worker(k):
        try:
            torch.cuda.set_device(d)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(3):
                    order = range(len(ops)) if k == 0 else reversed(range(len(ops)))
                    for i in order:
                        results[k].append((i, ops[i]()))
            s.synchronize()
        except Exception as exc:                           # reported below, in the test's thread
            errors.append(exc)

    say("threads: two host threads, one stream each")
    threads = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for k in (0, 1):
        assert len(results[k]) == 3 * len(ops)
        for i, out in results[k]:
            assert _same(out, ref[i]), f"call {i} from thread {k} differs"
