#!/usr/bin/env python3
"""Benchmark of the grouped MXFP8 weight gradient (and the other passes).

Default (the headline): E=8 experts, M=N=K=8192, per-expert token counts
[3200, 1536, 1024, 640, 512, 512, 384, 384] (Zipf(1.1) in 128-token units),
g^T and x^T ~ normal(0,1) with 1% of entries x64, MX-quantised on the GPU by
moe_gg_mx_quantize before timing.  One step = one moe_gg_wgrad_mxfp8 call
(expert bounds, operand staging, scale packing, block-scaled MFMA, bf16
epilogue) over resident inputs.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --pass dgrad --workload 5      # other passes / workloads
  python bench.py --pass quantize --workload 4

Timing: HIP events on the stream the kernels are launched on (torch's
current stream), bracketing the K timed steps after a synchronize.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

# MI355X published dense peaks (per GPU)
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

KERNEL_SOURCES = {
    "wgrad": ["wgrad_mxfp8.hip", "mx_gemm_core.hpp", "common.hpp"],
    "dgrad": ["dgrad_f32.hip", "common.hpp"],
    "quantize": ["mx_quantize.hip", "common.hpp"],
    "quantize_t": ["mx_quantize.hip", "common.hpp"],
    "quantize4": ["mx_quantize.hip", "common.hpp"],
    "grouped": ["grouped_mxfp8.hip", "mx_gemm_core.hpp", "common.hpp"],
    "forward": ["grouped_mxfp8.hip", "mx_gemm_core.hpp", "common.hpp"],
    "a8w4": ["grouped_mxfp8.hip", "mx_gemm_core.hpp", "common.hpp"],
}
KERNEL_NAMES = {"wgrad": "wgrad_mxfp8_kernel", "dgrad": "dgrad_f32_kernel", "quantize": "mx_quantize_kernel",
                "quantize_t": "mx_quantize_t_kernel", "quantize4": "mx4_quantize_kernel",
                "grouped": "grouped_mxfp8_kernel",
                "forward": "grouped_mxfp8_kernel", "a8w4": "grouped_mxfp8_kernel"}


def code_text(src: str) -> str:
    """A kernel source without its comments, trailing blanks and empty lines, so
    that comment edits do not mark a measured kernel as changed."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in src.splitlines())
    return "\n".join(line for line in lines if line)


def source_digest(pass_name: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[pass_name]:
        with open(os.path.join(ROOT, "moe_grouped_gemm_mxfp8_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(pass_name: str, workload: int):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernel."""
    path = os.path.join(ROOT, "profiles", f"{pass_name}_w{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest(pass_name):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"])
    except Exception:
        pass
    return os.cpu_count() or 1


LAUNCH_DIST = {}     # per-launch times of the last timed region (ms): median, p10, p90


def quantiles(ms_list):
    q = sorted(ms_list)
    pick = lambda f: q[int(round(f * (len(q) - 1)))]
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4), "n": len(q)}


def time_steps(torch, fn, steps, warmup):
    """W untimed warm-ups, then exactly K timed launches on torch's current stream
    (the stream the library launches on), bracketed by two events.  Afterwards,
    outside the timed region, K more launches with an event between each give
    the per-launch distribution."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    LAUNCH_DIST.clear()
    LAUNCH_DIST.update(quantiles([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    return ms  # ms per step of the timed region


def time_cold(torch, fn, reps=20, scratch_bytes=512 << 20):
    """Each launch timed alone after a 512 MB write that evicts L2 and the MALL."""
    d = torch.device("cuda:0")
    scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device=d)
    stream = torch.cuda.current_stream()
    out = []
    for r in range(reps):
        scratch.fill_(r & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del scratch
    return quantiles(out)


def bind_roofline(line, flop, nbytes, ms):
    """Switch a GEMM line's roofline to HBM when the algorithmic bytes take longer
    at the HBM peak than the useful FLOP at the fp8 MFMA peak (the binding roofline
    is the larger floor); the fp8 fraction stays beside it."""
    if nbytes / (PEAK_HBM_GBS * 1e9) <= flop / (PEAK_FP8_TFLOPS * 1e12):
        return
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flop / (ms * 1e-3) / 1e12
    line["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "fp8_frac": round(tf / PEAK_FP8_TFLOPS, 4)})


def bench_wgrad(torch, mg, idx, steps, warmup, cpu_baseline, fast=False):
    w = wl.WORKLOADS[idx]
    inp = wl.make_wgrad_inputs(idx)
    d = torch.device("cuda:0")
    off_np = inp["off"]
    gT = torch.from_numpy(inp["gT"]).to(d)
    xT = torch.from_numpy(inp["xT"]).to(d)
    qa, sa = mg.mx_quantize(gT)
    qb, sb = mg.mx_quantize(xT)
    off = torch.from_numpy(off_np).to(d)
    del gT, xT
    out = torch.empty((w.E * w.N, w.K), dtype=torch.bfloat16, device=d)
    torch.cuda.synchronize()
    ms = time_steps(torch, lambda: mg.wgrad_mxfp8(qa, qb, sa, sb, off, out=out, fast=fast), steps, warmup)
    tokens = int(off_np[-1] - off_np[0])
    flop = 2.0 * w.N * w.K * tokens
    algo_bytes = (w.N + w.K) * w.M + (w.N + w.K) * (w.M // 32) + 2 * w.E * w.N * w.K
    tflops = flop / (ms * 1e-3) / 1e12
    line = {
        "metric": "TFLOP/s + % of fp8 MFMA peak, MXFP8 wgrad M=N=K=8192 E=8 (1 GPU)" if idx == 4
        else f"TFLOP/s, MXFP8 grouped wgrad workload {idx}",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "pct_of_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2),
        "ms_per_step": round(ms, 4),
        "dtype": "fp8e4m3*fp8e4m3->f32 acc, bf16 out" if fast else "mxfp8 (e4m3+e8m0) -> bf16 MFMA, f32 acc, bf16 out",
        "mode": "block-scaled fp8 MFMA (hardware run-of-8 rounding)" if fast
        else "E4M3 x E8M0 converted exactly to bf16, bf16 MFMA (exact sum up to f32-level accumulation error)",
        "config": {"workload": w.name, "E": w.E, "M": w.M, "N": w.N, "K": w.K,
                   "tokens_per_expert": [int(c) for c in np.diff(off_np)]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": None if fast else read_traffic("wgrad", idx),
                     "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (fp8)" if fast else "v_mfma_f32_32x32x16_bf16",
                     "frac_of_mfma_dtype_peak": round(tflops / (PEAK_FP8_TFLOPS if fast else PEAK_BF16_TFLOPS), 4),
                     "algorithmic_bytes": algo_bytes, "algorithmic_flop": flop,
                     "hbm_gbs_algorithmic": round(algo_bytes / (ms * 1e-3) / 1e9, 1)},
    }
    # the aligned 2048^3 and the 64-expert workloads: the bf16 output's stores
    # outweigh the MFMA work
    bind_roofline(line, flop, algo_bytes, ms)
    if idx == 3:
        # also cold: each launch alone after a 512 MB write (L2 and MALL evicted)
        line["cold_ms"] = time_cold(torch, lambda: mg.wgrad_mxfp8(qa, qb, sa, sb, off, out=out, fast=fast))
    if cpu_baseline:
        line["cpu_baseline"] = cpu_wgrad_baseline(inp)
    return line


def cpu_wgrad_baseline(inp):
    """The oracle (numpy fp64) on the whole workload, timed on this host."""
    import oracle
    gT, xT, off = inp["gT"], inp["xT"], inp["off"]
    ca, sa = oracle.mx_quantize(gT)          # input preparation, not timed
    cb, sb = oracle.mx_quantize(xT)
    t0 = time.perf_counter()
    ref = oracle.wgrad(ca, sa, cb, sb, off)   # dequantise + per-expert fp64 GEMM
    dt = time.perf_counter() - t0
    del ref
    tokens = int(off[-1] - off[0])
    flop = 2.0 * gT.shape[0] * xT.shape[0] * tokens
    return {"value": round(flop / dt / 1e12, 4), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2), "cpu": cpu_info(),
            "sample": "the whole workload: MX dequantise to fp64 + one fp64 matmul per expert "
                      "(oracle.wgrad); quantisation of the inputs not timed"}


def bench_dgrad(torch, mg, idx, steps, warmup, cpu_baseline):
    w = wl.WORKLOADS[idx]
    inp = wl.make_dgrad_inputs(idx)
    d = torch.device("cuda:0")
    g = torch.from_numpy(inp["g"]).to(d)
    W = torch.from_numpy(inp["W"]).to(d)
    off = torch.from_numpy(inp["off"]).to(d)
    out = torch.empty((w.M, w.K), dtype=torch.float32, device=d)
    ms = time_steps(torch, lambda: mg.dgrad_f32(g, W, off, out=out), steps, warmup)
    flop = 2.0 * w.M * w.N * w.K
    nonempty = int(np.count_nonzero(np.diff(inp["off"])))
    algo_bytes = 4 * (w.M * w.N + nonempty * w.N * w.K + w.M * w.K)
    tflops = flop / (ms * 1e-3) / 1e12
    line = {
        "metric": f"TFLOP/s, f32 grouped dgrad workload {idx}",
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "pct_of_f32_peak": round(100 * tflops / PEAK_F32_TFLOPS, 2),
        "ms_per_step": round(ms, 4), "dtype": "f32",
        "config": {"workload": w.name, "E": w.E, "M": w.M, "N": w.N, "K": w.K},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_F32_TFLOPS, 4),
                     "traffic": read_traffic("dgrad", idx), "algorithmic_bytes": algo_bytes},
    }
    if cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        oracle.dgrad(inp["g"], inp["W"], inp["off"])
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(flop / dt / 1e12, 4), "unit": "TFLOP/s", "cores": blas_threads(),
                                "kind": "oracle", "seconds": round(dt, 2), "cpu": cpu_info(),
                                "sample": "the whole workload (oracle.dgrad, fp64)"}
    return line


def bench_grouped(torch, mg, idx, steps, warmup, cpu_baseline, fast=False):
    """The expert-grouped MXFP8 GEMM as an MXFP8 data gradient of a dgrad workload:
    dx = g W_e with A = MX(g) along N and B[e] = MX(W_e^T) along N (both quantised on the GPU)."""
    inp = wl.make_dgrad_inputs(idx)
    d = torch.device("cuda:0")
    g = torch.from_numpy(inp["g"]).to(d)
    W = torch.from_numpy(inp["W"]).to(d)
    off = torch.from_numpy(inp["off"]).to(d)
    M, N = g.shape
    E, _, K = W.shape
    qa, sa = mg.mx_quantize(g)                                   # [M, N] along N
    qb = torch.empty((E, K, N), dtype=torch.uint8, device=d)
    sb = torch.empty((E, K, N // 32), dtype=torch.uint8, device=d)
    for e in range(E):
        mg.mx_quantize_t(W[e], qb[e], sb[e])                     # W_e [N, K] -> [K, N] along N
    torch.cuda.synchronize()
    del W
    out = torch.empty((M, K), dtype=torch.bfloat16, device=d)
    ms = time_steps(torch, lambda: mg.grouped_mxfp8(qa, qb, sa, sb, off, out=out, fast=fast), steps, warmup)
    flop = 2.0 * M * N * K
    tf = flop / (ms * 1e-3) / 1e12
    nbytes = M * N + M * N // 32 + 2 * M * K + sum(
        (N * K + N * K // 32) for e in range(E) if inp["off"][e + 1] > inp["off"][e])
    line = {"metric": f"TFLOP/s, expert-grouped MXFP8 GEMM as the data gradient of workload {idx} (1 GPU)",
            "value": round(tf, 2), "unit": "TFLOP/s", "pct_of_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
            "ms_per_step": round(ms, 4), "dtype": "fp8e4m3*fp8e4m3->f32 acc, bf16 out" if fast else "mxfp8 (e4m3+e8m0) -> bf16 MFMA, f32 acc, bf16 out",
            "mode": "single block-scaled fp8 MFMA pass" if fast else "exact: MX operands converted to bf16, bf16 MFMA",
            "config": {"workload": wl.WORKLOADS[idx].name, "E": E, "M": M, "contraction": N, "N_out": K},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": None if fast else read_traffic("grouped", idx),
                         "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (fp8)" if fast else "v_mfma_f32_32x32x16_bf16",
                         "frac_of_mfma_dtype_peak": round(tf / (PEAK_FP8_TFLOPS if fast else PEAK_BF16_TFLOPS), 4),
                         "algorithmic_bytes": int(nbytes), "algorithmic_flop": flop}}
    bind_roofline(line, flop, nbytes, ms)
    if cpu_baseline:
        import oracle
        qa_h, sa_h = qa.cpu().numpy(), sa.cpu().numpy()
        rows = int(inp["off"][E // 8])                            # the tokens of the first E/8 experts
        sub_off = inp["off"][: E // 8 + 1]
        qb_h, sb_h = qb[: E // 8].cpu().numpy(), sb[: E // 8].cpu().numpy()
        t0 = time.perf_counter()
        oracle.grouped_gemm(qa_h[:rows], sa_h[:rows], qb_h, sb_h, sub_off)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(2.0 * rows * N * K / dt / 1e12, 4), "unit": "TFLOP/s",
                                "cores": blas_threads(), "kind": "oracle", "seconds": round(dt, 2),
                                "cpu": cpu_info(),
                                "sample": f"the {rows} token rows of experts 0..{E // 8 - 1} (oracle.grouped_gemm, fp64)"}
    return line


def bench_forward(torch, mg, idx, steps, warmup, cpu_baseline, fast=False, fp4=False):
    """The MoE forward y = x W_e^T on the expert-grouped GEMM: A = MX(x) along K, B[e] = MXFP8(W_e)
    or, with fp4, MXFP4(W_e) (a8w4); operands quantised on the GPU."""
    inp = wl.make_forward_inputs(idx)
    d = torch.device("cuda:0")
    x = torch.from_numpy(inp["x"]).to(d)
    W = torch.from_numpy(inp["W"]).to(d)
    off = torch.from_numpy(inp["off"]).to(d)
    M, K = x.shape
    E, N, _ = W.shape
    qa, sa = mg.mx_quantize(x)
    if fp4:
        qb, sb = mg.mx4_quantize(W.view(E * N, K))
        qb, sb = qb.view(E, N, K // 2), sb.view(E, N, K // 32)
    else:
        qb, sb = mg.mx_quantize(W.view(E * N, K))
        qb, sb = qb.view(E, N, K), sb.view(E, N, K // 32)
    torch.cuda.synchronize()
    del x, W
    out = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    ms = time_steps(torch, lambda: mg.grouped_mxfp8(qa, qb, sa, sb, off, out=out, fast=fast, b_fp4=fp4),
                    steps, warmup)
    flop = 2.0 * M * N * K
    tf = flop / (ms * 1e-3) / 1e12
    wbytes = N * K // 2 if fp4 else N * K
    nonempty = int(np.count_nonzero(np.diff(inp["off"])))
    nbytes = M * K + M * K // 32 + nonempty * (wbytes + N * K // 32) + 2 * M * N
    name = "a8w4" if fp4 else "forward"
    line = {"metric": f"TFLOP/s, MoE forward y = x W_e^T ({'MXFP4' if fp4 else 'MXFP8'} weights) on workload {idx} (1 GPU)",
            "value": round(tf, 2), "unit": "TFLOP/s", "pct_of_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
            "ms_per_step": round(ms, 4),
            "dtype": (("fp8e4m3*fp4e2m1" if fp4 else "fp8e4m3*fp8e4m3") + "->f32 acc, bf16 out") if fast
                     else ("mxfp8 x mxfp4" if fp4 else "mxfp8 x mxfp8") + " -> bf16 MFMA, f32 acc, bf16 out",
            "mode": "single block-scaled fp8 MFMA pass" if fast else "exact: MX operands converted to bf16, bf16 MFMA",
            "config": {"workload": wl.WORKLOADS[idx].name, "E": E, "M": M, "K_in": K, "N_out": N},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": None if fast else read_traffic(name, idx),
                         "mfma": "v_mfma_scale_f32_32x32x64_f8f6f4 (fp8)" if fast else "v_mfma_f32_32x32x16_bf16",
                         "frac_of_mfma_dtype_peak": round(tf / (PEAK_FP8_TFLOPS if fast else PEAK_BF16_TFLOPS), 4),
                         "algorithmic_bytes": int(nbytes), "algorithmic_flop": flop}}
    bind_roofline(line, flop, nbytes, ms)
    if cpu_baseline:
        import oracle
        rows = int(inp["off"][E // 8])                            # the tokens of the first E/8 experts
        qa_h, sa_h = qa[:rows].cpu().numpy(), sa[:rows].cpu().numpy()
        qb_h, sb_h = qb[: E // 8].cpu().numpy(), sb[: E // 8].cpu().numpy()
        t0 = time.perf_counter()
        oracle.grouped_gemm(qa_h, sa_h, qb_h, sb_h, inp["off"][: E // 8 + 1], b_format="e2m1" if fp4 else "e4m3")
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(2.0 * rows * N * K / dt / 1e12, 4), "unit": "TFLOP/s",
                                "cores": blas_threads(), "kind": "oracle", "seconds": round(dt, 2),
                                "cpu": cpu_info(),
                                "sample": f"the {rows} token rows of experts 0..{E // 8 - 1} (oracle.grouped_gemm, fp64)"}
    return line


def bench_quantize(torch, mg, idx, steps, warmup, cpu_baseline, rule="floor", fp4=False):
    """The MX quantiser on x^T (MXFP8 with the floor or round-up scale rule, or MXFP4)."""
    inp = wl.make_wgrad_inputs(idx)
    d = torch.device("cuda:0")
    x = torch.from_numpy(inp["xT"]).to(d)
    R, L = x.shape
    q = torch.empty((R, L // 2 if fp4 else L), dtype=torch.uint8, device=d)
    s = torch.empty((R, L // 32), dtype=torch.uint8, device=d)
    if fp4:
        ms = time_steps(torch, lambda: mg.mx4_quantize(x, q, s), steps, warmup)
        nbytes = 4 * R * L + R * L // 2 + R * L // 32
    else:
        ms = time_steps(torch, lambda: mg.mx_quantize(x, q, s, rule=rule), steps, warmup)
        nbytes = 4 * R * L + R * L + R * L // 32
    gbs = nbytes / (ms * 1e-3) / 1e9
    what = "MXFP4 quantise" if fp4 else ("MX quantise (round-up scale rule)" if rule == "roundup" else "MX quantise")
    line = {"metric": f"GB/s, {what} of x^T, workload {idx}", "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "dtype": "f32->e2m1+e8m0" if fp4 else "f32->e4m3+e8m0",
            "config": {"workload": wl.WORKLOADS[idx].name, "R": R, "L": L},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
                         "traffic": read_traffic("quantize4" if fp4 else "quantize", idx)
                         if (fp4 or rule == "floor") else None}}
    if cpu_baseline:
        import oracle
        sub = inp["xT"][: max(1, R // 8)]
        t0 = time.perf_counter()
        if fp4:
            oracle.mx4_quantize(sub)
        else:
            oracle.mx_quantize(sub, rule=rule)
        dt = time.perf_counter() - t0
        per_elem = nbytes / (R * L)
        line["cpu_baseline"] = {"value": round(per_elem * sub.size / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "seconds": round(dt, 2), "cpu": cpu_info(),
                                "sample": f"rows 0..{sub.shape[0]} of x^T "
                                          f"({'oracle.mx4_quantize' if fp4 else 'oracle.mx_quantize'})"}
    return line


def bench_quantize_t(torch, mg, idx, steps, warmup, cpu_baseline, rule="floor"):
    """The transposing quantiser on g [M, N] -> g^T codes [N, M] (the weight gradient's A operand)."""
    inp = wl.make_wgrad_inputs(idx)
    d = torch.device("cuda:0")
    g = torch.from_numpy(inp["gT"]).to(d).t().contiguous()           # [M, N] token rows
    del inp
    R, L = g.shape
    q = torch.empty((L, R), dtype=torch.uint8, device=d)
    s = torch.empty((L, R // 32), dtype=torch.uint8, device=d)
    ms = time_steps(torch, lambda: mg.mx_quantize_t(g, q, s, rule=rule), steps, warmup)
    nbytes = 4 * R * L + R * L + R * L // 32
    gbs = nbytes / (ms * 1e-3) / 1e9
    what = "transposing MX quantise (round-up scale rule)" if rule == "roundup" else "transposing MX quantise"
    line = {"metric": f"GB/s, {what} of g, workload {idx}", "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "dtype": "f32->e4m3+e8m0",
            "config": {"workload": wl.WORKLOADS[idx].name, "R": R, "L": L},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic("quantize_t", idx) if rule == "floor" else None}}
    if cpu_baseline:
        import oracle
        sub = g[:, : max(32, L // 8)].cpu().numpy()
        t0 = time.perf_counter()
        oracle.mx_quantize(np.ascontiguousarray(sub.T), rule=rule)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(5.03125 * sub.size / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                "kind": "oracle", "seconds": round(dt, 2), "cpu": cpu_info(),
                                "sample": f"features 0..{sub.shape[1]} of g (oracle.mx_quantize of the transpose)"}
    return line


def bench_copy(torch, mg, idx, steps, warmup, cpu_baseline):
    """A plain device copy of a known size: calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    nbytes = 1 << 30
    d = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=d).fill_(1)
    dst = torch.empty_like(src)
    ms = time_steps(torch, lambda: dst.copy_(src), steps, warmup)
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"metric": "GB/s, device copy of 1 GiB (counter calibration)", "value": round(gbs, 1),
            "unit": "GB/s", "ms_per_step": round(ms, 4), "dtype": "u8",
            "config": {"workload": "copy_1GiB", "bytes": nbytes},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": 2 * nbytes}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--pass", dest="pass_name", choices=["wgrad", "grouped", "forward", "a8w4", "dgrad", "quantize", "quantize_t", "quantize4", "copy"], default="wgrad")
    ap.add_argument("--workload", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fast", action="store_true", help="GEMM passes: the single-pass entry point")
    ap.add_argument("--rule", choices=["floor", "roundup"], default="floor", help="quantise passes: the scale rule")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the kernels run on a single MI355X and the library "
              "has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_gemm_mxfp8_amd as mg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    idx = args.workload or {"wgrad": 4, "grouped": 5, "forward": 5, "a8w4": 5, "dgrad": 5, "quantize": 4,
                            "quantize_t": 4, "quantize4": 4, "copy": 0}[args.pass_name]
    fn = {"wgrad": bench_wgrad, "grouped": bench_grouped, "forward": bench_forward, "a8w4": bench_forward,
          "dgrad": bench_dgrad, "quantize": bench_quantize, "quantize_t": bench_quantize_t,
          "quantize4": bench_quantize, "copy": bench_copy}[args.pass_name]
    kw = {"fast": True} if (args.fast and args.pass_name in ("wgrad", "grouped", "forward", "a8w4")) else {}
    if args.pass_name in ("a8w4", "quantize4"):
        kw["fp4"] = True
    if args.pass_name in ("quantize", "quantize_t") and args.rule != "floor":
        kw["rule"] = args.rule
    line = fn(torch, mg, idx, args.steps, args.warmup, not args.no_cpu_baseline, **kw)
    line.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                 "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                 "data": "synthetic (seeded numpy generators, workload recipe)",
                 "kernel": KERNEL_NAMES.get(args.pass_name, "torch copy"),
                 "kernel_source_digest": source_digest(args.pass_name) if args.pass_name in KERNEL_SOURCES else None})
    if LAUNCH_DIST:
        line["per_launch_ms"] = dict(LAUNCH_DIST)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
