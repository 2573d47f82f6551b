"""Build the HIP library libmoe_gg.so for gfx950, in-tree, with hipcc.

Usage: python -m moe_grouped_gemm_mxfp8_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_gg.so")
SOURCES = ["wgrad_mxfp8.hip", "grouped_mxfp8.hip", "dgrad_f32.hip", "mx_quantize.hip", "status.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any generated code.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source into libmoe_gg.so (always recompiles)."""
    cc = hipcc()
    objs = []
    tmpdir = os.path.join(ROOT, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmpdir, src + ".o")
        cmd = [cc, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc, "-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"),
                   "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build_probe() -> str:
    """The single-instruction MFMA probe used by the GPU tests."""
    src = os.path.join(ROOT, "tests", "probes", "mfma_probe.hip")
    out = os.path.join(ROOT, "tests", "probes", "libmfma_probe.so")
    _run([hipcc(), *HIP_FLAGS, "-shared", src, "-o", out])
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())
