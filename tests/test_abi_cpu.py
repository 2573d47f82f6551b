"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects invalid arguments on the host before touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_gg.h")
LIB = os.path.join(ROOT, "moe_grouped_gemm_mxfp8_amd", "libmoe_gg.so")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_GG_API\s+[\w\s\*]+?\b(moe_gg_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoe_gg.so not built (run __graft_entry__.build())")
    from moe_grouped_gemm_mxfp8_amd import _lib
    return _lib.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for want in ("moe_gg_wgrad_mxfp8", "moe_gg_wgrad_mxfp8_fast", "moe_gg_grouped_mxfp8",
                 "moe_gg_grouped_mxfp8_fast", "moe_gg_dgrad_f32", "moe_gg_mx_quantize",
                 "moe_gg_mx_quantize_t", "moe_gg_mx_quantize_roundup", "moe_gg_mx_quantize_t_roundup",
                 "moe_gg_grouped_a8w4", "moe_gg_grouped_a8w4_fast", "moe_gg_mx4_quantize", "moe_gg_mx4_quantize_t",
                 "moe_gg_row_experts", "moe_gg_status_string"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else leaks out of the library's namespace
    assert {n for n in exported if n.startswith("moe_gg")} == set(_declared())


def test_binding_signatures_cover_the_header():
    from moe_grouped_gemm_mxfp8_amd import _lib
    assert set(_lib.SIGNATURES) == set(_declared())


def test_status_strings(lib):
    from moe_grouped_gemm_mxfp8_amd import status_string
    assert status_string(0) == "ok"
    for st in (-1, -2, -3, 7):
        assert isinstance(status_string(st), str) and status_string(st)


@pytest.mark.parametrize("name", ["moe_gg_wgrad_mxfp8", "moe_gg_wgrad_mxfp8_fast"])
def test_host_validation_wgrad(lib, name):
    f = getattr(lib, name)
    p = ctypes.c_void_p(16)     # never dereferenced: validation rejects before any launch
    ok = (256, 256, 256, 2)
    assert f(None, p, p, p, p, p, *ok, None) == -1
    assert f(p, p, p, p, p, None, *ok, None) == -1
    assert f(p, p, p, p, p, p, -128, 256, 256, 2, None) == -1
    assert f(p, p, p, p, p, p, 256, 256, 256, 0, None) == -1
    assert f(p, p, p, p, p, p, 80, 256, 256, 2, None) == -1        # M % 32: partial scale block
    assert f(p, p, p, p, p, p, 96, 256, 256, 2, None) == -2        # M % 128: not tiled
    assert f(p, p, p, p, p, p, 256, 200, 256, 2, None) == -2       # N % 256
    assert f(p, p, p, p, p, p, 256, 256, 384, 2, None) == -2       # K % 256
    assert f(p, p, p, p, p, p, 256, 256, 256, 2000, None) == -2    # E above the ranking table
    assert f(p, p, p, p, p, p, 1 << 24, 256, 256, 2, None) == -2    # 256 rows x M beyond 32-bit offsets
    assert f(p, p, p, p, p, p, 256, 256, 1 << 22, 2, None) == -2    # a 256-row bf16 output tile beyond 2^31 B


@pytest.mark.parametrize("name", ["moe_gg_grouped_mxfp8", "moe_gg_grouped_mxfp8_fast", "moe_gg_grouped_a8w4",
                                  "moe_gg_grouped_a8w4_fast"])
def test_host_validation_grouped(lib, name):
    f = getattr(lib, name)
    p = ctypes.c_void_p(16)
    ok = (300, 256, 256, 3)                                         # M need not be a tile multiple
    assert f(None, p, p, p, p, p, *ok, None) == -1
    assert f(p, p, p, p, p, None, *ok, None) == -1
    assert f(p, p, p, p, p, p, -1, 256, 256, 3, None) == -1
    assert f(p, p, p, p, p, p, 300, 256, 256, 0, None) == -1
    assert f(p, p, p, p, p, p, 300, 256, 48, 3, None) == -1        # K % 32
    assert f(p, p, p, p, p, p, 300, 200, 256, 3, None) == -2       # N % 256
    assert f(p, p, p, p, p, p, 300, 256, 160, 3, None) == -2       # K % 128
    assert f(p, p, p, p, p, p, 300, 256, 256, 2049, None) == -2    # E > 2048 (LDS tables)
    assert f(p, p, p, p, p, p, 300, 256, 256, 2048, None) not in (-1, -2)


def test_host_validation_dgrad_quantize_rows(lib):
    p = ctypes.c_void_p(16)
    assert lib.moe_gg_dgrad_f32(None, p, p, p, 8, 8, 8, 1, None) == -1
    assert lib.moe_gg_dgrad_f32(p, p, p, p, 8, -8, 8, 1, None) == -1
    assert lib.moe_gg_dgrad_f32(p, p, p, p, 8, 8, 6, 1, None) == -2
    assert lib.moe_gg_mx_quantize(p, p, None, 4, 64, None) == -1
    assert lib.moe_gg_mx_quantize(p, p, p, 4, 48, None) == -1
    assert lib.moe_gg_mx_quantize(p, p, p, -4, 64, None) == -1
    assert lib.moe_gg_mx_quantize_t(p, p, None, 64, 8, None) == -1
    assert lib.moe_gg_mx_quantize_t(p, p, p, 48, 8, None) == -1      # R % 32
    assert lib.moe_gg_mx_quantize_t(p, p, p, 64, -8, None) == -1
    assert lib.moe_gg_mx_quantize_t(p, p, p, 64, 6, None) == -2      # L % 4
    assert lib.moe_gg_mx_quantize_roundup(p, p, p, 4, 48, None) == -1
    assert lib.moe_gg_mx_quantize_roundup(None, p, p, 4, 64, None) == -1
    assert lib.moe_gg_mx_quantize_t_roundup(p, p, p, 48, 8, None) == -1
    assert lib.moe_gg_mx_quantize_t_roundup(p, p, p, 64, 6, None) == -2
    assert lib.moe_gg_mx4_quantize(p, p, None, 4, 64, None) == -1
    assert lib.moe_gg_mx4_quantize(p, p, p, 4, 48, None) == -1
    assert lib.moe_gg_mx4_quantize(p, p, p, -4, 64, None) == -1
    assert lib.moe_gg_mx4_quantize_t(p, p, None, 64, 8, None) == -1
    assert lib.moe_gg_mx4_quantize_t(p, p, p, 48, 8, None) == -1     # R % 32
    assert lib.moe_gg_mx4_quantize_t(p, p, p, 64, 6, None) == -2     # L % 4
    assert lib.moe_gg_row_experts(p, 0, 10, p, None) == -1
    assert lib.moe_gg_row_experts(None, 2, 10, p, None) == -1


def test_empty_outputs_return_ok_without_a_launch(lib):
    """A call with no output element returns 0 before any HIP call (so also
    here, without a GPU); pointers to zero-size buffers may be NULL, the
    offsets may not; negative sizes stay invalid."""
    p = ctypes.c_void_p(16)
    for name in ("moe_gg_wgrad_mxfp8", "moe_gg_wgrad_mxfp8_fast"):
        f = getattr(lib, name)
        assert f(None, None, None, None, None, p, 256, 0, 256, 2, None) == 0       # N = 0
        assert f(None, None, None, None, None, p, 256, 256, 0, 2, None) == 0       # K = 0
        assert f(None, None, None, None, None, None, 256, 0, 256, 2, None) == -1   # offsets still required
        assert f(None, None, None, None, None, p, 256, -256, 256, 2, None) == -1
        assert f(p, p, None, p, p, p, 0, 256, 256, 2, None) == -1                  # M = 0 writes C: C required
    for name in ("moe_gg_grouped_mxfp8", "moe_gg_grouped_mxfp8_fast", "moe_gg_grouped_a8w4",
                 "moe_gg_grouped_a8w4_fast"):
        f = getattr(lib, name)
        assert f(None, None, None, None, None, p, 0, 256, 256, 3, None) == 0       # M = 0
        assert f(None, None, None, None, None, p, 300, 0, 256, 3, None) == 0       # N = 0
        assert f(None, None, None, None, None, None, 0, 256, 256, 3, None) == -1
        assert f(p, p, p, p, p, p, 300, 256, -32, 3, None) == -1
        assert f(None, None, None, None, None, p, 300, 256, 0, 3, None) == -1      # K = 0 writes C: C required
    assert lib.moe_gg_dgrad_f32(None, None, None, p, 0, 8, 8, 1, None) == 0       # M = 0
    assert lib.moe_gg_dgrad_f32(None, None, None, p, 8, 8, 0, 1, None) == 0       # K = 0
    assert lib.moe_gg_dgrad_f32(None, None, None, None, 0, 8, 8, 1, None) == -1
    assert lib.moe_gg_dgrad_f32(None, None, None, p, 8, 0, 8, 1, None) == -1      # N = 0 writes dx: dx required
    for name in ("moe_gg_mx_quantize", "moe_gg_mx_quantize_roundup", "moe_gg_mx4_quantize",
                 "moe_gg_mx_quantize_t", "moe_gg_mx_quantize_t_roundup", "moe_gg_mx4_quantize_t"):
        f = getattr(lib, name)
        assert f(None, None, None, 0, 64, None) == 0
        assert f(None, None, None, 64, 0, None) == 0
        assert f(None, None, None, 0, 0, None) == 0
        assert f(None, None, None, -32, 64, None) == -1
    assert lib.moe_gg_row_experts(p, 2, 0, None, None) == 0
    assert lib.moe_gg_row_experts(p, 2, -1, p, None) == -1
    assert lib.moe_gg_row_experts(None, 2, 0, None, None) == -1


def test_python_binding_refuses_cpu_tensors():
    import torch
    import moe_grouped_gemm_mxfp8_amd as mg
    with pytest.raises(ValueError):
        mg.mx_quantize(torch.zeros(4, 64))
    with pytest.raises(ValueError):
        mg.mx_quantize_t(torch.zeros(64, 4))
    with pytest.raises(ValueError):
        mg.dgrad_f32(torch.zeros(4, 4), torch.zeros(1, 4, 4), torch.zeros(2, dtype=torch.int32))
