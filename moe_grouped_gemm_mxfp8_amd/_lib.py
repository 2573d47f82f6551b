"""ctypes binding of libmoe_gg.so (the C ABI declared in include/moe_gg.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Tensors are torch CUDA (HIP) tensors; the library
sees their device pointers and torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gg.so")

OK, EINVAL, EUNSUPPORTED, ELAUNCH = 0, -1, -2, -3

_lib = None

_VP = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "moe_gg_wgrad_mxfp8": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_wgrad_mxfp8_fast": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_grouped_mxfp8": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_grouped_mxfp8_fast": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_grouped_a8w4": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_grouped_a8w4_fast": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_dgrad_f32": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _VP]),
    "moe_gg_mx_quantize": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "moe_gg_mx_quantize_t": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "moe_gg_mx_quantize_roundup": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "moe_gg_mx4_quantize": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "moe_gg_mx4_quantize_t": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "moe_gg_mx_quantize_t_roundup": (_I, [_VP, _VP, _VP, _I, _I, _VP]),
    "moe_gg_row_experts": (_I, [_VP, _I, _I, _VP, _VP]),
    "moe_gg_status_string": (ctypes.c_char_p, [_I]),
}


class MoeGGError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m moe_grouped_gemm_mxfp8_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().moe_gg_status_string(int(status)).decode()


def call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != OK:
        raise MoeGGError(name, st)
