"""Shared helpers of the GPU tests (device transfer, sampling, printing)."""
import os
import sys

import numpy as np
import pytest


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_mxfp8_amd as mg   # fails loudly if the library is missing
    mg._lib.lib()
    return torch, mg


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def say(*args):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()

