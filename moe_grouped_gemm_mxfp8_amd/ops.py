"""torch-tensor wrappers of the C ABI (checks dtypes/devices, passes pointers)."""
from __future__ import annotations

import torch

from ._lib import call

__all__ = ["wgrad_mxfp8", "grouped_mxfp8", "dgrad_f32", "mx_quantize", "mx_quantize_t", "mx4_quantize",
           "mx4_quantize_t", "row_experts"]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/hip) tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_U8 = (torch.uint8, torch.float8_e4m3fn, torch.float8_e8m0fnu) if hasattr(torch, "float8_e8m0fnu") \
    else (torch.uint8, torch.float8_e4m3fn)


def wgrad_mxfp8(a, b, scale_a, scale_b, expert_off, out=None, fast=False):
    """grad_w[E*N, K] (bf16) from g^T codes a[N, M], x^T codes b[K, M], E8M0 scales [.., M/32].

    fast=False: bf16 MFMAs on the exactly converted MX operands (the exact sum up to
    f32-level accumulation error and the bf16 rounding).
    fast=True: the block-scaled fp8 MFMA with the hardware's 8-token truncating reduction.
    """
    _dev(a, "a", _U8); _dev(b, "b", _U8)
    _dev(scale_a, "scale_a", _U8); _dev(scale_b, "scale_b", _U8)
    _dev(expert_off, "expert_off", (torch.int32,))
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("a must be [N, M] and b [K, M]")
    N, M = a.shape
    K = b.shape[0]
    E = expert_off.numel() - 1
    if scale_a.shape != (N, M // 32) or scale_b.shape != (K, M // 32):
        raise ValueError("scales must be [N, M/32] and [K, M/32]")
    if out is None:
        out = torch.empty((E * N, K), dtype=torch.bfloat16, device=a.device)
    _dev(out, "out", (torch.bfloat16,))
    if out.shape != (E * N, K):
        raise ValueError("out must be [E*N, K]")
    call("moe_gg_wgrad_mxfp8_fast" if fast else "moe_gg_wgrad_mxfp8", a.data_ptr(), b.data_ptr(), out.data_ptr(), scale_a.data_ptr(),
         scale_b.data_ptr(), expert_off.data_ptr(), M, N, K, E, _stream())
    return out


def dgrad_f32(g, w, expert_off, out=None):
    """dx[M, K] (f32) = g[M, N] . W[e(r)] with W [E, N, K]."""
    _dev(g, "g", (torch.float32,)); _dev(w, "w", (torch.float32,))
    _dev(expert_off, "expert_off", (torch.int32,))
    if g.dim() != 2 or w.dim() != 3 or w.shape[1] != g.shape[1]:
        raise ValueError("g must be [M, N] and w [E, N, K]")
    M, N = g.shape
    E, _, K = w.shape
    if expert_off.numel() != E + 1:
        raise ValueError("expert_off must have E+1 entries")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=g.device)
    _dev(out, "out", (torch.float32,))
    if out.shape != (M, K):
        raise ValueError("out must be [M, K]")
    call("moe_gg_dgrad_f32", g.data_ptr(), w.data_ptr(), out.data_ptr(), expert_off.data_ptr(),
         M, N, K, E, _stream())
    return out


def grouped_mxfp8(a, b, scale_a, scale_b, expert_off, out=None, fast=False, b_fp4=False):
    """Expert-grouped MX GEMM: out[m] = deq(a)[m] @ deq(b[e(m)]).T as bf16 [M, N].

    a: uint8 E4M3 [M, K]; b: uint8 E4M3 [E, N, K], or with b_fp4 packed E2M1 [E, N, K/2]
    (moe_gg_grouped_a8w4); scale_a [M, K/32], scale_b [E, N, K/32]; expert_off int32 [E+1].
    """
    for t, name in ((a, "a"), (b, "b"), (scale_a, "scale_a"), (scale_b, "scale_b")):
        _dev(t, name, _U8)
    _dev(expert_off, "expert_off", (torch.int32,))
    if a.dim() != 2 or b.dim() != 3 or b.shape[2] * (2 if b_fp4 else 1) != a.shape[1]:
        raise ValueError("a must be [M, K] and b [E, N, K] ([E, N, K/2] packed fp4)")
    M, K = a.shape
    E, N, _ = b.shape
    if scale_a.shape != (M, K // 32) or scale_b.shape != (E, N, K // 32):
        raise ValueError("scale_a must be [M, K/32] and scale_b [E, N, K/32]")
    if expert_off.numel() != E + 1:
        raise ValueError("expert_off must have E+1 entries")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _dev(out, "out", (torch.bfloat16,))
    if out.shape != (M, N):
        raise ValueError("out must be [M, N]")
    name = "moe_gg_grouped_a8w4" if b_fp4 else "moe_gg_grouped_mxfp8"
    call(name + ("_fast" if fast else ""), a.data_ptr(), b.data_ptr(),
         out.data_ptr(), scale_a.data_ptr(), scale_b.data_ptr(), expert_off.data_ptr(), M, N, K, E, _stream())
    return out


_RULES = {"floor": "", "roundup": "_roundup"}


def _rule_suffix(rule):
    if rule not in _RULES:
        raise ValueError("rule must be 'floor' or 'roundup'")
    return _RULES[rule]


def mx_quantize(x, q=None, s=None, rule="floor"):
    """MX-quantise f32 x[R, L] along L: (E4M3 codes uint8 [R, L], E8M0 scales uint8 [R, L/32]).

    rule: "floor" (2^(floor(log2 max) - 8)) or "roundup" (ceil_pow2(max / 448)).
    """
    suffix = _rule_suffix(rule)
    _dev(x, "x", (torch.float32,))
    if x.dim() != 2:
        raise ValueError("x must be [R, L]")
    R, L = x.shape
    if q is None:
        q = torch.empty((R, L), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((R, max(L // 32, 1)), dtype=torch.uint8, device=x.device)
    _dev(q, "q", _U8); _dev(s, "s", _U8)
    if q.shape != (R, L) or s.shape != (R, max(L // 32, 1)):
        raise ValueError("q must be [R, L] and s [R, L/32]")
    call("moe_gg_mx_quantize" + suffix, x.data_ptr(), q.data_ptr(), s.data_ptr(), R, L, _stream())
    return q, s


def mx4_quantize(x, q=None, s=None):
    """MXFP4-quantise f32 x[R, L] along L: (E2M1 codes uint8 [R, L/2], two per byte, E8M0 scales [R, L/32])."""
    _dev(x, "x", (torch.float32,))
    if x.dim() != 2:
        raise ValueError("x must be [R, L]")
    R, L = x.shape
    if q is None:
        q = torch.empty((R, max(L // 2, 1)), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((R, max(L // 32, 1)), dtype=torch.uint8, device=x.device)
    _dev(q, "q", _U8); _dev(s, "s", _U8)
    if q.numel() != R * (L // 2) or s.numel() != R * (L // 32):
        raise ValueError("q must hold R*L/2 bytes and s R*L/32")
    call("moe_gg_mx4_quantize", x.data_ptr(), q.data_ptr(), s.data_ptr(), R, L, _stream())
    return q, s


def mx4_quantize_t(x, q=None, s=None):
    """MXFP4-quantise the transpose of f32 x[R, L] along R: (E2M1 codes uint8 [L, R/2], scales uint8 [L, R/32])."""
    _dev(x, "x", (torch.float32,))
    if x.dim() != 2:
        raise ValueError("x must be [R, L]")
    R, L = x.shape
    if q is None:
        q = torch.empty((L, max(R // 2, 1)), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((L, max(R // 32, 1)), dtype=torch.uint8, device=x.device)
    _dev(q, "q", _U8); _dev(s, "s", _U8)
    if q.numel() != L * (R // 2) or s.numel() != L * (R // 32):
        raise ValueError("q must hold L*R/2 bytes and s L*R/32")
    call("moe_gg_mx4_quantize_t", x.data_ptr(), q.data_ptr(), s.data_ptr(), R, L, _stream())
    return q, s


def mx_quantize_t(x, q=None, s=None, rule="floor"):
    """MX-quantise the transpose of f32 x[R, L] along R: (codes uint8 [L, R], scales uint8 [L, R/32])."""
    suffix = _rule_suffix(rule)
    _dev(x, "x", (torch.float32,))
    if x.dim() != 2:
        raise ValueError("x must be [R, L]")
    R, L = x.shape
    if q is None:
        q = torch.empty((L, R), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((L, max(R // 32, 1)), dtype=torch.uint8, device=x.device)
    _dev(q, "q", _U8); _dev(s, "s", _U8)
    if q.shape != (L, R) or s.shape != (L, max(R // 32, 1)):
        raise ValueError("q must be [L, R] and s [L, R/32]")
    call("moe_gg_mx_quantize_t" + suffix, x.data_ptr(), q.data_ptr(), s.data_ptr(), R, L, _stream())
    return q, s


def row_experts(expert_off, M, out=None):
    """int32 [M]: the expert of each token row (the data-gradient kernel's lookup)."""
    _dev(expert_off, "expert_off", (torch.int32,))
    E = expert_off.numel() - 1
    if out is None:
        out = torch.empty((M,), dtype=torch.int32, device=expert_off.device)
    _dev(out, "out", (torch.int32,))
    if out.numel() != M:
        raise ValueError("out must hold M entries")
    call("moe_gg_row_experts", expert_off.data_ptr(), E, int(M), out.data_ptr(), _stream())
    return out
