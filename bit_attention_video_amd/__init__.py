"""VC-Attention hot path on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libvcattn.so, whose C ABI is declared in include/vc_attn.h.
This module only marshals arguments: it checks dtypes, shapes and devices of torch
tensors, allocates outputs and workspaces with torch, and passes raw device pointers and
torch's current HIP stream to the library.  Every step of the method runs in the HIP
kernels; there is no CPU or PyTorch fallback, and a missing library is an error.

Entry points (same names as the C ABI):
  vc_vsmooth_group         k-means grouping + stable label sort (Sec. 3.2, Eq. 3)
  vc_vsmooth_demean_quant  K smoothing, V block demeaning, E4M3 operands (Eq. 4, App. B)
  vc_attn_fwd              FP8 attention with ExpCast-FP8 and mean restore (Eq. 1, 6, 7)
  vc_test_*                single-stage hooks for testing
plus vc_attention(Q, K, V, perm), which chains demean_quant and attn_fwd.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = ["VCError", "lib", "vc_vsmooth_group", "vc_vsmooth_demean_quant", "vc_attn_fwd",
           "vc_attention", "vc_vsmooth_demean_quant_mx4", "vc_attn_fwd_mx4", "vc_attention_mx4",
           "vc_test_fp4_encode", "vc_test_mfma_fp8_rate", "unpack_fp4", "pack_fp4", "vc_test_expcast", "vc_test_e4m3_encode", "vc_test_kmeans_assign",
           "vc_test_label_sort", "rq_tiled_to_natural", "rq_natural_to_tiled", "LIB_PATH",
           "VC_ATTN_NO_MEAN", "VC_ATTN_EXP_THEN_CAST", "VC_ATTN_HADAMARD", "VC_DQ_NO_DEMEAN",
           "VC_DQ_HADAMARD", "STATUS", "vc_workspace_size", "vc_validate_perm", "vc_test_quantize_q",
           "vc_test_attn_fwd_clock", "VC_OP_GROUP", "VC_OP_DEMEAN_QUANT", "VC_OP_DEMEAN_QUANT_MX4",
           "VC_OP_ATTN_FWD", "VC_OP_ATTN_FWD_MX4", "VC_OP_VALIDATE_PERM", "wall_clock_mhz",
           "vc_vsmooth_group_static", "vc_vsmooth_demean_quant_mx6", "vc_attn_fwd_mx6", "vc_attention_mx6",
           "vc_test_fp6_encode", "unpack_fp6", "pack_fp6", "VC_OP_DEMEAN_QUANT_MX6", "VC_OP_ATTN_FWD_MX6"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvcattn.so")

VC_ATTN_NO_MEAN = 0x1
VC_ATTN_EXP_THEN_CAST = 0x2
VC_ATTN_HADAMARD = 0x4
VC_DQ_NO_DEMEAN = 0x1
VC_DQ_HADAMARD = 0x2
VC_OP_GROUP = 1
VC_OP_DEMEAN_QUANT = 2
VC_OP_DEMEAN_QUANT_MX4 = 3
VC_OP_ATTN_FWD = 4
VC_OP_ATTN_FWD_MX4 = 5
VC_OP_VALIDATE_PERM = 6
VC_OP_DEMEAN_QUANT_MX6 = 7
VC_OP_ATTN_FWD_MX6 = 8
STATUS = {"VC_OK": 0, "VC_ERR_NULL": -1, "VC_ERR_SHAPE": -2, "VC_ERR_K": -3, "VC_ERR_ITERS": -4,
          "VC_ERR_WORKSPACE": -5, "VC_ERR_OVERFLOW": -6, "VC_ERR_FLAGS": -7, "VC_ERR_HIP": -8}

_P = ctypes.c_void_p
_I = ctypes.c_int
_U = ctypes.c_uint
_Z = ctypes.c_size_t
_F = ctypes.c_float

_SIGNATURES = {
    "vc_strerror": (ctypes.c_char_p, [_I]),
    "vc_last_hip_error": (_I, []),
    "vc_group_workspace_size": (_Z, [_I, _I, _I, _I]),
    "vc_vsmooth_group": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "vc_demean_quant_workspace_size": (_Z, [_I, _I, _I]),
    "vc_vsmooth_demean_quant": (_I, [_P, _P, _P, _I, _I, _I, _I, _U, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "vc_attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P]),
    "vc_vsmooth_demean_quant_mx4": (_I, [_P, _P, _P, _I, _I, _I, _I, _U, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "vc_attn_fwd_mx4": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P]),
    "vc_vsmooth_demean_quant_mx6": (_I, [_P, _P, _P, _I, _I, _I, _I, _U, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "vc_attn_fwd_mx6": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P]),
    "vc_test_fp4_encode": (_I, [_P, _P, _Z, _P]),
    "vc_test_fp6_encode": (_I, [_P, _P, _P, _Z, _P]),
    "vc_test_mfma_fp8_rate": (_I, [_P, _I, _I, _P, _P]),
    "vc_test_expcast": (_I, [_P, _P, _Z, _P]),
    "vc_test_e4m3_encode": (_I, [_P, _P, _Z, _P]),
    "vc_test_kmeans_assign": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "vc_test_label_sort": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "vc_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "vc_vsmooth_group_static": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "vc_validate_perm": (_I, [_P, _I, _I, _I, _P, _P, _Z, _P]),
    "vc_test_quantize_q": (_I, [_P, _I, _I, _I, _I, _F, _U, _P, _P, _P]),
    "vc_test_attn_clock_slots": (_Z, [_I, _I, _I]),
    "vc_test_wall_clock_khz": (_I, [ctypes.POINTER(_I)]),
    "vc_test_attn_fwd_clock": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _U, _P, _P, _P]),
}

_lib = None


class VCError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().vc_strerror(status).decode()
        if status == STATUS["VC_ERR_HIP"]:
            msg += f" (hipError_t {lib().vc_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


def lib() -> ctypes.CDLL:
    """Load libvcattn.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != 0:
        raise VCError(rc, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _bhnd(x: torch.Tensor, name: str):
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    _need(x, name, torch.bfloat16)
    return tuple(x.shape)


def vc_vsmooth_group(V: torch.Tensor, k: int, iters: int, C_init: Optional[torch.Tensor] = None,
                     objective: bool = True):
    """k-means grouping of value tokens and pi = stable argsort(labels) (Sec. 3.2, Eq. 3)."""
    B, H, N, d = _bhnd(V, "V")
    dev = V.device
    if C_init is not None:
        _need(C_init, "C_init", torch.float32, (B, H, k, d))
    C = torch.empty((B, H, k, d), dtype=torch.float32, device=dev)
    labels = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    offsets = torch.empty((B, H, k + 1), dtype=torch.int32, device=dev)
    J = torch.empty((B, H), dtype=torch.float64, device=dev) if objective else None
    nws = lib().vc_group_workspace_size(B, H, N, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _check(lib().vc_vsmooth_group(_ptr(V), B, H, N, d, k, iters, _ptr(C_init), _ptr(C), _ptr(labels),
                                  _ptr(perm), _ptr(offsets), _ptr(J), _ptr(ws), nws, _stream()),
           "vc_vsmooth_group")
    return {"C": C, "labels": labels, "perm": perm, "offsets": offsets, "J": J}


def vc_vsmooth_group_static(V: torch.Tensor, k: int, iters: int, C_init: Optional[torch.Tensor] = None,
                            objective: bool = True):
    """vc_vsmooth_group on the library's own device scratch: the library allocates nothing (the
    outputs are the caller's).  Calls overlapping on one GPU race on that scratch."""
    B, H, N, d = _bhnd(V, "V")
    dev = V.device
    if C_init is not None:
        _need(C_init, "C_init", torch.float32, (B, H, k, d))
    C = torch.empty((B, H, k, d), dtype=torch.float32, device=dev)
    labels = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    offsets = torch.empty((B, H, k + 1), dtype=torch.int32, device=dev)
    J = torch.empty((B, H), dtype=torch.float64, device=dev) if objective else None
    _check(lib().vc_vsmooth_group_static(_ptr(V), B, H, N, d, k, iters, _ptr(C_init), _ptr(C), _ptr(labels),
                                         _ptr(perm), _ptr(offsets), _ptr(J), _stream()), "vc_vsmooth_group_static")
    return {"C": C, "labels": labels, "perm": perm, "offsets": offsets, "J": J}


def vc_vsmooth_demean_quant(K: torch.Tensor, V: torch.Tensor, perm: Optional[torch.Tensor] = None,
                            no_demean: bool = False, hadamard: bool = False):
    """E4M3 operands of the VC path from bf16 K, V and pi (Sec. 3.2, Eq. 4; App. B).

    hadamard=True quantises the rotated keys (K[pi] - kbar) H with the scale divided by 128."""
    B, H, N, d = _bhnd(K, "K")
    _need(V, "V", torch.bfloat16, (B, H, N, d))
    if perm is not None:
        _need(perm, "perm", torch.int32, (B, H, N))
    dev = K.device
    T = N // 128 if N % 128 == 0 else 0
    Kq = torch.empty((B, H, N, d), dtype=torch.uint8, device=dev)
    sK = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    Rq = torch.empty((B, H, T, d, 128), dtype=torch.uint8, device=dev)
    mu = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    sV = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    nws = lib().vc_demean_quant_workspace_size(B, H, N)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    flags = (VC_DQ_NO_DEMEAN if no_demean else 0) | (VC_DQ_HADAMARD if hadamard else 0)
    _check(lib().vc_vsmooth_demean_quant(_ptr(K), _ptr(V), _ptr(perm), B, H, N, d, flags, _ptr(Kq), _ptr(sK),
                                         _ptr(Rq), _ptr(mu), _ptr(sV), _ptr(ws), nws, _stream()),
           "vc_vsmooth_demean_quant")
    return {"Kq": Kq, "sK": sK, "Rq": Rq, "mu": mu, "sV": sV}


def vc_attn_fwd(Q: torch.Tensor, Kq: torch.Tensor, sK: torch.Tensor, Rq: torch.Tensor,
                mu: Optional[torch.Tensor], sV: torch.Tensor, softmax_scale: float = 0.0,
                no_mean: bool = False, out: Optional[torch.Tensor] = None,
                exp_then_cast: bool = False, hadamard: bool = False) -> torch.Tensor:
    """FP8 attention with ExpCast-FP8 (or exp-then-cast P) and the online mean restore (Eq. 1, 6, 7).

    hadamard=True rotates the queries by H before quantising them; the keys must then come from
    vc_vsmooth_demean_quant(..., hadamard=True)."""
    B, H, N, d = _bhnd(Q, "Q")
    T = N // 128 if N % 128 == 0 else 0
    _need(Kq, "Kq", torch.uint8, (B, H, N, d))
    _need(sK, "sK", torch.float32, (B, H, T))
    _need(Rq, "Rq", torch.uint8, (B, H, T, d, 128))
    if mu is not None or not no_mean:
        _need(mu, "mu", torch.bfloat16, (B, H, T, d))
    _need(sV, "sV", torch.float32, (B, H, d))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=Q.device)
    else:
        _need(out, "out", torch.bfloat16, (B, H, N, d))
    flags = ((VC_ATTN_NO_MEAN if no_mean else 0) | (VC_ATTN_EXP_THEN_CAST if exp_then_cast else 0)
             | (VC_ATTN_HADAMARD if hadamard else 0))
    _check(lib().vc_attn_fwd(_ptr(Q), _ptr(Kq), _ptr(sK), _ptr(Rq), _ptr(mu), _ptr(sV), B, H, N, d,
                             float(softmax_scale), flags, _ptr(out), _stream()), "vc_attn_fwd")
    return out


def vc_attention(Q, K, V, perm=None, softmax_scale: float = 0.0, no_demean: bool = False,
                 hadamard: bool = False):
    """demean_quant then attn_fwd: O = attention(Q, K, V) on the VC path for a given pi."""
    ops = vc_vsmooth_demean_quant(K, V, perm, no_demean=no_demean, hadamard=hadamard)
    return vc_attn_fwd(Q, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"], softmax_scale,
                       no_mean=no_demean, hadamard=hadamard)


def vc_workspace_size(op: int, B: int, H: int, N: int, d: int = 128, k: int = 1) -> int:
    """Scratch bytes the call `op` (VC_OP_*) needs for this shape."""
    return int(lib().vc_workspace_size(op, B, H, N, d, k))


def vc_validate_perm(perm: torch.Tensor) -> torch.Tensor:
    """Per (b, h): entries of pi outside [0, N) plus repeats (0 = a permutation), as int32 [B, H]."""
    if perm.dim() != 3:
        raise ValueError("perm must be [B, H, N]")
    _need(perm, "perm", torch.int32)
    B, H, N = perm.shape
    bad = torch.empty((B, H), dtype=torch.int32, device=perm.device)
    nws = vc_workspace_size(VC_OP_VALIDATE_PERM, B, H, N)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=perm.device)
    _check(lib().vc_validate_perm(_ptr(perm), B, H, N, _ptr(bad), _ptr(ws), nws, _stream()), "vc_validate_perm")
    return bad


def vc_test_quantize_q(Q: torch.Tensor, softmax_scale: float = 0.0, hadamard: bool = False):
    """The attention kernel's query prologue alone: (E4M3 codes [B,H,N,d], block scales [B,H,N/128])."""
    B, H, N, d = _bhnd(Q, "Q")
    Qq = torch.empty((B, H, N, d), dtype=torch.uint8, device=Q.device)
    sQ = torch.empty((B, H, N // 128 if N % 128 == 0 else 0), dtype=torch.float32, device=Q.device)
    _check(lib().vc_test_quantize_q(_ptr(Q), B, H, N, d, float(softmax_scale), VC_ATTN_HADAMARD if hadamard else 0,
                                    _ptr(Qq), _ptr(sQ), _stream()), "vc_test_quantize_q")
    return Qq, sQ


def vc_test_attn_fwd_clock(Q, Kq, sK, Rq, mu, sV, softmax_scale: float = 0.0, no_mean: bool = False,
                           out: Optional[torch.Tensor] = None, clk: Optional[torch.Tensor] = None):
    """vc_attn_fwd's kernel with its clock stamps on.  Returns (O, clk) with clk int64
    [workgroups, 4] = (start cycles, start ticks, end cycles, end ticks) per workgroup."""
    B, H, N, d = _bhnd(Q, "Q")
    T = N // 128 if N % 128 == 0 else 0
    _need(Kq, "Kq", torch.uint8, (B, H, N, d))
    _need(sK, "sK", torch.float32, (B, H, T))
    _need(Rq, "Rq", torch.uint8, (B, H, T, d, 128))
    if mu is not None or not no_mean:
        _need(mu, "mu", torch.bfloat16, (B, H, T, d))
    _need(sV, "sV", torch.float32, (B, H, d))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=Q.device)
    n = int(lib().vc_test_attn_clock_slots(B, H, N))
    if clk is None:
        clk = torch.zeros((max(n, 4) // 4, 4), dtype=torch.int64, device=Q.device)
    _need(clk, "clk", torch.int64, (n // 4, 4))
    _check(lib().vc_test_attn_fwd_clock(_ptr(Q), _ptr(Kq), _ptr(sK), _ptr(Rq), _ptr(mu), _ptr(sV), B, H, N, d,
                                        float(softmax_scale), VC_ATTN_NO_MEAN if no_mean else 0, _ptr(out),
                                        _ptr(clk), _stream()), "vc_test_attn_fwd_clock")
    return out, clk


def wall_clock_mhz() -> float:
    """Frequency of the device's constant-rate counter (the clock probe's time base), in MHz."""
    khz = _I(0)
    _check(lib().vc_test_wall_clock_khz(ctypes.byref(khz)), "vc_test_wall_clock_khz")
    return khz.value * 1e-3


def vc_vsmooth_demean_quant_mx4(K: torch.Tensor, V: torch.Tensor, perm: Optional[torch.Tensor] = None,
                                no_demean: bool = False, hadamard: bool = False):
    """4-bit (MX E2M1, per-32 E8M0 scales) operands of the VC path (Sec. 3.2 Eq. 4; App. B)."""
    B, H, N, d = _bhnd(K, "K")
    _need(V, "V", torch.bfloat16, (B, H, N, d))
    if perm is not None:
        _need(perm, "perm", torch.int32, (B, H, N))
    dev = K.device
    T = N // 128 if N % 128 == 0 else 0
    Kq4 = torch.empty((B, H, N, d // 2), dtype=torch.uint8, device=dev)
    sK4 = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device=dev)
    Rq4 = torch.empty((B, H, T, d, 64), dtype=torch.uint8, device=dev)
    sR4 = torch.empty((B, H, T, d, 4), dtype=torch.uint8, device=dev)
    mu = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    nws = lib().vc_demean_quant_workspace_size(B, H, N)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    flags = (VC_DQ_NO_DEMEAN if no_demean else 0) | (VC_DQ_HADAMARD if hadamard else 0)
    _check(lib().vc_vsmooth_demean_quant_mx4(_ptr(K), _ptr(V), _ptr(perm), B, H, N, d, flags, _ptr(Kq4),
                                             _ptr(sK4), _ptr(Rq4), _ptr(sR4), _ptr(mu), _ptr(ws), nws, _stream()),
           "vc_vsmooth_demean_quant_mx4")
    return {"Kq4": Kq4, "sK4": sK4, "Rq4": Rq4, "sR4": sR4, "mu": mu}


def vc_attn_fwd_mx4(Q: torch.Tensor, Kq4: torch.Tensor, sK4: torch.Tensor, Rq4: torch.Tensor,
                    sR4: torch.Tensor, mu: Optional[torch.Tensor], softmax_scale: float = 0.0,
                    no_mean: bool = False, hadamard: bool = False,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """4-bit attention: MX E2M1 Q, K, P and residual, P = 2^(S L4 - m), mean restore (Eq. 1, 6)."""
    B, H, N, d = _bhnd(Q, "Q")
    T = N // 128 if N % 128 == 0 else 0
    _need(Kq4, "Kq4", torch.uint8, (B, H, N, d // 2))
    _need(sK4, "sK4", torch.uint8, (B, H, N, d // 32))
    _need(Rq4, "Rq4", torch.uint8, (B, H, T, d, 64))
    _need(sR4, "sR4", torch.uint8, (B, H, T, d, 4))
    if mu is not None or not no_mean:
        _need(mu, "mu", torch.bfloat16, (B, H, T, d))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=Q.device)
    else:
        _need(out, "out", torch.bfloat16, (B, H, N, d))
    flags = (VC_ATTN_NO_MEAN if no_mean else 0) | (VC_ATTN_HADAMARD if hadamard else 0)
    _check(lib().vc_attn_fwd_mx4(_ptr(Q), _ptr(Kq4), _ptr(sK4), _ptr(Rq4), _ptr(sR4), _ptr(mu), B, H, N, d,
                                 float(softmax_scale), flags, _ptr(out), _stream()), "vc_attn_fwd_mx4")
    return out


def vc_vsmooth_demean_quant_mx6(K: torch.Tensor, V: torch.Tensor, perm: Optional[torch.Tensor] = None,
                                no_demean: bool = False, hadamard: bool = False):
    """6-bit (MX E2M3, per-32 E8M0 scales, 32-byte groups) operands of the VC path."""
    B, H, N, d = _bhnd(K, "K")
    _need(V, "V", torch.bfloat16, (B, H, N, d))
    if perm is not None:
        _need(perm, "perm", torch.int32, (B, H, N))
    dev = K.device
    T = N // 128 if N % 128 == 0 else 0
    Kq6 = torch.empty((B, H, N, d), dtype=torch.uint8, device=dev)
    sK6 = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device=dev)
    Rq6 = torch.empty((B, H, T, d, 128), dtype=torch.uint8, device=dev)
    sR6 = torch.empty((B, H, T, d, 4), dtype=torch.uint8, device=dev)
    mu = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    nws = lib().vc_demean_quant_workspace_size(B, H, N)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    flags = (VC_DQ_NO_DEMEAN if no_demean else 0) | (VC_DQ_HADAMARD if hadamard else 0)
    _check(lib().vc_vsmooth_demean_quant_mx6(_ptr(K), _ptr(V), _ptr(perm), B, H, N, d, flags, _ptr(Kq6),
                                             _ptr(sK6), _ptr(Rq6), _ptr(sR6), _ptr(mu), _ptr(ws), nws, _stream()),
           "vc_vsmooth_demean_quant_mx6")
    return {"Kq6": Kq6, "sK6": sK6, "Rq6": Rq6, "sR6": sR6, "mu": mu}


def vc_attn_fwd_mx6(Q: torch.Tensor, Kq6: torch.Tensor, sK6: torch.Tensor, Rq6: torch.Tensor,
                    sR6: torch.Tensor, mu: Optional[torch.Tensor], softmax_scale: float = 0.0,
                    no_mean: bool = False, hadamard: bool = False,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """6-bit attention: MX E2M3 Q, K, P and residual, P = 2^(S L4 - m), mean restore (Eq. 1, 6)."""
    B, H, N, d = _bhnd(Q, "Q")
    T = N // 128 if N % 128 == 0 else 0
    _need(Kq6, "Kq6", torch.uint8, (B, H, N, d))
    _need(sK6, "sK6", torch.uint8, (B, H, N, d // 32))
    _need(Rq6, "Rq6", torch.uint8, (B, H, T, d, 128))
    _need(sR6, "sR6", torch.uint8, (B, H, T, d, 4))
    if mu is not None or not no_mean:
        _need(mu, "mu", torch.bfloat16, (B, H, T, d))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=Q.device)
    else:
        _need(out, "out", torch.bfloat16, (B, H, N, d))
    flags = (VC_ATTN_NO_MEAN if no_mean else 0) | (VC_ATTN_HADAMARD if hadamard else 0)
    _check(lib().vc_attn_fwd_mx6(_ptr(Q), _ptr(Kq6), _ptr(sK6), _ptr(Rq6), _ptr(sR6), _ptr(mu), B, H, N, d,
                                 float(softmax_scale), flags, _ptr(out), _stream()), "vc_attn_fwd_mx6")
    return out


def vc_attention_mx6(Q, K, V, perm=None, softmax_scale: float = 0.0, no_demean: bool = False,
                     hadamard: bool = False):
    """6-bit demean_quant then 6-bit attention for a given pi."""
    ops = vc_vsmooth_demean_quant_mx6(K, V, perm, no_demean=no_demean, hadamard=hadamard)
    return vc_attn_fwd_mx6(Q, ops["Kq6"], ops["sK6"], ops["Rq6"], ops["sR6"], ops["mu"], softmax_scale,
                           no_mean=no_demean, hadamard=hadamard)


def vc_test_fp6_encode(x: torch.Tensor, scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Words 6i .. 6i+5 (int32) = E2M3 codes of x[32i .. 32i+31] (value k in bits 6k .. 6k+5),
    converted with scale[i] as the conversion's scale operand when given."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or x.numel() % 32:
        raise ValueError("x must be a contiguous float32 device tensor of a multiple of 32 values")
    n = x.numel() // 32
    if scale is not None:
        _need(scale, "scale", torch.float32, (n,))
    out = torch.empty(6 * n, dtype=torch.int32, device=x.device)
    _check(lib().vc_test_fp6_encode(_ptr(x), _ptr(scale), _ptr(out), n, _stream()), "vc_test_fp6_encode")
    return out


def _fp6_fields(codes: np.ndarray) -> np.ndarray:
    """E2M3 codes [..., 32 g] -> the 24-byte fields [..., g, 24]: value k in bits 6k .. 6k+5."""
    g = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 32, 32))
    bits = ((g[..., None] >> np.arange(6, dtype=np.uint8)) & 1).astype(np.uint8).reshape(g.shape[:-1] + (192,))
    return np.packbits(bits, axis=-1, bitorder="little")


def _fp6_codes(fields: np.ndarray) -> np.ndarray:
    """24-byte fields [..., g, 24] -> E2M3 codes [..., 32 g]."""
    bits = np.unpackbits(fields, axis=-1, bitorder="little").reshape(fields.shape[:-1] + (32, 6))
    codes = (bits << np.arange(6, dtype=np.uint8)).sum(-1).astype(np.uint8)
    return codes.reshape(fields.shape[:-2] + (fields.shape[-2] * 32,))


# Byte offsets in a 6-bit row of 128 bytes (four groups): group g's first 16 code bytes at 16 g,
# its last 8 at 64 + 16 (g % 2) + 8 (g // 2); bytes 96 .. 127 are zero.
_FP6_HEAD = [16 * g for g in range(4)]
_FP6_TAIL = [64 + 16 * (g % 2) + 8 * (g // 2) for g in range(4)]


def unpack_fp6(b) -> np.ndarray:
    """The 6-bit layout -> E2M3 codes uint8.  A last axis that is a multiple of 128 is read as the
    operand rows of vc_vsmooth_demean_quant_mx6 (128 bytes per four groups, see _FP6_HEAD/_TAIL);
    a last axis of 24 code bytes per group (vc_test_fp6_encode's words) as plain fields.  Value k of
    a group is in bits 6k .. 6k+5 of its 192-bit little-endian field."""
    a = b.cpu().numpy() if isinstance(b, torch.Tensor) else np.asarray(b)
    a = a.astype(np.uint8)
    n = a.shape[-1]
    if n % 128 == 0:
        r = a.reshape(a.shape[:-1] + (n // 128, 128))
        f = np.stack([np.concatenate([r[..., h:h + 16], r[..., t:t + 8]], axis=-1)
                      for h, t in zip(_FP6_HEAD, _FP6_TAIL)], axis=-2)          # [..., rows, 4, 24]
        return _fp6_codes(f.reshape(a.shape[:-1] + (4 * (n // 128), 24)))
    if n % 24 == 0:
        return _fp6_codes(a.reshape(a.shape[:-1] + (n // 24, 24)))
    raise ValueError(f"6-bit data with a last axis of {n} bytes (need a multiple of 128 or of 24)")


def pack_fp6(codes) -> np.ndarray:
    """E2M3 codes uint8 [..., 128 r] -> the operand rows of vc_vsmooth_demean_quant_mx6 uint8
    [..., 128 r] (per row of four groups: the first 16 code bytes of group g at 16 g, its last 8 at
    64 + 16 (g % 2) + 8 (g // 2), zero bytes 96 .. 127)."""
    c = codes.cpu().numpy() if isinstance(codes, torch.Tensor) else np.asarray(codes)
    c = c.astype(np.uint8)
    n = c.shape[-1]
    if n % 128:
        raise ValueError(f"6-bit rows need a last axis that is a multiple of 128 codes, got {n}")
    f = _fp6_fields(c).reshape(c.shape[:-1] + (n // 128, 4, 24))
    out = np.zeros(c.shape[:-1] + (n // 128, 128), np.uint8)
    for g, (h, t) in enumerate(zip(_FP6_HEAD, _FP6_TAIL)):
        out[..., h:h + 16] = f[..., g, :16]
        out[..., t:t + 8] = f[..., g, 16:]
    return out.reshape(c.shape)


def vc_attention_mx4(Q, K, V, perm=None, softmax_scale: float = 0.0, no_demean: bool = False,
                     hadamard: bool = False):
    """4-bit demean_quant then 4-bit attention for a given pi."""
    ops = vc_vsmooth_demean_quant_mx4(K, V, perm, no_demean=no_demean, hadamard=hadamard)
    return vc_attn_fwd_mx4(Q, ops["Kq4"], ops["sK4"], ops["Rq4"], ops["sR4"], ops["mu"], softmax_scale,
                           no_mean=no_demean, hadamard=hadamard)


def vc_test_fp4_encode(x: torch.Tensor) -> torch.Tensor:
    """Byte i = E2M1 codes of (x[2i], x[2i+1]), x[2i] in the low nibble."""
    _need(x, "x", torch.float32)
    n = x.numel()
    codes = torch.empty(n // 2, dtype=torch.uint8, device=x.device)
    _check(lib().vc_test_fp4_encode(_ptr(x), _ptr(codes), n, _stream()), "vc_test_fp4_encode")
    return codes


def vc_test_mfma_fp8_rate(workgroups: int, iters: int, device="cuda", clock: bool = False):
    """Dense FP8 matrix-instruction loop (workgroups x iters x 4,194,304 FLOP); time it on the
    current stream to get the attainable FP8 rate.  Returns the per-thread outputs, and with
    clock=True also the shader clock (MHz) each workgroup's first wave sustained in its loop."""
    out = torch.empty(workgroups * 512, dtype=torch.float32, device=device)
    mhz = torch.empty(workgroups, dtype=torch.float32, device=device) if clock else None
    _check(lib().vc_test_mfma_fp8_rate(_ptr(out), workgroups, iters, _ptr(mhz) if clock else None, _stream()),
           "vc_test_mfma_fp8_rate")
    return (out, mhz) if clock else out


def vc_test_expcast(u: torch.Tensor) -> torch.Tensor:
    _need(u, "u", torch.float32)
    codes = torch.empty(u.shape, dtype=torch.uint8, device=u.device)
    _check(lib().vc_test_expcast(_ptr(u), _ptr(codes), u.numel(), _stream()), "vc_test_expcast")
    return codes


def vc_test_e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    _need(x, "x", torch.float32)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().vc_test_e4m3_encode(_ptr(x), _ptr(codes), x.numel(), _stream()), "vc_test_e4m3_encode")
    return codes


def vc_test_kmeans_assign(V: torch.Tensor, C: torch.Tensor):
    B, H, N, d = _bhnd(V, "V")
    k = C.shape[2]
    _need(C, "C", torch.float32, (B, H, k, d))
    labels = torch.empty((B, H, N), dtype=torch.int32, device=V.device)
    dist = torch.empty((B, H, N), dtype=torch.float32, device=V.device)
    nws = lib().vc_group_workspace_size(B, H, N, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=V.device)
    _check(lib().vc_test_kmeans_assign(_ptr(V), _ptr(C), B, H, N, d, k, _ptr(labels), _ptr(dist), _ptr(ws),
                                       nws, _stream()), "vc_test_kmeans_assign")
    return labels, dist


def vc_test_label_sort(labels: torch.Tensor, k: int):
    if labels.dim() != 3:
        raise ValueError("labels must be [B, H, N]")
    _need(labels, "labels", torch.int32)
    B, H, N = labels.shape
    perm = torch.empty((B, H, N), dtype=torch.int32, device=labels.device)
    offsets = torch.empty((B, H, k + 1), dtype=torch.int32, device=labels.device)
    nws = lib().vc_group_workspace_size(B, H, N, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=labels.device)
    _check(lib().vc_test_label_sort(_ptr(labels), B, H, N, k, _ptr(perm), _ptr(offsets), _ptr(ws), nws,
                                    _stream()), "vc_test_label_sort")
    return perm, offsets


# ---- layout of the tile-transposed residual operand (include/vc_attn.h, Rq) ----

def _key_of_slot() -> np.ndarray:
    s = np.arange(128)
    p, g, i = s // 64, (s // 32) % 2, s % 32
    return 64 * p + 32 * (i // 16) + 8 * ((i % 16) // 4) + 4 * g + (i % 4)


KEY_OF_SLOT = _key_of_slot()
SLOT_OF_KEY = np.argsort(KEY_OF_SLOT)


def rq_tiled_to_natural(Rq: torch.Tensor) -> torch.Tensor:
    """[B,H,T,d,128 slots] -> [B,H,N,d] with rows in permuted token order (pure indexing)."""
    B, H, T, d, _ = Rq.shape
    nat = Rq.permute(0, 1, 2, 4, 3)                                   # [B,H,T,slot,d]
    idx = torch.as_tensor(SLOT_OF_KEY, device=Rq.device)
    return nat.index_select(3, idx).reshape(B, H, T * 128, d).contiguous()


def rq_natural_to_tiled(R: torch.Tensor) -> torch.Tensor:
    """[B,H,N,d] (permuted token order) -> [B,H,T,d,128 slots] (pure indexing)."""
    B, H, N, d = R.shape
    T = N // 128
    t = R.reshape(B, H, T, 128, d)
    idx = torch.as_tensor(KEY_OF_SLOT, device=R.device)
    return t.index_select(3, idx).permute(0, 1, 2, 4, 3).contiguous()


def unpack_fp4(x: torch.Tensor) -> torch.Tensor:
    """Two E2M1 codes per byte (even index in the low nibble) -> one code per byte; last dim x2."""
    lo, hi = x & 0xF, x >> 4
    return torch.stack([lo, hi], dim=-1).reshape(*x.shape[:-1], 2 * x.shape[-1])


def pack_fp4(c: torch.Tensor) -> torch.Tensor:
    """One E2M1 code per byte -> two per byte (even index in the low nibble); last dim / 2."""
    c = c.reshape(*c.shape[:-1], c.shape[-1] // 2, 2)
    return (c[..., 0] | (c[..., 1] << 4)).contiguous()
