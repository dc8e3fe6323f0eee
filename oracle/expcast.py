"""ExpCast-FP8 (oracle; test infrastructure only).

VC-Attention, Sec. 3.3, Eq. 7: for the log-domain score u = (s - m') log2(e) <= 0
(row maximum subtracted, Eq. 1) and a probability scaled by 2^8 so the row
maximum lands at 256, the E4M3 byte is

    c(u) = clip_[0,120]( Round( 8 (u + 8) + 56 + beta ) ),   beta = -0.35,

with Round = round to nearest even (Sec. 3.3 below Eq. 7; Fig. 2 caption).
Read as E4M3 the byte encodes approximately 2^(u+8) (Sec. 3.3, the affine
log relation 8e + m = 8 log2 v + 56 + eps(m)).

Fixed precision.  The kernels evaluate the argument in float32 with one
rounding, t = fl32(8u + C) where C = fl32(120 + beta) = fl32(119.65) (8u is
exact in float32), then round t to the nearest even integer and clip.  The
bit-exact contract between kernel and oracle is this float32 form.  The
real-arithmetic form ``expcast_code_real`` differs from it only when t lies
within one float32 ulp of a rounding boundary (a test pins that).

Non-finite inputs are defined too: NaN -> 0, +inf -> 120, -inf -> 0.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_encode, e4m3_decode, fl32

BETA = -0.35
C_F32 = np.float32(120.0 + BETA)          # fl32(119.65): the FMA constant b of the Fig. 2 caption


def expcast_code(u) -> np.ndarray:
    """c(u) of Eq. 7 in the float32 form (bit-exact contract). u: float32 array."""
    u = np.asarray(u, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        t = np.float32(8.0) * u + C_F32             # float32 multiply (exact) and add (one rounding)
        r = np.rint(t)                              # round half to even
        r = np.where(np.isnan(r), np.float32(0), r)
        c = np.clip(r, 0.0, 120.0)
    return c.astype(np.uint8)


def expcast_code_real(u) -> np.ndarray:
    """c(u) of Eq. 7 evaluated in float64 with beta = -0.35 (for the pins)."""
    u = np.asarray(u, dtype=np.float64)
    t = 8.0 * (u + 8.0) + 56.0 + BETA
    return np.clip(np.rint(t), 0.0, 120.0).astype(np.uint8)


def exp_then_cast_code(u) -> np.ndarray:
    """Conventional path of Fig. 2 (left) / Fig. 5a: exponentiate 2^(u+8) in float32, then E4M3 RNE."""
    u = np.asarray(u, dtype=np.float64)
    return e4m3_encode(fl32(np.exp2(u + 8.0)))


def decoded(codes) -> np.ndarray:
    """Value a code stands for, with the common 2^8 scale removed (App. D, w-hat)."""
    return e4m3_decode(codes) / 256.0
