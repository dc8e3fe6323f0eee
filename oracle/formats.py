"""Number formats used by the method (oracle; test infrastructure only).

E2M1 (the 4-bit element of the MX formats, the analogue of the pages' NVFP4 elements in the
4-bit path, Sec. 3.2 after Eq. 4 and App. A) is defined at e2m1_decode.

E4M3 is the OCP 8-bit float E4M3FN that the pages' E4M3 refers to: a byte
with sign s, 4-bit exponent field e and 3-bit mantissa field m stores
2^(e-7) * (1 + m/8) for e >= 1 (VC-Attention, Sec. 3.3, the decoding rule
before Eq. 7), 2^-6 * m/8 for e = 0 (subnormals), and NaN for e = 15, m = 7.
The largest finite magnitude is 448.

Encoding rounds to the nearest representable value, ties to the even code,
and saturates finite values beyond 448 to +-448 (the quantisers scale blocks
so |x| <= 448 anyway).  The sign bit is the sign bit of the input, so -0.0 and
negative values that round to zero give 0x80.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values, from the field definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)
    return sign * val


# All finite non-negative E4M3 values, indexed by code 0..126 (monotone increasing).
_POS_VALUES = e4m3_decode(np.arange(127))


def e4m3_encode(x) -> np.ndarray:
    """Values -> E4M3 codes (uint8): nearest finite value, ties to even code, saturating.

    Written as a search over the table of representable magnitudes, so it is
    correct by inspection rather than by bit manipulation.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS_VALUES[hi], hi, code)
    code = code.astype(np.uint8)
    out = np.where(neg, code | 0x80, code).astype(np.uint8)
    out = np.where(np.isnan(x), np.uint8(0x7F), out)
    return out


E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 (OCP MX FP4) codes (low nibble of uint8) -> float64 values, from the field layout:
    sign bit 3, exponent field e = bits 2-1 (bias 1), mantissa bit 0; 2^(e-1) (1 + m/2) for
    e >= 1, m/2 for e = 0.  No infinities or NaNs; the largest magnitude is 6."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    val = np.where(e == 0, m / 2.0, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return sign * val


_E2M1_POS = e2m1_decode(np.arange(8))       # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(x) -> np.ndarray:
    """Values -> E2M1 codes (uint8, 0..15): nearest value, ties to the even code, saturating at
    +-6; the sign bit is the input's (a negative value that rounds to zero gives 0x8)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E2M1_MAX)
    hi = np.minimum(np.searchsorted(_E2M1_POS, a, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E2M1_POS[lo]
    dhi = _E2M1_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E2M1_POS[hi], hi, code).astype(np.uint8)
    return np.where(neg, code | 0x8, code).astype(np.uint8)


E2M3_MAX = 7.5


def e2m3_decode(codes) -> np.ndarray:
    """E2M3 (OCP MX FP6) codes (low six bits of uint8) -> float64 values, from the field layout:
    sign bit 5, exponent field e = bits 4-3 (bias 1), mantissa m = bits 2-0; 2^(e-1) (1 + m/8)
    for e >= 1, m/8 for e = 0.  No infinities or NaNs; the largest magnitude is 7.5."""
    c = np.asarray(codes, dtype=np.int64) & 0x3F
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> 3) & 0x3
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, (e - 1).astype(np.int64)))
    return sign * val


_E2M3_POS = e2m3_decode(np.arange(32))      # 0, 0.125, ..., 0.875, 1, 1.125, ..., 7.5


def e2m3_encode(x) -> np.ndarray:
    """Values -> E2M3 codes (uint8, 0..63): nearest value, ties to the even code, saturating at
    +-7.5; the sign bit is the input's (a negative value that rounds to zero gives 0x20)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E2M3_MAX)
    hi = np.minimum(np.searchsorted(_E2M3_POS, a, side="left"), 31)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E2M3_POS[lo]
    dhi = _E2M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E2M3_POS[hi], hi, code).astype(np.uint8)
    return np.where(neg, code | 0x20, code).astype(np.uint8)


def fl32(x) -> np.ndarray:
    """Round to the nearest float32 (ties to even); returned as float32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round finite values to the nearest bf16 (8 significant bits), ties to even.

    bf16 keeps float32's exponent range: normal magnitudes have spacing
    2^(E-7) in the binade [2^E, 2^(E+1)); below 2^-126 the spacing is 2^-133.
    Returned as float64 (exact).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = f * 2^e, f in [0.5, 1)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(x / ulp) * ulp


def bf16_bits_from_value(v) -> np.ndarray:
    """Exact bf16 values -> uint16 bit patterns."""
    return (fl32(v).view(np.uint32) >> 16).astype(np.uint16)


def bf16_value_from_bits(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
