"""4-bit (and 6-bit) V-Smooth on MX formats (oracle; test infrastructure only).

VC-Attention (arXiv 2609.15810):
  Sec. 3.2 after Eq. 4: the residual goes through the host kernel's value
      quantiser, 4-bit microscaled elements (NVFP4) at 4 bits.
  Sec. 4.1 "Implementation": the 4-bit configuration runs V-Smooth alone; P is
      a 4-bit operand whose per-block scale is computed on the fly, so ExpCast
      does not apply (App. A, "Scope of ExpCast-FP8").
  App. B: at 4 bits the microscales are applied inside the matrix instruction,
      so the block means are added unscaled.

The MX analogue built here (readings, all documented in the design notes):
  * Elements are E2M1 (formats.e2m1_*); each group of 32 elements along a
    product's reduction axis shares a power-of-two scale 2^E (an E8M0 value):
    Q and K per 32 channels of a row, P per 32 keys of a query row, R per 32
    keys of a channel.  (NVFP4's per-16 E4M3 scale has no MI355X matrix
    instruction; MX's per-32 E8M0 scale does.)
  * 2^E is the smallest power of two with amax <= 6 * 2^E, so no element
    saturates; E >= -100; an all-zero group takes E = 0.  Elements are
    E2M1_RNE(x / 2^E), the division exact.
  * The 32-key groups of P and R: in a 128-key tile, the keys of one 64-key
    half whose index has the same bit 2, group(k) = 2 (k // 64) + ((k >> 2) & 1).
    These are the keys one lane holds in the PV matrix instruction's operand
    order, so the same groups serve both operands of PV.
  * Slope: L4 = fl32(log2(e) softmax_scale) multiplies Q before quantisation,
    so scores are in log2 units: P = 2^(S - m), alpha = 2^(m - m').  The
    running maximum is the maximum of the float32 scores of the tiles so far.
  * K is centred by the key channel mean (as at 8 bits); the optional QK
    rotation is rotation.rotate on Q L4 and on the centred K, the key scale
    exponent lowered by 7 (H^-T = H / 128).
  * V: the block means mu_j of Eq. 4 (float32, exact sum rounded once) are
    stored as bf16(mu_j), unscaled; R = V' - mu_j (float32) is quantised.
  * r = the row sum of the dequantised P; l = alpha l + r;
    A = alpha A + P^ R^ + r mu~ (mu~ the stored bf16 means); O = bf16(A / l).
  * MXFP6: the same path with E2M3 elements (formats.e2m3_*, largest magnitude
    7.5, so the scale is the smallest 2^E with amax <= 7.5 * 2^E); every function
    takes fmt = "e2m3" for it.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import rotation
from .formats import E2M1_MAX, E2M3_MAX, bf16_round, e2m1_decode, e2m1_encode, e2m3_decode, e2m3_encode, fl32
from .vsmooth import block_means, key_channel_mean

G = 32     # elements per microscale group
BT = 128   # keys per tile (= B_v)

# element formats: largest magnitude, encoder, decoder
FORMATS = {"e2m1": (E2M1_MAX, e2m1_encode, e2m1_decode), "e2m3": (E2M3_MAX, e2m3_encode, e2m3_decode)}


def mx_exponent(amax, fmt: str = "e2m1") -> np.ndarray:
    """E of the smallest power of two 2^E with amax <= X * 2^E, X the format's largest magnitude
    (6 for E2M1, 7.5 for E2M3); E >= -100; 0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    X = FORMATS[fmt][0]
    with np.errstate(divide="ignore"):
        E = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / X)).astype(np.int64)
    # guard the logarithm's last-bit rounding with the defining inequality
    E = np.where(amax > np.ldexp(X, E), E + 1, E)
    E = np.where(amax <= np.ldexp(X, E - 1), E - 1, E)
    E = np.maximum(E, -100)
    return np.where(amax > 0, E, 0).astype(np.int64)


def quantize_row_groups(X32, fmt: str = "e2m1") -> tuple:
    """float32 rows (N, 128) -> codes (N, 128) and exponents E (N, 4) per 32-channel group."""
    X = np.asarray(X32, dtype=np.float32)
    N, d = X.shape
    Xg = X.reshape(N, d // G, G).astype(np.float64)
    E = mx_exponent(np.abs(Xg).max(axis=2), fmt)
    codes = FORMATS[fmt][1](Xg / np.ldexp(1.0, E)[:, :, None])
    return codes.reshape(N, d), E


def dequant_row_groups(codes, E, fmt: str = "e2m1") -> np.ndarray:
    N, d = codes.shape
    return (FORMATS[fmt][2](codes).reshape(N, d // G, G) * np.ldexp(1.0, E)[:, :, None]).reshape(N, d)


def log2e_scale4(softmax_scale, d: int = 128) -> np.float32:
    """L4 = fl32(log2(e) softmax_scale); softmax_scale None means 1/sqrt(d)."""
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    return np.float32(np.log2(np.e) * softmax_scale)


def quantize_q4(Q, softmax_scale=None, hadamard: bool = False, fmt: str = "e2m1"):
    """Q path: X = fl32(Q L4) (rotated by H when hadamard), MX elements per 32 channels."""
    Q = np.asarray(Q, dtype=np.float64)
    X = (fl32(Q) * log2e_scale4(softmax_scale, Q.shape[1])).astype(np.float32)
    if hadamard:
        X = rotation.rotate(X)
    return quantize_row_groups(X, fmt)


def quantize_k4(K, perm, hadamard: bool = False, fmt: str = "e2m1"):
    """K path: centring by the key channel mean, gather by pi, optional rotation (exponent - 7),
    MX elements per 32 channels of each permuted row."""
    kbar = key_channel_mean(K)
    Kp = fl32(np.asarray(K, dtype=np.float64)[perm])
    Ks = (Kp - kbar[None, :]).astype(np.float32)
    if not hadamard:
        return quantize_row_groups(Ks, fmt)
    codes, E = quantize_row_groups(rotation.rotate(Ks), fmt)
    return codes, E - 7


def key_group(k) -> np.ndarray:
    """32-key group of key k (0..127) inside its tile: 2 (k // 64) + ((k >> 2) & 1)."""
    k = np.asarray(k)
    return 2 * (k // 64) + ((k >> 2) & 1)


def quantize_v4(V, perm, demean: bool = True, fmt: str = "e2m1"):
    """V path: gather by pi, block means (Eq. 4), residual per (channel, 32-key group) in MX elements.

    Returns dict with
      codes  (N, d) uint8     R-hat codes in permuted row order
      E      (N/128, d, 4)    exponent of each (tile, channel, key group)
      mu     (N/128, d)       float32 block means (zeros when demean=False)
      mu_b   (N/128, d)       bf16(mu), the stored means (exact bf16 values, float64)
    """
    Vp = fl32(np.asarray(V, dtype=np.float64)[perm])
    N, d = Vp.shape
    T = N // BT
    mu = block_means(Vp) if demean else np.zeros((T, d), np.float32)
    R = (Vp.reshape(T, BT, d) - mu[:, None, :]).astype(np.float32).astype(np.float64)
    grp = key_group(np.arange(BT))
    E = np.zeros((T, d, 4), np.int64)
    codes = np.zeros((T, BT, d), np.uint8)
    for g in range(4):
        rows = np.nonzero(grp == g)[0]
        Eg = mx_exponent(np.abs(R[:, rows, :]).max(axis=1), fmt)           # (T, d)
        E[:, :, g] = Eg
        codes[:, rows, :] = FORMATS[fmt][1](R[:, rows, :] / np.ldexp(1.0, Eg)[:, None, :])
    return {"codes": codes.reshape(N, d), "E": E, "mu": mu, "mu_b": bf16_round(mu)}


def dequant_v4(codes, E, fmt: str = "e2m1") -> np.ndarray:
    N, d = codes.shape
    T = N // BT
    grp = key_group(np.arange(BT))
    vals = FORMATS[fmt][2](codes).reshape(T, BT, d)
    scale = np.ldexp(1.0, E)[:, :, grp]                                       # (T, d, BT)
    return (vals * np.transpose(scale, (0, 2, 1))).reshape(N, d)


def quantize_p4(P, fmt: str = "e2m1") -> np.ndarray:
    """Dequantised P of one tile (rows, 128 keys): MX elements per (row, 32-key group)."""
    P = np.asarray(P, dtype=np.float64)
    _, enc, dec = FORMATS[fmt]
    grp = key_group(np.arange(P.shape[1]))
    out = np.empty_like(P)
    for g in range(4):
        cols = np.nonzero(grp == g)[0]
        Eg = mx_exponent(P[:, cols].max(axis=1), fmt)
        out[:, cols] = dec(enc(P[:, cols] / np.ldexp(1.0, Eg)[:, None])) * np.ldexp(1.0, Eg)[:, None]
    return out


def attention_tiled_mx4(Qv, Kv, Rv, mu_b, rows: Optional[Sequence[int]] = None, p_mode: str = "mx4",
                        round_output: bool = True, fmt: str = "e2m1"):
    """Emulated tiled 4-bit VC attention for one (batch, head).

    Qv (N, d): dequantised query operand (Q L4, log2 units); Kv (N, d): dequantised keys in
    permuted order; Rv (N, d): dequantised residuals in permuted order; mu_b (N/128, d): the
    means added back.  p_mode "mx4": P quantised per 32-key group in the element format fmt
    (float32 scores and P);
    "exact": float64 throughout, P unquantised (then Qv = Q L4, Kv = K, Rv = V' - mu, mu_b = mu
    give exact attention).
    """
    Qv = np.asarray(Qv, dtype=np.float64)
    Kv = np.asarray(Kv, dtype=np.float64)
    Rv = np.asarray(Rv, dtype=np.float64)
    mu_b = np.asarray(mu_b, dtype=np.float64)
    N, d = Kv.shape
    rows = np.arange(Qv.shape[0]) if rows is None else np.asarray(rows)
    Qr = Qv[rows]
    nq = len(rows)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    A = np.zeros((nq, d))
    for j in range(N // BT):
        ks = slice(j * BT, (j + 1) * BT)
        s = Qr @ Kv[ks].T
        if p_mode == "exact":
            m_new = np.maximum(m, s.max(axis=1))
            P = np.exp2(s - m_new[:, None])
        elif p_mode == "mx4":
            s = fl32(s).astype(np.float64)                               # float32 scores
            m_new = np.maximum(m, s.max(axis=1))
            P = quantize_p4(fl32(np.exp2(fl32(s - m_new[:, None]).astype(np.float64))), fmt)
        else:
            raise ValueError(p_mode)
        alpha = np.exp2(m - m_new)                                       # 0 on the first tile
        r = P.sum(axis=1)
        A = alpha[:, None] * A + P @ Rv[ks] + r[:, None] * mu_b[j][None, :]
        l = alpha * l + r
        m = m_new
    O = A / l[:, None]
    return bf16_round(O) if round_output else O


def vc_attention_mx4_emulated(Q, K, V, perm, scale=None, rows=None, demean: bool = True,
                              hadamard: bool = False, round_output: bool = True, fmt: str = "e2m1"):
    """Whole emulated MX VC path for one (batch, head) from bf16 values Q, K, V and pi, in the
    element format fmt (E2M1 at 4 bits, E2M3 at 6 bits).  demean=False with the identity pi is
    the unsmoothed baseline.  Returns (O, operands)."""
    N = Q.shape[0]
    perm = np.arange(N) if perm is None else np.asarray(perm)
    qc, qE = quantize_q4(Q, scale, hadamard, fmt)
    kc, kE = quantize_k4(K, perm, hadamard, fmt)
    vq = quantize_v4(V, perm, demean, fmt)
    O = attention_tiled_mx4(dequant_row_groups(qc, qE, fmt), dequant_row_groups(kc, kE, fmt),
                            dequant_v4(vq["codes"], vq["E"], fmt), vq["mu_b"], rows, "mx4", round_output, fmt)
    return O, {"qc": qc, "qE": qE, "kc": kc, "kE": kE, **vq}
