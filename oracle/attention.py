"""Attention (oracle; test infrastructure only).

VC-Attention (arXiv 2609.15810):
  Sec. 3.1: S = Q K^T / sqrt(d), P = softmax(S), O = P V (non-causal).
  Sec. 3.1, Eq. 1: FlashAttention's online recurrence over key/value tiles j,
      m' = max(m, rowmax S_ij), alpha = exp(m - m'), P~ = exp(S_ij - m'),
      A <- alpha A + P~ V_j, l <- alpha l + P~ 1, O = A / l.
  Sec. 3.2, Eq. 6: with V'_j = R_j + 1 mu_j^T the numerator update becomes
      A <- alpha A + P~_q R_q,j + r mu_j^T,  l <- alpha l + r,  r = P~ 1.
  Sec. 3.3, Eq. 7 and the Fig. 2 caption: the E4M3 probability code is written
      by one FMA t = a S + b with a = 8 log2(e) and b = 120 + beta - a m' (the
      row maximum folded into b), then round-to-nearest-even and clip to [0, 120].
  App. B: means are stored divided by the per-channel value scale s_V, so one
      epilogue multiply by s_V serves both terms of Eq. 6.

The emulated path follows those steps in that order, tile by tile (tiles of 128
keys, j increasing), on the same quantised operands the kernel receives.  Its
float32 steps are the ones that decide a code; everything else is float64.
The query operand already carries L = fl32(8 log2(e) softmax_scale) (it is
quantised as fl32(Q L), see vsmooth.quantize_q), so with power-of-two block
scales the slope of Eq. 7 is exact:

  a    = s_Q * s_K[j]             one scale per (query block, key tile)
  s    = fl32(Q-hat . K-hat)      the FP32 score of two E4M3 operands
  xhat = fl32(a * rowmax_j s)     running maximum, in units of 8 log2(e) S
  m'   = max(m, xhat);  b = fl32(C - m'),  C = fl32(120 + beta)
  t    = fl32(a * s + b)          one FMA (emulated in float64, then rounded)
  code = clip(rint(t), 0, 120);  P = E4M3 value of code (2^8 = row maximum)
  r    = sum P;  alpha = 2^((m - m') / 8)
  A    = alpha A + P R-hat + r mu~;  l = alpha l + r
  O    = bf16(s_V * A / l)

``p_mode`` selects the probability path: "expcast" (above), "exp_cast" (the
conventional FP32 exponential 2^(t'/8), t' = fl32(a s - m') + 64, then an E4M3
cast, i.e. Fig. 2 left), or "exact" (P = 2^((a s - m')/8) in float64, no
quantisation of P; with unquantised operands this must reproduce exact attention).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .formats import e4m3_decode, e4m3_encode, fl32, bf16_round
from .expcast import C_F32

BK = 128   # key/value tile = B_v (Sec. 3.2, Eq. 4); the running max is updated per tile
BQ = 128   # query quantisation block


def softmax_scale_default(d: int) -> float:
    return 1.0 / np.sqrt(d)


def attention_exact(Q, K, V, scale: Optional[float] = None, rows: Optional[Sequence[int]] = None):
    """O = softmax(Q K^T * scale) V in float64 (Sec. 3.1). Q, K, V: (N, d) arrays of values."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = softmax_scale_default(Q.shape[1])
    if rows is not None:
        Q = Q[np.asarray(rows)]
    out = np.empty((Q.shape[0], V.shape[1]))
    for i0 in range(0, Q.shape[0], 256):
        S = (Q[i0:i0 + 256] @ K.T) * scale
        S -= S.max(axis=1, keepdims=True)
        P = np.exp(S)
        out[i0:i0 + 256] = (P @ V) / P.sum(axis=1, keepdims=True)
    return out


def _log2e_scale(scale: float) -> np.float32:
    return np.float32(8.0 * np.log2(np.e) * scale)


def attention_tiled(Qv, sQ, Kv, sK, Rv, mu_t, sV, scale: Optional[float] = None,
                    p_mode: str = "expcast", rows: Optional[Sequence[int]] = None,
                    round_output: bool = True, q_prescaled: bool = True):
    """Emulated tiled VC attention for one (batch, head).

    Qv   (N, d)      query operand values (decoded E4M3 codes of fl32(Q L) / s_Q when
                     q_prescaled, else raw query values that still need L)
    sQ   (N/128,)    query block scales
    Kv   (N, d)      key operand values in permuted order
    sK   (N/128,)    key tile scales
    Rv   (N, d)      residual operand values in permuted order
    mu_t (N/128, d)  stored means mu / s_V (or zeros)
    sV   (d,)        per-channel value scale
    rows             query rows to compute (default: all)

    Returns O (len(rows), d) as float64 (bf16-rounded values if round_output).
    """
    Qv = np.asarray(Qv, dtype=np.float64)
    Kv = np.asarray(Kv, dtype=np.float64)
    Rv = np.asarray(Rv, dtype=np.float64)
    mu_t = np.asarray(mu_t, dtype=np.float64)
    N, d = Kv.shape
    if scale is None:
        scale = softmax_scale_default(d)
    rows = np.arange(Qv.shape[0]) if rows is None else np.asarray(rows)
    nq = len(rows)
    L = _log2e_scale(scale)
    sQr = np.asarray(sQ)[rows // BQ]
    if q_prescaled:
        qa = fl32(sQr)                                                     # L is inside Q-hat
        qa64 = qa.astype(np.float64)                                       # exact: powers of two
    else:
        qa = fl32(np.float32(L) * fl32(sQr))                               # (nq,) float32
        qa64 = 8.0 * np.log2(np.e) * scale * np.asarray(sQr, dtype=np.float64)  # exact mode only
    Qr = Qv[rows]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    A = np.zeros((nq, d))
    for j in range(N // BK):
        ks = slice(j * BK, (j + 1) * BK)
        a = fl32(qa * np.float32(sK[j]))                                 # (nq,) float32
        s = Qr @ Kv[ks].T                                                # exact for E4M3 operands
        if p_mode != "exact":
            s = fl32(s).astype(np.float64)                               # FP32 scores
        a64 = a.astype(np.float64)
        if p_mode == "exact":
            a64 = qa64 * float(sK[j])
            xhat = a64 * s.max(axis=1)
            m_new = np.maximum(m, xhat)
            P = np.exp2((a64[:, None] * s - m_new[:, None]) / 8.0)
        else:
            xhat = fl32(a * fl32(s.max(axis=1))).astype(np.float64)
            m_new = np.maximum(m, xhat)
            b = fl32(C_F32 - fl32(m_new)).astype(np.float64)
            if p_mode == "expcast":
                t = fl32(a64[:, None] * s + b[:, None])                  # FMA, one rounding
                code = np.clip(np.rint(t), 0.0, 120.0).astype(np.uint8)
            elif p_mode == "exp_cast":
                y = fl32(a64[:, None] * s - m_new[:, None])              # FMA a*s - m', one rounding
                code = e4m3_encode(fl32(np.exp2(y.astype(np.float64) / 8.0 + 8.0)))
            else:
                raise ValueError(p_mode)
            P = e4m3_decode(code)
        alpha = np.exp2((m - m_new) / 8.0)                               # 0 on the first tile
        r = P.sum(axis=1)
        A = alpha[:, None] * A + P @ Rv[ks] + r[:, None] * mu_t[j][None, :]
        l = alpha * l + r
        m = m_new
    O = (A * np.asarray(sV, dtype=np.float64)[None, :]) / l[:, None]
    return bf16_round(O) if round_output else O


def vc_attention_emulated(Q, K, V, perm, scale=None, p_mode="expcast", rows=None,
                          demean: bool = True, k_smooth: bool = True, round_output: bool = True,
                          hadamard: bool = False):
    """Whole emulated VC path for one (batch, head) from bf16 values Q, K, V (N, d) and pi.

    Quantises with the oracle's own quantisers (vsmooth), then runs attention_tiled.
    demean=False, perm = identity is the unsmoothed sequence-order FP8 baseline.
    hadamard=True rotates Q by H and the centred K by H / d before their quantisers (App. B).
    Returns (O, operands dict).
    """
    from . import vsmooth
    N = Q.shape[0]
    perm = np.arange(N) if perm is None else np.asarray(perm)
    qc, sQ = vsmooth.quantize_q(Q, scale, hadamard=hadamard)
    if k_smooth:
        kc, sK = vsmooth.quantize_k(K, perm, hadamard=hadamard)
    elif hadamard:
        raise ValueError("the rotation is defined on the centred keys")
    else:
        kc, sK = vsmooth.quantize_rows_per_block(fl32(np.asarray(K, dtype=np.float64)[perm]))
    vq = vsmooth.quantize_v(V, perm, demean=demean)
    O = attention_tiled(e4m3_decode(qc), sQ, e4m3_decode(kc), sK, e4m3_decode(vq["codes"]),
                        vq["mu_t"], vq["sV"], scale, p_mode, rows, round_output)
    ops = {"qc": qc, "sQ": sQ, "kc": kc, "sK": sK, **vq}
    return O, ops


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))
