"""Closed forms behind ExpCast-FP8 and V-Smooth (oracle; test infrastructure only).

Sources, all in VC-Attention (arXiv 2609.15810):
  Sec. 3.3        eps(m) = m - 8 log2(1 + m/8), the offset of the byte from 8 log2 v + 56
  App. C, Fig. 8  range of that offset and its minimax centring shift
  App. D, Eq. 9   e(f) = 8 [f - (2^f - 1)], Mitchell's error in codes
  App. D, Eq. 10  decoded-to-exact ratio r(f) = (1 + Round(8f - 0.35)/8) / 2^f
  App. D, Eq. 11  bounds of r
  App. D, Eq. 12-13  total-variation bound of an endpoint reweighting
  App. D, Eq. 14-15  underflow tail and output bound
  Sec. 3.2, Eq. 5 energy identity of block demeaning
  Sec. 3.1, Eq. 2 output error split into probability and value terms
"""
from __future__ import annotations

import numpy as np


def eps_m(m):
    """Sec. 3.3: offset of byte 8e+m from 8 log2 v + 56, per mantissa field m."""
    m = np.asarray(m, dtype=np.float64)
    return m - 8.0 * np.log2(1.0 + m / 8.0)


def mitchell_e(f):
    """App. D, Eq. 9: e(f) = 8 [f - (2^f - 1)] for f in [0, 1)."""
    f = np.asarray(f, dtype=np.float64)
    return 8.0 * (f - (np.exp2(f) - 1.0))


def ratio_r(f, beta=-0.35):
    """App. D, Eq. 10: decoded-to-exact ratio for fractional part f of z = u + 8."""
    f = np.asarray(f, dtype=np.float64)
    return (1.0 + np.rint(8.0 * f + beta) / 8.0) / np.exp2(f)


def ratio_bounds(beta=-0.35, eps=1e-12):
    """Both one-sided limits of r at every rounding boundary f = (j + 1/2 - beta)/8 in [0, 1],
    including the carry cell j = 8, plus the interval ends (App. D, text before Eq. 11).

    r is continuous and decreasing inside each rounding cell, so its extrema over
    [0, 1) are among these limits.  Returns (inf r, sup r).
    """
    pts = [0.0, 1.0 - eps]
    for j in range(-1, 9):
        fb = (j + 0.5 - beta) / 8.0
        if 0.0 < fb < 1.0:
            pts += [fb - eps, fb + eps]
    vals = ratio_r(np.array(pts), beta)
    return float(vals.min()), float(vals.max())


def tv(p, q) -> np.ndarray:
    """Total variation distance along the last axis."""
    return 0.5 * np.abs(np.asarray(p) - np.asarray(q)).sum(axis=-1)


def tv_endpoint(q, a, b):
    """App. D, Eq. 12: TV when a fraction q of the mass is reweighted by b and the rest by a."""
    return q * (1.0 - q) * (b - a) / (a + q * (b - a))


def tv_bound(a, b):
    """App. D, Eq. 13: max over q of Eq. 12 = (sqrt b - sqrt a)/(sqrt b + sqrt a)."""
    return (np.sqrt(b) - np.sqrt(a)) / (np.sqrt(b) + np.sqrt(a))


def diam2(V) -> float:
    """Largest Euclidean distance between two rows (App. D, Eq. 15)."""
    V = np.asarray(V, dtype=np.float64)
    sq = (V * V).sum(1)
    d2 = sq[:, None] + sq[None, :] - 2.0 * V @ V.T
    return float(np.sqrt(max(d2.max(), 0.0)))


def block_energy_split(Vb):
    """Sec. 3.2, Eq. 4-5 for one block: (mean mu, residual R, ||V||^2, ||R||^2, mean share)."""
    Vb = np.asarray(Vb, dtype=np.float64)
    Bv = Vb.shape[0]
    mu = Vb.sum(0) / Bv
    R = Vb - mu[None, :]
    e_v = float((Vb * Vb).sum())
    e_r = float((R * R).sum())
    share = Bv * float(mu @ mu) / e_v if e_v > 0 else 0.0
    return mu, R, e_v, e_r, share


def output_error_split(P, Pq, V, Vq):
    """Sec. 3.1, Eq. 2: O - Oq = (P - Pq) V + Pq (V - Vq); returns (prob term, value term)."""
    return (P - Pq) @ V, Pq @ (V - Vq)
