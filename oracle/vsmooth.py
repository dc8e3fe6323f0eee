"""V-Smooth preprocessing (oracle; test infrastructure only).

VC-Attention (arXiv 2609.15810):
  Sec. 3.2 "Value-guided permutation", Eq. 3: per batch and head, k-means over
      the value tokens gives labels z; pi = argsort(z); K' = K[pi], V' = V[pi];
      Q keeps its order.
  Sec. 3.2 "Block demeaning", Eq. 4: blocks of B_v = 128 permuted rows;
      mu_j = (1/B_v) V'_j^T 1 and R_j = V'_j - 1 mu_j^T; only R goes through the
      value quantiser (per-channel E4M3 at 8 bits).
  App. B: K fuses the centering statistics (the key channel mean, Sec. 2),
      the gather by pi, mean subtraction and quantisation; V fuses the gather,
      block demeaning and quantisation and writes the block means divided by
      the per-channel value scale, so one epilogue multiply serves both terms
      of Eq. 6.
  Sec. 4.1 "Baselines": the quantisers round each operand to the nearest code
      per block.

Readings taken where the pages are silent (all documented in the design notes):
  * k-means is batch Lloyd (assign, then recompute means) for `iters` rounds,
    squared Euclidean distance, ties to the lowest cluster index, an empty
    cluster keeps its centroid; default start = rows floor((c + 1/2) N / k).
    Labels are those of the last assignment; the objective J uses those labels
    and the means recomputed from them.
  * pi is the stable argsort (ties keep token order).
  * K and Q scales: one per 128-row block, the smallest power of two 2^E with
    amax <= 448 * 2^E (an E8M0 block scale); the Q block is quantised after
    multiplying by L = fl32(8 log2(e) softmax_scale), so Q-hat . K-hat times
    s_Q s_K is the score in the units of Eq. 7's FMA.  V scale: one per
    (batch, head, channel) over all N tokens, amax|R|/448.  A zero amax gives
    scale 1.  Means are float32 (an exact sum rounded once), stored for the
    kernel as bf16(mu / s_V).
  * Quantisation decisions are taken in float32: x/s is one correctly rounded
    float32 division (exact for the power-of-two scales), then E4M3
    round-to-nearest-even.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import rotation
from .formats import E4M3_MAX, e4m3_encode, fl32, bf16_round

BV = 128  # hardware value block (Sec. 3.2, Eq. 4)


# ----------------------------------------------------------------------------------------------
# k-means grouping (Sec. 3.2, Eq. 3)
# ----------------------------------------------------------------------------------------------

def kmeans_init_strided(V: np.ndarray, k: int) -> np.ndarray:
    """Deterministic start: centroid c = row floor((c + 1/2) N / k) of V (float64 copy)."""
    N = V.shape[0]
    rows = ((2 * np.arange(k) + 1) * N) // (2 * k)
    return np.asarray(V, dtype=np.float64)[rows].copy()


def sq_distances(V: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Squared Euclidean distances (N, k) in float64 (expanded form; one matmul)."""
    V = np.asarray(V, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    return (V * V).sum(1)[:, None] - 2.0 * (V @ C.T) + (C * C).sum(1)[None, :]


def kmeans_assign(V, C) -> np.ndarray:
    """Nearest centroid per token, ties to the lowest index (np.argmin returns the first)."""
    return np.argmin(sq_distances(V, C), axis=1).astype(np.int32)


def kmeans_update(V, labels, C_prev) -> np.ndarray:
    """Mean of the tokens of each cluster; an empty cluster keeps its previous centroid."""
    V = np.asarray(V, dtype=np.float64)
    k, d = C_prev.shape
    sums = np.zeros((k, d))
    np.add.at(sums, labels, V)
    counts = np.bincount(labels, minlength=k)
    C = np.array(C_prev, dtype=np.float64, copy=True)
    nz = counts > 0
    C[nz] = sums[nz] / counts[nz, None]
    return C


def kmeans_objective(V, labels, C) -> float:
    """J = sum_t ||v_t - c_{z_t}||^2 (float64, direct differences)."""
    diff = np.asarray(V, dtype=np.float64) - np.asarray(C, dtype=np.float64)[labels]
    return float((diff * diff).sum())


def kmeans_lloyd(V, k: int, iters: int, C_init: Optional[np.ndarray] = None):
    """Batch Lloyd k-means. Returns (labels int32 (N,), centroids (k, d) float64, J, J history).

    J history holds J after each round (labels of that round, means recomputed from them).
    """
    V = np.asarray(V, dtype=np.float64)
    C = kmeans_init_strided(V, k) if C_init is None else np.array(C_init, dtype=np.float64)
    hist = []
    labels = None
    for _ in range(iters):
        labels = kmeans_assign(V, C)
        C = kmeans_update(V, labels, C)
        hist.append(kmeans_objective(V, labels, C))
    return labels, C, hist[-1], hist


def stable_argsort(labels) -> np.ndarray:
    """pi = argsort(z), ties in token order (Eq. 3)."""
    return np.argsort(np.asarray(labels), kind="stable").astype(np.int32)


def cluster_offsets(labels, k: int) -> np.ndarray:
    """Start of each cluster's run in the sorted order; offsets[k] = N."""
    counts = np.bincount(np.asarray(labels), minlength=k)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


# ----------------------------------------------------------------------------------------------
# Quantisers (Sec. 3.1 X_q = s_X * X-hat; Sec. 4.1 nearest code per block; App. B)
# ----------------------------------------------------------------------------------------------

def _scale_from_amax(amax) -> np.ndarray:
    """s = fl32(amax / 448), and 1 where amax == 0 (float32)."""
    amax = fl32(amax)
    s = amax / np.float32(E4M3_MAX)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def pow2_scale(amax) -> np.ndarray:
    """Smallest power of two 2^E with amax <= 448 * 2^E (1 where amax == 0), as float32.

    With amax = m 2^e (m in [0.5, 1)): 448 * 2^(e-8) = 1.75 * 2^e always fits, 448 * 2^(e-10)
    never does, so E is e - 9 when amax <= 448 * 2^(e-9) and e - 8 otherwise.  E is kept at
    or above -100 so the scale and its inverse are normal floats (blocks that small are
    all-but-zero; their codes underflow either way).
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    E = e.astype(np.int64) - 8
    E = np.where(amax <= np.ldexp(E4M3_MAX, E - 1), E - 1, E)
    E = np.maximum(E, -100)
    return np.where(amax > 0, np.ldexp(1.0, E), 1.0).astype(np.float32)


def quantize_rows_per_block(X32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per 128-row block of a float32 (N, d) array: s_b = pow2_scale(amax), codes = E4M3(x / s_b)."""
    N, d = X32.shape
    blocks = X32.reshape(N // BV, BV, d)
    s = pow2_scale(np.abs(blocks).max(axis=(1, 2)))
    codes = e4m3_encode(blocks / s[:, None, None])         # exact float32 scaling, then E4M3 RNE
    return codes.reshape(N, d), s


def key_channel_mean(K) -> np.ndarray:
    """Key channel mean over all N tokens: fl32(sum / N), the sum taken in float64 (exact for bf16 data)."""
    K = np.asarray(K, dtype=np.float64)
    return fl32(K.sum(0) / K.shape[0])


def quantize_k(K, perm, hadamard: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """K path of App. B: centering stats, gather by pi, mean subtraction, per-block E4M3.

    hadamard=True adds App. B's rotation: the centred rows are rotated by H (rotation.rotate)
    and quantised per block; the scale then carries the 1/d of H^-T = H / d, so
    codes * s_K = (K[pi] - kbar) H / d up to the E4M3 rounding.

    Returns (codes (N, d) uint8 in permuted order, s_K (N/128,) float32).
    """
    kbar = key_channel_mean(K)
    Kp = fl32(np.asarray(K, dtype=np.float64)[perm])
    Ks = (Kp - kbar[None, :]).astype(np.float32)              # one float32 subtraction
    if not hadamard:
        return quantize_rows_per_block(Ks)
    codes, s = quantize_rows_per_block(rotation.rotate(Ks))
    return codes, (s / np.float32(Ks.shape[1])).astype(np.float32)   # exact: d is a power of two


def log2e_scale(softmax_scale: float, d: int = 128) -> np.float32:
    """L = fl32(8 log2(e) softmax_scale): Eq. 7's slope a = 8 log2(e) times the softmax scale."""
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    return np.float32(8.0 * np.log2(np.e) * softmax_scale)


def quantize_q(Q, softmax_scale=None, hadamard: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Q path: fl32(Q * L), then per 128-row block E4M3 (Q keeps its token order, Eq. 3).

    hadamard=True rotates fl32(Q * L) by H (rotation.rotate) before the quantiser (App. B).
    """
    Q = np.asarray(Q, dtype=np.float64)
    L = log2e_scale(softmax_scale, Q.shape[1])
    X = (fl32(Q) * L).astype(np.float32)
    return quantize_rows_per_block(rotation.rotate(X) if hadamard else X)


def block_means(Vp) -> np.ndarray:
    """Eq. 4: mu_j per 128-row block, fl32 of the float64 block sum divided by 128."""
    Vp = np.asarray(Vp, dtype=np.float64)
    N, d = Vp.shape
    return fl32(Vp.reshape(N // BV, BV, d).sum(1) / BV)


def quantize_v(V, perm, demean: bool = True):
    """V path of App. B: gather by pi, block demeaning (Eq. 4), per-channel E4M3 residual.

    Returns dict with
      codes  (N, d) uint8   R-hat in permuted order
      sV     (d,) float32   per-channel scale amax_t |R[t, c]| / 448
      mu     (N/128, d) float32   block means (zeros when demean=False)
      mu_t   (N/128, d) float64   bf16(mu / sV), the stored means (exact bf16 values)
    demean=False is the unsmoothed baseline (mu = 0, raw V' quantised).
    """
    Vp = fl32(np.asarray(V, dtype=np.float64)[perm])
    N, d = Vp.shape
    if demean:
        mu = block_means(Vp)
    else:
        mu = np.zeros((N // BV, d), np.float32)
    R = (Vp.reshape(N // BV, BV, d) - mu[:, None, :]).astype(np.float32).reshape(N, d)
    sV = _scale_from_amax(np.abs(R).max(axis=0))
    codes = e4m3_encode(R / sV[None, :])                     # float32 division, then E4M3 RNE
    mu_t = bf16_round(mu / sV[None, :])                      # float32 division, then bf16 RNE
    return {"codes": codes, "sV": sV, "mu": mu, "mu_t": mu_t}


def vsmooth_group(V, k: int, iters: int, C_init=None):
    """Grouping step for one (batch, head): labels, centroids, J, pi, offsets."""
    labels, C, J, hist = kmeans_lloyd(V, k, iters, C_init)
    return {"labels": labels, "C": C, "J": J, "J_hist": hist,
            "perm": stable_argsort(labels), "offsets": cluster_offsets(labels, k)}
