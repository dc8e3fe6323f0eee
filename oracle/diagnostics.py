"""Error diagnostics of a workload (oracle; test infrastructure only, CPU).

The quantities VC-Attention (arXiv 2609.15810) measures on captured tensors to motivate its two
prescriptions, computed here with the oracle's own quantisers and recurrence:

  * Sec. 3.1, Eq. 2 and Fig. 3a: the low-bit output error splits into a probability term
    (P - P_q) V and a value term P_q (V - V_q).
  * Sec. 3.2, Eq. 5 and Fig. 4: the share of a block's energy that its mean carries, under
    three token orders (sequence, static spatiotemporal cubes, k-means).
  * Sec. 3.2, Table 1: the value quantiser's error under each token order, every order with
    block demeaning and per-channel E4M3 V.
  * Sec. 3.3, the paragraph after Prop. 3.1: the total variation between a softmax row and its
    ExpCast-normalised row, with the row's underflow mass tau.

Readings (the pages print these figures for their own tensors and leave the definitions
partly open):
  * The static cube order (Table 1's DeltaQuant row) numbers tokens cube by cube over the
    (T, H, W) token grid, 2 x 8 x 8 = 128 tokens a cube, tokens inside a cube in grid order;
    tokens past T*H*W continue the grid into a further (partial) frame.
  * The value error is the relative mean squared error ||V_hat - V'||^2 / ||V'||^2 of the
    dequantised operand the kernel uses (residual codes times s_V plus the stored mean).
  * Eq. 2 is taken with P the exact softmax of the unquantised scores and P_q the tiled ExpCast
    recurrence on the quantised Q and K, so P_q V is that recurrence with the exact V' as its
    value operand; the two terms then add up to O - O_q exactly.
  * The row TV compares the softmax of the quantised scores with the normalised decoded codes
    of the same row taken against the row's own maximum (one pass), so it isolates ExpCast.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .analysis import block_energy_split, tv
from .attention import attention_exact, attention_tiled, softmax_scale_default
from .expcast import decoded, exp_then_cast_code, expcast_code
from .formats import e4m3_decode, fl32
from .rotation import hadamard
from . import vsmooth

BV = 128


def static_cube_order(grid: Tuple[int, int, int], N: int, cube=(2, 8, 8)) -> np.ndarray:
    """Token order cube by cube over the (T, H, W) grid (token n = t H W + y W + x)."""
    T, Hh, W = grid
    n = np.arange(N)
    t, y, x = n // (Hh * W), (n // W) % Hh, n % W
    ct, cy, cx = cube
    nyc, nxc = -(-Hh // cy), -(-W // cx)
    cid = ((t // ct) * nyc + y // cy) * nxc + x // cx
    inner = ((t % ct) * cy + y % cy) * cx + x % cx
    return np.lexsort((inner, cid))


def block_mean_share(Vp) -> float:
    """Eq. 5 share B_v ||mu||^2 / ||V_j||^2 averaged over the 128-row blocks of Vp (permuted rows)."""
    Vp = np.asarray(Vp, dtype=np.float64)
    shares = [block_energy_split(Vp[j * BV:(j + 1) * BV])[4] for j in range(Vp.shape[0] // BV)]
    return float(np.mean(shares))


def dequantized_v(vq) -> np.ndarray:
    """The value operand the kernel uses, (R_hat + mu / s_V) s_V per channel, in permuted order."""
    codes = e4m3_decode(vq["codes"])
    N, d = codes.shape
    mu_rows = np.repeat(np.asarray(vq["mu_t"], dtype=np.float64), BV, axis=0)
    return (codes + mu_rows) * np.asarray(vq["sV"], dtype=np.float64)[None, :]


def value_rel_mse(V, perm, demean: bool = True, rotate: bool = False) -> float:
    """Table 1: ||V_hat - V'||^2 / ||V'||^2 of the V quantiser in the order perm.

    rotate=True is Table 1's "Hadamard on V": the rows are rotated by the orthonormal H/sqrt(d)
    before the quantiser (the error is measured in the rotated frame, which the rotation leaves
    unchanged in norm)."""
    V = np.asarray(V, dtype=np.float64)
    if rotate:
        d = V.shape[1]
        V = fl32(V @ hadamard(d) / np.sqrt(d)).astype(np.float64)
    perm = np.arange(V.shape[0]) if perm is None else np.asarray(perm)
    vq = vsmooth.quantize_v(V, perm, demean=demean)
    Vp = fl32(V[perm]).astype(np.float64)
    err = dequantized_v(vq) - Vp
    return float((err * err).sum() / (Vp * Vp).sum())


def output_error_terms(Q, K, V, perm, rows: Sequence[int], demean: bool = True,
                       hadamard_qk: bool = False, scale: Optional[float] = None) -> Dict[str, float]:
    """Eq. 2 on the given query rows: norms of O, of the probability term O - P_q V and of the value
    term P_q V - O_q, each relative to ||O|| (Frobenius over the rows)."""
    N = Q.shape[0]
    perm = np.arange(N) if perm is None else np.asarray(perm)
    rows = np.asarray(rows)
    O = attention_exact(Q, K, V, scale, rows=rows)
    qc, sQ = vsmooth.quantize_q(Q, scale, hadamard=hadamard_qk)
    kc, sK = vsmooth.quantize_k(K, perm, hadamard=hadamard_qk)
    vq = vsmooth.quantize_v(V, perm, demean=demean)
    Qv, Kv = e4m3_decode(qc), e4m3_decode(kc)
    d = V.shape[1]
    Oq = attention_tiled(Qv, sQ, Kv, sK, e4m3_decode(vq["codes"]), vq["mu_t"], vq["sV"], scale,
                         rows=rows, round_output=False)
    Vp = fl32(np.asarray(V, dtype=np.float64)[perm]).astype(np.float64)
    PqV = attention_tiled(Qv, sQ, Kv, sK, Vp, np.zeros((N // BV, d)), np.ones(d), scale,
                          rows=rows, round_output=False)
    nO = float(np.linalg.norm(O))
    prob = float(np.linalg.norm(O - PqV)) / nO
    val = float(np.linalg.norm(PqV - Oq)) / nO
    return {"prob_term": prob, "value_term": val, "total": float(np.linalg.norm(O - Oq)) / nO,
            "value_share": val / (prob + val) if prob + val > 0 else 0.0}


def row_tv(Q, K, rows: Sequence[int], scale: Optional[float] = None,
           hadamard_qk: bool = False) -> Dict[str, np.ndarray]:
    """Sec. 3.3 after Prop. 3.1: per query row, TV(p, p_hat) for ExpCast and for exp-then-cast, and
    the underflow mass tau (p's mass on the keys whose ExpCast code is 0).

    The scores are those of the quantised operands (key order does not matter here);
    u = (a s - max) / 8 in log2 units, p = 2^u normalised in float64, p_hat = decoded codes
    normalised."""
    N, d = Q.shape
    if scale is None:
        scale = softmax_scale_default(d)
    qc, sQ = vsmooth.quantize_q(Q, scale, hadamard=hadamard_qk)
    kc, sK = vsmooth.quantize_k(K, np.arange(N), hadamard=hadamard_qk)
    rows = np.asarray(rows)
    Qr = e4m3_decode(qc)[rows] * np.asarray(sQ, dtype=np.float64)[rows // BV][:, None]
    Kd = e4m3_decode(kc) * np.repeat(np.asarray(sK, dtype=np.float64), BV)[:, None]
    x = Qr @ Kd.T                                       # a s in Eq. 7's units (8 log2 per unit of u)
    u = (x - x.max(axis=1, keepdims=True)) / 8.0
    p = np.exp2(u)
    p /= p.sum(axis=1, keepdims=True)
    uf = u.astype(np.float32)
    codes = expcast_code(uf)
    w = decoded(codes)
    we = decoded(exp_then_cast_code(uf))
    out = {"tv_expcast": np.array([tv(p[i], w[i] / w[i].sum()) for i in range(len(rows))]),
           "tv_exp_then_cast": np.array([tv(p[i], we[i] / we[i].sum()) for i in range(len(rows))]),
           "tau": (p * (codes == 0)).sum(axis=1)}
    return out
