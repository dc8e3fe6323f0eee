"""QK Hadamard rotation (oracle; test infrastructure only).

VC-Attention (arXiv 2609.15810):
  Sec. 4.1 "Baselines": the 8-bit baselines run with a fused QK Hadamard
      transform, the rotation of both operands of the score product.
  Sec. 4.2 and Sec. 4.3: the rotation leaves the score unchanged, costs no
      time when fused, and changes fidelity little.
  App. B: the Q pass rotates before quantising; the K pass computes the
      centering statistics, gathers by pi, rotates, subtracts the mean and
      quantises.

Readings taken where the pages are silent (all documented in the design notes):
  * H is the Sylvester-ordered Hadamard matrix of order d = 128:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]; entries +-1, H symmetric,
    H H^T = d I.
  * The rotation pair is (H, H^-T) = (H, H / d): queries are multiplied by H,
    centred keys by H / d, so the score product is unchanged in exact
    arithmetic.  Both factors are +-1 times a power of two, so the 1/d rides
    on the key's power-of-two block scale and moves no code.  (An orthonormal
    H / sqrt(d) on both sides is not a power of two and would shift every
    code's rounding grid.)
  * Rotation is linear, so rotating the centred key equals centring the
    rotated key; the K pass rotates the float32 centred key K[pi] - kbar.
  * A rotated value is the float32 rounding of the exact product: the sum of
    d float32 terms with signs +-1 is taken in float64, which is exact (hence
    independent of summation order) whenever a row's terms span fewer than
    about 53 - 24 - 7 = 22 binades, and rounded to float32 once.
"""
from __future__ import annotations

import numpy as np

from .formats import fl32

D = 128


def hadamard(n: int = D) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), int64 entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def rotate(X) -> np.ndarray:
    """fl32(X H) for float32 rows X (..., d): the sum taken in float64, rounded once."""
    X = np.asarray(X, dtype=np.float32)
    H = hadamard(X.shape[-1]).astype(np.float64)
    return fl32(X.astype(np.float64) @ H)
