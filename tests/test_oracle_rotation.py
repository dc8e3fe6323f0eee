"""Pins of the QK Hadamard rotation (Sec. 4.1 "Baselines", Sec. 4.2, App. B): the matrix against
a library routine and its closed form, the rotation against brute force, the score product's
invariance, and the rotated quantisers against the exact centred operands."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import attention as T
from oracle import formats as F
from oracle import rotation as R
from oracle import vsmooth as S


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 128])
def test_hadamard_matches_library(n):
    assert np.array_equal(R.hadamard(n), scipy.linalg.hadamard(n))


def test_hadamard_closed_form():
    H = R.hadamard(128)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    popc = np.vectorize(lambda x: bin(int(x)).count("1"))(i & j)
    assert np.array_equal(H, np.where(popc % 2 == 0, 1, -1))
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    with pytest.raises(ValueError):
        R.hadamard(96)


def test_rotate_special_vectors():
    H = R.hadamard(128)
    ones = np.ones((1, 128), np.float32)
    e0 = np.zeros(128)
    e0[0] = 128
    assert np.array_equal(R.rotate(ones)[0], e0)                    # the constant row lands on channel 0
    X = np.zeros((3, 128), np.float32)
    X[0, 5] = 1.0
    X[1, 77] = -2.0
    X[2] = H[9]
    Y = R.rotate(X)
    assert np.array_equal(Y[0], H[5])
    assert np.array_equal(Y[1], -2.0 * H[77])
    e9 = np.zeros(128)
    e9[9] = 128
    assert np.array_equal(Y[2], e9)                                 # H H = 128 I


def test_rotate_against_brute_force():
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((3, 128)) * np.exp(rng.uniform(-3, 3, (3, 128)))).astype(np.float32)
    Y = R.rotate(X)
    for r in range(3):
        for j in range(128):
            exact = sum((Fraction(float(X[r, c])) if bin(c & j).count("1") % 2 == 0
                         else -Fraction(float(X[r, c]))) for c in range(128))
            assert Fraction(float(exact)) == exact                 # representable in float64: no double rounding
            assert Y[r, j] == np.float32(float(exact))


def test_score_product_invariance():
    rng = np.random.default_rng(3)
    Q = F.bf16_round(rng.standard_normal((256, 128)))
    K = F.bf16_round(rng.standard_normal((256, 128)) + 2.0 * rng.standard_normal(128))
    Xq = F.fl32(Q)
    Xk = (F.fl32(K) - S.key_channel_mean(K)).astype(np.float32)
    ref = Xq.astype(np.float64) @ Xk.astype(np.float64).T
    rot = R.rotate(Xq).astype(np.float64) @ R.rotate(Xk).astype(np.float64).T / 128.0
    assert np.max(np.abs(rot - ref)) <= 1e-5 * np.max(np.abs(ref))
    # rotation is linear: rotating the centred key equals centring the rotated key
    kbar = S.key_channel_mean(K)
    lin = R.rotate(F.fl32(K)).astype(np.float64) - R.rotate(kbar[None, :]).astype(np.float64)
    assert np.max(np.abs(lin - R.rotate(Xk))) <= 1e-5 * np.max(np.abs(lin))


def _outlier_qk(seed, N=512):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((N, 128))
    K = rng.standard_normal((N, 128)) + 1.5 * rng.standard_normal(128)
    oc = rng.choice(128, 4, replace=False)
    Q[:, oc] *= 25.0
    K[:, oc] *= 25.0
    return F.bf16_round(Q), F.bf16_round(K)


@pytest.mark.parametrize("hadamard", [False, True])
def test_rotated_quantisers_reproduce_the_centred_scores(hadamard):
    Q, K = _outlier_qk(5)
    perm = np.random.default_rng(6).permutation(len(K))
    qc, sQ = S.quantize_q(Q, hadamard=hadamard)
    kc, sK = S.quantize_k(K, perm, hadamard=hadamard)
    L = float(S.log2e_scale(None))
    Kc = F.fl32(K)[perm] - S.key_channel_mean(K)[None, :]
    ref = L * (Q @ Kc.T.astype(np.float64))
    Qd = F.e4m3_decode(qc) * np.repeat(sQ, 128)[:, None]
    Kd = F.e4m3_decode(kc) * np.repeat(sK, 128)[:, None]
    err = np.linalg.norm(Qd @ Kd.T - ref) / np.linalg.norm(ref)
    assert err < 0.05                                               # E4M3 on both operands
    # block scales stay powers of two; the rotated key scale carries the 1/128 of H / 128
    assert np.all(np.frexp(sK)[0] == 0.5) and np.all(np.frexp(sQ)[0] == 0.5)
    if hadamard:
        Kr = R.rotate((F.fl32(K)[perm] - S.key_channel_mean(K)[None, :]).astype(np.float32))
        half_step = np.ldexp(1.0, np.frexp(np.abs(Kr) + 1e-30)[1] - 5) / 128.0   # E4M3 half ulp, >= exact
        dq = F.e4m3_decode(kc) * np.repeat(sK, 128)[:, None]
        sub = np.repeat(sK, 128)[:, None] * 2.0 ** -10               # subnormal half step
        assert np.all(np.abs(dq - Kr / 128.0) <= np.maximum(half_step, sub) * 1.0000001)
        # the centred keys sum to ~0 over the tokens, and so do the rotated ones
        assert np.abs(Kr.astype(np.float64).sum(0)).max() < 1e-3 * np.abs(Kr).max()


def test_rotation_spreads_channel_outliers():
    """Sec. 4.1: the rotation is the strongest training-free treatment of the score product.
    With a few outlier channels in Q and K, the rotated quantisers' score error is lower."""
    errs = {}
    for had in (False, True):
        e = []
        for seed in range(3):
            Q, K = _outlier_qk(20 + seed)
            perm = np.arange(len(K))
            qc, sQ = S.quantize_q(Q, hadamard=had)
            kc, sK = S.quantize_k(K, perm, hadamard=had)
            L = float(S.log2e_scale(None))
            ref = L * (Q @ (F.fl32(K) - S.key_channel_mean(K)[None, :]).T.astype(np.float64))
            Qd = F.e4m3_decode(qc) * np.repeat(sQ, 128)[:, None]
            Kd = F.e4m3_decode(kc) * np.repeat(sK, 128)[:, None]
            e.append(np.linalg.norm(Qd @ Kd.T - ref) / np.linalg.norm(ref))
        errs[had] = np.mean(e)
    assert errs[True] < 0.8 * errs[False]


def test_rotated_attention_stays_close_to_exact():
    rng = np.random.default_rng(8)
    N = 384
    Q = F.bf16_round(rng.standard_normal((N, 128)))
    K = F.bf16_round(rng.standard_normal((N, 128)) + 1.5 * rng.standard_normal(128))
    V = F.bf16_round(rng.standard_normal((N, 128)) + 2.0 * rng.standard_normal(128))
    perm = np.random.default_rng(9).permutation(N)
    rows = np.arange(0, N, 7)
    exact = T.attention_exact(Q, K, V, rows=rows)
    O0, _ = T.vc_attention_emulated(Q, K, V, perm, rows=rows)
    O1, ops = T.vc_attention_emulated(Q, K, V, perm, rows=rows, hadamard=True)
    e0, e1 = T.rel_l2(O0, exact), T.rel_l2(O1, exact)
    assert e1 < 0.05 and e1 < 1.5 * e0
    with pytest.raises(ValueError):
        T.vc_attention_emulated(Q, K, V, perm, rows=rows, hadamard=True, k_smooth=False)
