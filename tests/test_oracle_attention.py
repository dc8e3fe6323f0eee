"""Pins of the oracle's attention: exact attention against a library routine, the tiled
recurrence (Eq. 1, Eq. 6) against exact attention, and the ExpCast path against Prop. 3.1."""
import numpy as np
import pytest
import torch

from oracle import analysis as A
from oracle import attention as T
from oracle import formats as F
from oracle import vsmooth as S


def _qkv(seed, N=384, d=128, v_offset=0.0):
    rng = np.random.default_rng(seed)
    Q = F.bf16_round(rng.standard_normal((N, d)))
    K = F.bf16_round(rng.standard_normal((N, d)) + 1.5 * rng.standard_normal(d))
    V = F.bf16_round(rng.standard_normal((N, d)) + v_offset * rng.standard_normal(d))
    return Q, K, V


def test_exact_attention_matches_torch_sdpa():
    Q, K, V = _qkv(0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None])[0, 0]
    assert np.allclose(T.attention_exact(Q, K, V), ref.numpy(), rtol=0, atol=1e-12)
    rows = [0, 5, 383]
    assert np.allclose(T.attention_exact(Q, K, V, rows=rows), ref.numpy()[rows], atol=1e-12)


def test_joint_permutation_invariance_eq3():
    Q, K, V = _qkv(1)
    perm = np.random.default_rng(2).permutation(len(K))
    assert np.allclose(T.attention_exact(Q, K[perm], V[perm]), T.attention_exact(Q, K, V), atol=1e-12)
    assert A.diam2(V[perm]) == pytest.approx(A.diam2(V), rel=1e-12)


def test_key_channel_mean_invariance():
    Q, K, V = _qkv(3)
    assert np.allclose(T.attention_exact(Q, K - K.mean(0), V), T.attention_exact(Q, K, V), atol=1e-12)


def test_mean_restore_identity_brute_force():
    rng = np.random.default_rng(4)
    for n, d in [(3, 2), (5, 4), (8, 3)]:
        P = rng.random((n, n))
        R = rng.standard_normal((n, d))
        mu = rng.standard_normal(d)
        lhs = P @ (R + np.ones((n, 1)) @ mu[None, :])
        rhs = P @ R + (P @ np.ones(n))[:, None] * mu[None, :]
        assert np.allclose(lhs, rhs, atol=1e-13)


@pytest.mark.parametrize("demean", [False, True])
def test_tiled_recurrence_exact_mode_equals_exact_attention(demean):
    # No quantisation anywhere and P = exact exponential: the tile loop of Eq. 1 with the
    # mean term of Eq. 6 must reproduce softmax attention on the un-permuted tokens.
    Q, K, V = _qkv(5, N=512, v_offset=4.0)
    N, d = K.shape
    perm = np.random.default_rng(6).permutation(N)
    Kp = K[perm] - K.mean(0)
    Vp = V[perm]
    if demean:
        mu = Vp.reshape(N // 128, 128, d).mean(1)
        R = (Vp.reshape(N // 128, 128, d) - mu[:, None, :]).reshape(N, d)
    else:
        mu = np.zeros((N // 128, d))
        R = Vp
    ones = np.ones(N // 128)
    O = T.attention_tiled(Q, ones, Kp, ones, R, mu, np.ones(d), p_mode="exact", round_output=False,
                          q_prescaled=False)
    assert np.allclose(O, T.attention_exact(Q, K, V), rtol=0, atol=1e-11)
    # scaling R and mu by 1/sV and multiplying back in the epilogue (App. B) changes nothing
    sV = np.exp(np.random.default_rng(7).uniform(-2, 2, d))
    O2 = T.attention_tiled(Q, ones, Kp, ones, R / sV, mu / sV, sV, p_mode="exact", round_output=False,
                           q_prescaled=False)
    assert np.allclose(O2, O, atol=1e-11)
    # a row subset gives the same rows
    rows = np.array([0, 127, 128, 511])
    O3 = T.attention_tiled(Q, ones, Kp, ones, R, mu, np.ones(d), p_mode="exact", rows=rows, round_output=False,
                           q_prescaled=False)
    assert np.allclose(O3, O[rows], atol=1e-13)


def test_tiled_expcast_rows_obey_prop31(golden):
    # ExpCast inside the tiled recurrence on unquantised operands: every row's output is
    # within (0.0364 + tau) diam2(V') of exact attention (Prop. 3.1, Eq. 14-15).
    g = golden("expcast_constants.txt")
    rng = np.random.default_rng(8)
    N, d = 640, 128
    for temp in (1.0, 3.0, 8.0):
        Q = rng.standard_normal((N, d)) * temp
        K = rng.standard_normal((N, d))
        V = rng.standard_normal((N, d)) * 2 + rng.standard_normal(d)
        ones = np.ones(N // 128)
        O = T.attention_tiled(Q, ones, K, ones, V, np.zeros((N // 128, d)), np.ones(d),
                              p_mode="expcast", round_output=False, q_prescaled=False)
        Oe = T.attention_exact(Q, K, V)
        S_ = (Q @ K.T) / np.sqrt(d)
        u = (S_ - S_.max(1, keepdims=True)) * np.log2(np.e)
        p = np.exp2(u)
        p /= p.sum(1, keepdims=True)
        tau = np.where(u < g["underflow_u"], p, 0).sum(1)       # p(T); p-hat(T) bounded below
        diam = A.diam2(V)
        err = np.linalg.norm(O - Oe, axis=1)
        assert np.all(err <= (g["tv_bound"] + 2 * tau + 1e-6) * diam)
        assert np.all(err[tau == 0] <= g["tv_bound"] * diam)


def test_emulated_vc_is_close_and_reduces_to_exact_without_quantisation():
    Q, K, V = _qkv(9, N=512, v_offset=3.0)
    perm = np.random.default_rng(10).permutation(512)
    O, ops = T.vc_attention_emulated(Q, K, V, perm)
    Oe = T.attention_exact(Q, K, V)
    assert T.rel_l2(O, Oe) < 0.05
    # rows subset gives identical rows
    rows = np.array([3, 200, 511])
    Or, _ = T.vc_attention_emulated(Q, K, V, perm, rows=rows)
    assert np.array_equal(Or, O[rows])
    # exact-exp P path on the same quantised operands is closer than ExpCast but still not exact
    Ox = T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                           F.e4m3_decode(ops["codes"]), ops["mu_t"], ops["sV"], p_mode="exact")
    assert T.rel_l2(Ox, Oe) < T.rel_l2(O, Oe)


def test_vsmooth_beats_unsmoothed_baseline_on_grouped_values():
    # Acceptance criterion 4 on a small structured input: grouped values with outlier tokens.
    rng = np.random.default_rng(11)
    N, d, G = 1024, 128, 8
    cent = rng.standard_normal((G, d)) * 2
    g = rng.integers(0, G, N)
    Vr = cent[g] + 0.3 * rng.standard_normal((N, d))
    out = rng.choice(N, 8, replace=False)
    Vr[np.ix_(out, rng.choice(d, 4, replace=False))] *= 30
    V = F.bf16_round(Vr)
    Q = F.bf16_round(rng.standard_normal((N, d)))
    K = F.bf16_round(rng.standard_normal((N, d)))
    grp = S.vsmooth_group(V, k=G, iters=10)
    Oe = T.attention_exact(Q, K, V)
    O_vc, _ = T.vc_attention_emulated(Q, K, V, grp["perm"])
    O_base, _ = T.vc_attention_emulated(Q, K, V, None, demean=False)
    assert T.rel_l2(O_vc, Oe) < T.rel_l2(O_base, Oe)


def test_prescaled_query_operand_equals_raw_query_path():
    # Folding the slope 8 log2(e) / sqrt(d) into the query operand (what vsmooth.quantize_q does
    # before quantising) gives the same attention as applying it in the recurrence.
    Q, K, V = _qkv(12, N=256)
    ones = np.ones(2)
    Qs = Q * (8 * np.log2(np.e) / np.sqrt(128))
    O = T.attention_tiled(Qs, ones, K, ones, V, np.zeros((2, 128)), np.ones(128), p_mode="exact",
                          round_output=False, q_prescaled=True)
    assert np.allclose(O, T.attention_exact(Q, K, V), atol=1e-11)
