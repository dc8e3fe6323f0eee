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


# ---- identity-value probes: with V = I the output row IS the normalised decoded P row, so the
# recurrence's probabilities can be read back and compared with the separately pinned codes ----

def _identity_probe(p_mode, maxima=(2.5, 5.0), nq=4, seed=20):
    """Two 128-key tiles, d = 256, V = I_256.  Scores (in Eq. 7 units, slope a = 1 exactly) are
    multiples of 1/16 with the row maxima of tile 0 and tile 1 at c_i * maxima[0] and
    c_i * maxima[1].  Returns (O, u0, u1, w): O from attention_tiled, u_j the log2-domain scores of
    tile j against its own running maximum, w = 2^((m0 - m1)/8) the tile-0 rescale."""
    rng = np.random.default_rng(seed)
    d = 256
    scale = 1.0 / (8.0 * np.log2(np.e))           # L = fl32(8 log2(e) scale) = 1 exactly
    assert T._log2e_scale(scale) == np.float32(1.0)
    c = np.array([1.0, 0.5, 0.25, 1.0])[:nq]
    base = np.concatenate([-rng.integers(0, 16 * 120, 128) / 16.0, -rng.integers(0, 16 * 120, 128) / 16.0])
    base[rng.integers(0, 128)] = maxima[0]
    base[128 + rng.integers(0, 128)] = maxima[1]
    Kv = np.zeros((256, d))
    Kv[:, 0] = base
    Qv = np.zeros((nq, d))
    Qv[:, 0] = c
    O = T.attention_tiled(Qv, np.ones(1), Kv, np.ones(2), np.eye(256), np.zeros((2, d)), np.ones(d), scale=scale,
                          p_mode=p_mode, round_output=False, q_prescaled=False)
    s = c[:, None] * base[None, :]
    m0 = s[:, :128].max(1)
    m1 = np.maximum(m0, s[:, 128:].max(1))
    u0 = (s[:, :128] - m0[:, None]) / 8.0
    u1 = (s[:, 128:] - m1[:, None]) / 8.0
    return O, u0, u1, np.exp2((m0 - m1) / 8.0)


@pytest.mark.parametrize("p_mode", ["expcast", "exp_cast"])
def test_tiled_probabilities_are_the_pinned_codes(p_mode):
    """The recurrence's P in each tile is the code of the pinned single-element function
    (expcast_code for Eq. 7, exp_then_cast_code for the exponentiate-then-cast path of Fig. 2/5a)
    taken against that tile's running maximum, rescaled by 2^((m - m')/8) when the maximum moves
    (Eq. 1), and normalised by the decoded row sum (Eq. 6's r, App. D's p-hat)."""
    from oracle import expcast as E
    for maxima in ((2.5, 5.0), (5.0, 2.5), (-3.0, 7.5)):
        O, u0, u1, w = _identity_probe(p_mode, maxima)
        code = E.expcast_code if p_mode == "expcast" else E.exp_then_cast_code
        cast = (lambda u: code(u.astype(np.float32))) if p_mode == "expcast" else code
        P0 = F.e4m3_decode(cast(u0)) * w[:, None]
        P1 = F.e4m3_decode(cast(u1))
        l = P0.sum(1) + P1.sum(1)
        want = np.concatenate([P0, P1], axis=1) / l[:, None]
        assert np.allclose(O, want, rtol=1e-14, atol=1e-300)
        # the larger maximum lands on code 120 (= 256) with zero error in both modes
        assert F.e4m3_decode(cast(np.zeros(1))).item() == 256.0


def test_tiled_exp_cast_rows_obey_e4m3_tv_bound():
    """P by exponentiate-then-cast on unquantised operands: in the normal range an E4M3 RNE value
    is within a relative half step 2^-4 of its argument (3 mantissa bits; Sec. 3.3's decode), so
    each weight's ratio lies in [1 - 2^-4, 1 + 2^-4] and App. D Eq. 12-13 bound the row's TV by
    (sqrt b - sqrt a)/(sqrt b + sqrt a) = 0.0313 (+ tau for the subnormal tail, u < -14), and the
    output by that times diam2(V) (Eq. 15)."""
    rng = np.random.default_rng(21)
    N, d = 640, 128
    slack = 1e-4                                       # float32 slope and score roundings
    a, b = (1 - 2.0 ** -4) * (1 - slack), (1 + 2.0 ** -4) * (1 + slack)
    bound = A.tv_bound(a, b)
    assert 0.031 < bound < 0.0314
    for temp in (1.0, 3.0, 8.0):
        Q = rng.standard_normal((N, d)) * temp
        K = rng.standard_normal((N, d))
        V = rng.standard_normal((N, d)) * 2 + rng.standard_normal(d)
        ones = np.ones(N // 128)
        O = T.attention_tiled(Q, ones, K, ones, V, np.zeros((N // 128, d)), np.ones(d),
                              p_mode="exp_cast", round_output=False, q_prescaled=False)
        Oe = T.attention_exact(Q, K, V)
        S_ = (Q @ K.T) / np.sqrt(d)
        u = (S_ - S_.max(1, keepdims=True)) * np.log2(np.e)
        p = np.exp2(u)
        p /= p.sum(1, keepdims=True)
        tau = np.where(u < -14, p, 0).sum(1)
        err = np.linalg.norm(O - Oe, axis=1)
        diam = A.diam2(V)
        assert np.all(err <= (bound + 2 * tau) * diam)
        assert np.all(err[tau == 0] <= bound * diam)


def test_tiled_expcast_rows_obey_prop31_prescaled_query(golden):
    """Prop. 3.1 (Eq. 8, 14-15) in the call form the GPU tests use: the query operand already
    carries L = fl32(8 log2(e)/sqrt(d)) (q_prescaled=True, unit block scales)."""
    g = golden("expcast_constants.txt")
    rng = np.random.default_rng(22)
    N, d = 640, 128
    L = float(S.log2e_scale(None))
    for temp in (1.0, 3.0, 8.0):
        Q = rng.standard_normal((N, d)) * temp
        K = rng.standard_normal((N, d))
        V = rng.standard_normal((N, d)) * 2 + rng.standard_normal(d)
        ones = np.ones(N // 128)
        Qs = F.fl32(Q * L).astype(np.float64)
        O = T.attention_tiled(Qs, ones, K, ones, V, np.zeros((N // 128, d)), np.ones(d),
                              p_mode="expcast", round_output=False, q_prescaled=True)
        Oe = T.attention_exact(Q, K, V)
        S_ = (Q @ K.T) / np.sqrt(d)
        u = (S_ - S_.max(1, keepdims=True)) * np.log2(np.e)
        p = np.exp2(u)
        p /= p.sum(1, keepdims=True)
        tau = np.where(u < g["underflow_u"], p, 0).sum(1)
        err = np.linalg.norm(O - Oe, axis=1)
        diam = A.diam2(V)
        assert np.all(err <= (g["tv_bound"] + 2 * tau + 1e-5) * diam)
        assert np.all(err[tau == 0] <= (g["tv_bound"] + 1e-5) * diam)


def test_output_error_split_eq2():
    """Sec. 3.1 Eq. 2: O - O_q = (P - P_q) V + P_q (V - V_q); each term vanishes when its
    operand is exact."""
    rng = np.random.default_rng(23)
    P = rng.random((6, 40))
    P /= P.sum(1, keepdims=True)
    Pq = P * (1 + 0.05 * rng.standard_normal(P.shape))
    V = rng.standard_normal((40, 8))
    Vq = V + 0.01 * rng.standard_normal(V.shape)
    prob, val = A.output_error_split(P, Pq, V, Vq)
    assert np.allclose(prob + val, P @ V - Pq @ Vq, rtol=0, atol=1e-13)
    assert np.allclose(prob, (P - Pq) @ V, atol=1e-15)
    p0, v0 = A.output_error_split(P, Pq, V, V)
    assert np.all(v0 == 0) and np.allclose(p0, P @ V - Pq @ V, atol=1e-13)
    p1, v1 = A.output_error_split(P, P, V, Vq)
    assert np.all(p1 == 0) and np.allclose(v1, P @ V - P @ Vq, atol=1e-13)
