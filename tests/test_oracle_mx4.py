"""Pins of the 4-bit (MX E2M1) V-Smooth oracle (Sec. 3.2 after Eq. 4; Sec. 4.1 "Implementation";
App. A "Scope of ExpCast-FP8"; App. B): the element format against its published value table
and brute-force rounding, the power-of-two scale rule, the key groups against the PV operand
order, the tiled recurrence against exact attention, the mean-restore identity, and V-Smooth's
gain at 4 bits."""
import numpy as np
import pytest

import synth
from oracle import attention as T
from oracle import formats as F
from oracle import mx4 as M
from oracle import vsmooth as S

# OCP Microscaling Formats (MX) v1.0, FP4 E2M1: the eight magnitudes of codes 0..7
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_value_table():
    vals = F.e2m1_decode(np.arange(16))
    assert vals[:8].tolist() == E2M1_TABLE
    assert (-vals[8:]).tolist() == E2M1_TABLE
    assert np.all(np.signbit(vals[8:]))


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(0)
    mids = [(a + b) / 2 for a, b in zip(E2M1_TABLE[:-1], E2M1_TABLE[1:])]
    xs = np.concatenate([rng.uniform(-7, 7, 20000), mids, np.negative(mids), E2M1_TABLE,
                         [6.5, 100.0, -1e9, 1e-30, -1e-30, 0.0, -0.0]])
    codes = F.e2m1_encode(xs)
    for x, c in zip(xs, codes):
        a = min(abs(x), 6.0)
        d = [abs(a - v) for v in E2M1_TABLE]
        best = min(d)
        cand = [i for i in range(8) if d[i] == best]
        want = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        if np.signbit(x):
            want |= 8
        assert c == want, (x, c, want)


@pytest.mark.parametrize("amax,E", [(6.0, 0), (np.nextafter(6.0, 7.0), 1), (3.0, -1),
                                    (np.nextafter(3.0, 4.0), 0), (1.0, -2), (0.75, -3), (1.5, -2),
                                    (1e-40, -100), (0.0, 0), (6.0 * 2.0 ** 20, 20)])
def test_mx_exponent_examples(amax, E):
    assert M.mx_exponent(amax) == E


def test_mx_exponent_defining_inequality():
    a = np.exp(np.random.default_rng(1).uniform(-40, 40, 5000))
    E = M.mx_exponent(a)
    assert np.all(a <= 6.0 * np.ldexp(1.0, E)) and np.all(a > 6.0 * np.ldexp(1.0, E - 1))


def test_row_group_quantiser_error_bound():
    rng = np.random.default_rng(2)
    X = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 1)))).astype(np.float32)
    codes, E = M.quantize_row_groups(X)
    D = M.dequant_row_groups(codes, E)
    scale = np.repeat(np.ldexp(1.0, E), 32, axis=1)
    u = np.abs(X) / scale
    half = np.where(u < 2, 0.25, np.where(u < 4, 0.5, 1.0)) * scale      # half the E2M1 spacing
    assert np.all(np.abs(D - X) <= half)
    assert np.all(np.abs(X) <= 6.0 * scale)                              # no element saturates
    assert np.all(np.abs(X).reshape(64, 4, 32).max(2) > 3.0 * np.ldexp(1.0, E))   # smallest scale


def test_key_groups_are_the_pv_operand_slot_groups():
    # slot s = 64 p + 32 g + i of a tile holds key 64 p + 32 (i/16) + 8 ((i%16)/4) + 4 g + i%4
    for s in range(128):
        p, g, i = s // 64, (s // 32) % 2, s % 32
        key = 64 * p + 32 * (i // 16) + 8 * ((i % 16) // 4) + 4 * g + i % 4
        assert M.key_group(key) == s // 32
    assert np.bincount(M.key_group(np.arange(128))).tolist() == [32] * 4


def test_v4_quantiser_groups_and_bound():
    cfg, = [synth.get_config("medium", H=1, N=1024, grid=(1, 32, 32), k_true=16)]
    _, _, V = synth.make_qkv(cfg)
    Vh = F.bf16_value_from_bits(V[0, 0])
    perm = np.random.default_rng(3).permutation(1024)
    vq = M.quantize_v4(Vh, perm)
    Vp = F.fl32(Vh[perm]).astype(np.float64)
    R = (Vp.reshape(8, 128, 128) - vq["mu"][:, None, :].astype(np.float64)).reshape(1024, 128)
    D = M.dequant_v4(vq["codes"], vq["E"])
    grp = M.key_group(np.arange(128))
    scale = np.transpose(np.ldexp(1.0, vq["E"])[:, :, grp], (0, 2, 1)).reshape(1024, 128)
    assert np.all(np.abs(D - R) <= scale)                                # at most one 2^E step
    assert np.all(np.abs(R) <= 6.0 * scale)
    for t in range(8):                                                   # E is each group's own
        for g in range(4):
            rows = 128 * t + np.nonzero(grp == g)[0]
            assert np.array_equal(vq["E"][t, :, g], M.mx_exponent(np.abs(R[rows]).max(0)))
    assert np.array_equal(vq["mu_b"], F.bf16_round(vq["mu"]))


def test_tiled_exact_mode_is_exact_attention():
    rng = np.random.default_rng(4)
    N = 384
    Q = F.bf16_round(rng.standard_normal((N, 128)))
    K = F.bf16_round(rng.standard_normal((N, 128)) + 1.0)
    V = F.bf16_round(rng.standard_normal((N, 128)) + 2.0 * rng.standard_normal(128))
    perm = rng.permutation(N)
    mu = S.block_means(V[perm]).astype(np.float64)
    R = V[perm] - np.repeat(mu, 128, axis=0)
    L4 = np.log2(np.e) / np.sqrt(128)
    O = M.attention_tiled_mx4(Q * L4, K[perm], R, mu, p_mode="exact", round_output=False)
    assert np.allclose(O, T.attention_exact(Q, K, V), atol=1e-12)


def test_mean_restore_identity_with_4bit_p():
    """With P quantised, P^(R + 1 mu) = P^ R + r mu needs r = the row sum of the dequantised P."""
    rng = np.random.default_rng(5)
    N = 256
    Qv = rng.standard_normal((N, 128)) * 0.2
    Kv = rng.standard_normal((N, 128))
    Vp = rng.standard_normal((N, 128)) + 3.0
    mu = Vp.reshape(2, 128, 128).mean(1)
    R = Vp - np.repeat(mu, 128, axis=0)
    a = M.attention_tiled_mx4(Qv, Kv, R, mu, round_output=False)
    b = M.attention_tiled_mx4(Qv, Kv, Vp, np.zeros_like(mu), round_output=False)
    assert np.allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())


def _rows_err(name, heads, demean, perm_kind, hadamard=False, rows=None):
    cfg = synth.get_config(name)
    Q, K, V = synth.make_qkv(cfg, heads)
    errs = []
    for h in range(len(heads)):
        Qh, Kh, Vh = (F.bf16_value_from_bits(x[0, h]) for x in (Q, K, V))
        if perm_kind == "kmeans":
            perm = S.vsmooth_group(Vh, cfg.k, 5)["perm"]
        else:
            perm = np.arange(cfg.N)
        r = np.arange(0, cfg.N, cfg.N // 128) if rows is None else rows
        O, _ = M.vc_attention_mx4_emulated(Qh, Kh, Vh, perm, rows=r, demean=demean, hadamard=hadamard)
        errs.append(T.rel_l2(O, T.attention_exact(Qh, Kh, Vh, rows=r)))
    return float(np.mean(errs))


def test_vsmooth_gain_at_4_bits():
    """Sec. 4.2: at 4 bits V-Smooth improves on the matched-precision baseline.  Two heads of the
    video workload (clusters of ~550 tokens, several blocks each), grouped + demeaned vs
    sequence-order unsmoothed, against exact attention: the value operand's own error (Q, K, P
    exact) drops by more than 2x, the whole 4-bit path's error by more than 10 %.  (With
    clusters of about one block, as in the medium workload, the per-32-key microscales already
    adapt and the gain vanishes.)"""
    cfg = synth.get_config("video")
    Q, K, V = synth.make_qkv(cfg, [0, 1])
    rows = np.arange(0, cfg.N, cfg.N // 128)
    L4 = float(M.log2e_scale4(None))
    e = {"vs": [], "base": [], "vs_v": [], "base_v": []}
    for h in range(2):
        Qh, Kh, Vh = (F.bf16_value_from_bits(x[0, h]) for x in (Q, K, V))
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        for name, perm, demean in (("vs", S.vsmooth_group(Vh, cfg.k, 5)["perm"], True),
                                   ("base", np.arange(cfg.N), False)):
            O, ops = M.vc_attention_mx4_emulated(Qh, Kh, Vh, perm, rows=rows, demean=demean)
            e[name].append(T.rel_l2(O, exact))
            Ov = M.attention_tiled_mx4(Qh * L4, Kh[perm], M.dequant_v4(ops["codes"], ops["E"]), ops["mu_b"],
                                       rows, p_mode="exact")
            e[name + "_v"].append(T.rel_l2(Ov, exact))
    m = {k: float(np.mean(v)) for k, v in e.items()}
    assert m["vs_v"] < 0.5 * m["base_v"]
    assert m["vs"] < 0.9 * m["base"]


def test_rotation_at_4_bits_on_channel_outliers():
    e_rot = _rows_err("qk_outlier", [0], True, "identity", hadamard=True)
    e_plain = _rows_err("qk_outlier", [0], True, "identity", hadamard=False)
    assert e_rot < e_plain


def _brute_p4(P):
    """Brute-force MX E2M1 quantiser of non-negative rows (rows, 128 keys): per (row, 32-key group
    of key_group) the exponent is found by scanning E upwards for the first 6 * 2^E >= group max
    (E >= -100; 0 for an all-zero group), then each element takes the nearest of the eight E2M1
    magnitudes times 2^E, a tie going to the even code (the OCP MX E2M1 table)."""
    out = np.empty_like(P)
    grp = M.key_group(np.arange(P.shape[1]))
    for r in range(P.shape[0]):
        for g in range(4):
            cols = np.nonzero(grp == g)[0]
            amax = P[r, cols].max()
            E = -100
            if amax == 0:
                E = 0
            else:
                while 6.0 * 2.0 ** E < amax:
                    E += 1
            for c in cols:
                x = P[r, c] / 2.0 ** E
                dist = [abs(x - v) for v in E2M1_TABLE]
                best = min(dist)
                cand = [i for i in range(8) if dist[i] == best]
                i = cand[0] if len(cand) == 1 else [j for j in cand if j % 2 == 0][0]
                out[r, c] = E2M1_TABLE[i] * 2.0 ** E
    return out


def test_quantize_p4_brute_force():
    """oracle.mx4.quantize_p4 equals the brute-force per-(row, 32-key group) quantiser, including
    exact ties, all-zero groups, tiny groups at the exponent floor and groups spanning many binades."""
    rng = np.random.default_rng(30)
    P = np.exp2(rng.uniform(-30, 0, (24, 128)))
    P[0] = 0.0                                                     # all groups zero
    P[1, :] = np.exp2(-140.0)                                      # below the exponent floor
    P[2] = np.exp2(rng.uniform(-3, 0, 128))                        # narrow range
    grp = M.key_group(np.arange(128))
    for r in range(3, 9):                                          # exact midpoints between codes
        for g in range(4):
            cols = np.nonzero(grp == g)[0]
            E = int(rng.integers(-20, 0))
            k = rng.integers(0, 7, len(cols))
            P[r, cols] = (np.array(E2M1_TABLE)[k] + np.array(E2M1_TABLE)[k + 1]) / 2 * 2.0 ** E
            P[r, cols[0]] = 6.0 * 2.0 ** E                         # the group maximum sets E exactly
    P[9, grp == 1] = 0.0                                           # one zero group in a live row
    assert np.array_equal(M.quantize_p4(P), _brute_p4(P))


def test_mx4_recurrence_closed_form():
    """The tiled 4-bit recurrence (Eq. 1 with Eq. 6's mean term) against its closed form: with
    m_j the running maximum after tile j and P_j the brute-force quantised 2^(S_j - m_j),
    O = sum_j 2^(m_j - m_T) (P_j R_j + r_j mu_j) / sum_j 2^(m_j - m_T) r_j, r_j = P_j 1."""
    rng = np.random.default_rng(31)
    N, d, nq = 512, 128, 6
    Qv = rng.standard_normal((nq, d)) * 0.4
    Kv = rng.standard_normal((N, d))
    Kv[300] *= 4.0                                                 # moves the running maximum late
    Rv = rng.standard_normal((N, d))
    mu = rng.standard_normal((N // 128, d)) * 3
    O = M.attention_tiled_mx4(Qv, Kv, Rv, mu, p_mode="mx4", round_output=False)
    m = -np.inf
    terms = []
    for j in range(N // 128):
        s = F.fl32(Qv @ Kv[128 * j:128 * (j + 1)].T).astype(np.float64)
        m = np.maximum(m, s.max(1))
        P = _brute_p4(F.fl32(np.exp2(F.fl32(s - m[:, None]).astype(np.float64))).astype(np.float64))
        terms.append((m.copy(), P @ Rv[128 * j:128 * (j + 1)] + P.sum(1)[:, None] * mu[j][None, :], P.sum(1)))
    mT = terms[-1][0]
    num = sum(np.exp2(mj - mT)[:, None] * a for mj, a, _ in terms)
    den = sum(np.exp2(mj - mT) * r for mj, _, r in terms)
    assert np.allclose(O, num / den[:, None], rtol=1e-12, atol=0)


def test_q4_k4_quantisers_fold_slope_and_centre():
    """The 4-bit Q path multiplies by L4 = fl32(log2(e)/sqrt(d)) before its per-32-channel
    quantiser, and the K path centres by the key channel mean and gathers by pi: each dequantised
    element lies within half an E2M1 step (at most the group scale, the half step of the 4..6
    binade) of fl32(Q) L4, resp. K[pi] - kbar."""
    rng = np.random.default_rng(32)
    N = 256
    Q = F.bf16_round(rng.standard_normal((N, 128)))
    K = F.bf16_round(rng.standard_normal((N, 128)) + 2.0 * rng.standard_normal(128))
    perm = rng.permutation(N)
    qc, qE = M.quantize_q4(Q)
    X = F.fl32(Q).astype(np.float64) * float(np.float32(np.log2(np.e) / np.sqrt(128)))
    sc = np.repeat(np.ldexp(1.0, qE), 32, axis=1)
    assert np.all(np.abs(M.dequant_row_groups(qc, qE) - X) <= sc + 1e-6 * np.abs(X))
    kc, kE = M.quantize_k4(K, perm)
    Kc = F.fl32(K[perm]).astype(np.float64) - S.key_channel_mean(K).astype(np.float64)[None, :]
    sc = np.repeat(np.ldexp(1.0, kE), 32, axis=1)
    assert np.all(np.abs(M.dequant_row_groups(kc, kE) - Kc) <= sc + 1e-6 * np.abs(Kc))
    assert np.abs(Kc.mean(0)).max() < 1e-5


def test_k4_rotated_keys_are_the_centred_keys_times_h_over_d():
    """With the QK rotation the 4-bit K path quantises fl32((K[pi] - kbar) H) per 32-channel group
    and stores its exponent lowered by 7, so the dequantised keys are (K[pi] - kbar) H / 128 = the
    centred keys times H^-T, within half an E2M1 step of the stored group scale (at most the
    scale)."""
    from oracle import rotation as R
    rng = np.random.default_rng(33)
    N = 256
    K = F.bf16_round(rng.standard_normal((N, 128)) + 2.0 * rng.standard_normal(128))
    perm = rng.permutation(N)
    kc, kE = M.quantize_k4(K, perm, hadamard=True)
    Kc = (F.fl32(K[perm]) - S.key_channel_mean(K)[None, :]).astype(np.float32)
    want = R.rotate(Kc).astype(np.float64) / 128.0
    sc = np.repeat(np.ldexp(1.0, kE), 32, axis=1)
    assert np.all(np.abs(M.dequant_row_groups(kc, kE) - want) <= sc)
    assert np.all(np.abs(want).reshape(N, 4, 32).max(2) > 3.0 * np.ldexp(1.0, kE))   # the smallest scale
