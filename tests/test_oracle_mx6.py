"""Pins of the 6-bit (MX E2M3) variant of the MX V-Smooth oracle: the element format against the
published OCP MX FP6 E2M3 value table and brute-force rounding, the scale rule with 7.5 as the
largest element, the quantisers' half-step bound, the tiled recurrence against exact attention,
the mean-restore identity with quantised P, and 6 bits against 4 bits on the same operands."""
import numpy as np
import pytest

import synth
from oracle import attention as T
from oracle import formats as F
from oracle import mx4 as M

# OCP Microscaling Formats (MX) v1.0, FP6 E2M3: the 32 magnitudes of codes 0..31 (subnormals
# m/8 for exponent field 0; then 1.000-1.875, 2.00-3.75, 4.0-7.5 in steps of 1/8, 1/4, 1/2)
E2M3_TABLE = ([m / 8 for m in range(8)] + [1 + m / 8 for m in range(8)] + [2 + m / 4 for m in range(8)]
              + [4 + m / 2 for m in range(8)])


def test_e2m3_value_table():
    vals = F.e2m3_decode(np.arange(64))
    assert vals[:32].tolist() == E2M3_TABLE
    assert (-vals[32:]).tolist() == E2M3_TABLE
    assert np.all(np.signbit(vals[32:]))
    assert E2M3_TABLE[-1] == F.E2M3_MAX == 7.5


def test_e2m3_encode_brute_force():
    rng = np.random.default_rng(0)
    mids = [(a + b) / 2 for a, b in zip(E2M3_TABLE[:-1], E2M3_TABLE[1:])]
    xs = np.concatenate([rng.uniform(-9, 9, 20000), mids, np.negative(mids), E2M3_TABLE,
                         [7.75, 100.0, -1e9, 1e-30, -1e-30, 0.0, -0.0]])
    codes = F.e2m3_encode(xs)
    for x, c in zip(xs, codes):
        a = min(abs(x), 7.5)
        d = [abs(a - v) for v in E2M3_TABLE]
        best = min(d)
        cand = [i for i in range(32) if d[i] == best]
        want = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        if np.signbit(x):
            want |= 0x20
        assert c == want, (x, c, want)


@pytest.mark.parametrize("amax,E", [(7.5, 0), (np.nextafter(7.5, 8.0), 1), (3.75, -1), (6.0, 0),
                                    (1.0, -2), (0.9375, -3), (1e-40, -100), (0.0, 0), (7.5 * 2.0 ** 9, 9)])
def test_mx_exponent_e2m3_examples(amax, E):
    assert M.mx_exponent(amax, "e2m3") == E


def test_mx_exponent_e2m3_defining_inequality():
    a = np.exp(np.random.default_rng(1).uniform(-40, 40, 5000))
    E = M.mx_exponent(a, "e2m3")
    assert np.all(a <= 7.5 * np.ldexp(1.0, E)) and np.all(a > 7.5 * np.ldexp(1.0, E - 1))


def test_row_group_quantiser_e2m3_error_bound():
    rng = np.random.default_rng(2)
    X = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 1)))).astype(np.float32)
    codes, E = M.quantize_row_groups(X, "e2m3")
    assert codes.max() < 64
    D = M.dequant_row_groups(codes, E, "e2m3")
    scale = np.repeat(np.ldexp(1.0, E), 32, axis=1)
    u = np.abs(X) / scale
    half = np.where(u < 2, 1 / 16, np.where(u < 4, 1 / 8, 1 / 4)) * scale    # half the E2M3 spacing
    assert np.all(np.abs(D - X) <= half)
    assert np.all(np.abs(X) <= 7.5 * scale)
    assert np.all(np.abs(X).reshape(64, 4, 32).max(2) > 3.75 * np.ldexp(1.0, E))


def test_p_quantiser_e2m3_brute_force():
    rng = np.random.default_rng(3)
    P = np.exp2(-rng.uniform(0, 12, (16, 128)))
    got = M.quantize_p4(P, "e2m3")
    for r in range(16):
        for g in range(4):
            cols = [k for k in range(128) if 2 * (k // 64) + ((k >> 2) & 1) == g]
            amax = P[r, cols].max()
            E = int(np.ceil(np.log2(amax / 7.5)))
            while amax > 7.5 * 2.0 ** E:
                E += 1
            while amax <= 7.5 * 2.0 ** (E - 1):
                E -= 1
            for k in cols:
                y = P[r, k] / 2.0 ** E
                d = [abs(y - v) for v in E2M3_TABLE]
                best = min(d)
                cand = [i for i in range(32) if d[i] == best]
                want = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
                assert got[r, k] == E2M3_TABLE[want] * 2.0 ** E


def _small(seed):
    cfg = synth.get_config("medium", H=1, N=1024, grid=(1, 32, 32), k_true=16)
    Q, K, V = (synth.bits_to_f32(x[0, 0]).astype(np.float64) for x in synth.make_qkv(cfg))
    return Q, K, V


def test_e2m3_tiled_exact_mode_is_exact_attention():
    Q, K, V = _small(0)
    N = Q.shape[0]
    perm = np.random.default_rng(4).permutation(N)
    L4 = float(M.log2e_scale4(None))
    rows = np.arange(0, N, 9)
    mu = np.zeros((N // 128, 128))
    O = M.attention_tiled_mx4(Q * L4, K[perm], V[perm], mu, rows, "exact", False, "e2m3")
    assert T.rel_l2(O, T.attention_exact(Q, K, V, rows=rows)) < 1e-6


def test_e2m3_mean_restore_identity_with_quantised_p():
    Q, K, V = _small(1)
    N = Q.shape[0]
    perm = np.arange(N)
    qc, qE = M.quantize_q4(Q, fmt="e2m3")
    kc, kE = M.quantize_k4(K, perm, fmt="e2m3")
    vq = M.quantize_v4(V, perm, fmt="e2m3")
    Qv, Kv = M.dequant_row_groups(qc, qE, "e2m3"), M.dequant_row_groups(kc, kE, "e2m3")
    Rv = M.dequant_v4(vq["codes"], vq["E"], "e2m3")
    rows = np.arange(0, N, 11)
    with_mean = M.attention_tiled_mx4(Qv, Kv, Rv, vq["mu_b"], rows, "mx4", False, "e2m3")
    folded = M.attention_tiled_mx4(Qv, Kv, Rv + np.repeat(vq["mu_b"], 128, axis=0), np.zeros_like(vq["mu_b"]),
                                   rows, "mx4", False, "e2m3")
    assert np.max(np.abs(with_mean - folded)) < 1e-9 * np.max(np.abs(folded))


def test_six_bits_closer_to_exact_than_four():
    Q, K, V = _small(2)
    rows = np.arange(0, Q.shape[0], 5)
    exact = T.attention_exact(Q, K, V, rows=rows)
    e4 = T.rel_l2(M.vc_attention_mx4_emulated(Q, K, V, None, rows=rows)[0], exact)
    e6 = T.rel_l2(M.vc_attention_mx4_emulated(Q, K, V, None, rows=rows, fmt="e2m3")[0], exact)
    assert e6 < 0.5 * e4
