"""Pins of ExpCast-FP8 (Sec. 3.3, Eq. 7) and its error analysis (App. C, App. D)."""
import numpy as np
import pytest

from oracle import analysis as A
from oracle import expcast as E
from oracle import formats as F


def test_worked_example(golden):
    g = golden("expcast_worked_example.txt")
    u = g["u"]
    assert 8 * (u + 8) + 56 + E.BETA == pytest.approx(g["fma_value"], abs=1e-9)
    code = int(E.expcast_code(np.float32(u)))
    assert code == g["code"] == 8 * g["exponent_field"] + g["mantissa_field"]
    assert F.e4m3_decode(code) == g["decoded_value"]
    exact = 2.0 ** (u + 8)
    assert exact == pytest.approx(g["exact_value"], abs=0.05)
    assert g["binade_lo"] <= exact < g["binade_hi"]
    assert F.e4m3_decode(E.exp_then_cast_code(u)) == g["decoded_value"]


def test_constants(golden):
    g = golden("expcast_constants.txt")
    assert E.BETA == g["beta"]
    assert g["bias_term"] == 8 * 7
    # u = 0 (the row maximum) lands at code 120 = 2^8 = 256, the clip's upper end
    assert int(E.expcast_code(np.float32(0.0))) == g["code_max"] == 120
    assert F.e4m3_decode(120) == 256.0
    # u = -14 is the first normal code (2^-6 * 2^8 = 2^-14 * 256); below -15 + 0.35/8 only zero
    assert int(E.expcast_code(np.float32(-14.0))) == 8
    assert F.e4m3_decode(8) / 256.0 == 2.0 ** -14
    assert int(E.expcast_code(np.float32(-15.0))) == 0


def test_specials():
    u = np.array([np.nan, np.inf, -np.inf, 1.0, 1e30, -1e30, -0.0], np.float32)
    assert E.expcast_code(u).tolist() == [0, 120, 0, 120, 120, 0, 120]


def test_float32_form_matches_real_form_off_boundaries():
    rng = np.random.default_rng(2)
    u = np.concatenate([rng.uniform(-16, 0, 2_000_000), -np.abs(rng.standard_normal(100000)) * 1e-6]).astype(np.float32)
    c32 = E.expcast_code(u)
    creal = E.expcast_code_real(u.astype(np.float64))
    t = 8.0 * (u.astype(np.float64) + 8.0) + 56.0 + E.BETA
    near = np.abs(t - np.floor(t) - 0.5) < 2e-5
    assert np.array_equal(c32[~near], creal[~near])
    assert np.all(np.abs(c32.astype(int) - creal.astype(int)) <= 1)


def test_same_byte_fraction_over_a_doubling(golden):
    g = golden("expcast_constants.txt")
    # one doubling of the probability = one unit interval of u; Fig. 5b says every unit looks the same
    for lo in (-2.0, -5.0, -9.0):
        u = lo + (np.arange(1_000_000) + 0.5) / 1_000_000
        ce = E.expcast_code(u.astype(np.float32)).astype(int)
        cx = E.exp_then_cast_code(u).astype(int)
        diff = ce - cx
        frac = np.mean(diff == 0)
        assert frac == pytest.approx(g["same_byte_fraction"], abs=0.001)
        assert np.max(np.abs(diff)) == g["max_code_diff"]
    # per element at most one code: relative error of the decoded value below 7.5% (Sec. 3.3)
    rel = np.abs(E.decoded(E.expcast_code(u.astype(np.float32))) / np.exp2(u) - 1.0)
    assert rel.max() < g["max_elem_rel_error"]


def test_mitchell_error_and_minimax_shift(golden):
    g = golden("expcast_constants.txt")
    f = np.linspace(0.0, 1.0, 2_000_001)
    e = A.mitchell_e(f)
    assert e.min() == pytest.approx(0.0, abs=1e-12)
    assert e.max() == pytest.approx(g["mitchell_max"], abs=5e-5)
    shift = -e.max() / 2
    assert shift == pytest.approx(g["minimax_shift"], abs=5e-5)
    # Eq. 7 uses beta = -0.35, within 0.01 of the minimax shift (App. C, Fig. 8 caption)
    assert abs(E.BETA - shift) < 0.01


def test_eps_m_is_minus_mitchell_and_below_one_code():
    m = np.arange(8)
    eps = A.eps_m(m)
    assert np.all(np.abs(eps) < 1.0) and np.all(eps <= 0)
    # at f = log2(1 + m/8) the byte's offset eps(m) equals -e(f) (App. D after Eq. 9)
    f = np.log2(1.0 + m / 8.0)
    assert np.allclose(eps, -A.mitchell_e(f), atol=1e-12)


def test_ratio_bounds(golden):
    g = golden("expcast_constants.txt")
    lo, hi = A.ratio_bounds()
    # Eq. 11 prints the bounds to four decimals (the true minimum 0.928999.. rounds to 0.9290,
    # the true maximum 1.074535.. is printed as 1.0746); the TV bound holds for the true extremes
    assert abs(lo - g["ratio_min"]) < 1e-4 and abs(hi - g["ratio_max"]) < 1e-4
    assert A.tv_bound(lo, hi) < g["tv_bound"]
    f = np.linspace(0.0, 1.0, 1_000_001)[:-1]
    r = A.ratio_r(f)
    assert r.min() >= lo - 1e-9 and r.max() <= hi + 1e-9


def test_ratio_formula_matches_code_decode():
    # Eq. 10 restated through Eq. 7 and the E4M3 decode: in the normal range the decoded
    # ExpCast value over 2^u is r(frac(u + 8)).
    rng = np.random.default_rng(3)
    u = rng.uniform(-13.9, 0.0, 200000)
    u32 = u.astype(np.float32)
    u = u32.astype(np.float64)
    t = 8.0 * u32.astype(np.float64) + np.float64(E.C_F32)
    away = np.abs(t - np.floor(t) - 0.5) > 1e-4
    ratio = E.decoded(E.expcast_code(u32)) / np.exp2(u)
    z = u + 8.0
    f = z - np.floor(z)
    assert np.allclose(ratio[away], A.ratio_r(f[away], beta=float(E.C_F32) - 120.0), rtol=0, atol=1e-12)


def test_tv_bound(golden):
    g = golden("expcast_constants.txt")
    a, b = g["ratio_min"], g["ratio_max"]
    bound = A.tv_bound(a, b)
    assert bound < g["tv_bound"]
    assert bound == pytest.approx(0.036383, abs=2e-6)
    q = np.linspace(0, 1, 100001)
    assert A.tv_endpoint(q, a, b).max() == pytest.approx(bound, abs=1e-9)
    qstar = np.sqrt(a) / (np.sqrt(a) + np.sqrt(b))
    assert A.tv_endpoint(qstar, a, b) == pytest.approx(bound, abs=1e-12)
    assert 2 * bound < g["l1_bound"]


def _row_probs(u):
    w = np.exp2(u)
    wh = E.decoded(E.expcast_code(u.astype(np.float32)))
    return w / w.sum(), wh / wh.sum()


@pytest.mark.parametrize("spread", [2.0, 5.0, 9.0, 14.0, 30.0])
def test_prop31_row_bound(golden, spread):
    g = golden("expcast_constants.txt")
    rng = np.random.default_rng(int(spread * 10))
    d = 16
    for _ in range(200):
        n = int(rng.integers(4, 512))
        u = -rng.uniform(0, spread, n)
        u[rng.integers(n)] = 0.0                             # row maximum subtracted
        u = u.astype(np.float32).astype(np.float64)
        p, ph = _row_probs(u)
        tail = u < g["underflow_u"]
        tau = max(p[tail].sum(), ph[tail].sum())
        t = A.tv(p, ph)
        if not tail.any():
            assert t < g["tv_bound"]
        assert t < g["tv_bound"] + tau
        V = rng.standard_normal((n, d))
        assert np.linalg.norm(ph @ V - p @ V) <= (g["tv_bound"] + tau) * A.diam2(V) + 1e-12


def test_energy_identity_eq5():
    rng = np.random.default_rng(4)
    Vb = rng.standard_normal((128, 32)) + rng.standard_normal(32)
    mu, R, e_v, e_r, share = A.block_energy_split(Vb)
    c = rng.standard_normal(32)
    lhs = ((Vb - c[None, :]) ** 2).sum()
    assert lhs == pytest.approx(e_r + 128 * ((c - mu) ** 2).sum(), rel=1e-12)
    assert e_r == pytest.approx(e_v - 128 * mu @ mu, rel=1e-12)
    assert 0.0 <= share <= 1.0
    # with c = 0 the identity gives the mean's share of the block energy as 1 - ||R||^2 / ||V||^2
    assert share == pytest.approx(1.0 - e_r / e_v, rel=1e-12)


def test_diam2_closed_form():
    # App. D Eq. 15: the largest distance between two rows (a 3-4-5 triangle, and a cube's diagonal)
    assert A.diam2(np.array([[0.0, 0.0], [3.0, 4.0], [1.0, 1.0]])) == pytest.approx(5.0, rel=1e-15)
    cube = np.array([[i, j, k] for i in (0, 1) for j in (0, 1) for k in (0, 1)], dtype=float)
    assert A.diam2(cube) == pytest.approx(np.sqrt(3.0), rel=1e-15)


def test_mean_storage_cost(golden):
    g = golden("expcast_constants.txt")
    assert 16 / g["block_rows"] == g["mean_bits_per_element"]
