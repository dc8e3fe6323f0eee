"""Pins of the oracle's diagnostics (CPU): the static cube order, Eq. 5's block share, the value
error by token order, Eq. 2's split and the row total variation of Sec. 3.3."""
import numpy as np

from oracle import analysis as A
from oracle import diagnostics as D
from oracle import formats as F
from oracle import vsmooth as S


def test_static_cube_order_is_a_permutation_of_whole_cubes():
    grid = (4, 16, 24)
    N = 4 * 16 * 24
    order = D.static_cube_order(grid, N)
    assert sorted(order.tolist()) == list(range(N))
    t, y, x = order // (16 * 24), (order // 24) % 16, order % 24
    for b in range(N // 128):       # every 128 consecutive tokens are one 2 x 8 x 8 cube
        s = slice(128 * b, 128 * (b + 1))
        assert len(set(zip((t[s] // 2).tolist(), (y[s] // 8).tolist(), (x[s] // 8).tolist()))) == 1
        assert len(set(zip(t[s].tolist(), y[s].tolist(), x[s].tolist()))) == 128


def test_static_cube_order_continues_a_partial_frame():
    grid = (3, 8, 8)
    N = 3 * 64 + 64 + 40                # one full extra frame of 64 and 40 tokens beyond it
    order = D.static_cube_order(grid, N)
    assert sorted(order.tolist()) == list(range(N))
    assert order[:128].tolist() == list(range(128))      # frames 0 and 1 form the first cube


def test_block_mean_share_extremes():
    rng = np.random.default_rng(0)
    row = rng.standard_normal(128)
    same = np.tile(row, (256, 1))
    assert abs(D.block_mean_share(same) - 1.0) < 1e-12          # identical rows: all energy in the mean
    half = rng.standard_normal((64, 128))
    sym = np.concatenate([half, -half])                            # zero-mean block
    assert D.block_mean_share(sym) < 1e-24
    # the share against a brute-force minimum over shifted means (Eq. 5: the mean leaves the least)
    Vb = rng.standard_normal((128, 8)) + 3.0
    best = min(((Vb - c) ** 2).sum() for c in [Vb.mean(0) + 0.01 * rng.standard_normal(8) for _ in range(50)])
    mu, R, e_v, e_r, share = A.block_energy_split(Vb)
    assert e_r <= best
    assert abs(D.block_mean_share(Vb) - share) < 1e-15


def test_value_error_of_grid_values_is_zero_and_bounded_otherwise():
    # block-constant rows whose means are bf16 values with s_V = 1: the residual is 0, so the
    # dequantised operand is V itself
    rng = np.random.default_rng(1)
    means = F.bf16_round(rng.standard_normal((4, 128)))
    V = np.repeat(means, 128, axis=0)
    assert D.value_rel_mse(V, None) == 0.0
    # values of one binade per channel stay in E4M3's normal range after the per-channel scale
    # (amax / 448 puts them in [224, 448]): relative error at most 2^-4 per element
    W = F.bf16_round(rng.uniform(1.0, 2.0, size=(512, 128)))
    e = D.value_rel_mse(W, None, demean=False)
    assert 0.0 < e <= 2.0 ** -8
    # without demeaning the per-channel scale sees all tokens, so the order does not matter
    p = rng.permutation(512)
    assert abs(D.value_rel_mse(W, p, demean=False) - e) < 1e-15


def test_value_error_falls_with_value_grouping():
    rng = np.random.default_rng(2)
    cent = rng.standard_normal((8, 128)) * 3.0
    lab = rng.integers(0, 8, 1024)
    V = F.bf16_round(cent[lab] + 0.1 * rng.standard_normal((1024, 128)))
    seq = D.value_rel_mse(V, None)
    grp = D.value_rel_mse(V, S.stable_argsort(lab))
    assert grp < 0.5 * seq
    assert abs(D.value_rel_mse(V, None, rotate=True) / seq - 1.0) < 0.5   # rotation: same order of error


def test_eq2_terms_add_up_and_value_term_vanishes_on_grid_values():
    rng = np.random.default_rng(3)
    N = 512
    Q = F.bf16_round(rng.standard_normal((N, 128)))
    K = F.bf16_round(rng.standard_normal((N, 128)))
    rows = np.arange(0, N, 7)
    means = F.bf16_round(rng.standard_normal((N // 128, 128)))
    Vg = np.repeat(means, 128, axis=0)
    t = D.output_error_terms(Q, K, Vg, None, rows)
    assert t["value_term"] < 1e-12 and t["prob_term"] > 1e-4
    assert abs(t["total"] - t["prob_term"]) < 1e-9
    V = F.bf16_round(rng.standard_normal((N, 128)))
    t = D.output_error_terms(Q, K, V, None, rows)
    assert t["value_term"] > 1e-4
    assert t["total"] <= t["prob_term"] + t["value_term"] + 1e-12          # triangle inequality
    assert t["total"] >= abs(t["prob_term"] - t["value_term"]) - 1e-12


def test_row_tv_obeys_prop31_and_the_e4m3_bound():
    rng = np.random.default_rng(4)
    N = 1024
    Q = F.bf16_round(0.5 * rng.standard_normal((N, 128)))
    K = F.bf16_round(0.5 * rng.standard_normal((N, 128)))
    r = D.row_tv(Q, K, np.arange(0, N, 5))
    assert np.all(r["tau"] == 0.0)                        # mild scores: nothing underflows
    assert r["tv_expcast"].max() < A.tv_bound(0.9290, 1.0746)     # Prop. 3.1 (Eq. 8)
    assert r["tv_exp_then_cast"].max() < A.tv_bound(1 - 2.0 ** -4, 1 + 2.0 ** -4)
    assert r["tv_expcast"].min() > 0.0
    # peaked rows: some mass underflows, and the bound extends by tau (Eq. 14)
    r = D.row_tv(F.bf16_round(8.0 * Q), K, np.arange(0, N, 5))
    assert r["tau"].max() > 0.0
    assert np.all(r["tv_expcast"] < A.tv_bound(0.9290, 1.0746) + r["tau"])
