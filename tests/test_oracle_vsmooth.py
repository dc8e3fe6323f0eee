"""Pins of V-Smooth's grouping, sort and quantisers (Sec. 3.2, Eq. 3-5; App. B)."""
import itertools

import numpy as np
import pytest

from oracle import formats as F
from oracle import vsmooth as S


def _example(golden):
    g = golden("vsmooth_4x4_example.txt")
    V = np.array([g["t0"], g["t1"], g["t2"], g["t3"]])
    return g, V


def test_4x4_example_sequence_and_sorted_blocks(golden):
    g, V = _example(golden)
    assert np.allclose(V[0:2].mean(0), g["seq_block_mean"], atol=1e-12)
    labels, C, J, _ = S.kmeans_lloyd(V, k=2, iters=5)
    perm = S.stable_argsort(labels)
    blocks = {frozenset(perm[i:i + 2].tolist()) for i in range(0, 4, 2)}
    page = [int(x) for x in g["perm"]]
    assert blocks == {frozenset(page[i:i + 2]) for i in range(0, 4, 2)}      # {t0,t2}, {t1,t3}
    mu = V[[1, 3]].mean(0)
    assert np.allclose(mu, g["sorted_block_mean_t1_t3"], atol=1e-12)
    res = V[1] - mu
    assert np.allclose(res, g["residual_t1"], atol=1e-12)
    assert np.abs(res).max() == pytest.approx(g["residual_abs_max"], abs=1e-12)


def _brute_force_kmeans(X, k):
    best = np.inf
    for lab in itertools.product(range(k), repeat=len(X)):
        lab = np.array(lab)
        if len(set(lab.tolist())) < k:
            continue
        J = sum(((X[lab == c] - X[lab == c].mean(0)) ** 2).sum() for c in range(k))
        if J < best:
            best, best_lab = J, lab
    return best, best_lab


@pytest.mark.parametrize("seed,n,k", [(0, 8, 2), (1, 9, 3), (2, 10, 2), (3, 7, 3)])
def test_kmeans_vs_brute_force(seed, n, k):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, 3)) + 3 * rng.integers(0, k, n)[:, None]
    Jopt, lab_opt = _brute_force_kmeans(X, k)
    labels, C, J, hist = S.kmeans_lloyd(X, k, iters=20)
    assert J >= Jopt - 1e-9
    assert all(hist[i + 1] <= hist[i] + 1e-12 for i in range(len(hist) - 1))      # Lloyd never increases J
    # started at the optimum's centroids, Lloyd stays there (fixed point) with J = Jopt
    Copt = np.stack([X[lab_opt == c].mean(0) for c in range(k)])
    lab2, C2, J2, _ = S.kmeans_lloyd(X, k, iters=3, C_init=Copt)
    assert J2 == pytest.approx(Jopt, rel=1e-12)
    assert np.array_equal(lab2, S.kmeans_assign(X, Copt))


def test_kmeans_fixed_point_properties():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((400, 8)) + 4 * rng.standard_normal((6, 8))[rng.integers(0, 6, 400)]
    labels, C, J, hist = S.kmeans_lloyd(X, 6, iters=60)
    D = ((X[:, None, :] - C[None, :, :]) ** 2).sum(-1)          # direct distances, not the expanded form
    assert np.array_equal(labels, D.argmin(1))                   # each point nearest its centroid
    for c in range(6):
        if (labels == c).any():
            assert np.allclose(C[c], X[labels == c].mean(0))      # each centroid its cluster mean
    assert J == pytest.approx(((X - C[labels]) ** 2).sum(), rel=1e-12)


def test_kmeans_ties_and_empty_clusters():
    X = np.array([[0.0, 0.0], [2.0, 0.0], [1.0, 0.0]])
    C0 = np.array([[0.0, 0.0], [2.0, 0.0], [50.0, 50.0]])
    lab = S.kmeans_assign(X, C0)
    assert lab.tolist() == [0, 1, 0]                             # the tie at x=1 goes to the lower index
    C1 = S.kmeans_update(X, lab, C0)
    assert np.array_equal(C1[2], C0[2])                          # empty cluster keeps its centroid
    assert np.allclose(C1[0], [0.5, 0.0])


def test_strided_init_rows():
    V = np.arange(20, dtype=float)[:, None] * np.ones((1, 2))
    C = S.kmeans_init_strided(V, 4)
    assert C[:, 0].tolist() == [2.0, 7.0, 12.0, 17.0]            # floor((c + 1/2) N / k)


def test_stable_sort_against_bucket_sort():
    rng = np.random.default_rng(6)
    for k in (1, 3, 64, 256):
        z = rng.integers(0, k, 5000).astype(np.int32)
        buckets = [[] for _ in range(k)]
        for i, c in enumerate(z.tolist()):
            buckets[c].append(i)
        ref = [i for b in buckets for i in b]
        assert S.stable_argsort(z).tolist() == ref
        off = S.cluster_offsets(z, k)
        assert off[0] == 0 and off[-1] == len(z)
        assert [off[c + 1] - off[c] for c in range(k)] == [len(b) for b in buckets]


def test_permuted_quantisers_blocks():
    rng = np.random.default_rng(7)
    N, d = 512, 128
    K = F.bf16_round(rng.standard_normal((N, d)) + 3.0)
    perm = rng.permutation(N)
    codes, sK = S.quantize_k(K, perm)
    Kp = F.fl32(K[perm]) - S.key_channel_mean(K)[None, :]
    deq = F.e4m3_decode(codes) * np.repeat(sK, 128)[:, None]
    # each block's largest entry lands in the top binade of E4M3 (power-of-two scale), every
    # element within half an E4M3 step
    for b in range(N // 128):
        blk = np.abs(F.e4m3_decode(codes[b * 128:(b + 1) * 128]))
        assert 224.0 <= blk.max() <= 448.0
    err = np.abs(deq - Kp)
    assert np.all(err <= np.abs(Kp) * 2.0 ** -4 + np.repeat(sK, 128)[:, None] * 2.0 ** -10 + 1e-12)
    # channel mean of the smoothed keys is ~0
    assert np.abs(Kp.mean(0)).max() < 1e-5


def test_quantize_v_demeaning():
    rng = np.random.default_rng(8)
    N, d = 384, 128
    V = F.bf16_round(rng.standard_normal((N, d)) * 0.3 + 5.0 * rng.standard_normal(d))
    perm = rng.permutation(N)
    q = S.quantize_v(V, perm)
    Vp = V[perm]
    mu = Vp.reshape(3, 128, d).mean(1)
    assert np.allclose(q["mu"], mu, rtol=1e-6)
    R = Vp.reshape(3, 128, d) - q["mu"][:, None, :]
    assert np.allclose(np.abs(R.reshape(N, d)).max(0) / 448.0, q["sV"], rtol=1e-6)
    # stored means: bf16 of mu / sV; dequantised V' = sV * (R-hat + mu~)
    assert np.allclose(q["mu_t"], q["mu"] / q["sV"][None, :], rtol=2 ** -8)
    rec = (F.e4m3_decode(q["codes"]).reshape(3, 128, d) + q["mu_t"][:, None, :]) * q["sV"]
    assert np.abs(rec.reshape(N, d) - Vp).max() < 0.08 * np.abs(R).max()
    q0 = S.quantize_v(V, perm, demean=False)
    assert np.all(q0["mu_t"] == 0) and np.allclose(q0["sV"], np.abs(Vp).max(0) / 448.0, rtol=1e-6)


def test_sorting_lowers_value_error_on_grouped_values():
    # The Table 1 trend on synthetic grouped values: k-means order + demeaning gives a
    # lower reconstruction error than sequence order + demeaning.
    rng = np.random.default_rng(9)
    N, d, G = 2048, 128, 16
    cent = rng.standard_normal((G, d)) * 3
    g = rng.integers(0, G, N)
    V = F.bf16_round(cent[g] + 0.3 * rng.standard_normal((N, d)))
    def rmse(perm):
        q = S.quantize_v(V, perm)
        rec = (F.e4m3_decode(q["codes"]).reshape(-1, 128, d) + q["mu_t"][:, None, :]) * q["sV"]
        return np.sqrt(((rec.reshape(N, d) - V[perm]) ** 2).mean())
    grp = S.vsmooth_group(V, k=G, iters=10)
    assert rmse(grp["perm"]) < 0.7 * rmse(np.arange(N))


def test_pow2_block_scale_definition():
    rng = np.random.default_rng(10)
    amax = np.concatenate([rng.uniform(0, 1e4, 10000), np.ldexp(448.0, np.arange(-20, 20)),
                           np.nextafter(np.ldexp(448.0, np.arange(-20, 20)), np.inf), [0.0, 1e-30]])
    s = S.pow2_scale(amax).astype(np.float64)
    m, e = np.frexp(s)
    assert np.all(m == 0.5)                                       # powers of two
    pos = amax > 0
    assert np.all(amax[pos] <= 448.0 * s[pos])                   # the block fits E4M3
    big = amax > 448.0 * 2.0 ** -101
    assert np.all(amax[big] > 224.0 * s[big])                    # and the scale is the smallest such
    assert np.all(s[pos & ~big] == 2.0 ** -100)                  # floor for all-but-zero blocks
    assert np.all(s[~pos] == 1.0)


def test_q_quantiser_folds_log2e_scale():
    rng = np.random.default_rng(11)
    Q = F.bf16_round(rng.standard_normal((256, 128)))
    codes, sQ = S.quantize_q(Q)
    L = np.float32(8.0 * np.log2(np.e) / np.sqrt(128))
    deq = F.e4m3_decode(codes) * np.repeat(sQ, 128)[:, None]
    Qs = F.fl32(Q) * L
    assert np.all(np.abs(deq - Qs) <= np.abs(Qs) * 2.0 ** -4 + np.repeat(sQ, 128)[:, None] * 2.0 ** -10)
    codes2, sQ2 = S.quantize_q(Q, softmax_scale=0.5)
    assert not np.array_equal(sQ2, sQ) or not np.array_equal(codes2, codes)


def test_quantize_v_zero_residual_and_constant_block():
    """Reading of the V scale for a channel with no residual (Sec. 3.2 Eq. 4; App. B): a channel
    that is constant inside every 128-row block has R = 0, so amax = 0 and s_V = 1, its codes are
    zero and its stored mean is bf16(mu) itself; a block constant in every channel contributes
    zero residual codes while the other blocks keep theirs."""
    rng = np.random.default_rng(12)
    N, d = 384, 128
    V = F.bf16_round(rng.standard_normal((N, d)))
    V[:, 5] = np.repeat(F.bf16_round(rng.standard_normal(3) * 4), 128)      # block-constant channel
    V[128:256] = F.bf16_round(rng.standard_normal(d))[None, :]            # constant block
    q = S.quantize_v(V, np.arange(N))
    assert q["sV"][5] == 1.0
    assert np.all(q["codes"][:, 5] == 0)
    assert np.array_equal(q["mu_t"][:, 5], F.bf16_round(V[::128, 5]))
    assert np.all((q["codes"][128:256] & 0x7F) == 0)
    assert np.any(q["codes"][:128] != 0) and np.any(q["codes"][256:] != 0)
    # per-channel scale is the residual's amax / 448 elsewhere (the E4M3 maximum is reached)
    live = np.arange(d) != 5
    assert np.all(np.abs(F.e4m3_decode(q["codes"][:, live])).max(0) == 448.0)


def test_key_channel_mean_closed_form():
    """The key channel mean (Sec. 2; App. B's centering statistics) of a matrix whose columns are
    known arithmetic sequences, and the centred rows' column sums."""
    N = 1024
    t = np.arange(N, dtype=np.float64)
    K = np.stack([t * 2.0 ** -6, -t * 2.0 ** -8 + 3.0, np.full(N, 7.25)] + [np.zeros(N)] * 125, axis=1)
    kbar = S.key_channel_mean(K)
    assert kbar[0] == np.float32((N - 1) / 2 * 2.0 ** -6)
    assert kbar[1] == np.float32(3.0 - (N - 1) / 2 * 2.0 ** -8)
    assert kbar[2] == np.float32(7.25) and np.all(kbar[3:] == 0)
