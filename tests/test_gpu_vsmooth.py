"""GPU parity of V-Smooth against the oracle: k-means assignment and update, the grouping
objective, and the K/V smoothing + E4M3 operands (bit-exact)."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import formats as F
from oracle import vsmooth as S

from gpu_util import DEV, bf16_dev, bf16_host_bits, config_inputs, note, values

pytestmark = pytest.mark.gpu

# The assignment takes its distances from bf16 x (bf16 hi + lo) products with float32
# accumulation: |error of v.c| <= 2^-16 ||v|| ||c|| + 128 * 2^-24 sum|v_i c_i|.  Labels are
# compared exactly wherever the oracle's best and second-best distances differ by more than
# TIE_TOL * (||v||^2 + ||c||^2); inside that band any of the tied centroids is valid.
TIE_TOL = 2.0 ** -13


def _check_labels(Vh, C, lab_gpu):
    D = S.sq_distances(Vh, C)
    best = D.min(1)
    scale = (Vh * Vh).sum(1) + (C * C).sum(1).max()
    ok = D[np.arange(len(Vh)), lab_gpu] <= best + TIE_TOL * scale
    assert ok.all(), f"{(~ok).sum()} labels not within tolerance of the nearest centroid"
    srt = np.sort(D, axis=1)
    clear = (srt[:, 1] - srt[:, 0]) > TIE_TOL * scale
    ref = np.argmin(D, axis=1)
    assert np.array_equal(lab_gpu[clear], ref[clear])
    return clear.mean()


@pytest.mark.parametrize("name,heads,k", [("tiny", None, 8), ("medium", [0, 5], 64), ("video", [3], 128),
                                          ("long", [1], 256), ("medium", [2], 5)])
def test_kmeans_assign(name, heads, k):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"kmeans assign {name} heads={heads} k={k}")
    Vd = bf16_dev(V)
    rng = np.random.default_rng(k)
    H = V.shape[1]
    C = np.stack([S.kmeans_init_strided(values(V[0, h]), k) + 0.05 * rng.standard_normal((k, 128))
                  for h in range(H)])[None].astype(np.float32)
    lab, dist = vc.vc_test_kmeans_assign(Vd, torch.from_numpy(C).to(DEV))
    lab, dist = lab.cpu().numpy(), dist.cpu().numpy()
    for h in range(H):
        Vh = values(V[0, h])
        frac = _check_labels(Vh, C[0, h].astype(np.float64), lab[0, h])
        assert frac > 0.99
        dref = ((Vh - C[0, h][lab[0, h]]) ** 2).sum(1)
        assert np.allclose(dist[0, h], dref, rtol=1e-4, atol=1e-3 * dref.mean())


@pytest.mark.parametrize("name,heads", [("tiny", None), ("medium", [0, 7])])
def test_group_one_iteration_matches_oracle(name, heads):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"group iters=1 {name}")
    g = vc.vc_vsmooth_group(bf16_dev(V), cfg.k, 1)
    lab, C, J = g["labels"].cpu().numpy(), g["C"].cpu().numpy(), g["J"].cpu().numpy()
    for h in range(V.shape[1]):
        Vh = values(V[0, h])
        C0 = S.kmeans_init_strided(Vh, cfg.k)
        _check_labels(Vh, C0, lab[0, h])
        ref_lab = S.kmeans_assign(Vh, C0)
        ref_C = S.kmeans_update(Vh, ref_lab, C0)
        if np.array_equal(ref_lab, lab[0, h]):
            # same labels: the centroids are float32 of the exact means, bit for bit
            assert np.array_equal(C[0, h], F.fl32(ref_C))
        assert J[0, h] == pytest.approx(S.kmeans_objective(Vh, ref_lab, ref_C), rel=1e-6)


@pytest.mark.parametrize("name,heads", [("tiny", None), ("medium", [0, 3]), ("video", [0]), ("long", [1])])
def test_group_full_objective_within_1e3(name, heads):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"group iters={cfg.iters} {name} heads={heads}")
    g = vc.vc_vsmooth_group(bf16_dev(V), cfg.k, cfg.iters)
    lab, perm, off = g["labels"].cpu().numpy(), g["perm"].cpu().numpy(), g["offsets"].cpu().numpy()
    C, J = g["C"].cpu().numpy(), g["J"].cpu().numpy()
    for h in range(V.shape[1]):
        Vh = values(V[0, h])
        ref = S.vsmooth_group(Vh, cfg.k, cfg.iters)
        assert J[0, h] == pytest.approx(ref["J"], rel=1e-3)
        # the GPU's own outputs are mutually consistent:
        z = lab[0, h]
        assert np.all(np.diff(z[perm[0, h]]) >= 0)                              # pi sorts the labels
        assert sorted(perm[0, h].tolist()) == list(range(cfg.N))                # pi is a permutation
        same = z[perm[0, h]][1:] == z[perm[0, h]][:-1]
        assert np.all(np.diff(perm[0, h])[same] > 0)                             # ties keep token order
        assert np.array_equal(off[0, h], np.concatenate([[0], np.cumsum(np.bincount(z, minlength=cfg.k))]))
        for c in np.unique(z)[:16]:
            assert np.array_equal(C[0, h, c], F.fl32(Vh[z == c].mean(0)))      # centroid = exact mean
        assert J[0, h] == pytest.approx(S.kmeans_objective(Vh, z, C[0, h].astype(np.float64)), rel=1e-9)


def test_group_warm_start_and_determinism():
    cfg, Q, K, V = config_inputs("medium", [1])
    Vd = bf16_dev(V)
    g1 = vc.vc_vsmooth_group(Vd, cfg.k, 4)
    g2 = vc.vc_vsmooth_group(Vd, cfg.k, 4)
    for key in ("labels", "perm", "offsets", "C", "J"):
        assert torch.equal(g1[key], g2[key]), key
    # warm start from the previous centroids (Sec. 3.2, "Unbalanced clusters cost little")
    w = vc.vc_vsmooth_group(Vd, cfg.k, 2, C_init=g1["C"])
    Vh = values(V[0, 0])
    ref = S.vsmooth_group(Vh, cfg.k, 2, C_init=g1["C"].cpu().numpy()[0, 0])
    assert w["J"].item() == pytest.approx(ref["J"], rel=1e-3)
    assert w["J"].item() <= g1["J"].item() * (1 + 1e-9)


def test_group_empty_clusters():
    """Four well-separated patterns of 256 rows, each periodic with period 128: the strided
    start rows floor((c + 1/2) N / k) of centroids 2i and 2i + 1 are identical rows, every
    token ties between them and goes to the lower index, so the odd clusters start empty
    (they keep their centroid and add nothing to J)."""
    rng = np.random.default_rng(7)
    N, k = 1024, 8
    base = 20.0 * rng.standard_normal((4, 128))
    wiggle = rng.standard_normal((128, 128))
    Vf = base[np.arange(N) // 256] + wiggle[np.arange(N) % 128]
    Vb = F.bf16_bits_from_value(Vf)[None, None]
    Vh = values(Vb[0, 0])
    assert np.array_equal(Vh[64], Vh[192])                                    # the tie is real
    for iters in (1, 3):
        note(f"group with empty clusters, iters={iters}")
        g = vc.vc_vsmooth_group(bf16_dev(Vb), k, iters)
        lab, off, C, J = (g["labels"].cpu().numpy()[0, 0], g["offsets"].cpu().numpy()[0, 0],
                          g["C"].cpu().numpy()[0, 0], g["J"].cpu().numpy()[0, 0])
        ref = S.vsmooth_group(Vh, k, iters)
        if iters == 1:
            assert np.all(np.diff(off)[1::2] == 0)                            # odd clusters empty
            C0 = S.kmeans_init_strided(Vh, k)
            assert np.array_equal(C[1::2], F.fl32(C0[1::2]))                  # and keep their start
        assert np.array_equal(lab, ref["labels"])
        assert J == pytest.approx(ref["J"], rel=1e-6)
        assert J == pytest.approx(S.kmeans_objective(Vh, lab, C.astype(np.float64)), rel=1e-9)


def test_group_small_ragged_batched():
    """B = 2, N = 256 (less than one 1024-token sort tile), k = 7 (centroid rows padded to 32):
    J per (b, h) against the oracle's Lloyd, and the outputs' own consistency."""
    rng = np.random.default_rng(11)
    B, H, N, k, iters = 2, 2, 256, 7, 4
    Vf = rng.standard_normal((B, H, N, 128)) + 3.0 * rng.standard_normal((B, H, 1, 128)) * (np.arange(N) % 5)[None, None, :, None]
    Vb = F.bf16_bits_from_value(Vf)
    g = vc.vc_vsmooth_group(bf16_dev(Vb), k, iters)
    lab, perm, off = g["labels"].cpu().numpy(), g["perm"].cpu().numpy(), g["offsets"].cpu().numpy()
    C, J = g["C"].cpu().numpy(), g["J"].cpu().numpy()
    for b in range(B):
        for h in range(H):
            Vh = values(Vb[b, h])
            ref = S.vsmooth_group(Vh, k, iters)
            assert J[b, h] == pytest.approx(ref["J"], rel=1e-3)
            z = lab[b, h]
            assert np.all(np.diff(z[perm[b, h]]) >= 0)
            assert sorted(perm[b, h].tolist()) == list(range(N))
            assert np.array_equal(off[b, h], np.concatenate([[0], np.cumsum(np.bincount(z, minlength=k))]))
            for c in np.unique(z):
                assert np.array_equal(C[b, h, c], F.fl32(Vh[z == c].mean(0)))
            assert J[b, h] == pytest.approx(S.kmeans_objective(Vh, z, C[b, h].astype(np.float64)), rel=1e-9)


def _oracle_perm(V, k, iters):
    return np.stack([S.vsmooth_group(values(V[0, h]), k, iters)["perm"] for h in range(V.shape[1])])[None]


@pytest.mark.parametrize("name,heads,perm_kind,no_demean",
                         [("tiny", None, "oracle", False), ("medium", [0, 4], "oracle", False),
                          ("medium", [1], "identity", False), ("medium", [2], "identity", True),
                          ("video", [5], "random", False), ("long", [2], "random", False)])
def test_demean_quant_bit_exact(name, heads, perm_kind, no_demean):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"demean_quant {name} heads={heads} perm={perm_kind} no_demean={no_demean}")
    H, N = V.shape[1], cfg.N
    if perm_kind == "oracle":
        perm = _oracle_perm(V, cfg.k, cfg.iters).astype(np.int32)
    elif perm_kind == "random":
        perm = np.stack([np.random.default_rng(h).permutation(N) for h in range(H)])[None].astype(np.int32)
    else:
        perm = None
    ops = vc.vc_vsmooth_demean_quant(bf16_dev(K), bf16_dev(V), None if perm is None else torch.from_numpy(perm).to(DEV),
                                     no_demean=no_demean)
    Kq, sK = ops["Kq"].cpu().numpy(), ops["sK"].cpu().numpy()
    Rq = vc.rq_tiled_to_natural(ops["Rq"]).cpu().numpy()
    mu_bits, sV = bf16_host_bits(ops["mu"]), ops["sV"].cpu().numpy()
    for h in range(H):
        p = np.arange(N) if perm is None else perm[0, h]
        kc, sk = S.quantize_k(values(K[0, h]), p)
        vq = S.quantize_v(values(V[0, h]), p, demean=not no_demean)
        assert np.array_equal(sK[0, h], sk)
        assert np.array_equal(Kq[0, h], kc)
        assert np.array_equal(sV[0, h], vq["sV"])
        assert np.array_equal(Rq[0, h], vq["codes"])
        assert np.array_equal(mu_bits[0, h], F.bf16_bits_from_value(vq["mu_t"]))


def test_zero_residual_channel_and_constant_block():
    """A channel constant inside every block has no residual: s_V = 1, zero codes, stored mean =
    bf16(mu) (the V scale's reading for a zero amax); a block constant in every channel gives zero
    codes.  GPU operands bit-exact against the oracle, attention within the parity tolerance."""
    from oracle import attention as T
    rng = np.random.default_rng(42)
    N = 512
    Vv = F.bf16_round(rng.standard_normal((N, 128)))
    Vv[:, 9] = np.repeat(F.bf16_round(rng.standard_normal(N // 128) * 3), 128)
    Vv[256:384] = F.bf16_round(rng.standard_normal(128))[None, :]
    Qv = F.bf16_round(rng.standard_normal((N, 128)))
    Kv = F.bf16_round(rng.standard_normal((N, 128)))
    bits = lambda x: F.bf16_bits_from_value(x)[None, None]
    perm = np.arange(N, dtype=np.int32)
    ops = vc.vc_vsmooth_demean_quant(bf16_dev(bits(Kv)), bf16_dev(bits(Vv)), torch.from_numpy(perm[None, None]).to(DEV))
    vq = S.quantize_v(Vv, perm)
    sV = ops["sV"].cpu().numpy()[0, 0]
    assert sV[9] == 1.0 and np.array_equal(sV, vq["sV"])
    R = vc.rq_tiled_to_natural(ops["Rq"]).cpu().numpy()[0, 0]
    assert np.array_equal(R, vq["codes"]) and np.all(R[:, 9] == 0) and np.all((R[256:384] & 0x7F) == 0)
    mu = values(bf16_host_bits(ops["mu"]))[0, 0]
    assert np.array_equal(mu, vq["mu_t"])
    O = values(bf16_host_bits(vc.vc_attn_fwd(bf16_dev(bits(Qv)), ops["Kq"], ops["sK"], ops["Rq"], ops["mu"],
                                             ops["sV"])))[0, 0]
    O_ref, _ = T.vc_attention_emulated(Qv, Kv, Vv, perm)
    assert T.rel_l2(O, O_ref) < 5e-3
