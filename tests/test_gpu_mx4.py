"""GPU parity of the 4-bit (MX E2M1) V-Smooth path against the oracle (Sec. 3.2 after Eq. 4;
Sec. 4.1 "Implementation"; App. A "Scope of ExpCast-FP8"; App. B): the E2M1 conversion and the
K/V quantisers bit for bit, the 4-bit attention against the emulated 4-bit recurrence on the
same operands (rel-L2 within 5e-3), and V-Smooth's gain at 4 bits on the video workload."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import attention as T
from oracle import formats as F
from oracle import mx4 as M
from oracle import vsmooth as S

from gpu_util import DEV, bf16_dev, bf16_host_bits, config_inputs, note, rows_sample, values

pytestmark = pytest.mark.gpu

TOL = 5e-3
# Without the rotation the kernel takes the oracle's steps one for one on the same operands, so
# it differs from the emulated recurrence only where a float32 summation order flips a P code:
# 1e-9 to 7e-5 measured.  A corrupted operand (a fragment register overwritten while its product
# still waits on the matrix unit) moved whole query blocks by 1e-3 to 3e-3, inside TOL, so the
# on-operand parity also holds this bound.
TIGHT = 5e-4


def test_fp4_conversion_matches_oracle():
    rng = np.random.default_rng(0)
    grid = F.e2m1_decode(np.arange(16))
    mids = (grid[1:8] + grid[:7]) / 2
    x = np.concatenate([rng.uniform(-6, 6, 200000), grid, mids, -mids, [1e-30, -1e-30, 0.0, -0.0, 0.2, -0.2]])
    x = x[: len(x) // 2 * 2].astype(np.float32)
    got = vc.vc_test_fp4_encode(torch.from_numpy(x).to(DEV)).cpu().numpy()
    want = F.e2m1_encode(x)
    want = want[0::2] | (want[1::2] << 4)
    bad = np.nonzero(got != want)[0]
    note(f"fp4 conversion: {len(bad)} mismatches of {len(got)} pairs"
         + (f"; first {x[2 * bad[0]]}, {x[2 * bad[0] + 1]} -> {got[bad[0]]:#x} want {want[bad[0]]:#x}" if len(bad) else ""))
    assert len(bad) == 0


def _perm(kind, N, H, seed):
    if kind == "identity":
        return None
    return np.stack([np.random.default_rng(seed + h).permutation(N) for h in range(H)])[None].astype(np.int32)


@pytest.mark.parametrize("name,heads,perm_kind,no_demean,had",
                         [("tiny", None, "random", False, False), ("medium", [0, 3], "random", False, False),
                          ("medium", [1], "identity", True, False), ("qk_outlier", [0], "random", False, True),
                          ("video", [5], "random", False, False)])
def test_mx4_quantisers_bit_exact(name, heads, perm_kind, no_demean, had):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"mx4 quantisers {name} heads={heads} perm={perm_kind} no_demean={no_demean} hadamard={had}")
    H, N = K.shape[1], cfg.N
    perm = _perm(perm_kind, N, H, 90)
    ops = vc.vc_vsmooth_demean_quant_mx4(bf16_dev(K), bf16_dev(V),
                                         None if perm is None else torch.from_numpy(perm).to(DEV),
                                         no_demean=no_demean, hadamard=had)
    kc_g = vc.unpack_fp4(ops["Kq4"]).cpu().numpy()
    sk_g = ops["sK4"].cpu().numpy().astype(np.int64) - 127
    rc_g = vc.rq_tiled_to_natural(vc.unpack_fp4(ops["Rq4"])).cpu().numpy()
    sr_g = ops["sR4"].cpu().numpy().astype(np.int64) - 127
    mu_g = bf16_host_bits(ops["mu"])
    for h in range(H):
        p = np.arange(N) if perm is None else perm[0, h]
        kc, kE = M.quantize_k4(values(K[0, h]), p, hadamard=had)
        vq = M.quantize_v4(values(V[0, h]), p, demean=not no_demean)
        assert np.array_equal(sk_g[0, h], kE)
        assert np.array_equal(kc_g[0, h], kc)
        assert np.array_equal(sr_g[0, h], vq["E"])
        mism = int((rc_g[0, h] != vq["codes"]).sum())
        note(f"  head {h}: residual code mismatches {mism}")
        assert mism == 0
        assert np.array_equal(mu_g[0, h], F.bf16_bits_from_value(vq["mu_b"]))


def _oracle_ops(Qh, Kh, Vh, perm, had=False, demean=True):
    qc, qE = M.quantize_q4(Qh, hadamard=had)
    kc, kE = M.quantize_k4(Kh, perm, hadamard=had)
    vq = M.quantize_v4(Vh, perm, demean)
    return {"qc": qc, "qE": qE, "kc": kc, "kE": kE, **vq}


def _emulated(ops, rows, mean=True):
    mu = ops["mu_b"] if mean else np.zeros_like(ops["mu_b"])
    return M.attention_tiled_mx4(M.dequant_row_groups(ops["qc"], ops["qE"]), M.dequant_row_groups(ops["kc"], ops["kE"]),
                                 M.dequant_v4(ops["codes"], ops["E"]), mu, rows)


def _dev_ops(ops_list):
    st = lambda key: np.stack([o[key] for o in ops_list])[None]
    Kq4 = vc.pack_fp4(torch.from_numpy(st("kc"))).to(DEV)
    sK4 = torch.from_numpy((st("kE") + 127).astype(np.uint8)).to(DEV)
    Rq4 = vc.pack_fp4(vc.rq_natural_to_tiled(torch.from_numpy(st("codes")))).to(DEV)
    sR4 = torch.from_numpy((st("E") + 127).astype(np.uint8)).to(DEV)
    mu = torch.from_numpy(F.bf16_bits_from_value(st("mu_b")).view(np.int16)).view(torch.bfloat16).to(DEV)
    return Kq4, sK4, Rq4, sR4, mu


@pytest.mark.parametrize("name,heads,nrows,had", [("tiny", None, 1024, False), ("medium", [0, 6], 1024, False),
                                                  ("qk_outlier", [2], 512, True), ("video", [7], 256, False)])
def test_mx4_attention_on_oracle_operands(name, heads, nrows, had):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"mx4 attention on oracle operands {name} heads={heads} hadamard={had}")
    H, N = Q.shape[1], cfg.N
    perm = _perm("random", N, H, 11)
    ops = [_oracle_ops(values(Q[0, h]), values(K[0, h]), values(V[0, h]), perm[0, h], had) for h in range(H)]
    O = values(bf16_host_bits(vc.vc_attn_fwd_mx4(bf16_dev(Q), *_dev_ops(ops), hadamard=had)))
    rows = rows_sample(N, nrows)
    for h in range(H):
        err = T.rel_l2(O[0, h][rows], _emulated(ops[h], rows))
        note(f"  head {h}: rel-L2 vs emulated = {err:.3e}")
        assert err < (TOL if had else TIGHT)


@pytest.mark.parametrize("name,heads,had", [("medium", [4], False), ("medium", [4], True),
                                           ("qk_outlier", [2], True), ("video", [7], True)])
def test_mx4_no_mean_flag(name, heads, had):
    """Without the mean term, plain and rotated."""
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"mx4 no-mean {name} heads={heads} hadamard={had}")
    N = cfg.N
    perm = _perm("random", N, 1, 3)
    ops = [_oracle_ops(values(Q[0, 0]), values(K[0, 0]), values(V[0, 0]), perm[0, 0], had)]
    Kq4, sK4, Rq4, sR4, mu = _dev_ops(ops)
    O = values(bf16_host_bits(vc.vc_attn_fwd_mx4(bf16_dev(Q), Kq4, sK4, Rq4, sR4, None, no_mean=True,
                                                 hadamard=had)))
    rows = rows_sample(N, 512 if N <= 8192 else 256)
    err = T.rel_l2(O[0, 0][rows], _emulated(ops[0], rows, mean=False))
    note(f"  no mean: rel-L2 vs emulated = {err:.3e}")
    assert err < (TOL if had else TIGHT)


def test_mx4_end_to_end_and_vsmooth_gain():
    """Full 4-bit GPU path (GPU grouping, 4-bit quantisers, 4-bit attention) on two video heads:
    matches the emulated oracle with the GPU's pi, and the grouped + demeaned path is closer to
    exact attention than the sequence-order unsmoothed 4-bit baseline."""
    cfg, Q, K, V = config_inputs("video", [0, 1])
    H, N = Q.shape[1], cfg.N
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
    O_vs = values(bf16_host_bits(vc.vc_attention_mx4(Qd, Kd, Vd, g["perm"])))
    O_base = values(bf16_host_bits(vc.vc_attention_mx4(Qd, Kd, Vd, None, no_demean=True)))
    perm = g["perm"].cpu().numpy()
    rows = rows_sample(N, 128)
    e_vs, e_base = [], []
    for h in range(H):
        Qh, Kh, Vh = values(Q[0, h]), values(K[0, h]), values(V[0, h])
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        e_vs.append(T.rel_l2(O_vs[0, h][rows], exact))
        e_base.append(T.rel_l2(O_base[0, h][rows], exact))
        err = T.rel_l2(O_vs[0, h][rows], _emulated(_oracle_ops(Qh, Kh, Vh, perm[0, h]), rows))
        note(f"  head {h}: vs exact V-Smooth {e_vs[-1]:.3e} unsmoothed {e_base[-1]:.3e}; vs emulated {err:.3e}")
        assert err < TOL
    assert np.mean(e_vs) < 0.9 * np.mean(e_base)


def test_mx4_small_and_ragged_shapes():
    for B, H, N in [(1, 1, 128), (2, 3, 384), (1, 2, 640), (1, 1, 2176)]:   # 2176 = 17 tiles: a full 16-tile mean group closes in the last matrix phase
        cfg, Q, K, V = config_inputs("medium", list(range(H)), B=B, N=N, grid=None, v_kind="iid")
        note(f"mx4 path B={B} H={H} N={N}")
        perm = np.stack([np.random.default_rng(b * H + h).permutation(N) for b in range(B) for h in range(H)])
        perm = perm.reshape(B, H, N).astype(np.int32)
        O = values(bf16_host_bits(vc.vc_attention_mx4(bf16_dev(Q), bf16_dev(K), bf16_dev(V),
                                                      torch.from_numpy(perm).to(DEV), softmax_scale=0.05)))
        for b in range(B):
            for h in range(H):
                Qh, Kh, Vh = values(Q[b, h]), values(K[b, h]), values(V[b, h])
                qc, qE = M.quantize_q4(Qh, 0.05)
                kc, kE = M.quantize_k4(Kh, perm[b, h])
                vq = M.quantize_v4(Vh, perm[b, h])
                ref = M.attention_tiled_mx4(M.dequant_row_groups(qc, qE), M.dequant_row_groups(kc, kE),
                                            M.dequant_v4(vq["codes"], vq["E"]), vq["mu_b"])
                err = T.rel_l2(O[b, h], ref)
                note(f"  b={b} h={h}: rel-L2 vs emulated = {err:.3e}")
                assert err < TIGHT


def test_mx4_empty_is_noop():
    Q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    out = vc.vc_attn_fwd_mx4(Q, torch.empty((1, 2, 0, 64), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 4), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 128, 64), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 128, 4), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV))
    assert out.shape == (1, 2, 0, 128)
