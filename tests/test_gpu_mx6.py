"""GPU parity of the 6-bit (MX E2M3) V-Smooth path against the oracle: the E2M3 conversion (with
unit scale and with the conversion's own power-of-two scale operand) and the K/V quantisers bit
for bit, the 6-bit attention against the oracle's emulated E2M3 recurrence on the same operands
(rel-L2 within 5e-3), the no-mean flag, small and ragged shapes, and V-Smooth's gain at 6 bits
on two video heads (Sec. 3.2 after Eq. 4; App. B)."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import attention as T
from oracle import formats as F
from oracle import mx4 as M

from gpu_util import DEV, bf16_dev, bf16_host_bits, config_inputs, note, rows_sample, values

pytestmark = pytest.mark.gpu

TOL = 5e-3
# Without the rotation the kernel takes the oracle's steps one for one on the same operands, so
# it differs from the emulated recurrence only where a float32 summation order flips a P code:
# 1e-9 to 7e-5 measured.  A corrupted operand (a fragment register overwritten while its product
# still waits on the matrix unit) moved whole query blocks by 1e-3 to 3e-3, inside TOL, so the
# on-operand parity also holds this bound.
TIGHT = 5e-4
FMT = "e2m3"


def test_fp6_conversion_matches_oracle():
    rng = np.random.default_rng(0)
    grid = F.e2m3_decode(np.arange(64))
    mids = (grid[1:32] + grid[:31]) / 2
    x = np.concatenate([rng.uniform(-7.5, 7.5, 320000), grid, mids, -mids,
                        [1e-30, -1e-30, 0.0, -0.0, 0.03, -0.03, 7.5, -7.5]])
    x = np.concatenate([x, np.zeros((-len(x)) % 32)]).astype(np.float32)
    got = vc.unpack_fp6(vc.vc_test_fp6_encode(torch.from_numpy(x).to(DEV)).cpu().numpy().view(np.uint8))
    want = F.e2m3_encode(x)
    bad = np.nonzero(got != want)[0]
    note(f"fp6 conversion: {len(bad)} mismatches of {len(x)}"
         + (f"; first {x[bad[0]]} -> {got[bad[0]]:#x} want {want[bad[0]]:#x}" if len(bad) else ""))
    assert len(bad) == 0
    # the scale operand divides: values times 2^E with scale 2^E give the codes of the values
    E = rng.integers(-20, 20, len(x) // 32)
    sc = np.ldexp(1.0, E).astype(np.float32)
    xs = (x.reshape(-1, 32) * sc[:, None]).astype(np.float32).reshape(-1)
    got2 = vc.unpack_fp6(vc.vc_test_fp6_encode(torch.from_numpy(xs).to(DEV), torch.from_numpy(sc).to(DEV))
                         .cpu().numpy().view(np.uint8))
    assert np.array_equal(got2, want)


def _perm(kind, N, H, seed):
    if kind == "identity":
        return None
    return np.stack([np.random.default_rng(seed + h).permutation(N) for h in range(H)])[None].astype(np.int32)


@pytest.mark.parametrize("name,heads,perm_kind,no_demean,had",
                         [("tiny", None, "random", False, False), ("medium", [0, 3], "random", False, False),
                          ("medium", [1], "identity", True, False), ("qk_outlier", [0], "random", False, True),
                          ("video", [5], "random", False, False)])
def test_mx6_quantisers_bit_exact(name, heads, perm_kind, no_demean, had):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"mx6 quantisers {name} heads={heads} perm={perm_kind} no_demean={no_demean} hadamard={had}")
    H, N = K.shape[1], cfg.N
    perm = _perm(perm_kind, N, H, 90)
    ops = vc.vc_vsmooth_demean_quant_mx6(bf16_dev(K), bf16_dev(V),
                                         None if perm is None else torch.from_numpy(perm).to(DEV),
                                         no_demean=no_demean, hadamard=had)
    kraw = ops["Kq6"].cpu().numpy()
    rraw = ops["Rq6"].cpu().numpy()
    assert not kraw.reshape(-1, 128)[:, 96:].any() and not rraw.reshape(-1, 128)[:, 96:].any()   # pad bytes
    kc_g = vc.unpack_fp6(kraw)
    sk_g = ops["sK6"].cpu().numpy().astype(np.int64) - 127
    rc_g = vc.rq_tiled_to_natural(torch.from_numpy(vc.unpack_fp6(rraw))).numpy()
    sr_g = ops["sR6"].cpu().numpy().astype(np.int64) - 127
    mu_g = bf16_host_bits(ops["mu"])
    for h in range(H):
        p = np.arange(N) if perm is None else perm[0, h]
        kc, kE = M.quantize_k4(values(K[0, h]), p, hadamard=had, fmt=FMT)
        vq = M.quantize_v4(values(V[0, h]), p, demean=not no_demean, fmt=FMT)
        assert np.array_equal(sk_g[0, h], kE)
        kmism = int((kc_g[0, h] != kc).sum())
        assert np.array_equal(sr_g[0, h], vq["E"])
        mism = int((rc_g[0, h] != vq["codes"]).sum())
        note(f"  head {h}: key code mismatches {kmism}, residual code mismatches {mism}")
        assert kmism == 0 and mism == 0
        assert np.array_equal(mu_g[0, h], F.bf16_bits_from_value(vq["mu_b"]))


def _oracle_ops(Qh, Kh, Vh, perm, had=False, demean=True, scale=None):
    qc, qE = M.quantize_q4(Qh, scale, hadamard=had, fmt=FMT)
    kc, kE = M.quantize_k4(Kh, perm, hadamard=had, fmt=FMT)
    vq = M.quantize_v4(Vh, perm, demean, fmt=FMT)
    return {"qc": qc, "qE": qE, "kc": kc, "kE": kE, **vq}


def _emulated(ops, rows, mean=True):
    mu = ops["mu_b"] if mean else np.zeros_like(ops["mu_b"])
    return M.attention_tiled_mx4(M.dequant_row_groups(ops["qc"], ops["qE"], FMT),
                                 M.dequant_row_groups(ops["kc"], ops["kE"], FMT),
                                 M.dequant_v4(ops["codes"], ops["E"], FMT), mu, rows, fmt=FMT)


def _dev_ops(ops_list):
    st = lambda key: np.stack([o[key] for o in ops_list])[None]
    Kq6 = torch.from_numpy(vc.pack_fp6(st("kc"))).to(DEV)
    sK6 = torch.from_numpy((st("kE") + 127).astype(np.uint8)).to(DEV)
    Rq6 = torch.from_numpy(vc.pack_fp6(vc.rq_natural_to_tiled(torch.from_numpy(st("codes"))).numpy())).to(DEV)
    sR6 = torch.from_numpy((st("E") + 127).astype(np.uint8)).to(DEV)
    mu = torch.from_numpy(F.bf16_bits_from_value(st("mu_b")).view(np.int16)).view(torch.bfloat16).to(DEV)
    return Kq6, sK6, Rq6, sR6, mu


@pytest.mark.parametrize("name,heads,nrows,had", [("tiny", None, 1024, False), ("medium", [0, 6], 1024, False),
                                                  ("qk_outlier", [2], 512, True), ("video", [7], 256, False)])
def test_mx6_attention_on_oracle_operands(name, heads, nrows, had):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"mx6 attention on oracle operands {name} heads={heads} hadamard={had}")
    H, N = Q.shape[1], cfg.N
    perm = _perm("random", N, H, 11)
    ops = [_oracle_ops(values(Q[0, h]), values(K[0, h]), values(V[0, h]), perm[0, h], had) for h in range(H)]
    O = values(bf16_host_bits(vc.vc_attn_fwd_mx6(bf16_dev(Q), *_dev_ops(ops), hadamard=had)))
    rows = rows_sample(N, nrows)
    for h in range(H):
        err = T.rel_l2(O[0, h][rows], _emulated(ops[h], rows))
        note(f"  head {h}: rel-L2 vs emulated = {err:.3e}")
        assert err < (TOL if had else TIGHT)


@pytest.mark.parametrize("name,heads,had", [("medium", [4], False), ("medium", [4], True),
                                           ("qk_outlier", [2], True), ("video", [7], True)])
def test_mx6_no_mean_flag(name, heads, had):
    """Without the mean term, plain and rotated: the rotated no-mean kernel is the one built at -O2
    (its -O3 code gave wrong outputs)."""
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"mx6 no-mean {name} heads={heads} hadamard={had}")
    N = cfg.N
    perm = _perm("random", N, 1, 3)
    ops = [_oracle_ops(values(Q[0, 0]), values(K[0, 0]), values(V[0, 0]), perm[0, 0], had)]
    Kq6, sK6, Rq6, sR6, mu = _dev_ops(ops)
    O = values(bf16_host_bits(vc.vc_attn_fwd_mx6(bf16_dev(Q), Kq6, sK6, Rq6, sR6, None, no_mean=True,
                                                 hadamard=had)))
    rows = rows_sample(N, 512 if N <= 8192 else 256)
    err = T.rel_l2(O[0, 0][rows], _emulated(ops[0], rows, mean=False))
    note(f"  no mean: rel-L2 vs emulated = {err:.3e}")
    assert err < (TOL if had else TIGHT)


def test_mx6_end_to_end_and_vsmooth_gain():
    """Full 6-bit GPU path on two video heads: matches the emulated oracle with the GPU's pi; the
    grouped + demeaned path is closer to exact attention than the unsmoothed 6-bit baseline, and
    less than half as far as the 4-bit V-Smooth path."""
    cfg, Q, K, V = config_inputs("video", [0, 1])
    H, N = Q.shape[1], cfg.N
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
    O_vs = values(bf16_host_bits(vc.vc_attention_mx6(Qd, Kd, Vd, g["perm"])))
    O_base = values(bf16_host_bits(vc.vc_attention_mx6(Qd, Kd, Vd, None, no_demean=True)))
    O_4 = values(bf16_host_bits(vc.vc_attention_mx4(Qd, Kd, Vd, g["perm"])))
    perm = g["perm"].cpu().numpy()
    rows = rows_sample(N, 128)
    e_vs, e_base, e_4 = [], [], []
    for h in range(H):
        Qh, Kh, Vh = values(Q[0, h]), values(K[0, h]), values(V[0, h])
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        e_vs.append(T.rel_l2(O_vs[0, h][rows], exact))
        e_base.append(T.rel_l2(O_base[0, h][rows], exact))
        e_4.append(T.rel_l2(O_4[0, h][rows], exact))
        err = T.rel_l2(O_vs[0, h][rows], _emulated(_oracle_ops(Qh, Kh, Vh, perm[0, h]), rows))
        note(f"  head {h}: vs exact 6-bit V-Smooth {e_vs[-1]:.3e}, unsmoothed {e_base[-1]:.3e}, "
             f"4-bit V-Smooth {e_4[-1]:.3e}; vs emulated {err:.3e}")
        assert err < TOL
    # at 6 bits the value operand's share of the error is smaller than at 4, so the gain is the
    # acceptance ordering (about 5 % here), not the 4-bit path's margin
    assert np.mean(e_vs) < np.mean(e_base)
    assert np.mean(e_vs) < 0.5 * np.mean(e_4)


def test_mx6_small_and_ragged_shapes():
    for B, H, N in [(1, 1, 128), (2, 3, 384), (1, 2, 640), (1, 1, 2176)]:
        cfg, Q, K, V = config_inputs("medium", list(range(H)), B=B, N=N, grid=None, v_kind="iid")
        note(f"mx6 path B={B} H={H} N={N}")
        perm = np.stack([np.random.default_rng(b * H + h).permutation(N) for b in range(B) for h in range(H)])
        perm = perm.reshape(B, H, N).astype(np.int32)
        O = values(bf16_host_bits(vc.vc_attention_mx6(bf16_dev(Q), bf16_dev(K), bf16_dev(V),
                                                      torch.from_numpy(perm).to(DEV), softmax_scale=0.05)))
        for b in range(B):
            for h in range(H):
                ops = _oracle_ops(values(Q[b, h]), values(K[b, h]), values(V[b, h]), perm[b, h], scale=0.05)
                ref = M.attention_tiled_mx4(M.dequant_row_groups(ops["qc"], ops["qE"], FMT),
                                            M.dequant_row_groups(ops["kc"], ops["kE"], FMT),
                                            M.dequant_v4(ops["codes"], ops["E"], FMT), ops["mu_b"], fmt=FMT)
                err = T.rel_l2(O[b, h], ref)
                note(f"  b={b} h={h}: rel-L2 vs emulated = {err:.3e}")
                assert err < TIGHT


def test_mx6_empty_is_noop():
    Q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    out = vc.vc_attn_fwd_mx6(Q, torch.empty((1, 2, 0, 128), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 4), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 128, 128), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 128, 4), dtype=torch.uint8, device=DEV),
                             torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV))
    assert out.shape == (1, 2, 0, 128)


@pytest.mark.parametrize("fmt_bits", [4, 6])
@pytest.mark.parametrize("mag", [1e-4, 1e4])
def test_mx_paths_extreme_magnitudes(fmt_bits, mag):
    """Inputs scaled by 1e-4 and 1e4 through the 4-bit and the 6-bit path: the per-32 scales
    follow, the quantised operands stay bit-exact and the output matches the emulated oracle."""
    fmt = "e2m1" if fmt_bits == 4 else "e2m3"
    rng = np.random.default_rng(15)
    N = 512
    Q = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((1, 1, N, 128)) * mag))
    K = F.bf16_bits_from_value(F.bf16_round((rng.standard_normal((1, 1, N, 128)) + 1.0) * mag))
    V = F.bf16_bits_from_value(F.bf16_round((rng.standard_normal((1, 1, N, 128)) + 2.0) * mag))
    perm = rng.permutation(N).astype(np.int32)
    Qh, Kh, Vh = values(Q[0, 0]), values(K[0, 0]), values(V[0, 0])
    scale = 1.0 / (mag * mag * np.sqrt(128.0))   # keeps the scores O(1)
    pd = torch.from_numpy(perm[None, None]).to(DEV)
    if fmt_bits == 4:
        dev = vc.vc_vsmooth_demean_quant_mx4(bf16_dev(K), bf16_dev(V), pd)
        kc_g = vc.unpack_fp4(dev["Kq4"]).cpu().numpy()[0, 0]
        O = vc.vc_attn_fwd_mx4(bf16_dev(Q), dev["Kq4"], dev["sK4"], dev["Rq4"], dev["sR4"], dev["mu"],
                               softmax_scale=float(scale))
        sk_g = dev["sK4"].cpu().numpy()[0, 0].astype(np.int64) - 127
    else:
        dev = vc.vc_vsmooth_demean_quant_mx6(bf16_dev(K), bf16_dev(V), pd)
        kc_g = vc.unpack_fp6(dev["Kq6"].cpu().numpy()[0, 0])
        O = vc.vc_attn_fwd_mx6(bf16_dev(Q), dev["Kq6"], dev["sK6"], dev["Rq6"], dev["sR6"], dev["mu"],
                               softmax_scale=float(scale))
        sk_g = dev["sK6"].cpu().numpy()[0, 0].astype(np.int64) - 127
    qc, qE = M.quantize_q4(Qh, scale, fmt=fmt)
    kc, kE = M.quantize_k4(Kh, perm, fmt=fmt)
    vq = M.quantize_v4(Vh, perm, fmt=fmt)
    assert np.array_equal(kc_g, kc) and np.array_equal(sk_g, kE)
    ref = M.attention_tiled_mx4(M.dequant_row_groups(qc, qE, fmt), M.dequant_row_groups(kc, kE, fmt),
                                M.dequant_v4(vq["codes"], vq["E"], fmt), vq["mu_b"], fmt=fmt)
    err = T.rel_l2(values(bf16_host_bits(O))[0, 0], ref)
    note(f"  {fmt_bits}-bit, magnitude {mag}: rel-L2 vs emulated {err:.3e}")
    assert err < TOL
