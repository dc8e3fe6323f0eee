"""GPU parity of the fused QK Hadamard rotation (App. B's Q and K passes; Sec. 4.1 "Baselines"):
the rotated key codes and scales bit for bit against the oracle, the rotated-query attention
against the emulated oracle with the same rotated operands (rel-L2 within the acceptance
tolerance 5e-3), and the effect the rotation exists for: on Q/K channel outliers the rotated
path is closer to exact attention than the unrotated one."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import attention as T
from oracle import formats as F
from oracle import vsmooth as S

from gpu_util import DEV, bf16_dev, bf16_host_bits, config_inputs, note, rows_sample, values

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _perm(N, H, seed):
    return np.stack([np.random.default_rng(seed + h).permutation(N) for h in range(H)])[None].astype(np.int32)


@pytest.mark.parametrize("name,heads", [("tiny", None), ("medium", [0, 3]), ("qk_outlier", [1]),
                                        ("video", [5])])
def test_rotated_key_codes_bit_exact(name, heads):
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"rotated K codes {name} heads={heads}")
    H, N = K.shape[1], cfg.N
    perm = _perm(N, H, 40)
    Kd, Vd, pd = bf16_dev(K), bf16_dev(V), torch.from_numpy(perm).to(DEV)
    rot = vc.vc_vsmooth_demean_quant(Kd, Vd, pd, hadamard=True)
    plain = vc.vc_vsmooth_demean_quant(Kd, Vd, pd)
    for key in ("Rq", "mu", "sV"):                  # the value operand does not see the flag
        assert torch.equal(rot[key], plain[key]), key
    Kq, sK = rot["Kq"].cpu().numpy(), rot["sK"].cpu().numpy()
    for h in range(H):
        kc, sk = S.quantize_k(values(K[0, h]), perm[0, h], hadamard=True)
        assert np.array_equal(sK[0, h], sk)
        mism = int((Kq[0, h] != kc).sum())
        note(f"  head {h}: code mismatches {mism} of {kc.size}")
        assert mism == 0


def _oracle_ops(Qh, Kh, Vh, perm):
    qc, sQ = S.quantize_q(Qh, hadamard=True)
    kc, sK = S.quantize_k(Kh, perm, hadamard=True)
    vq = S.quantize_v(Vh, perm)
    return {"qc": qc, "sQ": sQ, "kc": kc, "sK": sK, **vq}


def _emulated(ops, rows, p_mode="expcast"):
    return T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                             F.e4m3_decode(ops["codes"]), ops["mu_t"], ops["sV"], p_mode=p_mode, rows=rows)


def _dev_ops(ops_list):
    Kq = torch.from_numpy(np.stack([o["kc"] for o in ops_list])[None]).to(DEV)
    sK = torch.from_numpy(np.stack([o["sK"] for o in ops_list])[None]).to(DEV)
    Rq = vc.rq_natural_to_tiled(torch.from_numpy(np.stack([o["codes"] for o in ops_list])[None])).to(DEV)
    mu = np.stack([F.bf16_bits_from_value(o["mu_t"]) for o in ops_list])[None]
    mu = torch.from_numpy(mu.view(np.int16)).view(torch.bfloat16).to(DEV)
    sV = torch.from_numpy(np.stack([o["sV"] for o in ops_list])[None]).to(DEV)
    return Kq, sK, Rq, mu, sV


@pytest.mark.parametrize("name,heads,nrows,etc", [("tiny", None, 1024, False), ("qk_outlier", [0, 2], 1024, False),
                                                  ("qk_outlier", [3], 512, True), ("video", [7], 256, False)])
def test_rotated_query_attention_on_oracle_operands(name, heads, nrows, etc):
    """The kernel rotates Q itself; K, R, mu come from the oracle's rotated quantisers."""
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"rotated-query attention on oracle operands {name} heads={heads} exp_then_cast={etc}")
    H, N = Q.shape[1], cfg.N
    perm = _perm(N, H, 70)
    ops = [_oracle_ops(values(Q[0, h]), values(K[0, h]), values(V[0, h]), perm[0, h]) for h in range(H)]
    O = values(bf16_host_bits(vc.vc_attn_fwd(bf16_dev(Q), *_dev_ops(ops), hadamard=True, exp_then_cast=etc)))
    rows = rows_sample(N, nrows)
    for h in range(H):
        ref = _emulated(ops[h], rows, "exp_cast" if etc else "expcast")
        err = T.rel_l2(O[0, h][rows], ref)
        note(f"  head {h}: rel-L2 vs emulated = {err:.3e}")
        assert err < TOL


def test_rotation_helps_on_channel_outliers():
    """Sec. 4.1: the rotation treats the score product.  Full GPU path (grouping, rotated
    quantisers, attention) with and without it, against exact attention."""
    cfg, Q, K, V = config_inputs("qk_outlier")
    H, N = Q.shape[1], cfg.N
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
    O_rot = values(bf16_host_bits(vc.vc_attention(Qd, Kd, Vd, g["perm"], hadamard=True)))
    O_plain = values(bf16_host_bits(vc.vc_attention(Qd, Kd, Vd, g["perm"])))
    rows = rows_sample(N, 256)
    perm = g["perm"].cpu().numpy()
    e_rot, e_plain = [], []
    for h in range(H):
        Qh, Kh, Vh = values(Q[0, h]), values(K[0, h]), values(V[0, h])
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        e_rot.append(T.rel_l2(O_rot[0, h][rows], exact))
        e_plain.append(T.rel_l2(O_plain[0, h][rows], exact))
        ref = _emulated(_oracle_ops(Qh, Kh, Vh, perm[0, h]), rows)
        err = T.rel_l2(O_rot[0, h][rows], ref)
        note(f"  head {h}: vs exact rotated {e_rot[-1]:.3e} plain {e_plain[-1]:.3e}; vs emulated {err:.3e}")
        assert err < TOL
    assert np.mean(e_rot) < np.mean(e_plain)


def test_rotation_small_and_ragged_shapes():
    """One and three tiles, an odd query-block count, two batch entries."""
    for B, H, N in [(1, 1, 128), (2, 3, 384), (1, 2, 640)]:
        cfg, Q, K, V = config_inputs("medium", list(range(H)), B=B, N=N, grid=None, v_kind="iid")
        note(f"rotated path B={B} H={H} N={N}")
        perm = np.stack([np.random.default_rng(b * H + h).permutation(N) for b in range(B) for h in range(H)])
        perm = perm.reshape(B, H, N).astype(np.int32)
        O = vc.vc_attention(bf16_dev(Q), bf16_dev(K), bf16_dev(V), torch.from_numpy(perm).to(DEV), hadamard=True)
        O = values(bf16_host_bits(O))
        for b in range(B):
            for h in range(H):
                Qh, Kh, Vh = values(Q[b, h]), values(K[b, h]), values(V[b, h])
                ref = _emulated(_oracle_ops(Qh, Kh, Vh, perm[b, h]), np.arange(N))
                assert T.rel_l2(O[b, h], ref) < TOL


def test_rotated_no_mean_path():
    """The rotation combined with the plain low-bit kernel (no mean term, unsmoothed V)."""
    cfg, Q, K, V = config_inputs("qk_outlier", [2])
    N = cfg.N
    O = values(bf16_host_bits(vc.vc_attention(bf16_dev(Q), bf16_dev(K), bf16_dev(V), None, no_demean=True,
                                              hadamard=True)))
    Qh, Kh, Vh = values(Q[0, 0]), values(K[0, 0]), values(V[0, 0])
    qc, sQ = S.quantize_q(Qh, hadamard=True)
    kc, sK = S.quantize_k(Kh, np.arange(N), hadamard=True)
    vq = S.quantize_v(Vh, np.arange(N), demean=False)
    rows = rows_sample(N, 512)
    ref = T.attention_tiled(F.e4m3_decode(qc), sQ, F.e4m3_decode(kc), sK, F.e4m3_decode(vq["codes"]),
                            np.zeros_like(vq["mu_t"]), vq["sV"], rows=rows)
    assert T.rel_l2(O[0, 0][rows], ref) < TOL
