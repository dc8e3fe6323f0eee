"""GPU parity of vc_attn_fwd against the oracle's emulated tiled VC attention (same operands,
same permutation): relative L2 within 5e-3 (the acceptance tolerance), plus the ordering of
errors against exact attention and the unsmoothed FP8 baseline."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import attention as T
from oracle import formats as F
from oracle import vsmooth as S

from gpu_util import DEV, bf16_dev, bf16_host_bits, config_inputs, note, rows_sample, values

pytestmark = pytest.mark.gpu

TOL = 5e-3   # acceptance: rel-L2 of the GPU output against the emulated oracle, same permutation


def _oracle_ops(Qh, Kh, Vh, perm, demean=True, scale=None):
    qc, sQ = S.quantize_q(Qh, scale)
    kc, sK = S.quantize_k(Kh, perm)
    vq = S.quantize_v(Vh, perm, demean=demean)
    return {"qc": qc, "sQ": sQ, "kc": kc, "sK": sK, **vq}


def _emulated(Qh, ops, rows, p_mode="expcast", mean=True):
    mu_t = ops["mu_t"] if mean else np.zeros_like(ops["mu_t"])
    return T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                             F.e4m3_decode(ops["codes"]), mu_t, ops["sV"], p_mode=p_mode, rows=rows)


def _dev_ops(ops_list):
    """Stack per-head oracle operands into the kernel's device layouts."""
    Kq = torch.from_numpy(np.stack([o["kc"] for o in ops_list])[None]).to(DEV)
    sK = torch.from_numpy(np.stack([o["sK"] for o in ops_list])[None]).to(DEV)
    R = torch.from_numpy(np.stack([o["codes"] for o in ops_list])[None])
    Rq = vc.rq_natural_to_tiled(R).to(DEV)
    mu = np.stack([F.bf16_bits_from_value(o["mu_t"]) for o in ops_list])[None]
    mu = torch.from_numpy(mu.view(np.int16)).view(torch.bfloat16).to(DEV)
    sV = torch.from_numpy(np.stack([o["sV"] for o in ops_list])[None]).to(DEV)
    return Kq, sK, Rq, mu, sV


@pytest.mark.parametrize("name,heads,nrows", [("tiny", None, 1024), ("medium", [0, 6], 1024),
                                              ("video", [7], 256), ("long", [4], 128)])
def test_attn_fwd_on_oracle_operands(name, heads, nrows):
    """Kernel alone: identical quantised operands in, compare O with the emulated recurrence."""
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"attn_fwd on oracle operands {name} heads={heads}")
    H, N = Q.shape[1], cfg.N
    rng = np.random.default_rng(3)
    perms = [rng.permutation(N) for _ in range(H)]
    ops = [_oracle_ops(values(Q[0, h]), values(K[0, h]), values(V[0, h]), perms[h]) for h in range(H)]
    O = vc.vc_attn_fwd(bf16_dev(Q), *_dev_ops(ops))
    O = values(bf16_host_bits(O))
    rows = rows_sample(N, nrows)
    for h in range(H):
        ref = _emulated(values(Q[0, h]), ops[h], rows)
        err = T.rel_l2(O[0, h][rows], ref)
        note(f"  head {h}: rel-L2 vs emulated = {err:.3e}")
        assert err < TOL


@pytest.mark.parametrize("no_mean", [False, True])
def test_attn_fwd_exp_then_cast_mode(no_mean):
    """VC_ATTN_EXP_THEN_CAST against the oracle's exp-then-cast recurrence (same operands)."""
    cfg, Q, K, V = config_inputs("medium", [1])
    N = cfg.N
    perm = np.random.default_rng(7).permutation(N)
    ops = [_oracle_ops(values(Q[0, 0]), values(K[0, 0]), values(V[0, 0]), perm)]
    Kq, sK, Rq, mu, sV = _dev_ops(ops)
    O = vc.vc_attn_fwd(bf16_dev(Q), Kq, sK, Rq, None if no_mean else mu, sV, no_mean=no_mean,
                       exp_then_cast=True)
    O = values(bf16_host_bits(O))
    rows = rows_sample(N, 512)
    ref = _emulated(values(Q[0, 0]), ops[0], rows, p_mode="exp_cast", mean=not no_mean)
    err = T.rel_l2(O[0, 0][rows], ref)
    note(f"  exp-then-cast no_mean={no_mean}: rel-L2 vs emulated = {err:.3e}")
    assert err < TOL


def test_attn_fwd_no_mean_flag():
    cfg, Q, K, V = config_inputs("medium", [3])
    N = cfg.N
    perm = np.random.default_rng(4).permutation(N)
    ops = [_oracle_ops(values(Q[0, 0]), values(K[0, 0]), values(V[0, 0]), perm)]
    Kq, sK, Rq, mu, sV = _dev_ops(ops)
    O = values(bf16_host_bits(vc.vc_attn_fwd(bf16_dev(Q), Kq, sK, Rq, None, sV, no_mean=True)))
    rows = rows_sample(N, 512)
    ref = _emulated(values(Q[0, 0]), ops[0], rows, mean=False)
    assert T.rel_l2(O[0, 0][rows], ref) < TOL


@pytest.mark.parametrize("name,heads", [("tiny", None), ("medium", [0, 5])])
def test_vc_path_end_to_end_and_error_ordering(name, heads):
    """GPU demean_quant + attn_fwd with the oracle's pi, against the emulated oracle; then the
    acceptance ordering: VC error vs exact below the unsmoothed sequence-order FP8 baseline's."""
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"end-to-end {name} heads={heads}")
    H, N = Q.shape[1], cfg.N
    perm = np.stack([S.vsmooth_group(values(V[0, h]), cfg.k, cfg.iters)["perm"] for h in range(H)])[None]
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    O = values(bf16_host_bits(vc.vc_attention(Qd, Kd, Vd, torch.from_numpy(perm.astype(np.int32)).to(DEV))))
    Ob = values(bf16_host_bits(vc.vc_attention(Qd, Kd, Vd, None, no_demean=True)))
    rows = rows_sample(N, 512)
    e_vc, e_base = [], []
    for h in range(H):
        Qh, Kh, Vh = values(Q[0, h]), values(K[0, h]), values(V[0, h])
        ref = _emulated(Qh, _oracle_ops(Qh, Kh, Vh, perm[0, h]), rows)
        err = T.rel_l2(O[0, h][rows], ref)
        note(f"  head {h}: rel-L2 vs emulated = {err:.3e}")
        assert err < TOL
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        e_vc.append(T.rel_l2(O[0, h][rows], exact))
        e_base.append(T.rel_l2(Ob[0, h][rows], exact))
        note(f"  head {h}: vs exact: VC {e_vc[-1]:.3e}  unsmoothed {e_base[-1]:.3e}")
    if name != "tiny":   # iid V (tiny) has no shared component to subtract; see the design notes
        assert np.mean(e_vc) < np.mean(e_base)


def test_attn_fwd_deterministic():
    cfg, Q, K, V = config_inputs("medium", [2])
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(cfg.N).astype(np.int32)[None, None]).to(DEV)
    O1 = vc.vc_attention(Qd, Kd, Vd, perm)
    O2 = vc.vc_attention(Qd, Kd, Vd, perm)
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))


def test_attn_fwd_small_and_ragged_shapes():
    """N = 128 (one tile), N = 384 (odd tile count), B = 2, several heads; explicit scale."""
    rng = np.random.default_rng(6)
    for B, H, N in [(1, 1, 128), (2, 3, 384)]:
        note(f"small shape B={B} H={H} N={N}")
        Q = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((B, H, N, 128))))
        K = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((B, H, N, 128)) + 1.0))
        V = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((B, H, N, 128)) * 2))
        perm = np.stack([np.stack([rng.permutation(N) for _ in range(H)]) for _ in range(B)]).astype(np.int32)
        O = vc.vc_attention(bf16_dev(Q), bf16_dev(K), bf16_dev(V), torch.from_numpy(perm).to(DEV),
                            softmax_scale=0.05)
        O = values(bf16_host_bits(O))
        for b in range(B):
            for h in range(H):
                Qh, Kh, Vh = values(Q[b, h]), values(K[b, h]), values(V[b, h])
                ops = _oracle_ops(Qh, Kh, Vh, perm[b, h], scale=0.05)
                ref = T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                                        F.e4m3_decode(ops["codes"]), ops["mu_t"], ops["sV"], scale=0.05)
                assert T.rel_l2(O[b, h], ref) < TOL


@pytest.mark.parametrize("N", [2048, 2176])
def test_attn_fwd_mean_group_boundaries(N):
    """The mean term's 16-tile groups at the key loop's end: N = 2048 (16 tiles: one full group,
    closed after the loop) and N = 2176 (17 tiles: the full group closes in the last matrix phase,
    then a one-tile group)."""
    rng = np.random.default_rng(N)
    note(f"mean-group boundary N={N}")
    Q = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((1, 1, N, 128))))
    K = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((1, 1, N, 128)) + 1.0))
    V = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((1, 1, N, 128)) * 2 + 3.0))
    perm = rng.permutation(N).astype(np.int32)[None, None]
    O = vc.vc_attention(bf16_dev(Q), bf16_dev(K), bf16_dev(V), torch.from_numpy(perm).to(DEV), softmax_scale=0.05)
    O = values(bf16_host_bits(O))[0, 0]
    Qh, Kh, Vh = values(Q[0, 0]), values(K[0, 0]), values(V[0, 0])
    ops = _oracle_ops(Qh, Kh, Vh, perm[0, 0], scale=0.05)
    ref = T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                            F.e4m3_decode(ops["codes"]), ops["mu_t"], ops["sV"], scale=0.05)
    assert T.rel_l2(O, ref) < TOL


def test_attn_fwd_empty_is_noop():
    Q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    Kq = torch.empty((1, 2, 0, 128), dtype=torch.uint8, device=DEV)
    out = vc.vc_attn_fwd(Q, Kq, torch.empty((1, 2, 0), device=DEV), torch.empty((1, 2, 0, 128, 128), dtype=torch.uint8, device=DEV),
                         torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV),
                         torch.empty((1, 2, 128), device=DEV))
    assert out.shape == (1, 2, 0, 128)


@pytest.mark.parametrize("scale", [0.5, 2.0])
def test_attn_fwd_peaked_softmax(scale):
    """Large softmax scales make the rows peaked and the running maximum move often (Eq. 1's
    rescale branch on most tiles); the kernel still matches the emulated recurrence."""
    cfg, Q, K, V = config_inputs("medium", [3])
    note(f"peaked softmax scale={scale}")
    N = cfg.N
    perm = np.random.default_rng(13).permutation(N)
    Qh, Kh, Vh = values(Q[0, 0]), values(K[0, 0]), values(V[0, 0])
    ops = _oracle_ops(Qh, Kh, Vh, perm, scale=scale)
    Kq, sK, Rq, mu, sV = _dev_ops([ops])
    O = values(bf16_host_bits(vc.vc_attn_fwd(bf16_dev(Q), Kq, sK, Rq, mu, sV, softmax_scale=scale)))
    rows = rows_sample(N, 512)
    ref = T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                            F.e4m3_decode(ops["codes"]), ops["mu_t"], ops["sV"], scale=scale, rows=rows)
    err = T.rel_l2(O[0, 0][rows], ref)
    note(f"  rel-L2 vs emulated = {err:.3e}")
    assert err < TOL


@pytest.mark.parametrize("mag", [1e-4, 1e4])
def test_vc_path_extreme_magnitudes(mag):
    """Inputs scaled by 1e-4 and 1e4: the power-of-two block scales and the V scale follow, the
    quantised operands stay bit-exact and the output matches the emulated oracle."""
    rng = np.random.default_rng(14)
    N = 512
    Q = F.bf16_bits_from_value(F.bf16_round(rng.standard_normal((1, 1, N, 128)) * mag))
    K = F.bf16_bits_from_value(F.bf16_round((rng.standard_normal((1, 1, N, 128)) + 1.0) * mag))
    V = F.bf16_bits_from_value(F.bf16_round((rng.standard_normal((1, 1, N, 128)) + 2.0) * mag))
    perm = rng.permutation(N).astype(np.int32)
    Qh, Kh, Vh = values(Q[0, 0]), values(K[0, 0]), values(V[0, 0])
    scale = 1.0 / (mag * mag * np.sqrt(128.0))   # keeps the scores O(1)
    ops_dev = vc.vc_vsmooth_demean_quant(bf16_dev(K), bf16_dev(V), torch.from_numpy(perm[None, None]).to(DEV))
    ops = _oracle_ops(Qh, Kh, Vh, perm, scale=scale)
    assert np.array_equal(ops_dev["Kq"].cpu().numpy()[0, 0], ops["kc"])
    assert np.array_equal(ops_dev["sK"].cpu().numpy()[0, 0], ops["sK"])
    assert np.array_equal(ops_dev["sV"].cpu().numpy()[0, 0], ops["sV"])
    O = values(bf16_host_bits(vc.vc_attn_fwd(bf16_dev(Q), ops_dev["Kq"], ops_dev["sK"], ops_dev["Rq"],
                                             ops_dev["mu"], ops_dev["sV"], softmax_scale=float(scale))))
    ref = T.attention_tiled(F.e4m3_decode(ops["qc"]), ops["sQ"], F.e4m3_decode(ops["kc"]), ops["sK"],
                            F.e4m3_decode(ops["codes"]), ops["mu_t"], ops["sV"], scale=float(scale))
    assert T.rel_l2(O[0, 0], ref) < TOL
