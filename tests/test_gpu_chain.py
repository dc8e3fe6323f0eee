"""The whole hot path on the GPU at the full sizes of the video (H=40, N=70,016) and long
(H=24, N=115,200) workloads, on four heads each: GPU grouping (k-means + label sort) -> GPU
demean/quantise -> GPU attention, against the oracle's emulated recurrence on the GPU's own
permutation (512 sampled query rows per head, rel-L2 within 5e-3), and the acceptance ordering
against FP64 exact attention: the VC path's error below that of the unsmoothed sequence-order
FP8 baseline with the same P path.  The exp-then-cast baseline (the 8-bit comparator that smooths
neither, VC-Attention Sec. 4.1 "Baselines" and Table 4) is reported beside it."""
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


def _emulated(Qh, Kh, Vh, perm, rows):
    qc, sQ = S.quantize_q(Qh)
    kc, sK = S.quantize_k(Kh, perm)
    vq = S.quantize_v(Vh, perm)
    return T.attention_tiled(F.e4m3_decode(qc), sQ, F.e4m3_decode(kc), sK, F.e4m3_decode(vq["codes"]),
                             vq["mu_t"], vq["sV"], rows=rows)


@pytest.mark.parametrize("name,heads", [("video", [0, 13, 26, 39]), ("long", [0, 8, 16, 23])])
def test_full_chain_at_scale(name, heads):
    cfg, Q, K, V = config_inputs(name, heads)
    N = cfg.N
    note(f"full chain {name} heads={heads} N={N} k={cfg.k}")
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    g = vc.vc_vsmooth_group(Vd, cfg.k, cfg.iters)
    assert not vc.vc_validate_perm(g["perm"]).any()
    ops = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"])
    O = values(bf16_host_bits(vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])))
    base = vc.vc_vsmooth_demean_quant(Kd, Vd, None, no_demean=True)
    Ob = values(bf16_host_bits(vc.vc_attn_fwd(Qd, base["Kq"], base["sK"], base["Rq"], None, base["sV"],
                                              no_mean=True)))
    Oe = values(bf16_host_bits(vc.vc_attn_fwd(Qd, base["Kq"], base["sK"], base["Rq"], None, base["sV"],
                                              no_mean=True, exp_then_cast=True)))
    perm = g["perm"].cpu().numpy()
    rows = rows_sample(N, 512)
    e = {"vc": [], "base": [], "etc": []}
    for h in range(len(heads)):
        Qh, Kh, Vh = values(Q[0, h]), values(K[0, h]), values(V[0, h])
        err = T.rel_l2(O[0, h][rows], _emulated(Qh, Kh, Vh, perm[0, h], rows))
        exact = T.attention_exact(Qh, Kh, Vh, rows=rows)
        e["vc"].append(T.rel_l2(O[0, h][rows], exact))
        e["base"].append(T.rel_l2(Ob[0, h][rows], exact))
        e["etc"].append(T.rel_l2(Oe[0, h][rows], exact))
        note(f"  head {heads[h]}: vs emulated {err:.2e}; vs exact: VC {e['vc'][-1]:.3e}, unsmoothed "
             f"{e['base'][-1]:.3e}, unsmoothed exp-then-cast {e['etc'][-1]:.3e}")
        assert err < TOL
    m = {k: float(np.mean(v)) for k, v in e.items()}
    note(f"  mean vs exact: VC {m['vc']:.3e}, unsmoothed {m['base']:.3e}, exp-then-cast {m['etc']:.3e}")
    assert m["vc"] < m["base"]
