"""The largest shape the C ABI accepts, B*H*N*d just below 2^31 (B=1, H=127, N=131,072, d=128:
2,130,706,432 elements, 4.3 GB per bf16 tensor): grouping -> demean/quantise -> attention on
the GPU, then the first and the last head checked against the oracle on sampled rows (emulated
VC attention on the GPU's pi within 5e-3) and the last head's k-means objective against the
oracle's Lloyd (1e-3).  The inputs are seeded device draws (torch's generator), copied back for
the checked heads only."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import attention as T
from oracle import vsmooth as S

from gpu_util import DEV, bf16_host_bits, note, rows_sample, values

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _emulated(Qh, Kh, Vh, perm, rows):
    from oracle import formats as F
    qc, sQ = S.quantize_q(Qh)
    kc, sK = S.quantize_k(Kh, perm)
    vq = S.quantize_v(Vh, perm)
    return T.attention_tiled(F.e4m3_decode(qc), sQ, F.e4m3_decode(kc), sK, F.e4m3_decode(vq["codes"]),
                             vq["mu_t"], vq["sV"], rows=rows)


def test_largest_shape_full_chain():
    B, H, N, d, k, iters = 1, 127, 131072, 128, 128, 10
    assert B * H * N * d < 2 ** 31 <= B * (H + 1) * N * d
    note(f"largest shape B={B} H={H} N={N}: {B * H * N * d} elements")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20260)
    draw = lambda: torch.randn((B, H, N, d), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    Qd = draw()
    Kd = draw()
    Vd = draw()
    torch.cuda.synchronize()
    g = vc.vc_vsmooth_group(Vd, k, iters)
    assert not vc.vc_validate_perm(g["perm"]).any()
    ops = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"])
    O = vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
    torch.cuda.synchronize()
    note("  GPU chain done")
    rows = rows_sample(N, 48)
    for h in (0, H - 1):
        Qh, Kh, Vh = (values(bf16_host_bits(t[0, h])) for t in (Qd, Kd, Vd))
        perm = g["perm"][0, h].cpu().numpy()
        Oh = values(bf16_host_bits(O[0, h]))
        err = T.rel_l2(Oh[rows], _emulated(Qh, Kh, Vh, perm, rows))
        note(f"  head {h}: rel-L2 vs emulated {err:.3e}")
        assert err < TOL
    Vh = values(bf16_host_bits(Vd[0, H - 1]))
    J_ref = S.vsmooth_group(Vh, k, iters)["J"]
    J = float(g["J"][0, H - 1])
    note(f"  head {H - 1}: J {J:.6e} vs oracle {J_ref:.6e}")
    assert abs(J - J_ref) <= 1e-3 * J_ref
