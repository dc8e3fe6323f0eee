"""GPU parity of the single stages against the oracle: ExpCast codes (bit-exact, exhaustive
over every float32 u in [-16, 0]), the E4M3 quantiser (bit-exact), the label sort (exact)."""
import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc
from oracle import expcast as E
from oracle import formats as F
from oracle import vsmooth as S

from gpu_util import DEV, note

pytestmark = pytest.mark.gpu

# float32 bit patterns of [-16, -0.0]: 0x80000000 (-0.0) .. 0xC1800000 (-16.0)
NEG_LO, NEG_HI = 0x80000000, 0xC1800000
NCHUNK = 10


@pytest.mark.parametrize("chunk", range(NCHUNK))
def test_expcast_exhaustive_negative_range(chunk):
    total = NEG_HI + 1 - NEG_LO
    step = -(-total // NCHUNK)
    lo = NEG_LO + chunk * step
    hi = min(NEG_LO + (chunk + 1) * step, NEG_HI + 1)
    note(f"expcast exhaustive chunk {chunk}: bits [{lo:#x}, {hi:#x})")
    for a in range(lo, hi, 1 << 26):
        b = min(a + (1 << 26), hi)
        u = np.arange(a, b, dtype=np.uint64).astype(np.uint32).view(np.float32)
        got = vc.vc_test_expcast(torch.from_numpy(u).to(DEV)).cpu().numpy()
        ref = E.expcast_code(u)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"u={u[bad[:5]]} gpu={got[bad[:5]]} oracle={ref[bad[:5]]}"


def test_expcast_specials_and_positive():
    u = np.array([0.0, -0.0, 1e-45, -1e-45, 0.001, 0.5, 1.0, 3.0, 1e30, np.inf, -np.inf, np.nan,
                  -15.0, -15.0625, -14.9, -14.0, -1.6, -0.05625], dtype=np.float32)
    rng = np.random.default_rng(0)
    u = np.concatenate([u, rng.uniform(-40, 40, 1_000_000).astype(np.float32)])
    got = vc.vc_test_expcast(torch.from_numpy(u).to(DEV)).cpu().numpy()
    assert np.array_equal(got, E.expcast_code(u))
    assert got[0] == 120 and got[12] == 0 and got[15] == 8 and got[16] == 107   # u = 0, -15, -14, -1.6


def test_e4m3_quantiser_bit_exact():
    rng = np.random.default_rng(1)
    pos = F.e4m3_decode(np.arange(127))
    mids = ((pos[1:] + pos[:-1]) / 2)
    x = np.concatenate([
        rng.uniform(-448, 448, 2_000_000), rng.standard_normal(1_000_000) * 3.0,
        rng.standard_normal(500_000) * 0.005, mids, -mids, pos, -pos,
        np.nextafter(mids, 0), np.nextafter(mids, 1000), [0.0, -0.0, 448.0, -448.0, 460.0, 1e9, -1e9],
    ]).astype(np.float32)
    got = vc.vc_test_e4m3_encode(torch.from_numpy(x).to(DEV)).cpu().numpy()
    ref = F.e4m3_encode(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"x={x[bad[:5]]} gpu={got[bad[:5]]} oracle={ref[bad[:5]]}"


@pytest.mark.parametrize("H,N,k", [(1, 128, 1), (2, 1152, 3), (3, 8192, 64), (2, 70016, 128),
                                   (1, 115200, 256), (1, 2048, 256)])
def test_label_sort_exact(H, N, k):
    note(f"label sort H={H} N={N} k={k}")
    rng = np.random.default_rng(N + k)
    z = rng.integers(0, k, (1, H, N)).astype(np.int32)
    if k > 2:
        z[0, 0, : N // 3] = k - 1          # a long run of one label, across tile boundaries
    perm, off = vc.vc_test_label_sort(torch.from_numpy(z).to(DEV), k)
    perm, off = perm.cpu().numpy(), off.cpu().numpy()
    for h in range(H):
        assert np.array_equal(perm[0, h], S.stable_argsort(z[0, h]))
        assert np.array_equal(off[0, h], S.cluster_offsets(z[0, h], k))


def test_mfma_fp8_rate_hook():
    """The FP8 matrix-instruction loop the bench times: it runs, its outputs are finite and the
    same on a second call."""
    o1 = vc.vc_test_mfma_fp8_rate(4, 3).cpu()
    o2, mhz = vc.vc_test_mfma_fp8_rate(4, 3, clock=True)
    assert torch.isfinite(o1).all()
    assert torch.equal(o1, o2.cpu())   # the clock stamps change nothing in the products
    # a loop long enough for the counters to resolve: a shader clock within MI355X's range
    _, mhz = vc.vc_test_mfma_fp8_rate(256, 500, clock=True)
    mhz = mhz.cpu()
    assert ((mhz > 300.0) & (mhz < 3000.0)).all(), mhz
