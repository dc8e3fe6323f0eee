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


@pytest.mark.parametrize("name,heads,scale,had", [("tiny", None, 0.0, False), ("medium", [0, 4], 0.0, False),
                                                  ("medium", [1], 0.37, False), ("video", [11], 0.0, False),
                                                  ("qk_outlier", [2], 0.0, True), ("video", [5], 0.0, True)])
def test_query_prologue_codes_bit_exact(name, heads, scale, had):
    """Row a8: the attention kernel's query prologue (its own code, run alone) against the oracle's
    quantize_q -- E4M3 codes and the power-of-two block scales bit for bit, with and without the
    QK rotation."""
    from gpu_util import bf16_dev, config_inputs, values
    cfg, Q, K, V = config_inputs(name, heads)
    note(f"query prologue {name} heads={heads} scale={scale} hadamard={had}")
    Qq, sQ = vc.vc_test_quantize_q(bf16_dev(Q), softmax_scale=scale, hadamard=had)
    Qq, sQ = Qq.cpu().numpy(), sQ.cpu().numpy()
    for h in range(Q.shape[1]):
        qc, s = S.quantize_q(values(Q[0, h]), None if scale == 0.0 else scale, hadamard=had)
        assert np.array_equal(sQ[0, h], s)
        bad = np.nonzero(Qq[0, h] != qc)
        assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][:3]}, {bad[1][:3]}"


def test_validate_perm_counts():
    """vc_validate_perm: 0 for permutations; out-of-range entries and every extra occurrence of a
    repeated value counted exactly (Sec. 3.2, Eq. 3 needs pi to be a permutation)."""
    rng = np.random.default_rng(40)
    B, H, N = 2, 3, 1000
    p = np.stack([np.stack([rng.permutation(N) for _ in range(H)]) for _ in range(B)]).astype(np.int32)
    bad = vc.vc_validate_perm(torch.from_numpy(p).to(DEV)).cpu().numpy()
    assert np.array_equal(bad, np.zeros((B, H), np.int32))
    q = p.copy()
    q[0, 1, 7] = N                 # out of range
    q[0, 1, 9] = -5                # out of range
    q[1, 2, 0] = q[1, 2, 1]        # one repeat (and one missing value)
    q[1, 0, 10:14] = q[1, 0, 3]    # a value occurring 5 times: 4 extra
    bad = vc.vc_validate_perm(torch.from_numpy(q).to(DEV)).cpu().numpy()
    assert bad.tolist() == [[0, 2, 0], [4, 0, 1]]


def test_demean_quant_reads_bad_perm_entries_as_token_zero():
    """Out-of-range pi entries are read as token 0 (no gather leaves the head): the operands equal
    the oracle's for the permutation with those entries replaced by 0."""
    from gpu_util import bf16_dev, config_inputs, values
    cfg, Q, K, V = config_inputs("tiny")
    N = cfg.N
    rng = np.random.default_rng(41)
    p = rng.permutation(N).astype(np.int32)
    p[[3, 200, 777]] = [N, -1, 1 << 30]
    ops = vc.vc_vsmooth_demean_quant(bf16_dev(K), bf16_dev(V), torch.from_numpy(p[None, None]).to(DEV))
    pc = np.where((p >= 0) & (p < N), p, 0)
    kc, sK = S.quantize_k(values(K[0, 0]), pc)
    vq = S.quantize_v(values(V[0, 0]), pc)
    assert np.array_equal(ops["Kq"].cpu().numpy()[0, 0], kc)
    assert np.array_equal(ops["sK"].cpu().numpy()[0, 0], sK)
    assert np.array_equal(vc.rq_tiled_to_natural(ops["Rq"]).cpu().numpy()[0, 0], vq["codes"])
    assert np.array_equal(ops["sV"].cpu().numpy()[0, 0], vq["sV"])


def test_attention_clock_probe():
    """The clock probe runs vc_attn_fwd's kernel with its stamps on: the output is bit-identical to
    vc_attn_fwd's, and every workgroup reports a shader clock within MI355X's range."""
    from gpu_util import bf16_dev, config_inputs
    cfg, Q, K, V = config_inputs("medium", [0, 1, 2, 3])
    Qd = bf16_dev(Q)
    ops = vc.vc_vsmooth_demean_quant(bf16_dev(K), bf16_dev(V), None)
    O1 = vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
    O2, clk = vc.vc_test_attn_fwd_clock(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    c = clk.cpu().numpy().astype(np.float64)
    assert c.shape == (4 * 32, 4)
    cyc, tick = c[:, 2] - c[:, 0], c[:, 3] - c[:, 1]
    assert np.all(cyc > 0) and np.all(tick > 0)
    mhz = vc.wall_clock_mhz()
    ghz = cyc.sum() / tick.sum() * mhz * 1e-3
    note(f"  attention kernel clock {ghz:.3f} GHz (wall-clock counter {mhz:.1f} MHz)")
    assert 0.3 < ghz < 3.0
