"""The C ABI: the built library exports every entry point declared in include/vc_attn.h, and
every argument error is reported on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import bit_attention_video_amd as vc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc_attn.h")
S = vc.STATUS
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails before any use


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s+(vc_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = vc.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
        assert n in vc._SIGNATURES, f"{n} has no binding"


def test_header_statuses_match_binding():
    text = open(HEADER).read()
    for name, val in S.items():
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
        assert m and int(m.group(1)) == val, name
    for name in ("VC_ATTN_NO_MEAN", "VC_ATTN_EXP_THEN_CAST", "VC_ATTN_HADAMARD", "VC_DQ_NO_DEMEAN",
                 "VC_DQ_HADAMARD"):
        m = re.search(rf"#define\s+{name}\s+(0x[0-9a-fA-F]+)u", text)
        assert m and int(m.group(1), 16) == getattr(vc, name), name


def test_strerror():
    lib = vc.lib()
    for v in S.values():
        assert lib.vc_strerror(v)
    assert lib.vc_strerror(12345) == b"unknown status"


def test_attn_fwd_argument_errors():
    lib = vc.lib()
    f = lib.vc_attn_fwd
    P = [FAKE] * 6
    assert f(*P, 1, 1, 128, 64, 0.0, 0, FAKE, None) == S["VC_ERR_SHAPE"]        # d != 128
    assert f(*P, 1, 1, 100, 128, 0.0, 0, FAKE, None) == S["VC_ERR_SHAPE"]       # N % 128
    assert f(*P, -1, 1, 128, 128, 0.0, 0, FAKE, None) == S["VC_ERR_SHAPE"]
    assert f(*P, 1, 1, 1 << 24, 128, 0.0, 0, FAKE, None) == S["VC_ERR_OVERFLOW"]
    assert f(None, *P[1:], 1, 1, 128, 128, 0.0, 0, FAKE, None) == S["VC_ERR_NULL"]
    assert f(*P, 1, 1, 128, 128, 0.0, 0, None, None) == S["VC_ERR_NULL"]
    # mu may be NULL only with VC_ATTN_NO_MEAN
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 128, 128, 0.0, 0, FAKE, None) == S["VC_ERR_NULL"]
    assert f(*P, 1, 1, 128, 128, 0.0, 0x8, FAKE, None) == S["VC_ERR_FLAGS"]
    # VC_ATTN_EXP_THEN_CAST (0x2), VC_ATTN_HADAMARD (0x4) and all of them together pass the flag
    # check (the bad scale is caught next)
    assert f(*P, 1, 1, 128, 128, -1.0, vc.VC_ATTN_EXP_THEN_CAST, FAKE, None) == S["VC_ERR_SHAPE"]
    assert f(*P, 1, 1, 128, 128, -1.0, vc.VC_ATTN_HADAMARD, FAKE, None) == S["VC_ERR_SHAPE"]
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 128, 128, -1.0, 0x7, FAKE, None) == S["VC_ERR_SHAPE"]
    assert f(*P, 1, 1, 128, 128, -1.0, 0, FAKE, None) == S["VC_ERR_SHAPE"]
    assert f(*P, 1, 1, 128, 128, float("nan"), 0, FAKE, None) == S["VC_ERR_SHAPE"]
    # empty problems are a no-op
    assert f(None, None, None, None, None, None, 0, 4, 128, 128, 0.0, 0, None, None) == S["VC_OK"]
    assert f(None, None, None, None, None, None, 1, 4, 0, 128, 0.0, 0, None, None) == S["VC_OK"]


def test_group_argument_errors():
    lib = vc.lib()
    f = lib.vc_vsmooth_group
    ws = lib.vc_group_workspace_size(1, 2, 1024, 8)
    assert ws > 0
    args = lambda N=1024, d=128, k=8, it=10, V=FAKE, nws=ws: (V, 1, 2, N, d, k, it, None, FAKE, FAKE, FAKE,
                                                                FAKE, FAKE, FAKE, nws, None)
    assert f(*args(d=127)) == S["VC_ERR_SHAPE"]
    assert f(*args(N=1000)) == S["VC_ERR_SHAPE"]
    assert f(*args(V=None)) == S["VC_ERR_NULL"]
    assert f(*args(k=0)) == S["VC_ERR_K"]
    assert f(*args(k=257)) == S["VC_ERR_K"]
    assert f(*args(N=128, k=200)) == S["VC_ERR_K"]                             # k > N
    assert f(*args(it=0)) == S["VC_ERR_ITERS"]
    assert f(*args(nws=ws - 1)) == S["VC_ERR_WORKSPACE"]
    assert f(*args(N=0)) == S["VC_OK"]


def test_demean_quant_argument_errors():
    lib = vc.lib()
    f = lib.vc_vsmooth_demean_quant
    ws = lib.vc_demean_quant_workspace_size(1, 2, 1024)
    assert ws > 0
    args = lambda N=1024, d=128, flags=0, K=FAKE, nws=ws: (K, FAKE, None, 1, 2, N, d, flags, FAKE, FAKE, FAKE,
                                                            FAKE, FAKE, FAKE, nws, None)
    assert f(*args(d=256)) == S["VC_ERR_SHAPE"]
    assert f(*args(N=129)) == S["VC_ERR_SHAPE"]
    assert f(*args(K=None)) == S["VC_ERR_NULL"]
    assert f(*args(flags=0x4)) == S["VC_ERR_FLAGS"]
    assert f(*args(flags=0x3, nws=0)) == S["VC_ERR_WORKSPACE"]      # both flags are known
    assert f(*args(nws=0)) == S["VC_ERR_WORKSPACE"]
    assert f(*args(N=0)) == S["VC_OK"]


def test_mx4_argument_errors():
    lib = vc.lib()
    f = lib.vc_vsmooth_demean_quant_mx4
    ws = lib.vc_demean_quant_workspace_size(1, 2, 1024)
    args = lambda N=1024, d=128, flags=0, K=FAKE, nws=ws, mu=FAKE: (K, FAKE, None, 1, 2, N, d, flags, FAKE, FAKE,
                                                                    FAKE, FAKE, mu, FAKE, nws, None)
    assert f(*args(d=64)) == S["VC_ERR_SHAPE"]
    assert f(*args(N=200)) == S["VC_ERR_SHAPE"]
    assert f(*args(K=None)) == S["VC_ERR_NULL"]
    assert f(*args(mu=None)) == S["VC_ERR_NULL"]
    assert f(*args(flags=0x4)) == S["VC_ERR_FLAGS"]
    assert f(*args(flags=0x3, nws=ws - 1)) == S["VC_ERR_WORKSPACE"]
    assert f(*args(N=0)) == S["VC_OK"]
    a = lib.vc_attn_fwd_mx4
    P = [FAKE] * 6
    assert a(*P, 1, 1, 128, 64, 0.0, 0, FAKE, None) == S["VC_ERR_SHAPE"]
    assert a(*P, 1, 1, 1 << 24, 128, 0.0, 0, FAKE, None) == S["VC_ERR_OVERFLOW"]
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 128, 0.0, 0, FAKE, None) == S["VC_ERR_NULL"]
    assert a(*P, 1, 1, 128, 128, 0.0, vc.VC_ATTN_EXP_THEN_CAST, FAKE, None) == S["VC_ERR_FLAGS"]   # no ExpCast at 4 bits
    assert a(*P, 1, 1, 128, 128, -1.0, vc.VC_ATTN_HADAMARD, FAKE, None) == S["VC_ERR_SHAPE"]
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 128, float("inf"), 0x5, FAKE, None) == S["VC_ERR_SHAPE"]
    assert a(None, None, None, None, None, None, 1, 4, 0, 128, 0.0, 0, None, None) == S["VC_OK"]
    assert lib.vc_test_fp4_encode(FAKE, FAKE, 3, None) == S["VC_ERR_SHAPE"]
    assert lib.vc_test_fp4_encode(None, FAKE, 4, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_fp4_encode(None, None, 0, None) == S["VC_OK"]
    assert lib.vc_test_mfma_fp8_rate(None, 1, 1, None, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_mfma_fp8_rate(FAKE, 0, 1, None, None) == S["VC_ERR_SHAPE"]
    assert lib.vc_test_mfma_fp8_rate(FAKE, 1, 0, None, None) == S["VC_ERR_SHAPE"]
    assert lib.vc_test_mfma_fp8_rate(FAKE, 2 ** 31 - 1, 2 ** 31 - 1, FAKE, None) == S["VC_ERR_SHAPE"]


def test_mx6_argument_errors():
    lib = vc.lib()
    f = lib.vc_vsmooth_demean_quant_mx6
    ws = lib.vc_demean_quant_workspace_size(1, 2, 1024)
    assert lib.vc_workspace_size(vc.VC_OP_DEMEAN_QUANT_MX6, 1, 2, 1024, 128, 0) == ws
    assert lib.vc_workspace_size(vc.VC_OP_ATTN_FWD_MX6, 1, 2, 1024, 128, 0) == 0
    args = lambda N=1024, d=128, flags=0, K=FAKE, nws=ws, mu=FAKE: (K, FAKE, None, 1, 2, N, d, flags, FAKE, FAKE,
                                                                    FAKE, FAKE, mu, FAKE, nws, None)
    assert f(*args(d=64)) == S["VC_ERR_SHAPE"]
    assert f(*args(N=200)) == S["VC_ERR_SHAPE"]
    assert f(*args(K=None)) == S["VC_ERR_NULL"]
    assert f(*args(mu=None)) == S["VC_ERR_NULL"]
    assert f(*args(flags=0x4)) == S["VC_ERR_FLAGS"]
    assert f(*args(flags=0x3, nws=ws - 1)) == S["VC_ERR_WORKSPACE"]
    assert f(*args(N=0)) == S["VC_OK"]
    a = lib.vc_attn_fwd_mx6
    P = [FAKE] * 6
    assert a(*P, 1, 1, 128, 64, 0.0, 0, FAKE, None) == S["VC_ERR_SHAPE"]
    assert a(*P, 1, 1, 1 << 24, 128, 0.0, 0, FAKE, None) == S["VC_ERR_OVERFLOW"]
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 128, 0.0, 0, FAKE, None) == S["VC_ERR_NULL"]
    assert a(*P, 1, 1, 128, 128, 0.0, vc.VC_ATTN_EXP_THEN_CAST, FAKE, None) == S["VC_ERR_FLAGS"]
    assert a(*P, 1, 1, 128, 128, -1.0, vc.VC_ATTN_HADAMARD, FAKE, None) == S["VC_ERR_SHAPE"]
    assert a(None, None, None, None, None, None, 1, 4, 0, 128, 0.0, 0, None, None) == S["VC_OK"]
    assert lib.vc_test_fp6_encode(None, None, FAKE, 4, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_fp6_encode(FAKE, None, None, 4, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_fp6_encode(FAKE, FAKE, FAKE, 1 << 35, None) == S["VC_ERR_OVERFLOW"]
    assert lib.vc_test_fp6_encode(None, None, None, 0, None) == S["VC_OK"]


def test_fp6_pack_roundtrip_and_layout():
    import numpy as np
    rng = np.random.default_rng(5)
    c = rng.integers(0, 64, (2, 3, 128)).astype(np.uint8)
    p = vc.pack_fp6(c)
    assert p.shape == c.shape and not p.reshape(-1, 128)[:, 96:].any()   # 32 zero bytes per row
    assert np.array_equal(vc.unpack_fp6(p), c)
    # group g of a row: its first 16 code bytes at 16 g, its last 8 at 64 + 16 (g % 2) + 8 (g // 2);
    # value k in bits 6k .. 6k+5 of the group's little-endian 192-bit field
    row = p.reshape(-1, 128)[0]
    for g in range(4):
        t = 64 + 16 * (g % 2) + 8 * (g // 2)
        field = int.from_bytes(bytes(row[16 * g:16 * g + 16].tolist() + row[t:t + 8].tolist()), "little")
        assert [(field >> (6 * k)) & 63 for k in range(32)] == c.reshape(-1, 32)[g].tolist()


def test_fp4_pack_roundtrip():
    import torch
    c = torch.randint(0, 16, (3, 5, 128), dtype=torch.uint8)
    p = vc.pack_fp4(c)
    assert p.shape == (3, 5, 64)
    assert torch.equal(vc.unpack_fp4(p), c)
    assert int(vc.pack_fp4(torch.tensor([[1, 2]], dtype=torch.uint8))[0, 0]) == 0x21   # even index low


def test_hook_argument_errors():
    lib = vc.lib()
    assert lib.vc_test_expcast(None, None, 0, None) == S["VC_OK"]
    assert lib.vc_test_expcast(None, FAKE, 10, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_e4m3_encode(FAKE, None, 10, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_kmeans_assign(FAKE, FAKE, 1, 1, 256, 128, 300, FAKE, None, FAKE, 1 << 30, None) == S["VC_ERR_K"]
    assert lib.vc_test_kmeans_assign(FAKE, FAKE, 1, 1, 256, 128, 8, FAKE, None, None, 0, None) == S["VC_ERR_NULL"]
    assert lib.vc_test_kmeans_assign(FAKE, FAKE, 1, 1, 256, 128, 8, FAKE, None, FAKE, 16, None) == S["VC_ERR_WORKSPACE"]
    ws = lib.vc_group_workspace_size(1, 1, 256, 4)
    assert lib.vc_test_label_sort(FAKE, 1, 1, 256, 4, FAKE, FAKE, FAKE, ws - 1, None) == S["VC_ERR_WORKSPACE"]


def test_workspace_sizes_grow():
    lib = vc.lib()
    a = lib.vc_group_workspace_size(1, 8, 8192, 64)
    b = lib.vc_group_workspace_size(1, 40, 70016, 128)
    assert 0 < a < b
    assert lib.vc_demean_quant_workspace_size(1, 8, 8192) < lib.vc_demean_quant_workspace_size(1, 40, 70016)
    assert lib.vc_group_workspace_size(0, 8, 8192, 64) == 0


def test_rq_layout_roundtrip_and_key_order():
    import numpy as np
    import torch
    R = torch.randint(0, 256, (1, 2, 384, 128), dtype=torch.uint8)
    T = vc.rq_natural_to_tiled(R)
    assert T.shape == (1, 2, 3, 128, 128)
    assert torch.equal(vc.rq_tiled_to_natural(T), R)
    assert sorted(vc.KEY_OF_SLOT.tolist()) == list(range(128))
    # slot s = 64p + 32g + i holds key 64p + 32(i/16) + 8((i%16)/4) + 4g + i%4
    assert vc.KEY_OF_SLOT[0] == 0 and vc.KEY_OF_SLOT[1] == 1 and vc.KEY_OF_SLOT[4] == 8
    assert vc.KEY_OF_SLOT[16] == 32 and vc.KEY_OF_SLOT[32] == 4 and vc.KEY_OF_SLOT[64] == 64
    assert np.array_equal(T[0, 1, 2, 5, :].numpy(), R[0, 1, 256 + vc.KEY_OF_SLOT, 5].numpy())   # [.., c, s]


def test_workspace_size_entry_matches_per_call_sizes():
    lib = vc.lib()
    for B, H, N, k in [(1, 8, 8192, 64), (1, 40, 70016, 128), (2, 3, 384, 7)]:
        assert lib.vc_workspace_size(vc.VC_OP_GROUP, B, H, N, 128, k) == lib.vc_group_workspace_size(B, H, N, k)
        dq = lib.vc_demean_quant_workspace_size(B, H, N)
        assert lib.vc_workspace_size(vc.VC_OP_DEMEAN_QUANT, B, H, N, 128, 0) == dq
        assert lib.vc_workspace_size(vc.VC_OP_DEMEAN_QUANT_MX4, B, H, N, 128, 0) == dq
        assert lib.vc_workspace_size(vc.VC_OP_ATTN_FWD, B, H, N, 128, 0) == 0
        assert lib.vc_workspace_size(vc.VC_OP_ATTN_FWD_MX4, B, H, N, 128, 0) == 0
        v = lib.vc_workspace_size(vc.VC_OP_VALIDATE_PERM, B, H, N, 128, 0)
        assert v >= B * H * ((N + 31) // 32) * 4 and v % 256 == 0
    assert lib.vc_workspace_size(vc.VC_OP_GROUP, 1, 1, 1024, 64, 8) == 0      # d != 128
    assert lib.vc_workspace_size(99, 1, 1, 1024, 128, 8) == 0                 # unknown op
    assert lib.vc_workspace_size(vc.VC_OP_VALIDATE_PERM, 1, 0, 1024, 128, 0) == 0


def test_validate_perm_argument_errors():
    lib = vc.lib()
    f = lib.vc_validate_perm
    ws = lib.vc_workspace_size(vc.VC_OP_VALIDATE_PERM, 1, 2, 1000, 128, 0)
    assert f(FAKE, -1, 2, 1000, FAKE, FAKE, ws, None) == S["VC_ERR_SHAPE"]
    assert f(FAKE, 1, 1 << 16, 1 << 16, FAKE, FAKE, ws, None) == S["VC_ERR_OVERFLOW"]
    assert f(None, 1, 2, 1000, FAKE, FAKE, ws, None) == S["VC_ERR_NULL"]
    assert f(FAKE, 1, 2, 1000, None, FAKE, ws, None) == S["VC_ERR_NULL"]
    assert f(FAKE, 1, 2, 1000, FAKE, FAKE, ws - 1, None) == S["VC_ERR_WORKSPACE"]
    assert f(None, 1, 2, 0, None, None, 0, None) == S["VC_OK"]      # any N works, empty is a no-op


def test_new_hook_argument_errors():
    lib = vc.lib()
    q = lib.vc_test_quantize_q
    assert q(FAKE, 1, 1, 100, 128, 0.0, 0, FAKE, FAKE, None) == S["VC_ERR_SHAPE"]
    assert q(None, 1, 1, 128, 128, 0.0, 0, FAKE, FAKE, None) == S["VC_ERR_NULL"]
    assert q(FAKE, 1, 1, 128, 128, 0.0, vc.VC_ATTN_NO_MEAN, FAKE, FAKE, None) == S["VC_ERR_FLAGS"]
    assert q(FAKE, 1, 1, 128, 128, -2.0, vc.VC_ATTN_HADAMARD, FAKE, FAKE, None) == S["VC_ERR_SHAPE"]
    assert q(None, 1, 1, 0, 128, 0.0, 0, None, None, None) == S["VC_OK"]
    c = lib.vc_test_attn_fwd_clock
    P = [FAKE] * 6
    assert lib.vc_test_attn_clock_slots(1, 40, 70016) == 4 * 40 * 274
    assert lib.vc_test_attn_clock_slots(1, 1, 100) == 0
    assert c(*P, 1, 1, 128, 128, 0.0, 0, FAKE, None, None) == S["VC_ERR_NULL"]      # clk required
    assert c(*P, 1, 1, 128, 64, 0.0, 0, FAKE, FAKE, None) == S["VC_ERR_SHAPE"]
    assert c(*P, 1, 1, 128, 128, 0.0, 0x10, FAKE, FAKE, None) == S["VC_ERR_FLAGS"]
