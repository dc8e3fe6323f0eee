"""Pins of the oracle's number formats against library routines and the field definition."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # field definition of Sec. 3.3: code 8e+m stores 2^(e-7)(1+m/8); 0x38 = 1.0, 0x78 = 256, max 448
    assert ours[0x38] == 1.0 and ours[0x78] == 256.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 30.0,
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(50000) * 0.01,          # subnormal range
        np.array([0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 456.0, 464.0]),
    ]).astype(np.float32)
    # every midpoint between adjacent finite magnitudes (ties go to the even code)
    pos = F.e4m3_decode(np.arange(127))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = F.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates():
    assert F.e4m3_encode(np.array([1e6, -1e6, 500.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E]


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(300000).astype(np.float32) * np.float32(10.0) ** rng.integers(-40, 38, 300000),
        (rng.standard_normal(10000) * 1e-39).astype(np.float32),     # float32 / bf16 subnormals
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_round(x), ref)


@pytest.mark.parametrize("v", [1.0, -3.140625, 0.0, 65504.0, 1e-40])
def test_bf16_bits_roundtrip(v):
    val = F.bf16_round(np.array([v]))
    assert F.bf16_value_from_bits(F.bf16_bits_from_value(val))[0] == val[0]
