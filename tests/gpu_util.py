"""Helpers for the GPU parity tests: moving seeded synthetic inputs to the device and
oracle results back to numpy.  No method arithmetic lives here."""
import sys

import numpy as np
import torch

import synth
from oracle import formats as F

DEV = "cuda:0"


def note(msg: str):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 patterns -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def values(bits: np.ndarray) -> np.ndarray:
    """bf16 patterns -> float64 values."""
    return F.bf16_value_from_bits(bits)


def config_inputs(name: str, heads=None, **over):
    cfg = synth.get_config(name, **over)
    Q, K, V = synth.make_qkv(cfg, heads)
    return cfg, Q, K, V


def rows_sample(N: int, n: int) -> np.ndarray:
    """n query rows spread over [0, N), always including the first and the last."""
    if n >= N:
        return np.arange(N)
    return np.unique(np.linspace(0, N - 1, n).round().astype(np.int64))
