"""Seeded synthetic inputs for the VC-Attention hot path.

This module only draws numbers: bf16 Q, K, V tensors shaped like the captured
post-RoPE attention operands of a video DiT (d = 128, tens of thousands of
spatiotemporal tokens on a (T, H, W) latent grid).  It holds none of the
method's arithmetic (no quantisation, clustering, softmax or scaling), so both
the CPU oracle and the GPU path may import it.

Recipe (one numpy Generator per (config, head, tensor), seeded by
``np.random.default_rng([cfg_id, head, tensor_id, step])``):

* Q ~ N(0, 1).  K ~ N(0, 1), plus a per-head channel bias ~ N(0, 2)
  (variance 2) where the config asks for it.
* V, "field" generator: per head, k_true centroid vectors c_g ~ N(0, I_d);
  a smooth scalar field over the token grid (the sum of four random
  low-frequency sinusoids in (t, y, x)) is cut at its quantiles into k_true
  equal-population groups g(n); V_n = c_{g(n)} + N(0, 0.3^2) noise.
* V, "iid" generator: V ~ N(0, 1).
* Outliers: round(f * N) tokens drawn without replacement; in each head a set
  of 4 channels is drawn and those channels of every outlier token are
  multiplied by a per-token factor U[20, 50] (or a fixed factor).
* Q/K channel outliers (the case a QK rotation is for): in each head a set of
  qk_outlier_channels channels is drawn and those channels of Q and K are
  multiplied by qk_outlier_scale for every token.
* Draws are float32, rounded once to bf16 (round to nearest even) by torch.

Tokens n <-> (t, y, x) in row-major order.  When N exceeds T*H*W (the N=70,016
video config pads 69,930 grid tokens to a multiple of 128) the extra tokens
continue the row-major flattening into a partial next frame, so no key
masking is needed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["Config", "CONFIGS", "get_config", "make_qkv", "make_head", "bf16_bits", "bits_to_f32",
           "make_reuse_steps"]


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    B: int
    H: int
    N: int
    d: int
    k: int                      # k-means clusters used by the method
    iters: int                  # Lloyd iterations
    grid: Optional[Tuple[int, int, int]]  # (T, H, W) token grid, None for iid
    v_kind: str                 # "iid" | "field"
    k_true: int = 0             # groups in the V field generator
    outlier_frac: float = 0.0
    outlier_factor: Optional[float] = None   # fixed factor, else U[20, 50]
    outlier_shared_channels: bool = False    # one channel set for every head
    k_bias_var: float = 0.0     # variance of the per-head K channel bias
    noise_std: float = 0.3
    steps: int = 1              # permutation-reuse steps
    step_noise_std: float = 0.05
    qk_outlier_channels: int = 0      # Q/K channels scaled by qk_outlier_scale in every token
    qk_outlier_scale: float = 1.0


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, 1, 1, 1024, 128, k=8, iters=10, grid=None, v_kind="iid",
                   outlier_frac=0.005, outlier_factor=30.0, outlier_shared_channels=True),
    "medium": Config("medium", 2, 1, 8, 8192, 128, k=64, iters=10, grid=(8, 32, 32), v_kind="field",
                     k_true=64, outlier_frac=0.005),
    "video": Config("video", 3, 1, 40, 70016, 128, k=128, iters=10, grid=(21, 45, 74), v_kind="field",
                    k_true=128, outlier_frac=0.003, k_bias_var=2.0),
    "reuse": Config("reuse", 4, 1, 24, 32768, 128, k=128, iters=10, grid=(8, 64, 64), v_kind="field",
                    k_true=128, outlier_frac=0.003, k_bias_var=2.0, steps=4),
    "long": Config("long", 5, 1, 24, 115200, 128, k=256, iters=10, grid=(30, 48, 80), v_kind="field",
                   k_true=256, outlier_frac=0.003, k_bias_var=2.0),
    "qk_outlier": Config("qk_outlier", 6, 1, 4, 8192, 128, k=64, iters=10, grid=(8, 32, 32), v_kind="field",
                         k_true=64, outlier_frac=0.003, k_bias_var=2.0, qk_outlier_channels=4,
                         qk_outlier_scale=25.0),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    if overrides:
        cfg = Config(**{**cfg.__dict__, **overrides})
    return cfg


def _rng(cfg: Config, head: int, tensor_id: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.cfg_id, head, tensor_id, step])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (round to nearest even, via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _token_coords(cfg: Config) -> np.ndarray:
    T, Hh, W = cfg.grid
    n = np.arange(cfg.N)
    t = n // (Hh * W)
    y = (n // W) % Hh
    x = n % W
    return np.stack([t / T, y / Hh, x / W], axis=1)  # normalised coordinates, (N, 3)


def _field_groups(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Quantile bins of a smooth random field over the token grid -> group id per token."""
    coords = _token_coords(cfg)
    f = np.zeros(cfg.N)
    for _ in range(4):
        freq = rng.uniform(0.5, 3.0, size=3) * rng.choice([-1.0, 1.0], size=3)
        phase = rng.uniform(0.0, 2.0 * np.pi)
        amp = rng.uniform(0.5, 1.0)
        f += amp * np.sin(2.0 * np.pi * coords @ freq + phase)
    order = np.argsort(f, kind="stable")
    g = np.empty(cfg.N, dtype=np.int64)
    g[order] = (np.arange(cfg.N) * cfg.k_true) // cfg.N
    return g


def _v_head(cfg: Config, head: int, step: int = 0) -> np.ndarray:
    rng = _rng(cfg, head, 2)
    N, d = cfg.N, cfg.d
    if cfg.v_kind == "iid":
        v = rng.standard_normal((N, d), dtype=np.float32)
    else:
        g = _field_groups(cfg, rng)
        cent = rng.standard_normal((cfg.k_true, d), dtype=np.float32)
        v = cent[g] + np.float32(cfg.noise_std) * rng.standard_normal((N, d), dtype=np.float32)
    n_out = int(round(cfg.outlier_frac * N))
    if n_out:
        orng = np.random.default_rng([cfg.cfg_id, 0 if cfg.outlier_shared_channels else head, 3])
        chans = orng.choice(d, size=4, replace=False)
        trng = _rng(cfg, head, 4)
        toks = trng.choice(N, size=n_out, replace=False)
        if cfg.outlier_factor is not None:
            fac = np.full(n_out, cfg.outlier_factor, dtype=np.float32)
        else:
            fac = trng.uniform(20.0, 50.0, size=n_out).astype(np.float32)
        v[np.ix_(toks, chans)] *= fac[:, None]
    for s in range(1, step + 1):   # permutation-reuse drift: V_t = V_{t-1} + N(0, sigma^2)
        srng = _rng(cfg, head, 5, s)
        v = v + np.float32(cfg.step_noise_std) * srng.standard_normal((N, d), dtype=np.float32)
    return v


def make_head(cfg: Config, head: int, step: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """bf16 bit patterns (uint16, shape (N, d)) of Q, K, V for one head."""
    N, d = cfg.N, cfg.d
    q = _rng(cfg, head, 0).standard_normal((N, d), dtype=np.float32)
    krng = _rng(cfg, head, 1)
    k = krng.standard_normal((N, d), dtype=np.float32)
    if cfg.k_bias_var > 0:
        k += np.float32(np.sqrt(cfg.k_bias_var)) * krng.standard_normal(d, dtype=np.float32)[None, :]
    if cfg.qk_outlier_channels > 0:
        ch = np.random.default_rng([cfg.cfg_id, head, 4]).choice(d, cfg.qk_outlier_channels, replace=False)
        q[:, ch] *= np.float32(cfg.qk_outlier_scale)
        k[:, ch] *= np.float32(cfg.qk_outlier_scale)
    v = _v_head(cfg, head, step)
    return bf16_bits(q), bf16_bits(k), bf16_bits(v)


def make_qkv(cfg: Config, heads: Optional[List[int]] = None, step: int = 0):
    """bf16 bit patterns (uint16) of shape (B, len(heads), N, d) for Q, K, V.

    Batch entries b > 0 reuse the head seeds offset by b * H.
    """
    if heads is None:
        heads = list(range(cfg.H))
    shape = (cfg.B, len(heads), cfg.N, cfg.d)
    Q = np.empty(shape, np.uint16)
    K = np.empty(shape, np.uint16)
    V = np.empty(shape, np.uint16)
    for b in range(cfg.B):
        for i, h in enumerate(heads):
            Q[b, i], K[b, i], V[b, i] = make_head(cfg, h + b * cfg.H, step)
    return Q, K, V


def make_reuse_steps(cfg: Config, heads: Optional[List[int]] = None):
    """Q, K fixed and V for each of cfg.steps consecutive steps (list of uint16 arrays)."""
    Q, K, V0 = make_qkv(cfg, heads, 0)
    Vs = [V0]
    for s in range(1, cfg.steps):
        Vs.append(make_qkv(cfg, heads, s)[2])
    return Q, K, Vs
