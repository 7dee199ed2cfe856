"""Seeded synthetic layers: the only code shared by the oracle-side tests and the GPU side.

This module draws random numbers and rounds them to bf16 storage. It holds none of the
quantization or matmul arithmetic: callers hand the arrays it returns to the CPU oracle
and, separately, to the HIP library.

Workload shapes and value structure follow the pages:
  * Llama-7B MLP up-projection (4096 -> 11008) and a 70B-shaped MLP (8192 -> 28672),
    weights ~ N(0, sigma) ("DL S067 · Quantization", §2 uses 4096x4096 weight matrices);
  * outlier input channels: about 0.1 % of feature dimensions 20-100x larger than the rest
    ("DL S067 · Quantization", "The origin story" and §3 "The outlier problem");
  * a few weight rows with larger magnitude ("LLM Weight Quantization - GPTQ, AWQ,
    SmoothQuant, FP8 & INT4/INT8 Trade-offs", "Granularity and outliers" snippet scales
    rows by 6 and channels by 50).

Every config draws, in this order, from ``np.random.default_rng(seed)``:
  1. W = normal(0, sigma, (N, K))
  2. if row outliers:      rows = choice(N, round(0.01 N), replace=False); W[rows] *= 10
  3. X = normal(0, 1, (M_max, K))
  4. if channel outliers:  ch = choice(K, round(0.001 K), replace=False); X[:, ch] *= f
     where f = uniform(20, 100, len(ch)) (config 2) or the config's constant factor
  5. W and X are rounded fp64 -> fp32 -> bf16 (round to nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "make_layer", "f64_to_bf16_bits", "bf16_bits_to_f32"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    N: int
    K: int
    M_max: int
    sigma: float
    g: int
    mode: str              # "asym" or "sym"
    seed: int
    row_outliers: bool = False
    n_channel_outliers: int = 0
    channel_factor: float | None = None   # None -> uniform(20, 100) per channel


# Index i is configuration i+1 of the workload list (seed = index).
CONFIGS = [
    LayerConfig("tiny 128x256 M=1 asym g64", 128, 256, 1, 0.02, 64, "asym", 0),
    LayerConfig("llama7b-up 11008x4096 M=1 asym g128", 11008, 4096, 1, 0.02, 128, "asym", 1,
                n_channel_outliers=4, channel_factor=None),
    LayerConfig("batched-decode 4096x4096 M=16 sym g128", 4096, 4096, 16, 0.02, 128, "sym", 2,
                row_outliers=True, n_channel_outliers=4, channel_factor=50.0),
    LayerConfig("70b-mlp 28672x8192 M<=8 asym g128", 28672, 8192, 8, 0.015, 128, "asym", 3,
                n_channel_outliers=8, channel_factor=50.0),
    LayerConfig("prefill 8192x8192 M=2048 asym g128", 8192, 8192, 2048, 0.02, 128, "asym", 4,
                n_channel_outliers=8, channel_factor=100.0),
]


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round an array to fp32 (RNE), then to bf16 (RNE); return the bf16 bit patterns (uint16).

    Storage conversion for generated inputs only.  NaN never occurs in generated data.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_layer(cfg: LayerConfig, M: int | None = None, rows: int | None = None):
    """Generate (W_bits[N, K], X_bits[M, K]) as bf16 bit patterns (uint16), per the recipe above.

    ``M`` selects the first M rows of the drawn X (so M in {1, 4, 8} nest for the 70B shape).
    ``rows`` truncates W to its first rows after the full draw (the draw order is unchanged).
    """
    rng = np.random.default_rng(cfg.seed)
    W = rng.normal(0.0, cfg.sigma, (cfg.N, cfg.K))
    if cfg.row_outliers:
        idx = rng.choice(cfg.N, int(round(0.01 * cfg.N)), replace=False)
        W[idx] *= 10.0
    X = rng.normal(0.0, 1.0, (cfg.M_max, cfg.K))
    if cfg.n_channel_outliers:
        ch = rng.choice(cfg.K, cfg.n_channel_outliers, replace=False)
        if cfg.channel_factor is None:
            fac = rng.uniform(20.0, 100.0, len(ch))
        else:
            fac = np.full(len(ch), cfg.channel_factor)
        X[:, ch] *= fac
    m = cfg.M_max if M is None else M
    if not 0 <= m <= cfg.M_max:
        raise ValueError(f"M={m} outside [0, {cfg.M_max}] for {cfg.name}")
    if rows is not None:
        W = W[:rows]
    return f64_to_bf16_bits(W), f64_to_bf16_bits(X[:m])


def random_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale) values rounded to bf16 bits, for small parity cases."""
    return f64_to_bf16_bits(rng.normal(0.0, scale, shape))
