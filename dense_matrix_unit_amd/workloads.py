"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers (numpy PCG64) and returns FP32 source
arrays; it holds none of the method's arithmetic (no rounding to BF16/FP8, no
scaling).  Tests and the benchmark both draw their inputs from here.

Recipes (value distributions follow the pages' experiments):
  * ``uniform_pm1``: U[-1, 1) drawn in FP64, stored as FP32 -- the input of the
    page "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured",
    Step 2 (uniform in [-1, 1), later rounded to BF16).
  * ``normal``: N(0, 1) in FP64, stored as FP32.
  * ``outlier_rows``: ``round(frac * rows)`` distinct row indices, drawn without
    replacement; the caller multiplies those rows by a factor (activations with
    a few large rows, the case fine-grained FP8 scaling is for).
  * ``small_ints``: integers in [lo, hi], exact in BF16 and FP8, so that a
    product computed in any order is exact.
  * ``expert_rows``: how many of ``total`` routed rows each of G experts gets
    in one step: a multinomial draw with probabilities proportional to
    exp(spread * z), z ~ N(0, 1) per expert (uneven load; some experts may
    get none).
Seeds: A = 1, B = 2 (the seeds of the handbook chapter's WMMA harness),
outlier rows = 3.
"""
from __future__ import annotations

import numpy as np

SEED_A = 1
SEED_B = 2
SEED_OUTLIERS = 3


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def uniform_pm1(shape, seed: int) -> np.ndarray:
    return _rng(seed).uniform(-1.0, 1.0, size=shape).astype(np.float32)


def normal(shape, seed: int) -> np.ndarray:
    return _rng(seed).standard_normal(size=shape).astype(np.float32)


def outlier_rows(rows: int, seed: int = SEED_OUTLIERS, frac: float = 0.01) -> np.ndarray:
    n = int(round(frac * rows))
    return np.sort(_rng(seed).choice(rows, size=n, replace=False)).astype(np.int64)


def normal_with_outlier_rows(shape, seed: int, factor: float = 100.0,
                             outlier_seed: int = SEED_OUTLIERS, frac: float = 0.01):
    """N(0,1) FP32 matrix with round(frac*rows) rows multiplied by `factor`
    (the product is formed in FP32).  Returns (X, outlier row indices)."""
    X = normal(shape, seed)
    idx = outlier_rows(shape[0], outlier_seed, frac)
    X[idx] *= np.float32(factor)
    return X, idx


def small_ints(shape, seed: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    return _rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def expert_rows(G: int, total: int, seed: int, spread: float = 0.5) -> np.ndarray:
    rng = _rng(seed)
    w = np.exp(spread * rng.standard_normal(G))
    return rng.multinomial(total, w / w.sum()).astype(np.int64)


SEED_ROUTING = 4

# The workloads: (name, M, N, K) with their input recipe.  B is stored N x K
# ("column-major B") unless a row-major variant is named.
WORKLOADS = {
    "bf16_256": dict(M=256, N=256, K=256, dist="uniform_pm1", out="f32"),
    "bf16_4096": dict(M=4096, N=4096, K=4096, dist="normal", out="bf16"),
    "fp8_4096": dict(M=4096, N=4096, K=4096, dist="normal", out="bf16"),
    "fp8_block_8192x7168x7168": dict(M=8192, N=7168, K=7168, dist="normal_outliers",
                                     out="bf16"),
    "llm_28672x8192": dict(Ms=(16, 128, 1024, 8192), N=28672, K=8192, dist="normal",
                           out="bf16"),
    "moe_bf16_32x16384x4096x7168": dict(G=32, total_rows=16384, N=4096, K=7168, dist="normal",
                                        routing="expert_rows(spread 0.5, seed 4)", out="bf16"),
    "attention_bf16_32x4096x4096x128": dict(heads=32, S=4096, d=128, dist="normal",
                                            scale="1/sqrt(d)", out="bf16"),
    "acc_sweep_256": dict(M=256, N=256, Ks=(256, 1024, 4096, 16384, 65536), dist="normal",
                          out="f32"),
}
