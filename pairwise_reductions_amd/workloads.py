"""Seeded synthetic workloads for the pairwise-reduction engine.

This module only draws random inputs; it holds none of the reductions' arithmetic, so the
device path, the CPU oracle and the benchmark can all share it.

The six workloads follow the sizes and distributions the pages use:
  * "Kernel matrix reduction" (concept page), Variants: Gaussian product, D=3, float32,
    10k / 100k / 1M points;
  * "Fast Gauss Sums via Flash Attention", Figure 1 (lower row): B=4, D=32, C=32, fp16, and
    Figure 2: forward and backward at B=4, D=32, C=1, fp16.
Points in the unit cube are drawn on the 2^-24 grid so that every coordinate is an exact
float32 value and no generator internals beyond integer draws are relied on.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

GRID_BITS = 24


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named workload: an operation, its sizes and the input distribution."""

    key: str
    op: str
    M: int
    N: int
    D: int
    C: int = 1
    B: int = 1
    K: int = 0
    sigma: float = 1.0
    dist: str = "uniform"
    seed: int = 0
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "gauss_sum_10k": Workload(
        key="gauss_sum_10k", op="gauss_sum", M=10_000, N=10_000, D=3, C=1, sigma=0.1,
        description="Gaussian kernel sum, M=N=1e4, D=3, C=1, fp32, uniform [0,1)^3, sigma=0.1"),
    "gauss_sum_grad_x_100k_mixture": Workload(
        key="gauss_sum_grad_x_100k_mixture", op="gauss_sum+grad_x", M=100_000, N=100_000, D=3,
        C=1, sigma=0.05, dist="mixture8",
        description="Gaussian kernel sum and its gradient w.r.t. x, M=N=1e5, D=3, C=1, fp32, "
                    "mixture of 8 isotropic Gaussians (std 0.05), sigma=0.05"),
    "gauss_sum_1m": Workload(
        key="gauss_sum_1m", op="gauss_sum", M=1_000_000, N=1_000_000, D=3, C=1, sigma=0.01,
        description="Gaussian kernel sum, M=N=1e6, D=3, C=1, fp32, uniform [0,1)^3, sigma=0.01"),
    "batched_gauss_sum_fp16": Workload(
        key="batched_gauss_sum_fp16", op="gauss_sum_batched", B=4, M=16_384, N=16_384, D=32,
        C=32, sigma=1.0, dist="normal_over_sqrt_d",
        description="Batched Gaussian kernel sum with signed weights, B=4, M=N=16384, D=32, "
                    "C=32, fp16 inputs, tau=1 (sigma=1)"),
    "batched_gauss_sum_fp16_fwd_bwd": Workload(
        key="batched_gauss_sum_fp16_fwd_bwd", op="gauss_sum_batched+backward", B=4, M=16_384, N=16_384,
        D=32, C=1, sigma=1.0, dist="normal_over_sqrt_d",
        description="Batched Gaussian kernel sum, forward and backward (gradients with respect "
                    "to x, y and b), B=4, M=N=16384, D=32, C=1, fp16 inputs, tau=1 (sigma=1)"),
    "argkmin_lse_100k": Workload(
        key="argkmin_lse_100k", op="argkmin+lse", M=100_000, N=100_000, D=3, K=10, sigma=0.1,
        description="Row-wise argKmin (K=10) of squared distance plus log-sum-exp of "
                    "-|x-y|^2/(2*0.1^2), M=N=1e5, D=3, fp32, uniform [0,1)^3"),
}


def grid24(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform draws on [0,1) that are exact multiples of 2^-24, as float32."""
    ints = rng.integers(0, 2 ** GRID_BITS, size=shape)
    return (ints * 2.0 ** -GRID_BITS).astype(np.float32)


def _mixture8(rng: np.random.Generator, centres: np.ndarray, n: int, d: int) -> np.ndarray:
    labels = rng.integers(0, centres.shape[0], n)
    noise = 0.05 * rng.standard_normal((n, d))
    return (centres[labels] + noise).astype(np.float32)


def make_inputs(key: str, M: Optional[int] = None, N: Optional[int] = None,
                B: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``key``; M, N, B and seed may be overridden.

    Draw order is fixed per workload so that a given (key, sizes, seed) always gives the
    same arrays on any machine:
      uniform:            x, y, then b (N, C) ~ N(0,1)
      mixture8:           8 centres ~ U[0,1)^3, x labels, x noise, y labels, y noise, then b
      normal_over_sqrt_d: q, k ~ N(0, I/D) as fp16, then v ~ N(0,1) as fp16
    Returns a dict with numpy arrays and the scalar parameters as numpy float32.
    """
    w = WORKLOADS[key]
    M = w.M if M is None else int(M)
    N = w.N if N is None else int(N)
    B = w.B if B is None else int(B)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = {"key": key, "M": M, "N": N, "D": w.D, "C": w.C, "B": B, "K": w.K,
           "sigma": np.float32(w.sigma)}
    if w.dist == "uniform":
        out["x"] = grid24(rng, (M, w.D))
        out["y"] = grid24(rng, (N, w.D))
        out["b"] = rng.standard_normal((N, w.C)).astype(np.float32)
    elif w.dist == "mixture8":
        centres = rng.random((8, w.D))
        out["x"] = _mixture8(rng, centres, M, w.D)
        out["y"] = _mixture8(rng, centres, N, w.D)
        out["b"] = rng.standard_normal((N, w.C)).astype(np.float32)
    elif w.dist == "normal_over_sqrt_d":
        scale = 1.0 / np.sqrt(w.D)
        out["x"] = (rng.standard_normal((B, M, w.D)) * scale).astype(np.float16)
        out["y"] = (rng.standard_normal((B, N, w.D)) * scale).astype(np.float16)
        out["b"] = rng.standard_normal((B, N, w.C)).astype(np.float16)
    else:  # pragma: no cover - table above is closed
        raise ValueError(w.dist)
    return out


def upstream_gradient(M: int, C: int, seed: int = 2, B: Optional[int] = None) -> np.ndarray:
    """A seeded upstream gradient g = dL/ds of shape (M, C), or (B, M, C) when B is given,
    float32 ~ N(0,1)."""
    shape = (M, C) if B is None else (B, M, C)
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def sample_rows(M: int, count: int, seed: int = 1, edge: int = 64) -> np.ndarray:
    """Sorted row indices for sampled checks: ``count`` seeded rows plus the first and
    last ``edge`` rows (so the tail of the last tile is always covered)."""
    rng = np.random.default_rng(seed)
    picks = rng.choice(M, size=min(count, M), replace=False)
    ends = np.concatenate([np.arange(min(edge, M)), np.arange(max(M - edge, 0), M)])
    return np.unique(np.concatenate([picks, ends]))
