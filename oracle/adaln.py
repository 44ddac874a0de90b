"""Plain fp64 CPU oracle for the fused AdaLN + residual step of a Swin3D block.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the build entry point
and the benchmark's CPU-baseline leg may import or run this module. The GPU
library never calls it and shares no code with it.

What it computes (Flash-Aurora README, "Kernel fusion for backbone memory
traffic", the AdaLN bullet and the paragraph after it): a LayerNorm of each
token's C channels, FiLM modulation of the normalised values, and a residual
add, with the result optionally kept in FP32 between blocks.

Readings taken where the pages leave the formula open (listed with their
reasons in the design notes of the repository):
  * LayerNorm without its own affine weights, biased variance (divide by C),
    epsilon inside the square root: xhat = (x - mean) / sqrt(var + eps);
  * FiLM is the plain feature-wise form gamma * xhat + beta, with gamma and
    beta given per batch element and channel (whatever produced them from the
    conditioning, e.g. 1 + scale, is outside this step);
  * the residual is added last: out = res + gamma * xhat + beta.

Everything runs in float64 on the exact values the GPU receives.
"""
from __future__ import annotations

import numpy as np


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis, biased variance, float64."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps)


def adaln_residual(x: np.ndarray, res: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                   eps: float) -> np.ndarray:
    """out[b, t, c] = res[b, t, c] + gamma[b, c] * layer_norm(x)[b, t, c] + beta[b, c].

    x, res: [B, T, C]; gamma, beta: [B, C]. Returns float64 [B, T, C]."""
    xhat = layer_norm(x, eps)
    g = np.asarray(gamma, dtype=np.float64)[:, None, :]
    b = np.asarray(beta, dtype=np.float64)[:, None, :]
    return np.asarray(res, dtype=np.float64) + g * xhat + b
