"""Seeded synthetic inputs for Swin3D shifted-window attention.

This module is the only code shared by the fp64 oracle and the GPU library's
tests and benchmark. It holds no attention arithmetic: it draws random
tensors, rounds them to the I/O dtype, and describes the workloads.

Workloads stand in for the ERA5 encoder activations of the Flash-Aurora
README ("CuTe DSL window attention": attention shapes (1800,8,144,64),
(450,16,144,64), (128,32,144,64) with window (2,6,12), N = 144). Those
activations need data and trained weights that are not available, so the
inputs here are seeded iid draws of the same shapes. The kernel has no
value-dependent control flow, so timing on them is faithful.

Generation recipe (every config):
  * one numpy Generator per (seed, tensor id, b, d) slice, tensor ids
    Q=0, K=1, V=2, so any [H, W, heads, head_dim] slice can be regenerated
    alone (the largest config is 3.3 GB per bf16 tensor);
  * float32 draws in C order, N(0,1) unless the config says otherwise;
  * bf16 configs round the float32 draw to bfloat16 with round-to-nearest-
    even and keep the 16-bit patterns (numpy uint16); a multiplier that is
    a power of two is applied after rounding, so it is exact.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: grid-layout Q/K/V of shape [B, D, H, W, heads, head_dim]."""

    name: str
    B: int
    D: int
    H: int
    W: int
    heads: int
    head_dim: int
    window: tuple
    shift: tuple
    dtype: str  # "f32" or "bf16": the I/O dtype
    seed: int
    qk_mult: float = 1.0  # power-of-two multiplier applied to Q and K after rounding
    v_dist: str = "normal"  # "normal" -> N(0,1); "uniform" -> U(-1, 1)
    plan: str = ""  # library dtype when it differs from the I/O dtype ("f32_split")

    @property
    def plan_dtype(self) -> str:
        return self.plan or self.dtype

    @property
    def shape(self):
        return (self.B, self.D, self.H, self.W, self.heads, self.head_dim)

    @property
    def tokens(self) -> int:
        return self.B * self.D * self.H * self.W

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim) rounded to float32, the value handed to the library."""
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))

    def with_shift(self, shift, name=None):
        return dataclasses.replace(self, shift=tuple(shift), name=name or self.name)


# The workloads. Sizes follow the three ERA5 encoder latent stages of a
# 0.25-degree grid (721x1440 -> 4 x 180 x 360 tokens at stage 1), one tiny fp32
# case for exhaustive checks and one high-resolution stress case with large
# logits (Q, K scaled by 8) and uniform V.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 12, 24, 2, 32, (2, 6, 12), (1, 3, 6), "f32", 0),
    "stage1": Workload("stage1", 1, 4, 180, 360, 8, 64, (2, 6, 12), (1, 3, 6), "bf16", 1),
    "stage2_s0": Workload("stage2_s0", 1, 4, 90, 180, 16, 64, (2, 6, 12), (0, 0, 0), "bf16", 2),
    "stage2": Workload("stage2", 1, 4, 90, 180, 16, 64, (2, 6, 12), (1, 3, 6), "bf16", 2),
    "stage3_pad": Workload("stage3_pad", 1, 4, 45, 90, 32, 64, (2, 6, 12), (1, 3, 6), "bf16", 3),
    "stress_hres": Workload("stress_hres", 2, 4, 450, 900, 8, 64, (2, 6, 12), (1, 3, 6), "bf16", 4,
                            qk_mult=8.0, v_dist="uniform"),
    # other window sizes and head_dim 128 on the stage-1 grid (the K/V-streaming kernel)
    "stage1_w2x12x12": Workload("stage1_w2x12x12", 1, 4, 180, 360, 8, 64, (2, 12, 12), (1, 6, 6), "bf16", 1),
    "stage1_h4d128": Workload("stage1_h4d128", 1, 4, 180, 360, 4, 128, (2, 6, 12), (1, 3, 6), "bf16", 1),
    "stage1_w4x12x24": Workload("stage1_w4x12x24", 1, 4, 180, 360, 8, 64, (4, 12, 24), (2, 6, 12), "bf16", 1),
    "stage1_w3x12x12_h4d128": Workload("stage1_w3x12x12_h4d128", 1, 4, 180, 360, 4, 128, (3, 12, 12), (1, 6, 6),
                                       "bf16", 1),
    # FP32-I/O runs of the stage shapes (unrounded float32 draws) for the split-bf16
    # matrix-core path and the exact fp32 path
    "stage1_f32_split": Workload("stage1_f32_split", 1, 4, 180, 360, 8, 64, (2, 6, 12), (1, 3, 6), "f32", 1,
                                 plan="f32_split"),
    "stage3_pad_f32_split": Workload("stage3_pad_f32_split", 1, 4, 45, 90, 32, 64, (2, 6, 12), (1, 3, 6),
                                     "f32", 3, plan="f32_split"),
    "stress_f32_split": Workload("stress_f32_split", 1, 4, 90, 180, 8, 64, (2, 6, 12), (1, 3, 6), "f32", 4,
                                 qk_mult=8.0, v_dist="uniform", plan="f32_split"),
    # the same shapes on the exact FP32 path (FP32 matrix-core products)
    "stage1_f32": Workload("stage1_f32", 1, 4, 180, 360, 8, 64, (2, 6, 12), (1, 3, 6), "f32", 1),
    "stage3_pad_f32": Workload("stage3_pad_f32", 1, 4, 45, 90, 32, 64, (2, 6, 12), (1, 3, 6), "f32", 3),
    "stress_f32": Workload("stress_f32", 1, 4, 90, 180, 8, 64, (2, 6, 12), (1, 3, 6), "f32", 4,
                           qk_mult=8.0, v_dist="uniform"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite draws, so NaN handling is not needed and not done."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _mult_bf16_bits(bits: np.ndarray, mult: float) -> np.ndarray:
    # Multiplying by a power of two only moves the exponent: exact for these magnitudes.
    m, e = np.frexp(mult)
    if m != 0.5:
        raise ValueError("multiplier must be a power of two to stay exact in bf16")
    f = bf16_bits_to_f32(bits) * np.float32(mult)
    out = f32_to_bf16_bits(f)
    assert np.array_equal(bf16_bits_to_f32(out), f)
    return out


def slice_f32(wl: Workload, tensor: str, b: int, d: int) -> np.ndarray:
    """The [H, W, heads, head_dim] slice (b, d) of tensor q/k/v as float32 draws (before rounding)."""
    rng = np.random.default_rng([wl.seed, TENSOR_IDS[tensor], b, d])
    shp = (wl.H, wl.W, wl.heads, wl.head_dim)
    if tensor == "v" and wl.v_dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shp).astype(np.float32)
    return rng.standard_normal(shp, dtype=np.float32)


def slice_io(wl: Workload, tensor: str, b: int, d: int) -> np.ndarray:
    """The (b, d) slice in the I/O dtype: float32 array, or uint16 bf16 bit patterns."""
    x = slice_f32(wl, tensor, b, d)
    if wl.dtype == "f32":
        if tensor in ("q", "k") and wl.qk_mult != 1.0:
            x = x * np.float32(wl.qk_mult)  # a power of two: exact
        return x
    bits = f32_to_bf16_bits(x)
    if tensor in ("q", "k") and wl.qk_mult != 1.0:
        bits = _mult_bf16_bits(bits, wl.qk_mult)
    return bits


def slice_f64(wl: Workload, tensor: str, b: int, d: int) -> np.ndarray:
    """The (b, d) slice exactly as the GPU receives it, widened to float64."""
    x = slice_io(wl, tensor, b, d)
    if wl.dtype == "bf16":
        x = bf16_bits_to_f32(x)
    return x.astype(np.float64)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def full_io(wl: Workload, tensor: str) -> np.ndarray:
    """Whole tensor [B, D, H, W, heads, head_dim] in the I/O dtype (float32 or uint16 bits)."""
    dt = np.float32 if wl.dtype == "f32" else np.uint16
    out = np.empty(wl.shape, dtype=dt)

    def fill(bd):
        b, d = bd
        out[b, d] = slice_io(wl, tensor, b, d)

    jobs = [(b, d) for b in range(wl.B) for d in range(wl.D)]
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(fill, jobs))
    return out


def full_f64(wl: Workload, tensor: str) -> np.ndarray:
    """Whole tensor widened to float64 (small workloads only)."""
    x = full_io(wl, tensor)
    if wl.dtype == "bf16":
        x = bf16_bits_to_f32(x)
    return x.astype(np.float64)


def to_torch(x: np.ndarray, dtype: str):
    """Host array in I/O representation -> CPU torch tensor of the I/O dtype (no rounding)."""
    import torch

    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def small_workload(name, B, D, H, W, heads, head_dim, window, shift, dtype, seed, **kw) -> Workload:
    """Ad-hoc workload for tests (same generation recipe)."""
    return Workload(name, B, D, H, W, heads, head_dim, tuple(window), tuple(shift), dtype, seed, **kw)


# ---- fused AdaLN + residual inputs ------------------------------------------

@dataclasses.dataclass(frozen=True)
class AdalnWorkload:
    """x, res: [B, rows, C] in their I/O dtypes; gamma, beta: [B, C] float32."""
    name: str
    B: int
    rows: int
    C: int
    x_dtype: str
    res_dtype: str
    out_dtype: str
    seed: int
    eps: float = 1e-5

    @property
    def shape(self):
        return (self.B, self.rows, self.C)


# The stage-1 token count and a 512-channel embedding (8 heads x 64): x is the
# bf16 output of the attention block's projection, the residual stream and the
# output stay in float32 between blocks.
ADALN_WORKLOADS = {
    "adaln_stage1": AdalnWorkload("adaln_stage1", 1, 4 * 180 * 360, 512, "bf16", "f32", "f32", 21),
}


def adaln_inputs(wl: AdalnWorkload) -> dict:
    """Seeded inputs in I/O representation (float32 arrays or uint16 bf16 bits). Each row of x has
    its own offset U(-1, 1) and spread U(0.5, 2) so that centering and scaling both matter;
    res ~ N(0, 1); gamma = 1 + 0.2 N(0, 1), beta = 0.2 N(0, 1)."""
    out = {"x": [], "res": [], "gamma": [], "beta": []}
    for b in range(wl.B):
        rng = np.random.default_rng([wl.seed, 10, b])
        mu = rng.uniform(-1.0, 1.0, size=(wl.rows, 1)).astype(np.float32)
        sd = rng.uniform(0.5, 2.0, size=(wl.rows, 1)).astype(np.float32)
        x = mu + sd * rng.standard_normal((wl.rows, wl.C), dtype=np.float32)
        res = np.random.default_rng([wl.seed, 11, b]).standard_normal((wl.rows, wl.C), dtype=np.float32)
        prng = np.random.default_rng([wl.seed, 12, b])
        out["gamma"].append(1.0 + 0.2 * prng.standard_normal(wl.C, dtype=np.float32))
        out["beta"].append(0.2 * prng.standard_normal(wl.C, dtype=np.float32))
        out["x"].append(f32_to_bf16_bits(x) if wl.x_dtype == "bf16" else x)
        out["res"].append(f32_to_bf16_bits(res) if wl.res_dtype == "bf16" else res)
    return {k: np.stack(v) for k, v in out.items()}


def io_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """I/O representation -> the float64 values it holds."""
    return (bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)
