"""GPU parity of the exact FP32 matrix-core kernel (plan dtype "f32", windows of up to 256 slots,
head_dim 32 or 64) against the fp64 oracle, with the FP32 bar (1e-5 max abs)."""
import math

import numpy as np
import pytest
import torch

import datagen
import swin3d_window_attention_amd as sw
from _gpu import (check, check_sampled, device_inputs, oracle_full, run_gpu, sample_windows, say,
                  to_f64)

pytestmark = pytest.mark.gpu

BIASES = [-100.0, -math.inf]
WL = datagen.WORKLOADS


def f32_workload(name, B, D, H, W, heads, dh, shift, seed, **kw):
    return datagen.small_workload(name, B, D, H, W, heads, dh, (2, 6, 12), shift, "f32", seed, **kw)


SMALL = [
    f32_workload("f32m_small", 1, 2, 12, 24, 2, 64, (1, 3, 6), 50),
    f32_workload("f32m_ragged", 2, 3, 7, 13, 3, 64, (1, 5, 11), 51),     # padding on every axis
    f32_workload("f32m_pad_ne_shift", 1, 4, 44, 30, 2, 64, (1, 3, 6), 52),
    f32_workload("f32m_one_token", 1, 1, 1, 1, 2, 64, (1, 3, 6), 53),
    f32_workload("f32m_noshift", 1, 2, 12, 36, 4, 32, (0, 0, 0), 54),
    f32_workload("f32m_dh32_ragged", 1, 5, 13, 25, 3, 32, (1, 4, 7), 55),
    f32_workload("f32m_stress_small", 1, 2, 12, 48, 2, 64, (1, 3, 6), 56, qk_mult=8.0, v_dist="uniform"),
]


OTHER_WINDOWS = [
    # windows of fewer than 144 slots: the last tile of 16 slots is partly padding (slots past N)
    datagen.small_workload("f32m_w2x6x6", 1, 4, 13, 20, 2, 64, (2, 6, 6), (1, 3, 3), "f32", 57),         # N = 72
    datagen.small_workload("f32m_w1x7x7", 2, 3, 15, 16, 2, 32, (1, 7, 7), (0, 3, 3), "f32", 58),         # N = 49
    datagen.small_workload("f32m_w2x4x4", 1, 4, 10, 13, 3, 64, (2, 4, 4), (1, 2, 3), "f32", 59),         # N = 32
    datagen.small_workload("f32m_w2x8x8", 1, 4, 17, 19, 2, 64, (2, 8, 8), (1, 4, 4), "f32", 60),         # N = 128
    datagen.small_workload("f32m_w1x1x3", 1, 2, 3, 7, 2, 32, (1, 1, 3), (0, 0, 1), "f32", 61),           # N = 3
    datagen.small_workload("f32m_w1x1x1", 1, 2, 3, 4, 2, 64, (1, 1, 1), (0, 0, 0), "f32", 62),           # N = 1
    datagen.small_workload("f32m_w3x5x9", 1, 5, 11, 20, 2, 32, (3, 5, 9), (2, 2, 4), "f32", 63),         # N = 135
    # windows of 145 to 256 slots: 10 tiles, or 12, 14, 16 with the tail as padding
    datagen.small_workload("f32m_w2x8x10", 1, 4, 13, 25, 2, 64, (2, 8, 10), (1, 4, 5), "f32", 64),       # N = 160
    datagen.small_workload("f32m_w2x10x10", 1, 3, 17, 23, 2, 32, (2, 10, 10), (1, 5, 5), "f32", 65),     # N = 200
    datagen.small_workload("f32m_w2x8x11", 1, 3, 17, 20, 2, 64, (2, 8, 11), (1, 4, 5), "f32", 69),       # N = 176
    datagen.small_workload("f32m_w1x13x14_dh32", 1, 2, 15, 30, 2, 32, (1, 13, 14), (0, 6, 7), "f32", 70),  # N = 182
    datagen.small_workload("f32m_w2x7x15", 1, 4, 15, 29, 2, 64, (2, 7, 15), (1, 3, 7), "f32", 66),       # N = 210
    datagen.small_workload("f32m_w4x8x8", 1, 5, 17, 9, 2, 64, (4, 8, 8), (2, 4, 4), "f32", 67),          # N = 256
    datagen.small_workload("f32m_w4x8x8_dh32", 2, 4, 8, 16, 3, 32, (4, 8, 8), (0, 0, 0), "f32", 68),     # N = 256
]


@pytest.mark.parametrize("wl", SMALL + OTHER_WINDOWS, ids=lambda w: w.name)
@pytest.mark.parametrize("bias", BIASES)
def test_small_whole_grid(wl, bias):
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="f32", scale=wl.scale)
    assert plan.info().kernel == 4
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    ref = oracle_full(wl, bias)
    check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"bias={bias}")


@pytest.mark.parametrize("name", ["stage3_pad_f32", "stress_f32"])
@pytest.mark.parametrize("bias", BIASES)
def test_stage_whole_grid(name, bias):
    wl = WL[name]
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    heads = [0, wl.heads - 1]
    ref = oracle_full(wl, bias, heads)
    check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"heads {heads} bias={bias}")


def test_stage1_full_size_sampled():
    wl = WL["stage1_f32"]
    x = device_inputs(wl, keep_host=True)
    o = run_gpu(wl, -100.0, x)
    assert not torch.isnan(o).any().item(), "an output element was never written"
    check_sampled(wl, -100.0, o, sample_windows(wl, 48, seed=9), x["host"])


def test_deterministic():
    """Two runs on the same inputs give the same bits."""
    wl = SMALL[1]
    x = device_inputs(wl)
    a = run_gpu(wl, -100.0, x)
    b = run_gpu(wl, -100.0, x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
