"""GPU parity of the FP32-I/O split-bf16 matrix-core kernel (plan dtype "f32_split")
against the fp64 oracle, with the tolerance derived in tests/test_split_model.py."""
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


def split_workload(name, B, D, H, W, heads, shift, seed, **kw):
    return datagen.small_workload(name, B, D, H, W, heads, 64, (2, 6, 12), shift, "f32", seed,
                                  plan="f32_split", **kw)


SMALL = [
    split_workload("split_small", 1, 2, 12, 24, 2, (1, 3, 6), 30),
    split_workload("split_ragged", 2, 3, 7, 13, 3, (1, 5, 11), 31),   # padding on every axis
    split_workload("split_pad_ne_shift", 1, 4, 44, 30, 2, (1, 3, 6), 32),
    split_workload("split_one_token", 1, 1, 1, 1, 2, (1, 3, 6), 33),
    split_workload("split_noshift", 1, 2, 12, 36, 4, (0, 0, 0), 34),
    split_workload("split_stress_small", 1, 2, 12, 48, 2, (1, 3, 6), 35, qk_mult=8.0, v_dist="uniform"),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("bias", BIASES)
def test_small_whole_grid(wl, bias):
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    ref = oracle_full(wl, bias)
    check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"bias={bias}")


@pytest.mark.parametrize("name", ["stage3_pad_f32_split", "stress_f32_split"])
@pytest.mark.parametrize("bias", BIASES)
def test_stage_whole_grid(name, bias):
    wl = WL[name]
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    heads = [0, wl.heads - 1]
    ref = oracle_full(wl, bias, heads)
    check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"heads {heads} bias={bias}")


def test_stage1_full_size_sampled():
    wl = WL["stage1_f32_split"]
    x = device_inputs(wl, keep_host=True)
    o = run_gpu(wl, -100.0, x)
    assert not torch.isnan(o).any().item(), "an output element was never written"
    check_sampled(wl, -100.0, o, sample_windows(wl, 48, seed=7), x["host"])


def test_between_exact_f32_and_tolerance():
    """On the same fp32 inputs the exact-fp32 kernel is closer to the oracle than the split
    kernel (splits cannot beat exact arithmetic), and the split kernel stays inside its bar."""
    wl = SMALL[0]
    x = device_inputs(wl)
    ref = oracle_full(wl, -100.0)
    err = lambda o: max(float(np.abs(to_f64(o)[..., h, :] - r).max()) for h, r in ref.items())
    e_split = err(run_gpu(wl, -100.0, x))
    plan32 = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="f32", scale=wl.scale)
    o32 = torch.empty_like(x["q"])
    plan32.run(x["q"], x["k"], x["v"], o32)
    torch.cuda.synchronize()
    e_f32 = err(o32)
    say(f"[gpu] split {e_split:.2e}  exact f32 {e_f32:.2e}")
    assert e_f32 <= e_split <= 5e-5


def test_strided_and_guard():
    """Fused-QKV strided input and a wide strided output give bit-identical results, and
    nothing outside the output positions is written."""
    wl = SMALL[1]
    x = device_inputs(wl)
    contiguous = run_gpu(wl, -100.0, x)
    B, D, H, W, h, dh = wl.shape
    fused = torch.stack([x["q"], x["k"], x["v"]], dim=4).contiguous()
    wide = torch.full((B, D, H, W, h * dh + 32), float("nan"), dtype=torch.float32, device="cuda")
    before = wide.view(torch.int32).clone()
    o = wide[..., :h * dh].unflatten(-1, (h, dh))
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="f32_split", scale=wl.scale)
    plan.run(fused[..., 0, :, :], fused[..., 1, :, :], fused[..., 2, :, :], o)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous().view(torch.int32), contiguous.view(torch.int32))
    assert torch.equal(wide.view(torch.int32)[..., h * dh:], before[..., h * dh:])


def test_binding_accepts_f32_tensors_only():
    wl = SMALL[0]
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="f32_split", scale=wl.scale)
    assert plan.info().kernel == 2
    xb = torch.zeros(wl.shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        plan.run(xb, xb, xb, torch.empty_like(xb))
