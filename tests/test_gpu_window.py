"""GPU parity of the whole-window bf16 kernel (kernel 5: K and V of a window staged in LDS once,
for N x head_dim = 144 x 128 and 288 x 64) against the fp64 oracle, with the bf16 acceptance bar."""
import math

import numpy as np
import pytest
import torch

import datagen
import swin3d_window_attention_amd as sw
from _gpu import check, check_sampled, device_inputs, oracle_full, run_gpu, sample_windows, say, to_f64

pytestmark = pytest.mark.gpu

BIASES = [-100.0, -math.inf]


def wl_of(name, B, D, H, W, heads, dh, window, shift, seed=43):
    return datagen.small_workload(name, B, D, H, W, heads, dh, window, shift, "bf16", seed)


SMALL = [
    wl_of("dh128", 1, 4, 12, 24, 2, 128, (2, 6, 12), (1, 3, 6)),            # N = 144, no padding
    wl_of("dh128_ragged", 2, 3, 13, 25, 2, 128, (2, 6, 12), (1, 3, 6)),     # padding on every axis
    wl_of("dh128_noshift", 1, 2, 12, 24, 3, 128, (2, 6, 12), (0, 0, 0)),    # no mask step at all
    wl_of("dh128_single_token", 1, 1, 1, 1, 2, 128, (2, 6, 12), (1, 3, 6)),  # 143 padding slots
    wl_of("w2x12x12", 1, 4, 24, 36, 2, 64, (2, 12, 12), (1, 6, 6)),         # N = 288, no padding
    wl_of("w2x12x12_ragged", 2, 3, 13, 17, 2, 64, (2, 12, 12), (1, 6, 6)),  # padding on every axis
    wl_of("w2x12x12_noshift", 1, 2, 24, 24, 2, 64, (2, 12, 12), (0, 0, 0)),
    wl_of("w4x6x12_dh64", 1, 4, 12, 24, 2, 64, (4, 6, 12), (2, 3, 6)),       # another 288-slot window
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("bias", BIASES)
def test_small_whole_grid(wl, bias):
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    assert plan.info().kernel == 5
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    ref = oracle_full(wl, bias)
    check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"bias={bias}")


LARGE_LOGITS = [
    # Q and K x 8, V ~ U(-1, 1): nearly one-hot rows with a logit spread of hundreds
    datagen.small_workload("dh128_qk8", 1, 4, 13, 25, 2, 128, (2, 6, 12), (1, 3, 6), "bf16", 49,
                           qk_mult=8.0, v_dist="uniform"),
    datagen.small_workload("w2x12x12_qk8", 1, 4, 13, 25, 2, 64, (2, 12, 12), (1, 6, 6), "bf16", 50,
                           qk_mult=8.0, v_dist="uniform"),
]


@pytest.mark.parametrize("wl", LARGE_LOGITS, ids=lambda w: w.name)
def test_large_logits(wl):
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    assert plan.info().kernel == 5
    x = device_inputs(wl)
    for bias in BIASES:
        o = to_f64(run_gpu(wl, bias, x))
        ref = oracle_full(wl, bias)
        check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"bias={bias}")


def test_stage2_grid_head_dim_128():
    """The stage-2 grid with 8 heads of 128 (same channel count as 16 x 64), heads 0 and 7."""
    wl = wl_of("stage2_dh128", 1, 4, 90, 180, 8, 128, (2, 6, 12), (1, 3, 6), seed=2)
    x = device_inputs(wl)
    for bias in BIASES:
        o = to_f64(run_gpu(wl, bias, x))
        ref = oracle_full(wl, bias, [0, 7])
        check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"heads 0,7 bias={bias}")


@pytest.mark.parametrize("name", ["stage1_h4d128", "stage1_w2x12x12"])
def test_stage1_grid_sampled(name):
    """The stage-1 grid in the launch configuration the benchmark times, on 24 sampled windows
    (every head), and every output element written."""
    wl = datagen.WORKLOADS[name]
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    assert plan.info().kernel == 5
    x = device_inputs(wl, keep_host=True)
    o = run_gpu(wl, -100.0, x)
    assert not torch.isnan(o).any().item()
    check_sampled(wl, -100.0, o, sample_windows(wl, 24, seed=9), x["host"])


@pytest.mark.parametrize("idx", [1, 5])
def test_strided_views(idx):
    """Q, K, V as views of one fused [.., 3, heads, head_dim] buffer and O inside a wider row:
    bit-identical to the contiguous run, and the bytes past O's row untouched."""
    wl = SMALL[idx]
    x = device_inputs(wl)
    contiguous = run_gpu(wl, -100.0, x)
    B, D, H, W, h, dh = wl.shape
    fused = torch.stack([x["q"], x["k"], x["v"]], dim=4).contiguous()
    wide = torch.full((B, D, H, W, h * dh + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = wide.view(torch.int16).clone()
    o = wide[..., :h * dh].unflatten(-1, (h, dh))
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    plan.run(fused[..., 0, :, :], fused[..., 1, :, :], fused[..., 2, :, :], o)
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous().view(torch.int16), contiguous.view(torch.int16))
    assert torch.equal(wide.view(torch.int16)[..., h * dh:], before[..., h * dh:])
    say(f"[gpu] whole-window strided run ({wl.name}) bit-identical, padding untouched")
