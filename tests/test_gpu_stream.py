"""GPU parity of the K/V-streaming bf16 kernel (kernel 3: bf16 windows whose K and V do not fit
the single-tile kernels, and head_dim 32) against the fp64 oracle, with the bf16 acceptance bar."""
import math

import numpy as np
import pytest
import torch

import datagen
import swin3d_window_attention_amd as sw
from _gpu import check, check_sampled, device_inputs, oracle_full, run_gpu, sample_windows, say, to_f64

pytestmark = pytest.mark.gpu

BIASES = [-100.0, -math.inf]


def wl_of(name, B, D, H, W, heads, dh, window, shift, seed=41):
    return datagen.small_workload(name, B, D, H, W, heads, dh, window, shift, "bf16", seed)


SMALL = [
    wl_of("w2x6x6", 1, 4, 12, 24, 2, 64, (2, 6, 6), (1, 3, 3)),        # N = 72: a partial second chunk
    wl_of("w4x8x8_ragged", 2, 5, 13, 17, 2, 128, (4, 8, 8), (2, 4, 4)),  # N = 256, padding on every axis
    wl_of("w1x7x7", 1, 3, 20, 30, 3, 64, (1, 7, 7), (0, 3, 3)),        # N = 49 < one chunk
    wl_of("w4x12x24", 1, 4, 24, 48, 1, 64, (4, 12, 24), (2, 6, 12)),   # N = 1152: 18 chunks
    wl_of("w2x6x6_noshift", 1, 2, 12, 18, 2, 64, (2, 6, 6), (0, 0, 0)),  # no mask step but a partial chunk
    wl_of("single_token", 1, 1, 1, 1, 2, 128, (2, 6, 6), (1, 3, 3)),
    wl_of("w3x12x12", 1, 6, 24, 24, 2, 128, (3, 12, 12), (1, 6, 6)),     # N = 432: 9 chunks of 48
    wl_of("w3x12x12_dh64", 1, 3, 13, 25, 2, 64, (3, 12, 12), (1, 6, 6)),  # the same at head_dim 64, padded
    wl_of("w2x6x4", 1, 4, 13, 15, 2, 64, (2, 6, 4), (1, 3, 2)),          # N = 48: one 48-key chunk
    wl_of("w16x16x16_max", 1, 16, 16, 20, 1, 64, (16, 16, 16), (8, 4, 10)),  # N = 4096, the largest window
    wl_of("dh32", 1, 4, 13, 25, 3, 32, (2, 6, 12), (1, 3, 6)),           # head_dim 32, N = 144
    wl_of("dh32_w2x6x6", 2, 3, 10, 14, 2, 32, (2, 6, 6), (1, 3, 3)),      # head_dim 32, N = 72
    # D padded 4 -> 6: in the second D-window two of three depth planes are padding, so whole
    # query blocks and whole 48-key chunks hold padding only (the skipping instance)
    wl_of("w3x12x12_d4pad", 1, 4, 24, 24, 2, 128, (3, 12, 12), (1, 6, 6)),
    # D padded 3 -> 4: the second D-window's first depth plane (64 slots) is padding, one whole
    # 64-key chunk of the four
    wl_of("w2x8x8_d3pad", 1, 3, 16, 24, 3, 64, (2, 8, 8), (1, 4, 4)),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("bias", BIASES)
def test_small_whole_grid(wl, bias):
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    assert plan.info().kernel == 3
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    ref = oracle_full(wl, bias)
    check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"bias={bias}")


LARGE_LOGITS = [
    # Q and K x 8, V ~ U(-1, 1): logits with a spread of hundreds, so the running max of a row
    # jumps many times across the chunks (the lazy rescale's move and keep branches both run)
    datagen.small_workload("w4x12x24_qk8", 1, 4, 24, 48, 1, 64, (4, 12, 24), (2, 6, 12), "bf16", 47,
                           qk_mult=8.0, v_dist="uniform"),
    datagen.small_workload("w3x12x12_dh128_qk8", 1, 3, 13, 25, 2, 128, (3, 12, 12), (1, 6, 6), "bf16", 48,
                           qk_mult=8.0, v_dist="uniform"),
]


@pytest.mark.parametrize("wl", LARGE_LOGITS, ids=lambda w: w.name)
def test_large_logits(wl):
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype="bf16", scale=wl.scale)
    assert plan.info().kernel == 3
    x = device_inputs(wl)
    for bias in BIASES:
        o = to_f64(run_gpu(wl, bias, x))
        ref = oracle_full(wl, bias)
        check(wl, np.stack([o[..., h, :] for h in ref]), np.stack(list(ref.values())), f"bias={bias}")


@pytest.mark.parametrize("name", ["stage1_w4x12x24", "stage1_w3x12x12_h4d128"])
def test_stage1_grid_streaming_sampled(name):
    """The stage-1 grid with window (4, 12, 24) (N = 1152, K and V of 295 KB per window and head:
    18 chunks), and with window (3, 12, 12) at 4 heads x 128 (N = 432 in nine 48-key chunks; the
    depth axis padded from 4 to 6), in the launch configuration the benchmark times, on 12 sampled
    windows each."""
    wl = datagen.WORKLOADS[name]
    x = device_inputs(wl, keep_host=True)
    o = run_gpu(wl, -100.0, x)
    assert not torch.isnan(o).any().item()
    check_sampled(wl, -100.0, o, sample_windows(wl, 12, seed=9), x["host"])


def test_strided_and_guard():
    wl = SMALL[2]
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
    say("[gpu] streaming strided run bit-identical, padding untouched")
