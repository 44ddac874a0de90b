"""GPU parity of the strided entry point: Q, K and V read straight out of a fused
projection buffer [B, D, H, W, 3, heads, head_dim], O written into a wider buffer.

The strided run must give bit-identical results to the contiguous run on the same
values (only addresses differ), match the fp64 oracle, and leave every element of
the wide output buffer outside the (token, head, dim) positions untouched."""
import math

import numpy as np
import pytest
import torch

import datagen
import swin3d_window_attention_amd as sw
from _gpu import check, device_inputs, oracle_full, run_gpu, say, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, D, H, W, heads, head_dim, shift, dtype, bias)
    ("stage3_pad", None, None, None, None, None, None, None, None, -100.0),
    ("tiny_f32", None, None, None, None, None, None, None, None, -math.inf),
    ("ragged_bf16", 2, 3, 7, 13, 3, 64, (1, 5, 11), "bf16", -math.inf),
    ("ragged_f32", 1, 4, 44, 30, 2, 32, (1, 3, 6), "f32", -100.0),
    ("ragged_f32_dh64", 2, 3, 7, 13, 3, 64, (1, 5, 11), "f32", -math.inf),
    ("f32_window_2x4x4", 1, 4, 10, 13, 2, 32, (1, 2, 3), "f32", -100.0, (2, 4, 4)),  # matrix cores, N = 32
    ("f32_window_2x8x10", 1, 4, 13, 25, 2, 32, (1, 4, 5), "f32", -100.0, (2, 8, 10)),  # matrix cores, N = 160
    ("bf16_stream_2x4x4", 1, 4, 10, 13, 2, 64, (1, 2, 3), "bf16", -100.0, (2, 4, 4)),  # K/V streaming, N = 32
    ("bf16_stream_3x12x12_dh128", 1, 4, 13, 14, 2, 128, (1, 6, 6), "bf16", -math.inf, (3, 12, 12)),  # N = 432
    ("bf16_window_2x12x12", 1, 2, 13, 25, 2, 64, (1, 6, 6), "bf16", -100.0, (2, 12, 12)),  # whole window, N = 288
]


def _workload(case):
    name, B, D, H, W, h, dh, shift, dt = case[:9]
    window = case[10] if len(case) > 10 else (2, 6, 12)
    if B is None:
        return datagen.WORKLOADS[name]
    return datagen.small_workload(name, B, D, H, W, h, dh, window, shift, dt, seed=23)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fused_qkv_and_wide_output(case):
    wl, bias = _workload(case), case[9]
    x = device_inputs(wl)
    contiguous = run_gpu(wl, bias, x)
    B, D, H, W, h, dh = wl.shape
    fused = torch.stack([x["q"], x["k"], x["v"]], dim=4).contiguous()  # [B, D, H, W, 3, h, dh]
    q, k, v = fused[..., 0, :, :], fused[..., 1, :, :], fused[..., 2, :, :]
    extra = 64  # elements of padding after each token's row in the output buffer
    wide = torch.full((B, D, H, W, h * dh + extra), float("nan"), dtype=x["q"].dtype, device="cuda")
    ibits = torch.int16 if wl.dtype == "bf16" else torch.int32
    before = wide.view(ibits).clone()
    o = wide[..., :h * dh].unflatten(-1, (h, dh))
    assert o.stride()[3] == h * dh + extra and q.stride()[3] == 3 * h * dh
    say(f"[gpu] strided {wl.name} shape={wl.shape} bias={bias}")
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.dtype, scale=wl.scale,
                   cross_region_bias=bias)
    plan.run(q, k, v, o)
    torch.cuda.synchronize()
    # same values as the contiguous path, bit for bit
    assert torch.equal(o.contiguous().view(ibits), contiguous.view(ibits))
    # the padding after each row is untouched
    assert torch.equal(wide.view(ibits)[..., h * dh:], before[..., h * dh:])
    # and the oracle agrees
    got = to_f64(o.contiguous())
    heads = [0, h - 1]
    ref = oracle_full(wl, bias, heads)
    check(wl, np.stack([got[..., i, :] for i in ref]), np.stack(list(ref.values())), f"strided heads {heads}")


def test_binding_rejects_uneven_views():
    wl = datagen.WORKLOADS["stage3_pad"]
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.dtype, scale=wl.scale)
    x = torch.zeros(wl.shape, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    with pytest.raises(ValueError):  # heads and head_dim swapped in memory
        plan.run(x.transpose(-1, -2).contiguous().transpose(-1, -2), x, x, o)
    with pytest.raises(ValueError):  # tokens not evenly spaced: the first 90 W columns of a wider grid
        wide = torch.zeros((1, 4, 45, 100, 32, 64), dtype=torch.bfloat16, device="cuda")
        plan.run(wide[:, :, :, :90], x, x, o)


# K and V at different token strides: the K/V-streaming kernel then addresses their rows with
# 64-bit offsets (equal strides take one 32-bit offset for both); every kernel must give the same
# bits as the contiguous run
UNEQUAL = [
    ("bf16_stream_2x4x4_kv", 1, 4, 10, 13, 2, 64, (1, 2, 3), "bf16", -100.0, (2, 4, 4)),
    ("bf16_stream_4x12x24_kv", 1, 4, 12, 24, 2, 64, (2, 6, 12), "bf16", -100.0, (4, 12, 24)),
    ("bf16_window_2x12x12_kv", 1, 2, 13, 25, 2, 64, (1, 6, 6), "bf16", -100.0, (2, 12, 12)),
    ("stage3_pad", None, None, None, None, None, None, None, None, -100.0),
]


@pytest.mark.parametrize("case", UNEQUAL, ids=lambda c: c[0])
def test_unequal_kv_strides(case):
    wl, bias = _workload(case), case[9]
    x = device_inputs(wl)
    contiguous = run_gpu(wl, bias, x)
    B, D, H, W, h, dh = wl.shape
    kq = torch.stack([x["q"], x["k"]], dim=4).contiguous()  # [B, D, H, W, 2, h, dh]: Q and K at stride 2 h dh
    vv = torch.zeros((B, D, H, W, h * dh + 128), dtype=x["v"].dtype, device="cuda")  # V at stride h dh + 128
    vv[..., :h * dh] = x["v"].flatten(-2)
    q, k = kq[..., 0, :, :], kq[..., 1, :, :]
    v = vv[..., :h * dh].unflatten(-1, (h, dh))
    assert k.stride()[3] == 2 * h * dh and v.stride()[3] == h * dh + 128
    o = torch.full_like(x["q"], float("nan"))
    say(f"[gpu] unequal K/V strides {wl.name} shape={wl.shape} window={wl.window} bias={bias}")
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.dtype, scale=wl.scale,
                   cross_region_bias=bias)
    plan.run(q, k, v, o)
    torch.cuda.synchronize()
    ibits = torch.int16 if wl.dtype == "bf16" else torch.int32
    assert torch.equal(o.view(ibits), contiguous.view(ibits))
