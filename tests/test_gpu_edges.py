"""GPU parity at the edges of the launch shape: the largest head count a plan accepts (65,535,
the y dimension of every attention kernel's launch grid), on a one-window grid, for the bf16
single-tile, the K/V-streaming, the whole-window (head_dim 128) and the exact FP32 kernels. Checked against the fp64 oracle on
the first, a middle and the last head."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw
from _gpu import check, say

pytestmark = pytest.mark.gpu

MAX_HEADS = 65535
CASES = [
    # (name, D, H, W, head_dim, window, shift, dtype, kernel)
    ("max_heads_bf16", 2, 6, 12, 64, (2, 6, 12), (1, 3, 6), "bf16", 1),
    ("max_heads_stream", 2, 6, 6, 64, (2, 6, 6), (1, 3, 3), "bf16", 3),
    ("max_heads_window", 2, 6, 12, 128, (2, 6, 12), (1, 3, 6), "bf16", 5),
    ("max_heads_f32", 2, 6, 12, 32, (2, 6, 12), (1, 3, 6), "f32", 4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_max_heads(case):
    name, D, H, W, dh, window, shift, dt, kernel = case
    wl = datagen.small_workload(name, 1, D, H, W, MAX_HEADS, dh, window, shift, dt, seed=71)
    plan = sw.Plan(*wl.shape, window=window, shift=shift, dtype=dt, scale=wl.scale, cross_region_bias=-math.inf)
    assert plan.info().kernel == kernel
    host = {t: datagen.full_io(wl, t) for t in "qkv"}
    x = {t: datagen.to_torch(host[t], dt).to("cuda") for t in "qkv"}
    o = torch.full_like(x["q"], float("nan"))
    say(f"[gpu] run {name} shape={wl.shape}")
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item(), "an output element was never written"
    heads = [0, MAX_HEADS // 2, MAX_HEADS - 1]
    widen = (lambda a: datagen.bf16_bits_to_f32(a).astype(np.float64)) if dt == "bf16" else \
        (lambda a: a.astype(np.float64))
    got = o[..., heads, :].float().cpu().numpy().astype(np.float64)
    for i, h in enumerate(heads):
        sl = (Ellipsis, slice(h, h + 1), slice(None))
        ref = oracle.swin3d_window_attention(widen(host["q"][sl]), widen(host["k"][sl]), widen(host["v"][sl]),
                                             window, shift, wl.scale, -math.inf)[..., 0, :]
        check(wl, got[..., i, :], ref, f"head {h}")
