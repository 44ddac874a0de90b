"""GPU parity with cross-region biases that do not vanish (the shifted-window bias as a real
additive term, not an exclusion) and a scale other than 1/sqrt(head_dim), on every attention
kernel. With the pages' -100 the cross-region weights are ~e^-100 and any error in how a kernel
forms the bias (bias / scale split into bf16 terms, the log2-domain conversion, the order of
scale and bias) would not show; with -0.5 .. -6 it does."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw
from _gpu import check, say, to_f64

pytestmark = pytest.mark.gpu

SCALE = 0.2
BIASES = [-0.5, -3.7, -6.0]
CASES = [
    # (name, B, D, H, W, heads, head_dim, window, shift, I/O dtype, plan dtype, kernel)
    # grids with padding and with real tokens on both sides of the region cuts
    ("bf16_tile", 1, 4, 13, 25, 2, 64, (2, 6, 12), (1, 3, 6), "bf16", "bf16", 1),
    ("f32_split", 1, 4, 13, 25, 2, 64, (2, 6, 12), (1, 3, 6), "f32", "f32_split", 2),
    ("stream_dh64", 1, 4, 12, 22, 2, 64, (2, 6, 6), (1, 3, 3), "bf16", "bf16", 3),
    ("stream_dh128", 1, 4, 12, 22, 2, 128, (2, 6, 6), (1, 3, 3), "bf16", "bf16", 3),
    ("window_dh128", 1, 4, 13, 25, 2, 128, (2, 6, 12), (1, 3, 6), "bf16", "bf16", 5),
    ("window_w2x12x12", 1, 4, 13, 25, 2, 64, (2, 12, 12), (1, 6, 6), "bf16", "bf16", 5),
    ("f32_mfma", 1, 4, 13, 25, 2, 64, (2, 6, 12), (1, 3, 6), "f32", "f32", 4),
    ("f32_mfma_w2x4x4", 1, 4, 10, 13, 2, 32, (2, 4, 4), (1, 2, 3), "f32", "f32", 4),
    ("f32_mfma_w2x8x10", 1, 4, 13, 25, 2, 32, (2, 8, 10), (1, 4, 5), "f32", "f32", 4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("bias", BIASES)
def test_nonvanishing_bias(case, bias):
    name, B, D, H, W, h, dh, window, shift, io, plan_dt, kernel = case
    wl = datagen.small_workload(name, B, D, H, W, h, dh, window, shift, io, seed=81,
                                **({"plan": plan_dt} if plan_dt != io else {}))
    plan = sw.Plan(*wl.shape, window=window, shift=shift, dtype=plan_dt, scale=SCALE, cross_region_bias=bias)
    assert plan.info().kernel == kernel and plan.info().n_masked_windows > 0
    x = {t: datagen.to_torch(datagen.full_io(wl, t), io).to("cuda") for t in "qkv"}
    o = torch.full_like(x["q"], float("nan"))
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    qkv = [datagen.full_f64(wl, t) for t in "qkv"]
    ref = oracle.swin3d_window_attention(*qkv, window, shift, SCALE, bias)
    # the case is not degenerate: the bias changes the result (real tokens meet across regions)
    excl = oracle.swin3d_window_attention(*qkv, window, shift, SCALE, -np.inf)
    assert np.abs(ref - excl).max() > 1e-3, "no cross-region pair of real tokens in this grid"
    say(f"[gpu] bias {name} bias={bias} scale={SCALE}")
    check(wl, to_f64(o), ref, f"bias={bias} scale={SCALE}")
