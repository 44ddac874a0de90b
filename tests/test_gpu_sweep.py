"""A seeded sweep of random problem shapes through every attention kernel against the fp64
oracle: window sizes and shapes, shifts (including none and shifts on single-window axes), grid
extents below, at and above a window multiple, batch, heads, head_dim, bias mode and dtype. The
list is drawn once from a fixed seed, so every run checks the same cases."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw
from _gpu import check, say, to_f64

pytestmark = pytest.mark.gpu


# windows whose K and V fill half the LDS (N x head_dim = 18432): the whole-window kernel
WHOLE_WINDOW = [((2, 6, 12), 128), ((1, 12, 12), 128), ((4, 6, 6), 128), ((2, 12, 12), 64), ((4, 6, 12), 64),
                ((2, 8, 18), 64), ((3, 8, 12), 64)]


def _cases(n=54, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = ["bf16", "bf16_144", "f32", "f32_144", "f32_split", "bf16_win"][len(out) % 6]
        if kind == "bf16_win":
            window, dh_win = WHOLE_WINDOW[int(rng.integers(len(WHOLE_WINDOW)))]
        elif kind in ("bf16_144", "f32_144", "f32_split"):
            window = [(2, 6, 12), (1, 12, 12), (4, 6, 6), (2, 8, 9), (3, 6, 8)][int(rng.integers(5))]
        else:
            while True:
                window = tuple(int(x) for x in rng.integers(1, 13, size=3))
                N = window[0] * window[1] * window[2]
                if (kind == "f32" and 1 <= N <= 256) or (kind == "bf16" and 8 <= N <= 600):
                    break
        shift = tuple(int(rng.integers(0, w)) if rng.random() < 0.8 else 0 for w in window)
        grid = tuple(int(max(1, rng.integers(1, 3 * w + 2))) for w in window)
        B = int(rng.integers(1, 3))
        heads = int(rng.integers(1, 4))
        if kind.startswith("bf16"):
            dh = 64 if kind == "bf16_144" else dh_win if kind == "bf16_win" else int(rng.choice([32, 64, 128]))
            io, plan = "bf16", "bf16"
        elif kind == "f32_split":
            dh, io, plan = 64, "f32", "f32_split"
        else:
            dh, io, plan = int(rng.choice([32, 64])), "f32", "f32"
        bias = [-100.0, -math.inf, -2.0][int(rng.integers(3))]
        out.append((len(out), B, grid, heads, dh, window, shift, io, plan, bias))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]:02d}_{c[8]}_w{'x'.join(map(str, c[5]))}_dh{c[4]}")
def test_sweep(case):
    i, B, grid, heads, dh, window, shift, io, plan_dt, bias = case
    wl = datagen.small_workload(f"sweep{i:02d}", B, *grid, heads, dh, window, shift, io, seed=100 + i,
                                **({"plan": plan_dt} if plan_dt != io else {}))
    plan = sw.Plan(*wl.shape, window=window, shift=shift, dtype=plan_dt, scale=wl.scale, cross_region_bias=bias)
    say(f"[gpu] sweep {i}: shape={wl.shape} window={window} shift={shift} {plan_dt} bias={bias} "
        f"kernel={plan.info().kernel}")
    x = {t: datagen.to_torch(datagen.full_io(wl, t), io).to("cuda") for t in "qkv"}
    o = torch.full_like(x["q"], float("nan"))
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    ref = oracle.swin3d_window_attention(*(datagen.full_f64(wl, t) for t in "qkv"), window, shift, wl.scale, bias)
    check(wl, to_f64(o), ref, f"sweep {i}")
