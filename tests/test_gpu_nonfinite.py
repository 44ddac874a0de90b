"""Padding slots are immune to what their stand-in token holds.

Every kernel fills a window's padding slots by loading a real stand-in token,
so that all loads are unconditional: the nearest real token (its coordinates
clamped to the grid), or token 0 in the K/V-streaming kernel.
The padding exclusion of the pages' scope (padded key positions masked out,
padded query rows cropped) must then hold for any input: here an Inf or NaN
is planted in Q, K and V of a real token that serves as such a stand-in for
the padding of neighbouring windows. In the fp64 oracle the non-finite values
stay in the planted token's own window; the GPU must give the oracle's
result, within the usual tolerance, everywhere else, in particular in the
neighbouring windows whose padding slots loaded that token. Every kernel
(bf16 single tile, split-bf16, K/V streaming with and without a partial last
chunk, exact FP32 with and without a partial last tile, whole window) and both
bias modes."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw
from _gpu import check, say

pytestmark = pytest.mark.gpu

CASES = [
    # (name, D, H, W, heads, head_dim, window, shift, io dtype, plan dtype, kernel)
    ("single_tile", 4, 15, 30, 2, 64, (2, 6, 12), (1, 3, 6), "bf16", "bf16", 1),
    ("split", 4, 15, 30, 2, 64, (2, 6, 12), (1, 3, 6), "f32", "f32_split", 2),
    ("stream", 4, 15, 15, 2, 64, (2, 6, 6), (1, 3, 3), "bf16", "bf16", 3),
    ("stream_tail", 3, 10, 10, 2, 64, (1, 7, 7), (0, 3, 3), "bf16", "bf16", 3),
    ("f32", 4, 15, 30, 2, 32, (2, 6, 12), (1, 3, 6), "f32", "f32", 4),
    ("f32_tail", 4, 15, 15, 2, 32, (2, 6, 6), (1, 3, 3), "f32", "f32", 4),
    ("window_d128", 4, 15, 30, 2, 128, (2, 6, 12), (1, 3, 6), "bf16", "bf16", 5),
    ("window_n288", 4, 15, 30, 2, 64, (2, 12, 12), (1, 6, 6), "bf16", "bf16", 5),
]


def _plant(host, dtype, coord):
    """+Inf in Q and K, NaN in V at grid position coord (every head)."""
    b, d, h, w = coord
    if dtype == "bf16":
        host["q"][b, d, h, w] = 0x7F80
        host["k"][b, d, h, w] = 0x7F80
        host["v"][b, d, h, w] = 0x7FC0
    else:
        host["q"][b, d, h, w] = np.inf
        host["k"][b, d, h, w] = np.inf
        host["v"][b, d, h, w] = np.nan


def _windows_touching(grid, window, shift, coord):
    """(own window, the other windows whose padding slots load coord as their stand-in)."""
    P = [oracle.padded_extent(x, w) for x, w in zip(grid, window)]
    own = tuple(((c - s) % p) // w for c, s, p, w in zip(coord, shift, P, window))
    nwin = [p // w for p, w in zip(P, window)]
    neighbours = []
    for kd in range(nwin[0]):
        for kh in range(nwin[1]):
            for kw in range(nwin[2]):
                g, valid, _ = oracle.window_slot_coords(grid, window, shift, (kd, kh, kw))
                clamped = np.minimum(g, np.asarray(grid)[None, :] - 1)
                if (kd, kh, kw) != own and np.any(~valid & np.all(clamped == np.asarray(coord), axis=1)):
                    neighbours.append((kd, kh, kw))
    return own, neighbours


@pytest.mark.parametrize("bias", [-100.0, -math.inf], ids=["bias-100", "bias-inf"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_nonfinite_stand_in_stays_in_its_window(case, bias):
    name, D, H, W, heads, dh, window, shift, io, plan_dt, kernel = case
    extra = {"plan": plan_dt} if plan_dt != io else {}
    wl = datagen.small_workload(f"nonfinite_{name}", 1, D, H, W, heads, dh, window, shift, io, seed=83, **extra)
    grid = (D, H, W)
    coord = (D - 1, H - 1, W - 1)
    own, neighbours = _windows_touching(grid, window, shift, coord)
    assert neighbours, own  # the planted token is a stand-in in other windows

    host = {t: datagen.full_io(wl, t) for t in "qkv"}
    _plant(host, io, (0,) + coord)
    x = {t: datagen.to_torch(host[t], io).to("cuda") for t in "qkv"}
    plan = sw.Plan(*wl.shape, window=window, shift=shift, dtype=plan_dt, scale=wl.scale, cross_region_bias=bias)
    assert plan.info().kernel == kernel
    o = torch.full_like(x["q"], float("nan"))
    say(f"[gpu] run {wl.name} shape={wl.shape} window={window} shift={shift} bias={bias} kernel={kernel}")
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)

    widen = (lambda a: datagen.bf16_bits_to_f32(a).astype(np.float64)) if io == "bf16" else \
        (lambda a: a.astype(np.float64))
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.swin3d_window_attention(widen(host["q"]), widen(host["k"]), widen(host["v"]), window, shift,
                                             wl.scale, bias)
    # the oracle keeps the non-finite values inside the planted token's own window
    own_coords = oracle.window_slot_coords(grid, window, shift, own)
    own_mask = np.zeros(grid, dtype=bool)
    g, valid, _ = own_coords
    own_mask[tuple(g[valid].T)] = True
    bad_ref = ~np.all(np.isfinite(ref[0]), axis=(-2, -1))
    assert bad_ref.any() and not np.any(bad_ref & ~own_mask), "oracle leaked outside the planted window"
    # everywhere else the GPU matches the oracle; the neighbouring windows are covered
    keep = ~own_mask
    for kd, kh, kw in neighbours:
        gn, vn, _ = oracle.window_slot_coords(grid, window, shift, (kd, kh, kw))
        assert keep[tuple(gn[vn].T)].all()
    check(wl, got[0][keep], ref[0][keep], f"outside the planted window, bias={bias}")


@pytest.mark.parametrize("bias", [-100.0, -math.inf], ids=["bias-100", "bias-inf"])
def test_stream_token0_stand_in(bias):
    """The K/V-streaming kernel loads token 0 for every padding slot (the same lines for all, from
    the caches): with Inf / NaN planted in token 0, every window that holds padding loads it, and
    all of them must still match the oracle."""
    grid, window, shift = (3, 10, 12), (2, 6, 8), (1, 3, 4)  # N = 96, padded to 4 x 12 x 16
    wl = datagen.small_workload("nonfinite_stream_token0", 1, *grid, 2, 64, window, shift, "bf16", seed=84)
    host = {t: datagen.full_io(wl, t) for t in "qkv"}
    _plant(host, "bf16", (0, 0, 0, 0))
    x = {t: datagen.to_torch(host[t], "bf16").to("cuda") for t in "qkv"}
    plan = sw.Plan(*wl.shape, window=window, shift=shift, dtype="bf16", scale=wl.scale, cross_region_bias=bias)
    assert plan.info().kernel == 3
    o = torch.full_like(x["q"], float("nan"))
    say(f"[gpu] run {wl.name} shape={wl.shape} window={window} shift={shift} bias={bias}")
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    widen = lambda a: datagen.bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.swin3d_window_attention(widen(host["q"]), widen(host["k"]), widen(host["v"]), window, shift,
                                             wl.scale, bias)
    P = [oracle.padded_extent(x_, w) for x_, w in zip(grid, window)]
    own = tuple(((0 - s) % p) // w for s, p, w in zip(shift, P, window))
    g, valid, _ = oracle.window_slot_coords(grid, window, shift, own)
    own_mask = np.zeros(grid, dtype=bool)
    own_mask[tuple(g[valid].T)] = True
    bad_ref = ~np.all(np.isfinite(ref[0]), axis=(-2, -1))
    assert bad_ref.any() and not np.any(bad_ref & ~own_mask), "oracle leaked outside the planted window"
    # windows other than the planted one that hold padding (and so load token 0 as a stand-in)
    padded_others = 0
    nwin = [p // w for p, w in zip(P, window)]
    for kd in range(nwin[0]):
        for kh in range(nwin[1]):
            for kw in range(nwin[2]):
                _, vn, _ = oracle.window_slot_coords(grid, window, shift, (kd, kh, kw))
                padded_others += (kd, kh, kw) != own and not vn.all()
    assert padded_others > 0
    check(wl, got[0][~own_mask], ref[0][~own_mask], f"outside the planted window, bias={bias}")
