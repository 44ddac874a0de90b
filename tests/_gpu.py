"""Helpers for the GPU parity tests: put seeded inputs on the device, run the
HIP library through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw

from _tolerances import BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_TOL, SPLIT_TOL  # noqa: F401


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def device_inputs(wl: datagen.Workload, keep_host: bool = False):
    """Seeded Q, K, V on the device (and, if asked, the host arrays they came from under 'host')."""
    host = {t: datagen.full_io(wl, t) for t in ("q", "k", "v")}
    x = {t: datagen.to_torch(host[t], wl.dtype).to("cuda") for t in ("q", "k", "v")}
    if keep_host:
        x["host"] = host
    return x


def io_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return (datagen.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def run_gpu(wl: datagen.Workload, bias: float, x: dict, fill=float("nan")) -> torch.Tensor:
    say(f"[gpu] run {wl.name} shape={wl.shape} shift={wl.shift} bias={bias}")
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.plan_dtype, scale=wl.scale,
                   cross_region_bias=bias)
    o = torch.full_like(x["q"], fill)
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    return o


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)) if diff.size else 0.0
    return max_abs, rel_l2


def check(wl: datagen.Workload, got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    assert np.all(np.isfinite(got)), f"{wl.name} {what}: non-finite output"
    max_abs, rel = errors(got, ref)
    say(f"[gpu] {wl.name} {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if wl.plan_dtype == "f32_split":
        tol_abs, tol_rel = SPLIT_TOL[wl.qk_mult]
        assert max_abs <= tol_abs, (wl.name, what, max_abs)
        assert rel <= tol_rel, (wl.name, what, rel)
    elif wl.dtype == "f32":
        tol_abs, tol_rel = F32_TOL[wl.qk_mult]
        assert max_abs <= tol_abs, (wl.name, what, max_abs)
        assert rel <= tol_rel, (wl.name, what, rel)
    else:
        assert max_abs <= BF16_MAX_ABS, (wl.name, what, max_abs)
        assert rel <= BF16_REL_L2, (wl.name, what, rel)


def oracle_full(wl: datagen.Workload, bias: float, heads=None) -> np.ndarray:
    """Oracle on the whole grid, one head at a time (heads are independent)."""
    q, k, v = (datagen.full_f64(wl, t) for t in ("q", "k", "v"))
    heads = range(wl.heads) if heads is None else heads
    out = {}
    for h in heads:
        sl = (Ellipsis, slice(h, h + 1), slice(None))
        out[h] = oracle.swin3d_window_attention(q[sl], k[sl], v[sl], wl.window, wl.shift, wl.scale, bias)[..., 0, :]
    return out


def sample_windows(wl: datagen.Workload, count: int, seed: int):
    """Seeded windows that cover every seam type: interior, and last along each
    subset of axes, in every batch; the rest drawn at random."""
    nwin = [oracle.padded_extent(x, w) // w for x, w in zip((wl.D, wl.H, wl.W), wl.window)]
    rng = np.random.default_rng(seed)
    picks = set()
    for b in range(wl.B):
        for last in range(8):
            idx = []
            for a in range(3):
                if last >> a & 1:
                    idx.append(nwin[a] - 1)
                else:
                    idx.append(int(rng.integers(0, max(1, nwin[a] - 1))))
            picks.add((b, *idx))
        picks.add((b, 0, 0, 0))
    while len(picks) < count:
        picks.add((int(rng.integers(0, wl.B)),) + tuple(int(rng.integers(0, n)) for n in nwin))
    return sorted(picks)


def check_sampled(wl: datagen.Workload, bias: float, o_dev: torch.Tensor, windows, host) -> None:
    """Compare the listed windows with the oracle; host holds the I/O arrays the device got."""
    fetch = lambda t, b, c: io_to_f64(host[t][b, c[:, 0], c[:, 1], c[:, 2]], wl.dtype)
    res = oracle.windows_attention(fetch, wl.B, (wl.D, wl.H, wl.W), wl.heads, wl.head_dim, wl.window,
                                   wl.shift, wl.scale, bias, windows)
    got, ref = [], []
    for b, coords, o_ref in res:
        idx = torch.from_numpy(coords).to(o_dev.device)
        g = o_dev[b][idx[:, 0], idx[:, 1], idx[:, 2]]
        got.append(to_f64(g))
        ref.append(o_ref)
    check(wl, np.concatenate(got), np.concatenate(ref), f"{len(windows)} sampled windows, bias={bias}")
