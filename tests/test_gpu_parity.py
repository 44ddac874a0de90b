"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on seeded inputs."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw
from _gpu import (check, check_sampled, device_inputs, oracle_full, run_gpu, sample_windows, say,
                  to_f64)

pytestmark = pytest.mark.gpu

BIASES = [-100.0, -math.inf]
WL = datagen.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sw.load_library()  # fails loudly when the HIP library is missing
    yield


# ---------------------------------------------------------------- whole-grid parity
@pytest.mark.parametrize("bias", BIASES)
def test_tiny_f32(bias):
    wl = WL["tiny_f32"]
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    ref = oracle_full(wl, bias)
    for h, r in ref.items():
        check(wl, o[..., h, :], r, f"head {h} bias={bias}")


@pytest.mark.parametrize("name", ["stage2_s0", "stage2", "stage3_pad"])
@pytest.mark.parametrize("bias", BIASES)
def test_bf16_stage_full(name, bias):
    wl = WL[name]
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    heads = [0, wl.heads - 1] if bias == -math.inf else range(wl.heads)
    ref = oracle_full(wl, bias, heads)
    got = np.stack([o[..., h, :] for h in ref])
    check(wl, got, np.stack(list(ref.values())), f"heads {list(ref)} bias={bias}")


RAGGED = [
    # (B, D, H, W, heads, dh, shift, dtype)
    (2, 3, 7, 13, 3, 64, (1, 5, 11), "bf16"),   # padding on every axis, large shifts (each window's
                                                #   real tokens lie in one region: a padding case)
    (1, 4, 44, 30, 2, 64, (1, 3, 6), "bf16"),   # pad != shift along H
    (1, 2, 6, 12, 1, 64, (0, 0, 0), "bf16"),    # a single unmasked window
    (1, 1, 1, 1, 2, 64, (1, 3, 6), "bf16"),     # a single real token
    (1, 2, 6, 12, 4, 64, (1, 3, 6), "bf16"),    # one window cut into 8 regions
    (3, 2, 12, 36, 2, 64, (0, 3, 0), "bf16"),   # shift along one axis only
    (2, 3, 7, 13, 3, 32, (1, 5, 11), "f32"),
    (1, 4, 44, 30, 2, 64, (1, 3, 6), "f32"),
    (1, 1, 1, 1, 1, 32, (0, 0, 0), "f32"),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "x".join(map(str, c[:6])) + f"_s{''.join(map(str, c[6]))}_{c[7]}")
@pytest.mark.parametrize("bias", BIASES)
def test_ragged(case, bias):
    B, D, H, W, h, dh, shift, dt = case
    wl = datagen.small_workload("ragged", B, D, H, W, h, dh, (2, 6, 12), shift, dt, seed=17)
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, bias, x))
    ref = oracle.swin3d_window_attention(*(datagen.full_f64(wl, t) for t in "qkv"), wl.window, shift,
                                         wl.scale, bias)
    check(wl, o, ref, f"bias={bias}")


@pytest.mark.parametrize("window,shift", [((1, 1, 1), (0, 0, 0)), ((2, 4, 4), (1, 2, 3)), ((4, 8, 8), (2, 7, 5))])
def test_f32_other_windows(window, shift):
    wl = datagen.small_workload("f32win", 2, 5, 9, 11, 2, 32, window, shift, "f32", seed=23)
    x = device_inputs(wl)
    o = to_f64(run_gpu(wl, -100.0, x))
    ref = oracle.swin3d_window_attention(*(datagen.full_f64(wl, t) for t in "qkv"), window, shift, wl.scale,
                                         -100.0)
    check(wl, o, ref, f"window={window}")


# ---------------------------------------------------------------- full sizes, sampled
def test_stage1_full_size():
    wl = WL["stage1"]
    x = device_inputs(wl, keep_host=True)
    o = run_gpu(wl, -100.0, x)
    assert not torch.isnan(o).any().item(), "an output element was never written"
    of = to_f64(o)
    ref = oracle_full(wl, -100.0, heads=[0, 5])
    check(wl, np.stack([of[..., h, :] for h in ref]), np.stack(list(ref.values())), "heads 0,5 whole grid")
    check_sampled(wl, -100.0, o, sample_windows(wl, 48, seed=1), x["host"])


@pytest.mark.parametrize("bias", BIASES)
def test_stress_full_size(bias):
    wl = WL["stress_hres"]
    say("[gpu] generating stress inputs (3 x 3.3 GB)")
    x = device_inputs(wl, keep_host=True)
    o = run_gpu(wl, bias, x)
    assert not torch.isnan(o).any().item(), "an output element was never written"
    assert torch.isfinite(o).all().item()
    check_sampled(wl, bias, o, sample_windows(wl, 40, seed=5 if bias == -100.0 else 6), x["host"])
    del x, o
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- properties at full size
def test_uniform_v_full_size():
    """V equal for every token (per head and dim): O == V up to bf16 rounding, everywhere."""
    wl = WL["stage1"]
    x = device_inputs(wl)
    c = x["v"][0, 0, 0, 0].clone()
    x["v"] = c.expand_as(x["v"]).contiguous()
    o = run_gpu(wl, -100.0, x)
    err = (o.float() - x["v"].float()).abs().max().item()
    assert err <= 1e-2 * c.float().abs().max().item() + 1e-3


def test_isolation_full_size():
    """-inf mode: changing K, V outside one corner window's region leaves that region's outputs bit-identical."""
    wl = WL["stage1"]
    x = device_inputs(wl)
    o1 = run_gpu(wl, -math.inf, x)
    # corner window (last along every axis): its 8 regions
    g, valid, labels = oracle.window_slot_coords((wl.D, wl.H, wl.W), wl.window, wl.shift, (1, 29, 29))
    target = labels[0]
    inside = g[(labels == target) & valid]
    outside = g[(labels != target) & valid]
    k2, v2 = x["k"].clone(), x["v"].clone()
    oi = torch.from_numpy(outside).cuda()
    k2[0, oi[:, 0], oi[:, 1], oi[:, 2]] = 30.0
    v2[0, oi[:, 0], oi[:, 1], oi[:, 2]] = -50.0
    o2 = run_gpu(wl, -math.inf, {"q": x["q"], "k": k2, "v": v2})
    ii = torch.from_numpy(inside).cuda()
    a = o1[0, ii[:, 0], ii[:, 1], ii[:, 2]]
    b = o2[0, ii[:, 0], ii[:, 1], ii[:, 2]]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # and the perturbed tokens' own outputs did change
    assert not torch.equal(o1[0, oi[:, 0], oi[:, 1], oi[:, 2]], o2[0, oi[:, 0], oi[:, 1], oi[:, 2]])


# ---------------------------------------------------------------- memory safety, determinism
@pytest.mark.parametrize("name", ["stage3_pad", "tiny_f32"])
def test_writes_exactly_the_output(name):
    """O sits between guard regions; every element of O is written and nothing outside it."""
    wl = WL[name]
    x = device_inputs(wl)
    n = x["q"].numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=x["q"].dtype, device="cuda")
    sentinel = buf.view(torch.int16 if wl.dtype == "bf16" else torch.int32).clone()
    o = buf[guard:guard + n].view(x["q"].shape)
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.dtype, scale=wl.scale)
    plan.run(x["q"], x["k"], x["v"], o)
    torch.cuda.synchronize()
    iv = buf.view(sentinel.dtype)
    assert torch.equal(iv[:guard], sentinel[:guard]) and torch.equal(iv[guard + n:], sentinel[guard + n:])
    assert not torch.isnan(o).any().item()


def test_deterministic_and_stream():
    wl = WL["stage2"]
    x = device_inputs(wl)
    o1 = run_gpu(wl, -100.0, x)
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.dtype, scale=wl.scale)
    s = torch.cuda.Stream()
    o2 = torch.empty_like(o1)
    with torch.cuda.stream(s):
        plan.run(x["q"], x["k"], x["v"], o2)
    s.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_binding_rejects_mismatched_tensors():
    wl = WL["stage3_pad"]
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.dtype, scale=wl.scale)
    q = torch.zeros(wl.shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        plan.run(q, q, q, torch.zeros(wl.shape, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        plan.run(q, q, q[:, :2].contiguous(), torch.empty_like(q))
    with pytest.raises(sw.Swin3dWattnError):
        plan.run(q, q, q, q)  # o overlaps q
