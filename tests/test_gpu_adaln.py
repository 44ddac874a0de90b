"""GPU parity of the fused AdaLN + residual kernel against the fp64 oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import swin3d_window_attention_amd as sw
from _gpu import say
from _tolerances import ADALN_BF16_REL, ADALN_F32_ABS

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dev(a, dtype):
    return datagen.to_torch(a, dtype).to("cuda")


def _check(wl, got, ref, what):
    err = np.abs(got - ref)
    say(f"[gpu] adaln {wl.name} {what}: max_abs={err.max():.3e}")
    if wl.out_dtype == "f32":
        assert err.max() <= ADALN_F32_ABS, (what, err.max())
    else:
        assert np.all(err <= ADALN_BF16_REL * np.abs(ref) + ADALN_F32_ABS), (what, err.max())


CASES = [
    # B, rows, C, x, res, out
    (1, 1001, 512, "bf16", "f32", "f32"),    # bf16 block output, FP32 residual stream
    (3, 257, 256, "f32", "f32", "f32"),
    (2, 130, 1024, "bf16", "bf16", "bf16"),
    (1, 3, 4096, "f32", "bf16", "f32"),
    (1, 1, 768, "bf16", "f32", "bf16"),
    (2, 65, 2048, "f32", "f32", "bf16"),     # 8 units per lane
    (1, 9, 1792, "bf16", "bf16", "f32"),     # 7 units: the guarded kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_parity(case):
    B, rows, C, xt, rt, ot = case
    wl = datagen.AdalnWorkload("case", B, rows, C, xt, rt, ot, seed=31)
    a = datagen.adaln_inputs(wl)
    x, res = _dev(a["x"], xt), _dev(a["res"], rt)
    g, b = (torch.from_numpy(a[k]).cuda() for k in ("gamma", "beta"))
    out = sw.adaln_residual(x, res, g, b, wl.eps, out_dtype=TORCH[ot])
    torch.cuda.synchronize()
    ref = oracle.adaln_residual(datagen.io_to_f64(a["x"], xt), datagen.io_to_f64(a["res"], rt),
                                a["gamma"], a["beta"], wl.eps)
    _check(wl, out.float().cpu().numpy().astype(np.float64), ref, "whole")


def test_in_place_residual_update():
    wl = datagen.AdalnWorkload("inplace", 2, 333, 512, "bf16", "f32", "f32", seed=32)
    a = datagen.adaln_inputs(wl)
    x, res = _dev(a["x"], "bf16"), _dev(a["res"], "f32")
    g, b = (torch.from_numpy(a[k]).cuda() for k in ("gamma", "beta"))
    sw.adaln_residual(x, res, g, b, wl.eps, out=res)
    torch.cuda.synchronize()
    ref = oracle.adaln_residual(datagen.io_to_f64(a["x"], "bf16"), a["res"], a["gamma"], a["beta"], wl.eps)
    _check(wl, res.cpu().numpy().astype(np.float64), ref, "in place")


def test_writes_exactly_the_output():
    wl = datagen.AdalnWorkload("guard", 1, 77, 256, "f32", "f32", "f32", seed=33)
    a = datagen.adaln_inputs(wl)
    n, guard = 77 * 256, 1024
    buf = torch.full((n + 2 * guard,), float("nan"), device="cuda")
    before = buf.view(torch.int32).clone()
    out = buf[guard:guard + n].view(1, 77, 256)
    sw.adaln_residual(_dev(a["x"], "f32"), _dev(a["res"], "f32"), torch.from_numpy(a["gamma"]).cuda(),
                      torch.from_numpy(a["beta"]).cuda(), wl.eps, out=out)
    torch.cuda.synchronize()
    iv = buf.view(torch.int32)
    assert torch.equal(iv[:guard], before[:guard]) and torch.equal(iv[guard + n:], before[guard + n:])
    assert not torch.isnan(out).any().item()


def test_stage1_size_sampled_rows():
    wl = datagen.ADALN_WORKLOADS["adaln_stage1"]
    a = datagen.adaln_inputs(wl)
    x, res = _dev(a["x"], wl.x_dtype), _dev(a["res"], wl.res_dtype)
    g, b = (torch.from_numpy(a[k]).cuda() for k in ("gamma", "beta"))
    out = sw.adaln_residual(x, res, g, b, wl.eps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    rows = np.sort(np.random.default_rng(3).choice(wl.rows, 4096, replace=False))
    rows[0], rows[-1] = 0, wl.rows - 1
    ref = oracle.adaln_residual(datagen.io_to_f64(a["x"][:, rows], wl.x_dtype), a["res"][:, rows],
                                a["gamma"], a["beta"], wl.eps)
    got = out[:, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    _check(wl, got, ref, "4096 sampled rows")


def test_binding_rejects_bad_shapes():
    x = torch.zeros((1, 4, 256), device="cuda")
    g = torch.zeros((1, 256), device="cuda")
    with pytest.raises(ValueError):
        sw.adaln_residual(x, x[:, :2], g, g)
    with pytest.raises(ValueError):
        sw.adaln_residual(x, x, g.double(), g)
    with pytest.raises(sw.Swin3dWattnError):
        sw.adaln_residual(torch.zeros((1, 4, 300), device="cuda"), torch.zeros((1, 4, 300), device="cuda"),
                          torch.zeros((1, 300), device="cuda"), torch.zeros((1, 300), device="cuda"))
