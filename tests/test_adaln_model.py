"""Where the AdaLN tolerance comes from (CPU only): a float32 NumPy model of the kernel's steps
(row sums in float32, two passes, rstd = 1 / sqrt(var + eps), FiLM and residual in float32) stays
well inside ADALN_F32_ABS against the fp64 oracle on the data class the GPU tests use."""
import numpy as np

import datagen
import oracle
from _tolerances import ADALN_F32_ABS


def model(x, res, gamma, beta, eps):
    x = x.astype(np.float32)
    C = np.float32(x.shape[-1])
    mean = x.sum(axis=-1, dtype=np.float32, keepdims=True) / C
    d = x - mean
    var = (d * d).sum(axis=-1, dtype=np.float32, keepdims=True) / C
    rstd = np.float32(1.0) / np.sqrt(var + np.float32(eps))
    return res.astype(np.float32) + gamma[:, None, :] * (d * rstd) + beta[:, None, :]


def test_model_error_well_inside_tolerance():
    worst = 0.0
    for C in (256, 512, 4096):
        wl = datagen.AdalnWorkload("model", 2, 200, C, "bf16", "f32", "f32", 5)
        a = datagen.adaln_inputs(wl)
        x = datagen.io_to_f64(a["x"], "bf16")
        ref = oracle.adaln_residual(x, a["res"], a["gamma"], a["beta"], wl.eps)
        got = model(x, a["res"], a["gamma"], a["beta"], wl.eps).astype(np.float64)
        worst = max(worst, float(np.abs(got - ref).max()))
    assert worst <= ADALN_F32_ABS / 3, worst
    assert worst >= ADALN_F32_ABS / 200, worst  # the model does round
