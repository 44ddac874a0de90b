"""Where the tolerance of the exact FP32 matrix-core path comes from (CPU only).

The FP32 kernel forms S^T = K Q^T and O^T = V^T P^T on FP32 matrix instructions: each
instruction adds a group of four FP32 products to an FP32 accumulator, the dims (for S) and the
keys (for O) taken in the kernel's order. The row max is subtracted in the units of Q K^T, then
the difference is scaled into the log2 domain and exponentiated in FP32; the row sum and 1/l are
FP32. This file models exactly those rounding points in NumPy and measures the error against the
fp64 oracle on random windows of both data classes the GPU tests use:
  * N(0,1) data: the model's worst error must sit far inside the FP32 bar of 1e-5 max abs;
  * Q, K scaled by 8 (logits ~64x larger): FP32 arithmetic itself cannot reach 1e-5 there (the
    model errs by ~2e-5), so the GPU bar for that class, F32_TOL[8.0], is about five times the
    model's worst case, as for the split-bf16 path.
It also checks that the model is not trivially exact.
"""
import numpy as np
import pytest

import oracle
from _tolerances import F32_TOL

N, DH = 144, 64
F32 = np.float32


def mfma_chain(a_groups, b_groups):
    """Sum of a_i @ b_i over four-wide groups, rounded to fp32 after each group."""
    c = np.zeros((a_groups[0].shape[0], b_groups[0].shape[1]), dtype=np.float32)
    for a, b in zip(a_groups, b_groups):
        c = (c.astype(np.float64) + a.astype(np.float64) @ b.astype(np.float64)).astype(np.float32)
    return c


def model_window(q, k, v, scale):
    c2 = F32(scale * np.log2(np.e))
    # S^T = K Q^T; k-step s of the four lane groups covers dims kk * 16 + s
    dims = [[kk * 16 + s for kk in range(4)] for s in range(DH // 4)]
    s = mfma_chain([k[:, d] for d in dims], [q[:, d].T for d in dims]).T  # queries x keys
    m = s.max(axis=1, keepdims=True)
    p = np.exp2(((s - m).astype(np.float32) * c2).astype(np.float32)).astype(np.float32)
    inv = (F32(1.0) / p.astype(np.float64).sum(axis=1).astype(np.float32)).astype(np.float32)
    # O^T = V^T P^T; k-step (kt, i) covers keys 16 kt + 4 kk + i
    keys = [[16 * kt + 4 * kk + i for kk in range(4)] for kt in range(N // 16) for i in range(4)]
    o = mfma_chain([v[kl, :].T for kl in keys], [p[:, kl].T for kl in keys]).T
    return (o * inv[:, None]).astype(np.float32)


@pytest.mark.parametrize("qk_mult", sorted(F32_TOL))
def test_model_error_well_inside_tolerance(qk_mult):
    rng = np.random.default_rng(11)
    scale = float(F32(1.0) / np.sqrt(F32(DH)))
    labels = np.zeros(N, dtype=np.int64)
    valid = np.ones(N, dtype=bool)
    worst_abs, worst_rel = 0.0, 0.0
    for _ in range(40):
        q = rng.standard_normal((N, DH)).astype(np.float32) * F32(qk_mult)
        k = rng.standard_normal((N, DH)).astype(np.float32) * F32(qk_mult)
        v = (rng.standard_normal((N, DH)) if qk_mult == 1.0 else rng.uniform(-1, 1, (N, DH))).astype(np.float32)
        ref = oracle.masked_window_attention(q[None, :, None].astype(np.float64), k[None, :, None].astype(np.float64),
                                             v[None, :, None].astype(np.float64), labels[None], valid[None],
                                             scale, -100.0)[0][0, :, 0]
        got = model_window(q, k, v, scale).astype(np.float64)
        worst_abs = max(worst_abs, float(np.abs(got - ref).max()))
        worst_rel = max(worst_rel, float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    tol_abs, tol_rel = F32_TOL[qk_mult]
    assert worst_abs <= tol_abs / 2 and worst_rel <= tol_rel / 2, (worst_abs, worst_rel)
    assert worst_abs >= tol_abs / 40, (worst_abs, "the model is suspiciously exact")
