"""Where the f32_split tolerance comes from (CPU only).

The split-bf16 kernel writes every fp32 operand as x = hi + lo with hi = bf16(x),
lo = bf16(x - hi) (round to nearest even) and forms each product as
Ah Bh + Al Bh + Ah Bl with fp32 accumulation; the softmax is fp32 and the row sum
adds the fp32 probabilities. This file models exactly those rounding points in
NumPy and checks, on random windows of both data classes the GPU tests use, that
the model's error against the fp64 oracle stays well inside the tolerance the
GPU tests apply (SPLIT_TOL in tests/_tolerances.py): the tolerance is about five times the
model's worst case. It also checks that the model is not trivially exact: its
error is far above fp32 rounding, so the tolerance is not hiding a broken model.
"""
import numpy as np
import pytest

import oracle
from _tolerances import SPLIT_TOL

N, DH = 144, 64


def bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split(x):
    h = bf16(x)
    return h, bf16(np.float32(x) - h)


def split_mm(a, b):
    """a @ b from the three split products, accumulated wide and rounded to fp32."""
    (ah, al), (bh, bl) = split(a), split(b)
    w = lambda x: x.astype(np.float64)
    return (w(ah) @ w(bh) + w(al) @ w(bh) + w(ah) @ w(bl)).astype(np.float32)


def model_window(q, k, v, scale):
    c2 = np.float32(scale * np.log2(np.e))
    s = split_mm(q, k.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp2(s * c2 - m * c2).astype(np.float32)
    l = p.astype(np.float64).sum(axis=1).astype(np.float32)
    return split_mm(p, v) / l[:, None]


@pytest.mark.parametrize("qk_mult", sorted(SPLIT_TOL))
def test_model_error_well_inside_tolerance(qk_mult):
    rng = np.random.default_rng(11)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(DH)))
    worst_abs, worst_rel = 0.0, 0.0
    labels = np.zeros(N, dtype=np.int64)
    valid = np.ones(N, dtype=bool)
    for _ in range(40):
        q = rng.standard_normal((N, DH)).astype(np.float32) * np.float32(qk_mult)
        k = rng.standard_normal((N, DH)).astype(np.float32) * np.float32(qk_mult)
        v = (rng.standard_normal((N, DH)) if qk_mult == 1.0 else rng.uniform(-1, 1, (N, DH))).astype(np.float32)
        ref, _, _ = oracle.masked_window_attention(q[None, :, None].astype(np.float64),
                                                   k[None, :, None].astype(np.float64),
                                                   v[None, :, None].astype(np.float64),
                                                   labels[None], valid[None], scale, -100.0)
        ref = ref[0, :, 0]
        got = model_window(q, k, v, scale).astype(np.float64)
        worst_abs = max(worst_abs, float(np.abs(got - ref).max()))
        worst_rel = max(worst_rel, float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    tol_abs, tol_rel = SPLIT_TOL[qk_mult]
    assert worst_abs <= tol_abs / 2 and worst_rel <= tol_rel / 2, (worst_abs, worst_rel)
    assert worst_abs >= tol_abs / 40, (worst_abs, "the model is suspiciously exact")
