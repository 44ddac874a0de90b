"""Plain fp64 CPU oracle for Swin3D shifted-window attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the build entry point
and the benchmark's CPU-baseline leg may import or run this module. The GPU
library never calls it and shares no code with it.

What it computes (Flash-Aurora README):
  * "Kernel fusion for backbone memory traffic": the Swin3D window layout is a
    cyclic shift, a pad to window multiples, a 3D window partition and, after
    attention, the inverse merge.
  * "CuTe DSL window attention": per window and head, S = scale * Q K^T, the
    optional Swin shifted-window mask added to S as the additive -100 bias of
    PyTorch's mask (so logits match scaled_dot_product_attention), a row
    softmax in FP32, and O = softmax(S) V; window (2, 6, 12) gives N = 144.
  * "Window attention kernels": attention layout (B * n_W, heads, N, D_h),
    where the leading dimension folds batch and window index.

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):
  * pad first, then roll over the padded extent; the inverse is merge, unroll,
    crop (the only order the stated inverse undoes);
  * padded key positions are excluded (-inf), padded query rows are cropped;
  * region labels are Swin's three slices per shifted axis,
    [0, P-w), [P-w, P-s), [P-s, P); a shift is applied as given, never clamped,
    even where the axis holds a single window;
  * the cross-region bias is a parameter: -100 (the pages' value) or -inf
    (exclusion); it is added after scaling;
  * scale is the caller's float (1/sqrt(head_dim) rounded to float32).

Everything runs in float64 on the exact values the GPU receives.
"""
from __future__ import annotations

import numpy as np


def padded_extent(n: int, w: int) -> int:
    """Smallest multiple of the window size w that holds n positions."""
    return ((n + w - 1) // w) * w


def pad_to_windows(x: np.ndarray, window, value: float = 0.0) -> np.ndarray:
    """Pad axes 1..3 (D, H, W) of x at the high end up to window multiples."""
    pads = [(0, 0)]
    for n, w in zip(x.shape[1:4], window):
        pads.append((0, padded_extent(n, w) - n))
    pads += [(0, 0)] * (x.ndim - 4)
    return np.pad(x, pads, mode="constant", constant_values=value)


def cyclic_shift(x: np.ndarray, shift) -> np.ndarray:
    """Swin's cyclic shift: roll the (padded) grid by -shift along D, H, W."""
    return np.roll(x, shift=tuple(-int(s) for s in shift), axis=(1, 2, 3))


def cyclic_unshift(x: np.ndarray, shift) -> np.ndarray:
    """Inverse of cyclic_shift."""
    return np.roll(x, shift=tuple(int(s) for s in shift), axis=(1, 2, 3))


def _axis_slices(n: int, w: int, s: int):
    if s == 0:
        return [slice(0, n)]
    return [slice(0, n - w), slice(n - w, n - s), slice(n - s, n)]


def region_labels(padded, window, shift) -> np.ndarray:
    """Integer region label of every position of the shifted, padded grid [PD, PH, PW].

    Swin's shifted-window mask: along each shifted axis the grid is cut into
    [0, P-w), [P-w, P-s), [P-s, P); a token's label is its triple of slices.
    Two tokens of one window attend without bias only if their labels match."""
    lab = np.zeros(tuple(padded), dtype=np.int64)
    count = 0
    for sd in _axis_slices(padded[0], window[0], shift[0]):
        for sh in _axis_slices(padded[1], window[1], shift[1]):
            for sw in _axis_slices(padded[2], window[2], shift[2]):
                lab[sd, sh, sw] = count
                count += 1
    return lab


def window_partition(x: np.ndarray, window) -> np.ndarray:
    """[B, PD, PH, PW, *rest] -> [B * n_windows, wd*wh*ww, *rest].

    Windows are numbered (b, kd, kh, kw) row-major; slots inside a window
    (od, oh, ow) row-major."""
    B, PD, PH, PW = x.shape[:4]
    rest = x.shape[4:]
    wd, wh, ww = window
    y = x.reshape(B, PD // wd, wd, PH // wh, wh, PW // ww, ww, *rest)
    y = y.transpose((0, 1, 3, 5, 2, 4, 6) + tuple(range(7, 7 + len(rest))))
    return y.reshape(B * (PD // wd) * (PH // wh) * (PW // ww), wd * wh * ww, *rest)


def window_merge(xw: np.ndarray, window, B: int, padded) -> np.ndarray:
    """Inverse of window_partition: [B * n_windows, N, *rest] -> [B, PD, PH, PW, *rest]."""
    PD, PH, PW = padded
    wd, wh, ww = window
    rest = xw.shape[2:]
    y = xw.reshape(B, PD // wd, PH // wh, PW // ww, wd, wh, ww, *rest)
    y = y.transpose((0, 1, 4, 2, 5, 3, 6) + tuple(range(7, 7 + len(rest))))
    return y.reshape(B, PD, PH, PW, *rest)


def masked_window_attention(qw, kw, vw, labels_w, valid_w, scale: float, bias: float):
    """Attention inside each window, every head on its own.

    qw, kw, vw: [n_windows, N, heads, dh] float64; labels_w, valid_w: [n_windows, N].
    S = scale * Q K^T; S += bias where the query and key labels differ;
    S = -inf where the key is padding; P = exp(S - rowmax); l = sum_j P;
    O = P V / l. Rows of padding queries are returned as 0.
    Returns (O [n_windows, N, heads, dh], l [n_windows, heads, N],
    rowsum of P / l [n_windows, heads, N])."""
    q = np.ascontiguousarray(qw.transpose(0, 2, 1, 3))  # [nW, h, N, dh]
    k = np.ascontiguousarray(kw.transpose(0, 2, 1, 3))
    v = np.ascontiguousarray(vw.transpose(0, 2, 1, 3))
    s = scale * np.matmul(q, k.transpose(0, 1, 3, 2))  # [nW, h, Nq, Nk]
    differ = labels_w[:, None, :, None] != labels_w[:, None, None, :]
    s = np.where(differ, s + bias, s)
    s = np.where(valid_w[:, None, None, :], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)  # only padding rows can be all -inf
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    qvalid = valid_w[:, None, :, None]
    safe_l = np.where(qvalid, l, 1.0)
    o = np.matmul(p, v) / safe_l
    o = np.where(qvalid, o, 0.0)
    rowsum = (p / safe_l).sum(axis=-1)
    return o.transpose(0, 2, 1, 3), l[..., 0], rowsum


def swin3d_window_attention(q, k, v, window, shift, scale: float, bias: float = -100.0,
                            pad_value: float = 0.0, return_stats: bool = False):
    """Swin3D shifted-window attention on grid-layout tensors [B, D, H, W, heads, dh].

    Steps, in the pages' order: pad to window multiples, cyclic shift, region
    labels, 3D window partition, masked softmax attention per window and head,
    inverse merge, inverse shift, crop. Returns O in float64 with the input's
    shape (and, if asked, l and the softmax row sums in windowed layout)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, D, H, W = q.shape[:4]
    padded = tuple(padded_extent(n, w) for n, w in zip((D, H, W), window))

    valid = pad_to_windows(np.ones((B, D, H, W), dtype=bool), window, value=False)
    qp = pad_to_windows(q, window, pad_value)
    kp = pad_to_windows(k, window, pad_value)
    vp = pad_to_windows(v, window, pad_value)

    qs, ks, vs = cyclic_shift(qp, shift), cyclic_shift(kp, shift), cyclic_shift(vp, shift)
    valid_s = cyclic_shift(valid, shift)
    labels = np.broadcast_to(region_labels(padded, window, shift), (B,) + padded)

    qw, kw, vw = window_partition(qs, window), window_partition(ks, window), window_partition(vs, window)
    valid_w = window_partition(valid_s, window)
    labels_w = window_partition(np.ascontiguousarray(labels), window)

    ow, l, rowsum = masked_window_attention(qw, kw, vw, labels_w, valid_w, scale, bias)

    o = window_merge(ow, window, B, padded)
    o = cyclic_unshift(o, shift)
    o = o[:, :D, :H, :W]
    if return_stats:
        return np.ascontiguousarray(o), {"l": l, "rowsum": rowsum, "valid_w": valid_w}
    return np.ascontiguousarray(o)


def window_count(B: int, grid, window) -> int:
    """Number of windows the partition produces (batch folded in)."""
    n = B
    for x, w in zip(grid, window):
        n *= padded_extent(x, w) // w
    return n


# ---------------------------------------------------------------------------
# Per-window evaluation at full size. Large grids do not fit a float64 copy,
# so the same attention is evaluated for a chosen set of windows. A window's
# slots are located by undoing the roll: shifted position p holds grid
# position g = (p + s) mod P; g outside the real grid is padding.
# ---------------------------------------------------------------------------

def window_slot_coords(grid, window, shift, win):
    """Grid coordinates [N, 3], validity [N] and region labels [N] of window win = (kd, kh, kw)."""
    padded = tuple(padded_extent(x, w) for x, w in zip(grid, window))
    wd, wh, ww = window
    od, oh, ow = np.meshgrid(np.arange(wd), np.arange(wh), np.arange(ww), indexing="ij")
    p = np.stack([win[0] * wd + od.ravel(), win[1] * wh + oh.ravel(), win[2] * ww + ow.ravel()], axis=1)
    g = (p + np.asarray(shift)[None, :]) % np.asarray(padded)[None, :]
    valid = np.all(g < np.asarray(grid)[None, :], axis=1)
    labels = region_labels(padded, window, shift)[p[:, 0], p[:, 1], p[:, 2]]
    return g, valid, labels


def windows_attention(fetch, B, grid, heads, dh, window, shift, scale, bias, windows):
    """Attention outputs of the listed windows.

    fetch(tensor, b, coords) returns the float64 rows [n, heads, dh] of tensor
    'q', 'k' or 'v' at batch b and grid coordinates coords [n, 3].
    windows: iterable of (b, kd, kh, kw).
    Returns a list of (b, coords [n, 3], O [n, heads, dh]) over real slots."""
    out = []
    for (b, kd, kh, kw) in windows:
        g, valid, labels = window_slot_coords(grid, window, shift, (kd, kh, kw))
        n = g.shape[0]
        gath = {}
        for t in ("q", "k", "v"):
            a = np.zeros((n, heads, dh), dtype=np.float64)
            a[valid] = fetch(t, b, g[valid])
            gath[t] = a
        o, _, _ = masked_window_attention(gath["q"][None], gath["k"][None], gath["v"][None],
                                          labels[None], valid[None], scale, bias)
        out.append((b, g[valid], o[0][valid]))
    return out
