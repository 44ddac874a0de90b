"""Independent formulations used to pin the oracle (test helpers, CPU only).

None of these calls the oracle's layout code: windows and regions are found
from grid coordinates with modular arithmetic, one token at a time, and the
softmax is written out again. They are slow and meant for tiny grids.
"""
from __future__ import annotations

import itertools
import math
from collections import defaultdict

import numpy as np


def _padded(n, w):
    return -(-n // w) * w


def token_groups(grid, window, shift, B):
    """Map every real token to (b, window id) with its per-axis region bits.

    Shifted position of grid coordinate g is p = (g - s) mod P; its window is
    p // w; along a shifted axis the tokens with p >= P - s form the second
    region of the last window (the part that wrapped around)."""
    P = [_padded(x, w) for x, w in zip(grid, window)]
    groups = defaultdict(list)
    for b in range(B):
        for g in itertools.product(range(grid[0]), range(grid[1]), range(grid[2])):
            p = [(g[a] - shift[a]) % P[a] for a in range(3)]
            win = tuple(p[a] // window[a] for a in range(3))
            bits = tuple(int(shift[a] > 0 and p[a] >= P[a] - shift[a]) for a in range(3))
            groups[(b, win)].append((g, bits))
    return groups


def grid_brute_force(q, k, v, window, shift, scale, bias):
    """Swin3D window attention computed token by token from grid coordinates."""
    B, D, H, W, h, dh = q.shape
    out = np.full(q.shape, np.nan)
    for (b, _win), toks in token_groups((D, H, W), window, shift, B).items():
        coords = np.array([t[0] for t in toks])
        bits = np.array([t[1] for t in toks])
        idx = (b, coords[:, 0], coords[:, 1], coords[:, 2])
        Q, K, V = q[idx], k[idx], v[idx]  # [n, h, dh]
        differ = np.any(bits[:, None, :] != bits[None, :, :], axis=2)
        for hh in range(h):
            s = scale * (Q[:, hh] @ K[:, hh].T)
            if np.isneginf(bias):
                s = np.where(differ, -np.inf, s)
            else:
                s = s + bias * differ
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[idx + (hh,)] = (p @ V[:, hh]) / p.sum(axis=1, keepdims=True)
    return out


def loop_attention_unshifted(q, k, v, window, scale):
    """Zero shift, no padding: explicit loops over windows, queries and keys with math.exp."""
    B, D, H, W, h, dh = q.shape
    wd, wh, ww = window
    out = np.zeros(q.shape)
    for b, kd, kh, kw in itertools.product(range(B), range(D // wd), range(H // wh), range(W // ww)):
        toks = [(kd * wd + a, kh * wh + c, kw * ww + e)
                for a in range(wd) for c in range(wh) for e in range(ww)]
        for hh in range(h):
            for ti in toks:
                qi = q[(b,) + ti + (hh,)]
                logits = [scale * float(np.dot(qi, k[(b,) + tj + (hh,)])) for tj in toks]
                mx = max(logits)
                ws = [math.exp(x - mx) for x in logits]
                tot = math.fsum(ws)
                acc = np.zeros(dh)
                for wgt, tj in zip(ws, toks):
                    acc += wgt * v[(b,) + tj + (hh,)]
                out[(b,) + ti + (hh,)] = acc / tot
    return out


def region_sizes(grid, window, shift, B=1):
    """Sorted region sizes per window (from the bit form)."""
    sizes = {}
    for key, toks in token_groups(grid, window, shift, B).items():
        cnt = defaultdict(int)
        for _, bits in toks:
            cnt[bits] += 1
        sizes[key] = sorted(cnt.values(), reverse=True)
    return sizes
