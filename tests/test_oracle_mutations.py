"""Planted mistakes in the oracle must be caught by the pins.

Each case swaps one oracle step for a plausible wrong variant (a sign, an
index, a transposed operand, a dropped term) and checks that the
brute-force / SDPA / invariant pins then fail. Runs on the CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.swin3d as osw
from _pins import grid_brute_force

WIN = (2, 6, 12)


def _qkv(shape, seed, qk=1.5):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal(shape) * s for s in (qk, qk, 1.0))


def pin_brute_force_error(bias=-100.0, shape=(1, 4, 15, 30, 2, 3), shift=(1, 3, 6), qk=1.5):
    q, k, v = _qkv(shape, 5, qk)
    o = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.3, bias)
    ref = grid_brute_force(q, k, v, WIN, shift, 0.3, bias)
    return float(np.max(np.abs(o - ref)))


def pin_padding_invariance_error():
    q, k, v = _qkv((1, 4, 15, 30, 1, 3), 6)
    o1 = oracle.swin3d_window_attention(q, k, v, WIN, (1, 3, 6), 0.3, -100.0, pad_value=0.0)
    o2 = oracle.swin3d_window_attention(q, k, v, WIN, (1, 3, 6), 0.3, -100.0, pad_value=1e3)
    return float(np.max(np.abs(o1 - o2)))


def pin_sdpa_zero_shift_error():
    q, k, v = _qkv((1, 2, 6, 12, 2, 4), 7)
    o = oracle.swin3d_window_attention(q, k, v, WIN, (0, 0, 0), 0.3, -100.0)
    t = lambda a: torch.from_numpy(a.reshape(144, 2, 4).transpose(1, 0, 2).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(t(q[0]), t(k[0]), t(v[0]), scale=0.3)
    return float(np.max(np.abs(o[0].reshape(144, 2, 4).transpose(1, 0, 2) - ref.numpy())))


def pin_roundtrip_error():
    x = np.random.default_rng(8).standard_normal((1, 4, 15, 30, 1, 1))
    B, D, H, W = x.shape[:4]
    padded = tuple(oracle.padded_extent(n, w) for n, w in zip((D, H, W), WIN))
    y = osw.window_partition(osw.cyclic_shift(osw.pad_to_windows(x, WIN), (1, 3, 6)), WIN)
    z = osw.cyclic_unshift(osw.window_merge(y, WIN, B, padded), (1, 3, 6))[:, :D, :H, :W]
    return float(np.max(np.abs(z - x)))


def all_pins():
    return {
        "brute_force_bias": pin_brute_force_error(-100.0),
        "brute_force_excl": pin_brute_force_error(-math.inf),
        # logits of std ~60, as in the stress workload: -100 no longer masks fully
        "brute_force_bias_large": pin_brute_force_error(-100.0, shape=(1, 2, 12, 24, 1, 16), qk=8.0),
        # a shift that is not half the window, so P - s and P - w + s differ
        "brute_force_odd_shift": pin_brute_force_error(-math.inf, shape=(1, 4, 12, 24, 1, 3), shift=(1, 2, 4)),
        "padding": pin_padding_invariance_error(),
        "sdpa": pin_sdpa_zero_shift_error(),
        "roundtrip": pin_roundtrip_error(),
    }


def test_unmutated_oracle_passes_every_pin():
    errs = all_pins()
    assert max(errs.values()) < 1e-12, errs


# ---- the mutations -------------------------------------------------------

def _shift_wrong_sign(x, shift):
    return np.roll(x, shift=tuple(int(s) for s in shift), axis=(1, 2, 3))


def _unshift_wrong_sign(x, shift):
    return np.roll(x, shift=tuple(-int(s) for s in shift), axis=(1, 2, 3))


def _labels_one_cut(padded, window, shift):
    # drops the cut at P - s: only [0, P-w) and [P-w, P) are told apart
    lab = np.zeros(tuple(padded), dtype=np.int64)
    c = 0
    cut = lambda n, w, s: [slice(0, n)] if s == 0 else [slice(0, n - w), slice(n - w, n)]
    for a in cut(padded[0], window[0], shift[0]):
        for b in cut(padded[1], window[1], shift[1]):
            for e in cut(padded[2], window[2], shift[2]):
                lab[a, b, e] = c
                c += 1
    return lab


def _labels_cut_at_w(padded, window, shift):
    # cuts at P - w and at s (a wrong index) instead of P - s
    lab = np.zeros(tuple(padded), dtype=np.int64)
    c = 0
    cut = lambda n, w, s: [slice(0, n)] if s == 0 else [slice(0, n - w), slice(n - w, n - w + s), slice(n - w + s, n)]
    for a in cut(padded[0], window[0], shift[0]):
        for b in cut(padded[1], window[1], shift[1]):
            for e in cut(padded[2], window[2], shift[2]):
                lab[a, b, e] = c
                c += 1
    return lab


def _partition_swapped_axes(x, window):
    # windows that are not spatial blocks: the slot order mixes window and in-window indices
    B, PD, PH, PW = x.shape[:4]
    rest = x.shape[4:]
    wd, wh, ww = window
    y = x.reshape(B, wd, PD // wd, wh, PH // wh, ww, PW // ww, *rest)
    y = y.transpose((0, 2, 4, 6, 1, 3, 5) + tuple(range(7, 7 + len(rest))))
    return y.reshape(B * (PD // wd) * (PH // wh) * (PW // ww), wd * wh * ww, *rest)


def _merge_swapped_axes(xw, window, B, padded):
    PD, PH, PW = padded
    wd, wh, ww = window
    rest = xw.shape[2:]
    y = xw.reshape(B, PD // wd, PH // wh, PW // ww, wd, wh, ww, *rest)
    y = y.transpose((0, 4, 1, 5, 2, 6, 3) + tuple(range(7, 7 + len(rest))))
    return y.reshape(B, PD, PH, PW, *rest)


def _make_attention(variant):
    def attn(qw, kw, vw, labels_w, valid_w, scale, bias):
        q = qw.transpose(0, 2, 1, 3)
        k = kw.transpose(0, 2, 1, 3)
        v = vw.transpose(0, 2, 1, 3)
        raw = np.matmul(q, k.transpose(0, 1, 3, 2))
        if variant == "transposed":
            raw = raw.transpose(0, 1, 3, 2)
        differ = labels_w[:, None, :, None] != labels_w[:, None, None, :]
        if variant == "bias_before_scale":
            s = scale * np.where(differ, raw + bias, raw)
        elif variant == "no_scale":
            s = np.where(differ, raw + bias, raw)
        else:
            s = scale * raw
            s = np.where(differ, s + bias, s)
        if variant != "no_pad_mask":
            s = np.where(valid_w[:, None, None, :], s, -np.inf)
        axis = -2 if variant == "softmax_wrong_axis" else -1
        m = s.max(axis=axis, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.exp(s - m)
        l = p.sum(axis=axis, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            o = np.matmul(p, v) / (l if axis == -1 else l.transpose(0, 1, 3, 2))
        o = np.where(valid_w[:, None, :, None], o, 0.0)
        return o.transpose(0, 2, 1, 3), l[..., 0] if axis == -1 else l[..., 0, :], p.sum(-1)
    return attn


MUTATIONS = {
    "shift_sign": [("cyclic_shift", _shift_wrong_sign), ("cyclic_unshift", _unshift_wrong_sign)],
    "labels_missing_cut": [("region_labels", _labels_one_cut)],
    "labels_wrong_index": [("region_labels", _labels_cut_at_w)],
    "partition_not_blocks": [("window_partition", _partition_swapped_axes),
                             ("window_merge", _merge_swapped_axes)],
    "transposed_scores": [("masked_window_attention", _make_attention("transposed"))],
    "bias_before_scale": [("masked_window_attention", _make_attention("bias_before_scale"))],
    "dropped_scale": [("masked_window_attention", _make_attention("no_scale"))],
    "no_padding_mask": [("masked_window_attention", _make_attention("no_pad_mask"))],
    "softmax_wrong_axis": [("masked_window_attention", _make_attention("softmax_wrong_axis"))],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(osw, attr, fn)
    errs = all_pins()
    assert max(errs.values()) > 1e-6, (name, errs)
