"""Pins of the oracle's layout steps: pad, cyclic shift, partition, merge, region labels."""
import json
import os

import numpy as np
import pytest

import datagen
import oracle
from _pins import region_sizes, token_groups

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _roundtrip(x, window, shift):
    B, D, H, W = x.shape[:4]
    padded = tuple(oracle.padded_extent(n, w) for n, w in zip((D, H, W), window))
    y = oracle.window_partition(oracle.cyclic_shift(oracle.pad_to_windows(x, window), shift), window)
    z = oracle.cyclic_unshift(oracle.window_merge(y, window, B, padded), shift)[:, :D, :H, :W]
    return y, z


def test_window_counts_match_pages():
    """B * n_W of the three ERA5 encoder shapes printed on the pages."""
    with open(os.path.join(GOLDEN, "window_counts.json")) as f:
        gold = json.load(f)
    wd, wh, ww = gold["window"]
    assert wd * wh * ww == gold["tokens_per_window"] == 144
    for case in gold["cases"]:
        wl = datagen.WORKLOADS[case["workload"]]
        assert tuple(wl.window) == tuple(gold["window"])
        n = oracle.window_count(wl.B, (wl.D, wl.H, wl.W), wl.window)
        assert [n, wl.heads, 144, wl.head_dim] == case["attention_shape"]


def test_window_counts_other_workloads():
    assert oracle.window_count(1, (2, 12, 24), (2, 6, 12)) == 4
    assert oracle.window_count(2, (4, 450, 900), (2, 6, 12)) == 22500


@pytest.mark.parametrize("name", sorted(datagen.WORKLOADS))
def test_roundtrip_identity_bit_exact(name):
    """crop . unshift . merge . partition . shift . pad == identity, for every workload's grid."""
    wl = datagen.WORKLOADS[name]
    rng = np.random.default_rng(7)
    x = rng.standard_normal((wl.B, wl.D, wl.H, wl.W, 1, 2))
    y, z = _roundtrip(x, wl.window, wl.shift)
    assert y.shape[1] == wl.window[0] * wl.window[1] * wl.window[2]
    assert z.dtype == x.dtype and np.array_equal(z, x)


@pytest.mark.parametrize("grid,shift", [((2, 12, 24), (1, 3, 6)), ((4, 45, 90), (1, 3, 6)),
                                        ((4, 44, 30), (1, 3, 6)), ((3, 7, 13), (1, 5, 11)),
                                        ((4, 45, 90), (0, 0, 0))])
def test_partition_is_bijection_onto_real_tokens(grid, shift):
    """Every real token sits in exactly one window slot; padding slots are exactly the rest."""
    B = 2
    window = (2, 6, 12)
    ids = np.arange(B * np.prod(grid), dtype=np.int64).reshape((B,) + grid) + 1
    y = oracle.window_partition(oracle.cyclic_shift(oracle.pad_to_windows(ids, window), shift), window)
    flat = y.ravel()
    real = flat[flat > 0]
    assert np.array_equal(np.sort(real), np.arange(1, B * np.prod(grid) + 1))
    padded = np.prod([oracle.padded_extent(n, w) for n, w in zip(grid, window)])
    assert (flat == 0).sum() == B * (padded - np.prod(grid))


@pytest.mark.parametrize("grid,shift", [((2, 12, 24), (1, 3, 6)), ((4, 48, 96), (1, 3, 6)),
                                        ((4, 18, 36), (1, 3, 6)), ((2, 12, 24), (0, 3, 0)),
                                        ((4, 44, 30), (1, 3, 6)), ((4, 12, 24), (1, 5, 11))])
def test_region_labels_match_bit_form(grid, shift):
    """Inside every window, the three-slice labels and the per-axis wrap bits
    (p >= P - s) induce the same partition of the real tokens."""
    window = (2, 6, 12)
    padded = tuple(oracle.padded_extent(n, w) for n, w in zip(grid, window))
    lab = oracle.region_labels(padded, window, shift)
    for (_, win), toks in token_groups(grid, window, shift, 1).items():
        labs, bits = [], []
        for g, bb in toks:
            p = [(g[a] - shift[a]) % padded[a] for a in range(3)]
            assert tuple(p[a] // window[a] for a in range(3)) == win
            labs.append(lab[p[0], p[1], p[2]])
            bits.append(bb)
        for i in range(len(toks)):
            for j in range(len(toks)):
                assert (labs[i] == labs[j]) == (bits[i] == bits[j])


def test_region_sizes_tiny():
    """Tiny workload (D = 2 = window depth, shift applied as given): each of the
    four windows splits into regions of 72, 36, 36 or 18 tokens."""
    sizes = region_sizes((2, 12, 24), (2, 6, 12), (1, 3, 6))
    got = sorted(tuple(v) for v in sizes.values())
    assert got == sorted([(72, 72), (36, 36, 36, 36), (36, 36, 36, 36), (18,) * 8])
    # and the oracle's label array agrees on the count of distinct labels per window
    lab = oracle.region_labels((2, 12, 24), (2, 6, 12), (1, 3, 6))
    lw = oracle.window_partition(lab[None], (2, 6, 12))
    assert sorted(len(np.unique(r)) for r in lw) == [2, 4, 4, 8]


def test_zero_shift_single_region():
    lab = oracle.region_labels((4, 90, 180), (2, 6, 12), (0, 0, 0))
    assert np.all(lab == 0)


def test_masked_window_count_stage1():
    """Windows that hold more than one region: the last along any shifted axis."""
    lab = oracle.region_labels((4, 180, 360), (2, 6, 12), (1, 3, 6))
    lw = oracle.window_partition(lab[None], (2, 6, 12))
    multi = sum(len(np.unique(r)) > 1 for r in lw)
    n_d, n_h, n_w = 2, 30, 30
    expected = sum(1 for kd in range(n_d) for kh in range(n_h) for kw in range(n_w)
                   if kd == n_d - 1 or kh == n_h - 1 or kw == n_w - 1)
    assert multi == expected == 959
