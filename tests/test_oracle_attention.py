"""Pins of the oracle's attention against brute force, PyTorch SDPA, closed forms and invariants."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from _pins import grid_brute_force, loop_attention_unshifted

WIN = (2, 6, 12)
NEG_INF = -math.inf


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _qkv(shape, seed, scale=1.0):
    return _rand(shape, seed, scale), _rand(shape, seed + 1, scale), _rand(shape, seed + 2)


# ---------------------------------------------------------------- P2: zero shift
def test_zero_shift_matches_loop_brute_force():
    q, k, v = _qkv((1, 2, 6, 24, 2, 4), 11)
    o = oracle.swin3d_window_attention(q, k, v, WIN, (0, 0, 0), 0.37, -100.0)
    ref = loop_attention_unshifted(q, k, v, WIN, 0.37)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


def test_zero_shift_matches_sdpa_per_window():
    """Each window is plain softmax attention: torch SDPA in float64 on the CPU."""
    q, k, v = _qkv((2, 4, 12, 24, 3, 8), 21)
    scale = 1 / math.sqrt(8)
    o = oracle.swin3d_window_attention(q, k, v, WIN, (0, 0, 0), scale, -100.0)
    for b in range(2):
        for kd in range(2):
            for kh in range(2):
                for kw in range(2):
                    sl = (b, slice(2 * kd, 2 * kd + 2), slice(6 * kh, 6 * kh + 6), slice(12 * kw, 12 * kw + 12))
                    tq = torch.from_numpy(q[sl].reshape(144, 3, 8).transpose(1, 0, 2).copy())
                    tk = torch.from_numpy(k[sl].reshape(144, 3, 8).transpose(1, 0, 2).copy())
                    tv = torch.from_numpy(v[sl].reshape(144, 3, 8).transpose(1, 0, 2).copy())
                    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
                    got = o[sl].reshape(144, 3, 8).transpose(1, 0, 2)
                    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P3: grid brute force
@pytest.mark.parametrize("bias", [-100.0, NEG_INF, -2.5])
@pytest.mark.parametrize("shape,shift", [
    ((1, 2, 12, 24, 2, 4), (1, 3, 6)),     # tiny workload grid, every window masked
    ((1, 4, 45, 90, 1, 3), (1, 3, 6)),     # stage-3 grid with padding (pad == shift per axis)
    ((1, 4, 44, 30, 1, 3), (1, 3, 6)),     # pad != shift along H: the pad-then-roll convention
    ((2, 3, 7, 13, 1, 2), (1, 5, 11)),     # odd sizes, pads on every axis, large shifts
    ((1, 2, 12, 24, 2, 4), (0, 3, 0)),     # shift along one axis only
])
def test_matches_grid_brute_force(shape, shift, bias):
    q, k, v = _qkv(shape, 31, 1.5)
    o = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.29, bias)
    ref = grid_brute_force(q, k, v, WIN, shift, 0.29, bias)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P4: SDPA with the mask
@pytest.mark.parametrize("bias", [-100.0, NEG_INF, -2.5])
def test_matches_sdpa_with_float_mask(bias):
    """Per window: SDPA (float64, CPU) with a float mask of `bias` where labels
    differ and -inf on padding keys equals the oracle on real query rows."""
    shape, shift = (1, 4, 9, 30, 2, 4), (1, 3, 6)
    q, k, v = _qkv(shape, 41, 2.0)
    scale = 0.41
    o = oracle.swin3d_window_attention(q, k, v, WIN, shift, scale, bias)
    B, D, H, W = shape[:4]
    padded = tuple(oracle.padded_extent(n, w) for n, w in zip((D, H, W), WIN))
    valid = oracle.pad_to_windows(np.ones((B, D, H, W), bool), WIN, False)
    lab = oracle.region_labels(padded, WIN, shift)
    part = lambda x: oracle.window_partition(oracle.cyclic_shift(oracle.pad_to_windows(x, WIN), shift), WIN)
    qw, kw, vw = part(q), part(k), part(v)
    vw_mask = oracle.window_partition(oracle.cyclic_shift(valid, shift), WIN)
    lw = oracle.window_partition(np.broadcast_to(lab, (B,) + padded).copy(), WIN)
    ow = part(o)  # the oracle's output, partitioned the same way, for comparison
    for w in range(qw.shape[0]):
        mask = np.where(lw[w][:, None] != lw[w][None, :], bias, 0.0)
        mask = np.where(vw_mask[w][None, :], mask, -np.inf)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a[w].transpose(1, 0, 2)))
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(qw), t(kw), t(vw), attn_mask=torch.from_numpy(mask), scale=scale).numpy()
        real = vw_mask[w]
        np.testing.assert_allclose(ow[w].transpose(1, 0, 2)[:, real], ref[:, real], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P5: uniform V
@pytest.mark.parametrize("bias", [-100.0, NEG_INF])
def test_uniform_v_gives_v(bias):
    shape = (1, 4, 45, 90, 2, 5)
    q, k, _ = _qkv(shape, 51, 3.0)
    c = np.random.default_rng(5).standard_normal((2, 5))
    v = np.broadcast_to(c, shape).copy()
    o = oracle.swin3d_window_attention(q, k, v, WIN, (1, 3, 6), 0.5, bias)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15 * 10)


# ---------------------------------------------------------------- P6: Q = 0
def test_q_zero_exclusion_gives_region_mean():
    """Under -inf, Q = 0 makes every allowed weight equal: O_i is the mean of V
    over i's region of i's window (region sizes 72/36/36/18 on the tiny grid)."""
    shape, shift = (1, 2, 12, 24, 1, 3), (1, 3, 6)
    v = _rand(shape, 61)
    z = np.zeros(shape)
    o = oracle.swin3d_window_attention(z, _rand(shape, 62), v, WIN, shift, 0.3, NEG_INF)
    from _pins import token_groups
    for (b, _), toks in token_groups((2, 12, 24), WIN, shift, 1).items():
        by_bits = {}
        for g, bits in toks:
            by_bits.setdefault(bits, []).append(g)
        for members in by_bits.values():
            idx = tuple(np.array(members).T)
            mean = v[(b,) + idx].mean(axis=0)
            np.testing.assert_allclose(o[(b,) + idx], np.broadcast_to(mean, o[(b,) + idx].shape),
                                       rtol=0, atol=1e-14)


@pytest.mark.parametrize("bias", [-100.0, -1.5])
def test_q_zero_bias_closed_form(bias):
    """Q = 0 under a finite bias b: O_i = (sum_same V + e^b sum_other V) / (n_same + e^b n_other)
    (at -100 the other regions all but vanish; at -1.5 they weigh in)."""
    shape, shift = (1, 2, 12, 24, 1, 2), (1, 3, 6)
    v = _rand(shape, 71)
    o = oracle.swin3d_window_attention(np.zeros(shape), _rand(shape, 72), v, WIN, shift, 0.3, bias)
    from _pins import token_groups
    e = math.exp(bias)
    for (b, _), toks in token_groups((2, 12, 24), WIN, shift, 1).items():
        coords = np.array([g for g, _ in toks])
        bits = [bb for _, bb in toks]
        V = v[b, coords[:, 0], coords[:, 1], coords[:, 2]]
        for i, (g, bi) in enumerate(toks):
            same = np.array([bj == bi for bj in bits])
            num = V[same].sum(0) + e * V[~same].sum(0)
            den = same.sum() + e * (~same).sum()
            np.testing.assert_allclose(o[(b,) + g], num / den, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- P7: softmax rows
@pytest.mark.parametrize("bias", [-100.0, NEG_INF])
def test_softmax_rows_sum_to_one(bias):
    q, k, v = _qkv((1, 4, 45, 90, 2, 4), 81, 4.0)
    _, st = oracle.swin3d_window_attention(q, k, v, WIN, (1, 3, 6), 0.5, bias, return_stats=True)
    real = np.broadcast_to(st["valid_w"][:, None, :], st["rowsum"].shape)
    np.testing.assert_allclose(st["rowsum"][real], 1.0, rtol=0, atol=1e-14)
    assert np.all(st["l"][real] >= 1.0)


# ---------------------------------------------------------------- P8: isolation
def _other_region_mask(grid, shift, target):
    """Boolean grid of tokens that share target's window but not its region, and tokens in other windows."""
    from _pins import token_groups
    same, other_win_region = set(), set()
    for key, toks in token_groups(grid, WIN, shift, 1).items():
        coords = [g for g, _ in toks]
        if target in coords:
            tb = dict(toks)[target]
            for g, bb in toks:
                (same if bb == tb else other_win_region).add(g)
    return same, other_win_region


def test_isolation_exclusion_bit_identical():
    """-inf mode: perturbing K, V of tokens outside a query's region leaves its output bit-identical."""
    shape, shift = (1, 2, 12, 24, 2, 4), (1, 3, 6)
    grid = shape[1:4]
    q, k, v = _qkv(shape, 91)
    target = (1, 11, 23)  # corner token: the last window along every axis, 8 regions
    same, other = _other_region_mask(grid, shift, target)
    assert len(same) == 18 and len(other) == 144 - 18
    k2, v2 = k.copy(), v.copy()
    for g in other:
        k2[(0,) + g] += 50.0
        v2[(0,) + g] *= -1e3
    # tokens of other windows too
    k2[0, :, :6, :12] += 7.0
    o1 = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.3, NEG_INF)
    o2 = oracle.swin3d_window_attention(q, k2, v2, WIN, shift, 0.3, NEG_INF)
    for g in same:
        assert np.array_equal(o1[(0,) + g], o2[(0,) + g])


def test_isolation_bias_within_bound():
    """-100 mode on N(0,1) data: the change is below 2 max|V| sum_j e^(S_ij - 100 - m_i)."""
    shape, shift = (1, 2, 12, 24, 1, 4), (1, 3, 6)
    grid = shape[1:4]
    q, k, v = _qkv(shape, 101)
    target = (1, 11, 23)
    same, other = _other_region_mask(grid, shift, target)
    v2 = v.copy()
    for g in other:
        v2[(0,) + g] += 3.0
    o1 = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.5, -100.0)
    o2 = oracle.swin3d_window_attention(q, k, v2, WIN, shift, 0.5, -100.0)
    for g in same:
        qi = q[(0,) + g + (0,)]
        s_same = [0.5 * qi @ k[(0,) + t + (0,)] for t in same]
        s_other = [0.5 * qi @ k[(0,) + t + (0,)] - 100.0 for t in other]
        m = max(s_same)
        bound = 2 * max(np.abs(v2).max(), np.abs(v).max()) * sum(math.exp(s - m) for s in s_other)
        assert bound < 1e-35
        assert np.max(np.abs(o1[(0,) + g] - o2[(0,) + g])) <= bound


@pytest.mark.parametrize("bias", [-100.0, NEG_INF])
def test_padding_values_never_matter(bias):
    """Padding keys are excluded in both modes: the pad fill value leaves the output bit-identical."""
    q, k, v = _qkv((1, 4, 45, 90, 2, 3), 111)
    o1 = oracle.swin3d_window_attention(q, k, v, WIN, (1, 3, 6), 0.5, bias, pad_value=0.0)
    o2 = oracle.swin3d_window_attention(q, k, v, WIN, (1, 3, 6), 0.5, bias, pad_value=1e6)
    assert np.array_equal(o1, o2)


# ---------------------------------------------------------------- P9: large logits
def test_large_logit_limit():
    """Where the top two allowed logits of a row differ by more than 40, O_i is V of the arg-max key."""
    shape, shift = (1, 2, 12, 24, 1, 8), (1, 3, 6)
    q, k, v = _qkv(shape, 121, 8.0)
    scale = 1 / math.sqrt(8)
    o = oracle.swin3d_window_attention(q, k, v, WIN, shift, scale, NEG_INF)
    assert np.all(np.isfinite(o))
    from _pins import token_groups
    checked = 0
    for (b, _), toks in token_groups((2, 12, 24), WIN, shift, 1).items():
        coords = np.array([g for g, _ in toks])
        bits = [bb for _, bb in toks]
        for i, (g, bi) in enumerate(toks):
            allowed = [j for j, bj in enumerate(bits) if bj == bi]
            s = np.array([scale * q[(b,) + g + (0,)] @ k[(b,) + tuple(coords[j]) + (0,)] for j in allowed])
            order = np.argsort(s)[::-1]
            if s[order[0]] - s[order[1]] > 40:
                j = allowed[order[0]]
                np.testing.assert_allclose(o[(b,) + g + (0,)], v[(b,) + tuple(coords[j]) + (0,)],
                                           rtol=0, atol=144 * math.exp(-40) * np.abs(v).max())
                checked += 1
    assert checked > 20


def test_stress_modes_differ():
    """At the stress workload's logit scale (Q, K x 8), -100 is not a mask: the two modes differ."""
    shape, shift = (1, 2, 12, 24, 1, 64), (1, 3, 6)
    q, k, v = _qkv(shape, 131, 8.0)
    o1 = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.125, -100.0)
    o2 = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.125, NEG_INF)
    assert np.max(np.abs(o1 - o2)) > 0.1


# ---------------------------------------------------------------- P10: equivariance
def test_permuting_slots_inside_window():
    rng = np.random.default_rng(141)
    nw, n, h, dh = 3, 144, 2, 4
    q, k, v = (rng.standard_normal((nw, n, h, dh)) for _ in range(3))
    lab = rng.integers(0, 3, size=(nw, n))
    valid = rng.random((nw, n)) > 0.1
    perm = rng.permutation(n)
    o1, _, _ = oracle.masked_window_attention(q, k, v, lab, valid, 0.4, -100.0)
    o2, _, _ = oracle.masked_window_attention(q[:, perm], k[:, perm], v[:, perm], lab[:, perm],
                                              valid[:, perm], 0.4, -100.0)
    np.testing.assert_allclose(o2, o1[:, perm], rtol=0, atol=1e-14)


def test_roll_by_whole_windows_rolls_output():
    q, k, v = _qkv((1, 4, 12, 36, 2, 4), 151)
    o = oracle.swin3d_window_attention(q, k, v, WIN, (0, 0, 0), 0.5)
    r = lambda x: np.roll(x, (2, 6, 12), axis=(1, 2, 3))
    o2 = oracle.swin3d_window_attention(r(q), r(k), r(v), WIN, (0, 0, 0), 0.5)
    np.testing.assert_allclose(o2, r(o), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- per-window formulation
@pytest.mark.parametrize("bias", [-100.0, NEG_INF])
@pytest.mark.parametrize("grid,shift", [((2, 12, 24), (1, 3, 6)), ((4, 45, 90), (1, 3, 6)),
                                        ((3, 7, 13), (1, 5, 11))])
def test_windows_attention_matches_full(grid, shift, bias):
    B, h, dh = 2, 2, 4
    shape = (B,) + grid + (h, dh)
    q, k, v = _qkv(shape, 161)
    o = oracle.swin3d_window_attention(q, k, v, WIN, shift, 0.5, bias)
    arrays = {"q": q, "k": k, "v": v}
    nwin = [oracle.padded_extent(x, w) // w for x, w in zip(grid, WIN)]
    wins = [(b, a, c, e) for b in range(B) for a in range(nwin[0]) for c in range(nwin[1]) for e in range(nwin[2])]
    fetch = lambda t, b, c: arrays[t][b, c[:, 0], c[:, 1], c[:, 2]]
    res = oracle.windows_attention(fetch, B, grid, h, dh, WIN, shift, 0.5, bias, wins)
    seen = 0
    for b, coords, ow in res:
        np.testing.assert_allclose(ow, o[b, coords[:, 0], coords[:, 1], coords[:, 2]], rtol=0, atol=1e-13)
        seen += len(coords)
    assert seen == B * np.prod(grid)


def test_datagen_bf16_is_exact_and_seeded():
    """The generator's bf16 rounding is round-to-nearest-even and the stress multiplier is exact."""
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -2.5, 3.0e-3], dtype=np.float32)
    bits = datagen.f32_to_bf16_bits(x)
    back = datagen.bf16_bits_to_f32(bits)
    # ties go to even mantissa, otherwise to nearest
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0078125)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(back, t)
    wl = datagen.WORKLOADS["stress_hres"]
    a = datagen.slice_f64(wl, "q", 1, 3)[:4, :4]
    b = datagen.slice_f64(wl, "q", 1, 3)[:4, :4]
    assert np.array_equal(a, b)
    raw = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(datagen.slice_f32(wl, "q", 1, 3)[:4, :4]))
    np.testing.assert_array_equal(a, raw.astype(np.float64) * 8)
