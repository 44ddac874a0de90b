"""The C-ABI library on the host: it loads, exports every declared symbol, and
validates arguments. No call here reaches a device."""
import ctypes
import math
import os
import re

import pytest

import datagen
import oracle
import swin3d_window_attention_amd as sw

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "swin3d_wattn.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(swin3d_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = sw.load_library()
    names = _declared_functions()
    assert names == sorted(["swin3d_wattn_create", "swin3d_wattn_run", "swin3d_wattn_run_strided",
                            "swin3d_wattn_destroy", "swin3d_wattn_strerror", "swin3d_wattn_get_info",
                            "swin3d_adaln_residual"])
    for n in names:
        assert hasattr(lib, n), n
        assert hasattr(sw, n), n  # the binding uses the same names


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("SWIN3D_WATTN_OK", "SWIN3D_WATTN_EINVAL", "SWIN3D_WATTN_EUNSUPPORTED", "SWIN3D_WATTN_ELAUNCH"):
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == getattr(sw, name)
    assert ctypes.sizeof(sw.Swin3dWattnDesc) == 4 * 15


def _create(**kw):
    base = dict(B=1, D=4, H=180, W=360, heads=8, head_dim=64, window=(2, 6, 12), shift=(1, 3, 6),
                dtype="bf16", scale=0.125, cross_region_bias=-100.0)
    base.update(kw)
    return sw.swin3d_wattn_create(sw.make_desc(**base))


def test_create_ok_and_info_matches_pages():
    for name, masked in [("stage1", 959), ("stage2", 254), ("stage2_s0", 0), ("stage3_pad", 79),
                         ("tiny_f32", 4), ("stress_hres", 11548)]:
        wl = datagen.WORKLOADS[name]
        rc, h = _create(B=wl.B, D=wl.D, H=wl.H, W=wl.W, heads=wl.heads, head_dim=wl.head_dim,
                        shift=wl.shift, dtype=wl.dtype, scale=wl.scale)
        assert rc == 0 and h
        rc, info = sw.swin3d_wattn_get_info(h)
        assert rc == 0
        assert info.n_windows == oracle.window_count(wl.B, (wl.D, wl.H, wl.W), wl.window)
        assert info.n_masked_windows == masked
        assert info.tokens_per_window == 144
        assert info.tokens == wl.tokens
        assert list(info.padded) == [oracle.padded_extent(x, w) for x, w in zip((wl.D, wl.H, wl.W), wl.window)]
        assert info.workgroups == info.n_windows * wl.heads
        assert sw.swin3d_wattn_destroy(h) == 0


def test_masked_window_count_matches_oracle_labels():
    """The plan's count of windows needing the mask path equals the windows whose
    oracle labels or validity are not uniform."""
    for grid, shift in [((4, 45, 90), (1, 3, 6)), ((3, 7, 13), (1, 5, 11)), ((4, 44, 30), (1, 3, 6)),
                        ((2, 12, 24), (0, 0, 0)), ((4, 18, 36), (0, 3, 0))]:
        rc, h = _create(D=grid[0], H=grid[1], W=grid[2], shift=shift, dtype="f32", head_dim=32)
        assert rc == 0
        _, info = sw.swin3d_wattn_get_info(h)
        padded = tuple(oracle.padded_extent(x, w) for x, w in zip(grid, (2, 6, 12)))
        import numpy as np
        lab = oracle.window_partition(oracle.region_labels(padded, (2, 6, 12), shift)[None], (2, 6, 12))
        val = oracle.window_partition(oracle.cyclic_shift(
            oracle.pad_to_windows(np.ones((1,) + grid, bool), (2, 6, 12), False), shift), (2, 6, 12))
        expected = sum(1 for w in range(lab.shape[0]) if len(np.unique(lab[w])) > 1 or not val[w].all())
        assert info.n_masked_windows == expected, (grid, shift)
        sw.swin3d_wattn_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(D=-1), -1), (dict(heads=0), -1), (dict(head_dim=0), -1),
    (dict(window=(0, 6, 12)), -1), (dict(shift=(2, 3, 6)), -1), (dict(shift=(-1, 0, 0)), -1),
    (dict(shift=(1, 6, 6)), -1), (dict(dtype=7), -1), (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1), (dict(scale=0.0), -1), (dict(scale=-0.1), -1),
    (dict(cross_region_bias=float("nan")), -1), (dict(cross_region_bias=1.0), -1),
    (dict(head_dim=256), -2), (dict(head_dim=16), -2), (dict(head_dim=96), -2), (dict(window=(2, 6, 6)), -1),
    (dict(window=(4, 8, 12), shift=(1, 3, 3), dtype="f32", head_dim=64), -2),
    (dict(dtype="f32", head_dim=48), -2),
    (dict(B=2, D=4, H=46341, W=46341), -2),
    (dict(dtype="f32", head_dim=32, window=(2, 8, 10), shift=(0, 0, 0), D=1, H=1, W=1, heads=65536), -2),
    (dict(dtype="f32", head_dim=64, window=(2, 8, 17), shift=(0, 0, 0)), -2),  # N = 272 > 256
    (dict(D=1, H=1, W=1, heads=65536), -2),
])
def test_create_rejects(kw, code):
    rc, h = _create(**kw)
    assert rc == code and h is None


def test_window_plans():
    """bf16 windows whose K and V fill half the LDS (N x head_dim = 144 x 128 or 288 x 64) go to
    the whole-window kernel (5): one workgroup of four waves per (window, head)."""
    for kw, wg in [(dict(head_dim=128), 1800 * 8),
                   (dict(head_dim=128, heads=4, shift=(0, 0, 0)), 1800 * 4),
                   (dict(window=(2, 12, 12), shift=(1, 6, 6)), 900 * 8),
                   (dict(window=(4, 6, 12), shift=(2, 3, 6), B=2), 2 * 30 * 30 * 8)]:
        rc, h = _create(**kw)
        assert rc == 0, kw
        rc2, info = sw.swin3d_wattn_get_info(h)
        assert (info.kernel, info.workgroups, info.threads_per_workgroup) == (5, wg, 256), (
            kw, info.kernel, info.workgroups, info.threads_per_workgroup)
        sw.swin3d_wattn_destroy(h)
    for kw in (dict(head_dim=128, dtype=0), dict(head_dim=128, dtype=2), dict(window=(2, 12, 12), dtype=0)):
        rc, h = _create(**kw)  # FP32 I/O never takes the bf16 kernels
        assert rc != 0 or sw.swin3d_wattn_get_info(h)[1].kernel != 5, kw
        if rc == 0:
            sw.swin3d_wattn_destroy(h)


def test_streaming_plans():
    """Other bf16 windows, and head_dim 32, go to the K/V-streaming kernel (3): 3 waves and 48-key
    chunks where N is a multiple of 48 but not of 64, else 4 waves and 64; 32 query slots per wave
    (two tiles of 16) at every head_dim."""
    for kw, wg, thr in [(dict(window=(2, 6, 6), shift=(1, 3, 3)), 3600 * 1 * 8, 256),     # N = 72: 1 x 128
                        (dict(window=(3, 12, 12), shift=(1, 6, 6), head_dim=128), 904 * 5 * 8, 192),  # 432: 5 x 96
                        (dict(window=(3, 12, 12), shift=(1, 6, 6)), 904 * 5 * 8, 192),    # N = 432: 5 x 96
                        (dict(window=(4, 12, 24), shift=(2, 6, 12)), 232 * 9 * 8, 256),   # N = 1152 = 9 x 128
                        (dict(window=(1, 7, 7), shift=(0, 3, 3), head_dim=128), 4 * 26 * 52 * 1 * 8, 256),
                        (dict(head_dim=32), 1800 * 2 * 8, 192)]:                          # N = 144: 2 x 96
        rc, h = _create(**kw)
        assert rc == 0, kw
        rc2, info = sw.swin3d_wattn_get_info(h)
        assert (info.kernel, info.workgroups, info.threads_per_workgroup) == (3, wg, thr), (
            kw, info.kernel, info.workgroups, info.threads_per_workgroup)
        sw.swin3d_wattn_destroy(h)
    rc, h = _create()
    assert sw.swin3d_wattn_get_info(h)[1].kernel == 1  # the production shape keeps its own kernel
    sw.swin3d_wattn_destroy(h)


def test_f32_split_plans():
    """FP32 I/O on the matrix cores: head_dim 64 and 144-slot windows only; kernel 2."""
    rc, h = _create(dtype=2)
    assert rc == 0
    rc2, info = sw.swin3d_wattn_get_info(h)
    assert rc2 == 0 and info.kernel == 2 and info.threads_per_workgroup == 256
    sw.swin3d_wattn_destroy(h)
    for kw in (dict(dtype=2, head_dim=32), dict(dtype=2, window=(2, 6, 6), shift=(1, 3, 3)),
               dict(dtype=2, D=1, H=1, W=1, heads=65536)):
        rc, h = _create(**kw)
        assert rc == -2 and h is None, kw
    assert sw.make_desc(1, 2, 6, 12, 1, 64, dtype="f32_split").dtype == sw.SWIN3D_WATTN_F32_SPLIT == 2


def test_create_accepts_edge_cases():
    for kw in [dict(cross_region_bias=-math.inf), dict(shift=(0, 0, 0)), dict(shift=(1, 5, 11)),
               dict(D=1, H=1, W=1), dict(D=1, H=1, W=1, heads=65535), dict(dtype="f32", head_dim=32, window=(1, 1, 1), shift=(0, 0, 0)),
               dict(dtype="f32", head_dim=64, window=(4, 8, 8), shift=(3, 7, 7))]:
        rc, h = _create(**kw)
        assert rc == 0, kw
        sw.swin3d_wattn_destroy(h)


def test_null_arguments():
    lib = sw.load_library()
    assert lib.swin3d_wattn_create(None, None) == -1
    out = ctypes.c_void_p(123)
    assert lib.swin3d_wattn_create(None, ctypes.byref(out)) == -1
    assert out.value is None
    assert sw.swin3d_wattn_destroy(None) == 0
    assert sw.swin3d_wattn_get_info(None)[0] == -1
    assert sw.swin3d_wattn_run(None, 16, 32, 48, 64, 0) == -1


def test_run_rejects_bad_pointers_before_launch():
    """Misaligned, null or overlapping buffers are refused on the host: nothing is launched."""
    rc, h = _create(B=1, D=2, H=6, W=12, heads=1)
    assert rc == 0
    n = 2 * 6 * 12 * 64 * 2
    base = 1 << 40
    q, k, v, o = base, base + 4 * n, base + 8 * n, base + 12 * n
    assert sw.swin3d_wattn_run(h, q + 2, k, v, o, 0) == -1   # misaligned
    assert sw.swin3d_wattn_run(h, q, k, v, o + 8, 0) == -1   # misaligned
    assert sw.swin3d_wattn_run(h, 0, k, v, o, 0) == -1       # null
    assert sw.swin3d_wattn_run(h, q, k, v, q + 16, 0) == -1  # o overlaps q
    assert sw.swin3d_wattn_run(h, q, k, v, v - n + 16, 0) == -1  # o overlaps v
    sw.swin3d_wattn_destroy(h)


def test_run_strided_rejects_before_launch():
    """Strides below heads*head_dim or not a multiple of 16 bytes, null strides and an O span that
    overlaps Q, K or V are refused on the host."""
    rc, h = _create(B=1, D=2, H=6, W=12, heads=2)  # bf16, 144 tokens, 128 elements per token
    assert rc == 0
    tokens, row = 2 * 6 * 12, 2 * 64
    S = sw.Swin3dWattnStrides
    base = 1 << 40
    fused = S(3 * row, 3 * row, 3 * row, row)
    q, k, v = base, base + row * 2, base + 2 * row * 2
    o = base + tokens * 3 * row * 2 + 4096          # just past the fused buffer
    run = lambda qq, kk, vv, oo, st: sw.swin3d_wattn_run_strided(h, qq, kk, vv, oo, st, 0)
    assert run(q, k, v, o, S(row - 8, 3 * row, 3 * row, row)) == -1      # stride below a token
    assert run(q, k, v, o, S(3 * row + 4, 3 * row, 3 * row, row)) == -1  # 8 bytes: not 16-aligned
    assert run(q, k, v, o, S(3 * row, 3 * row, 3 * row, 0)) == -1
    assert run(q, k, v, o, S(3 * row, 1 << 31, 3 * row, row)) == -1     # stride of 2^31 elements
    assert run(q, k, v, o + 8, fused) == -1                              # misaligned pointer
    assert sw.load_library().swin3d_wattn_run_strided(h, q, k, v, o, None, 0) == -1
    span_v = ((tokens - 1) * 3 * row + row) * 2
    assert run(q, k, v, v + span_v - 16, fused) == -1                    # o starts inside v's span
    assert run(q, k, v, q - ((tokens - 1) * row + row) * 2 + 16, fused) == -1  # o ends inside q's span
    assert run(0, k, v, o, fused) == -1
    sw.swin3d_wattn_destroy(h)


def test_run_strided_rejects_oversized_span():
    """A span beyond 2^46 elements is refused before any arithmetic on it could overflow."""
    rc, h = _create(B=1, D=1024, H=1024, W=1020, heads=1, head_dim=64, window=(2, 6, 12), shift=(1, 3, 6))
    assert rc == 0                                          # 2^30 - 4 Mi tokens
    S = sw.Swin3dWattnStrides
    base = 1 << 44
    big = (1 << 31) - 8                                     # allowed stride, span ~2^61 elements
    run = lambda st: sw.swin3d_wattn_run_strided(h, base, base, base, base + (1 << 47), st, 0)
    assert run(S(64, 64, 64, big)) == -1
    assert run(S(big, 64, 64, 64)) == -1
    sw.swin3d_wattn_destroy(h)


def test_f32_plans():
    """F32 I/O: windows of up to 256 slots run on the FP32 matrix-core kernel (4)."""
    for kw, kern, wg in [(dict(dtype="f32", head_dim=64), 4, 1800 * 8), (dict(dtype="f32", head_dim=32), 4, 1800 * 8),
                         (dict(dtype="f32", head_dim=64, window=(2, 4, 4), shift=(1, 2, 2)), 4, 2 * 45 * 90 * 8),
                         (dict(dtype="f32", head_dim=32, window=(1, 1, 1), shift=(0, 0, 0)), 4, 4 * 180 * 360 * 8),
                         (dict(dtype="f32", head_dim=64, window=(2, 8, 9), shift=(1, 4, 4)), 4, 2 * 23 * 40 * 8),
                         (dict(dtype="f32", head_dim=64, window=(2, 8, 10), shift=(1, 4, 5)), 4, 2 * 23 * 36 * 8),
                         (dict(dtype="f32", head_dim=32, window=(4, 8, 8), shift=(2, 4, 4)), 4, 1 * 23 * 45 * 8)]:
        rc, h = _create(**kw)
        assert rc == 0, kw
        info = sw.swin3d_wattn_get_info(h)[1]
        assert info.kernel == kern, (kw, info.kernel)
        if kern == 4:
            assert (info.threads_per_workgroup, info.workgroups) == (256, wg), kw
        sw.swin3d_wattn_destroy(h)


def test_grid_extent_limit():
    """Each grid extent must stay below 2^24 (the kernels' index arithmetic)."""
    rc, h = _create(B=1, D=2, H=6, W=(1 << 24) - 12)
    assert rc == 0
    sw.swin3d_wattn_destroy(h)
    assert _create(B=1, D=2, H=6, W=1 << 24)[0] == -2
    assert _create(B=1, D=2, H=(1 << 24) + 6, W=12)[0] == -2


def test_work_item_limit():
    """A launch counts the work-items of its first grid dimension in 32 bits: plans whose grid
    x extent times threads per workgroup reaches 2^32 are refused at create time (EUNSUPPORTED)
    rather than under-dispatched at run time."""
    # exact FP32, window (1, 1, 1): one window per token, 256 threads each
    ok = dict(dtype="f32", head_dim=32, window=(1, 1, 1), shift=(0, 0, 0), heads=1, B=1, D=1)
    rc, h = _create(H=4096, W=4095, **ok)  # 16,773,120 windows x 256 < 2^32
    assert rc == 0
    assert sw.swin3d_wattn_get_info(h)[1].workgroups == 4096 * 4095
    sw.swin3d_wattn_destroy(h)
    assert _create(H=4096, W=4097, **ok)[0] == -2   # 16,781,312 x 256 >= 2^32
    assert _create(H=4096, W=4096, **ok)[0] == -2   # exactly 2^24 windows: 2^32 work-items
    # bf16 K/V streaming, windows (2, 2, 2) and (1, 2, 2): x extent = windows padded to 8 x 1 query block
    st = dict(head_dim=64, heads=1, B=1, shift=(0, 0, 0))
    assert _create(window=(2, 2, 2), D=2, H=4096, W=8190, **st)[0] == 0       # 8,386,560 x 256 < 2^32
    assert _create(window=(2, 2, 2), D=8, H=8192, W=8192, **st)[0] == -2      # 67M tokens
    assert _create(window=(1, 2, 2), D=1, H=8192, W=16384, **st)[0] == -2     # 134M tokens
    assert _create(window=(1, 2, 2), D=1, H=4096, W=16380, **st)[0] == 0      # 16,773,120 windows / 4 x 256


def test_strerror():
    assert sw.swin3d_wattn_strerror(0) == "success"
    for c in (-1, -2, -3):
        assert sw.swin3d_wattn_strerror(c) and sw.swin3d_wattn_strerror(c) != "success"
    assert "unknown" in sw.swin3d_wattn_strerror(42)


def test_adaln_rejects_before_launch():
    """Bad descriptors, null or misaligned pointers and overlaps are refused on the host."""
    D = sw.Swin3dAdalnDesc
    base = 1 << 40
    n = 2 * 100 * 512
    x, res, out = base, base + 4 * n + 4096, base + 8 * n + 8192   # f32 spans of 4n bytes
    g, b = base + 16 * n, base + 16 * n + 8192
    ok = D(100, 2, 512, 1, 0, 0, 1e-5)
    run = lambda d, *p: sw.swin3d_adaln_residual(d, *p, 0)
    assert run(D(100, 2, 300, 1, 0, 0, 1e-5), x, res, g, b, out) == -2    # C not a multiple of 256
    assert run(D(100, 2, 8192, 1, 0, 0, 1e-5), x, res, g, b, out) == -2   # C above 4096
    assert run(D(100, 2, 512, 1, 0, 0, 0.0), x, res, g, b, out) == -1     # eps
    assert run(D(100, 2, 512, 1, 0, 0, float("nan")), x, res, g, b, out) == -1
    assert run(D(0, 2, 512, 1, 0, 0, 1e-5), x, res, g, b, out) == -1
    assert run(D(100, 2, 512, 2, 0, 0, 1e-5), x, res, g, b, out) == -1    # no split dtype here
    assert run(D(1 << 30, 4, 256, 1, 0, 0, 1e-5), x, res, g, b, out) == -2  # too many rows
    assert run(D(1 << 62, 4, 256, 1, 0, 0, 1e-5), x, res, g, b, out) == -2  # rows * B would overflow
    assert run(ok, 0, res, g, b, out) == -1
    assert run(ok, x + 8, res, g, b, out) == -1                            # misaligned
    assert run(ok, x, res, g, b, x + 16) == -1                             # out overlaps x
    assert run(ok, x, res, g, b, res + 16) == -1                           # partial overlap with res
    assert run(D(100, 2, 512, 1, 0, 1, 1e-5), x, res, g, b, res) == -1     # in place needs the same dtype
    assert run(ok, x, res, g, b, g) == -1                                  # out overlaps gamma
    assert sw.load_library().swin3d_adaln_residual(None, x, res, g, b, out, 0) == -1
