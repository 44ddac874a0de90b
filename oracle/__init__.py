"""fp64 CPU oracle for Swin3D shifted-window attention and the fused AdaLN +
residual step (test infrastructure only).

Only the tests, the build entry point's smoke check and the benchmark's CPU
baseline may import this package; the GPU library never does.
"""
from .swin3d import (  # noqa: F401
    cyclic_shift,
    cyclic_unshift,
    masked_window_attention,
    pad_to_windows,
    padded_extent,
    region_labels,
    swin3d_window_attention,
    window_count,
    window_merge,
    window_partition,
    window_slot_coords,
    windows_attention,
)
from .adaln import adaln_residual, layer_norm  # noqa: F401
