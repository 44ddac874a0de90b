"""Python binding of libswin3d_wattn (Swin3D shifted-window attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the shared library. PyTorch is used for device memory and the
current stream. There is no CPU fallback: if the library is missing, every
call raises.

The C entry points are exposed under their own names
(swin3d_wattn_create / _run / _destroy / _strerror / _get_info) plus a small
convenience layer (Plan, window_attention).
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = [
    "SWIN3D_WATTN_OK", "SWIN3D_WATTN_EINVAL", "SWIN3D_WATTN_EUNSUPPORTED", "SWIN3D_WATTN_ELAUNCH",
    "SWIN3D_WATTN_F32", "SWIN3D_WATTN_BF16", "SWIN3D_WATTN_F32_SPLIT", "Swin3dWattnDesc", "Swin3dWattnInfo",
    "Swin3dWattnStrides", "Swin3dWattnError", "lib_path", "load_library", "swin3d_wattn_create",
    "swin3d_wattn_run", "swin3d_wattn_run_strided", "swin3d_wattn_destroy",
    "swin3d_wattn_strerror", "swin3d_wattn_get_info", "Plan", "window_attention",
    "Swin3dAdalnDesc", "swin3d_adaln_residual", "adaln_residual",
]

SWIN3D_WATTN_OK = 0
SWIN3D_WATTN_EINVAL = -1
SWIN3D_WATTN_EUNSUPPORTED = -2
SWIN3D_WATTN_ELAUNCH = -3
SWIN3D_WATTN_F32 = 0
SWIN3D_WATTN_BF16 = 1
SWIN3D_WATTN_F32_SPLIT = 2

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libswin3d_wattn.so"


class Swin3dWattnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32 * 3), ("shift", ctypes.c_int32 * 3),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("cross_region_bias", ctypes.c_float),
    ]


class Swin3dWattnInfo(ctypes.Structure):
    _fields_ = [
        ("padded", ctypes.c_int32 * 3), ("windows_per_axis", ctypes.c_int32 * 3),
        ("n_windows", ctypes.c_int64), ("n_masked_windows", ctypes.c_int64),
        ("tokens_per_window", ctypes.c_int32), ("tokens", ctypes.c_int64),
        ("workgroups", ctypes.c_int64), ("threads_per_workgroup", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
    ]


class Swin3dWattnStrides(ctypes.Structure):
    """Token strides (elements) of Q, K, V, O: swin3d_wattn_strides_t."""
    _fields_ = [("q", ctypes.c_int64), ("k", ctypes.c_int64), ("v", ctypes.c_int64), ("o", ctypes.c_int64)]


class Swin3dAdalnDesc(ctypes.Structure):
    """swin3d_adaln_desc_t: fused AdaLN + residual over [B, rows, C]."""
    _fields_ = [("rows", ctypes.c_int64), ("B", ctypes.c_int32), ("C", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("res_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("eps", ctypes.c_float)]


class Swin3dWattnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {swin3d_wattn_strerror(code)} ({code})")


_lib = None
_lib_lock = threading.Lock()


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library():
    """Load the in-tree shared library (built by swin3d_window_attention_amd.build)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m swin3d_window_attention_amd.build`")
        lib = ctypes.CDLL(path)
        lib.swin3d_wattn_create.argtypes = [ctypes.POINTER(Swin3dWattnDesc), ctypes.POINTER(ctypes.c_void_p)]
        lib.swin3d_wattn_create.restype = ctypes.c_int
        lib.swin3d_wattn_run.argtypes = [ctypes.c_void_p] * 6
        lib.swin3d_wattn_run.restype = ctypes.c_int
        lib.swin3d_wattn_run_strided.argtypes = [ctypes.c_void_p] * 5 + [ctypes.POINTER(Swin3dWattnStrides),
                                                                         ctypes.c_void_p]
        lib.swin3d_wattn_run_strided.restype = ctypes.c_int
        lib.swin3d_wattn_destroy.argtypes = [ctypes.c_void_p]
        lib.swin3d_wattn_destroy.restype = ctypes.c_int
        lib.swin3d_wattn_strerror.argtypes = [ctypes.c_int]
        lib.swin3d_wattn_strerror.restype = ctypes.c_char_p
        lib.swin3d_wattn_get_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(Swin3dWattnInfo)]
        lib.swin3d_wattn_get_info.restype = ctypes.c_int
        lib.swin3d_adaln_residual.argtypes = [ctypes.POINTER(Swin3dAdalnDesc)] + [ctypes.c_void_p] * 6
        lib.swin3d_adaln_residual.restype = ctypes.c_int
        _lib = lib
        return lib


# ---- the C entry points, same names -------------------------------------

def swin3d_wattn_create(desc: Swin3dWattnDesc):
    """Returns (code, plan handle or None)."""
    h = ctypes.c_void_p()
    rc = load_library().swin3d_wattn_create(ctypes.byref(desc), ctypes.byref(h))
    return rc, (h.value if rc == 0 else None)


def swin3d_wattn_run(plan, q: int, k: int, v: int, o: int, stream: int = 0) -> int:
    return load_library().swin3d_wattn_run(plan, q, k, v, o, stream)


def swin3d_wattn_run_strided(plan, q: int, k: int, v: int, o: int, strides: Swin3dWattnStrides,
                             stream: int = 0) -> int:
    return load_library().swin3d_wattn_run_strided(plan, q, k, v, o, ctypes.byref(strides), stream)


def swin3d_adaln_residual(desc: Swin3dAdalnDesc, x: int, res: int, gamma: int, beta: int, out: int,
                          stream: int = 0) -> int:
    return load_library().swin3d_adaln_residual(ctypes.byref(desc), x, res, gamma, beta, out, stream)


def swin3d_wattn_destroy(plan) -> int:
    return load_library().swin3d_wattn_destroy(plan)


def swin3d_wattn_strerror(code: int) -> str:
    return load_library().swin3d_wattn_strerror(code).decode()


def swin3d_wattn_get_info(plan):
    info = Swin3dWattnInfo()
    rc = load_library().swin3d_wattn_get_info(plan, ctypes.byref(info))
    return rc, info


# ---- convenience layer --------------------------------------------------

def _dtype_code(dtype) -> int:
    """Plan dtype code: "f32" (exact FP32 arithmetic), "bf16", or "f32_split" (FP32 I/O with
    split-bf16 matrix-core products); a torch dtype maps to "f32" or "bf16"."""
    import torch

    if dtype in (torch.float32, "f32", "float32"):
        return SWIN3D_WATTN_F32
    if dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return SWIN3D_WATTN_BF16
    if dtype == "f32_split":
        return SWIN3D_WATTN_F32_SPLIT
    raise ValueError(f"unsupported dtype {dtype}")


def _io_code(code: int) -> int:
    """The tensor dtype code a plan dtype reads and writes."""
    return SWIN3D_WATTN_F32 if code == SWIN3D_WATTN_F32_SPLIT else code


def make_desc(B, D, H, W, heads, head_dim, window=(2, 6, 12), shift=(0, 0, 0), dtype="bf16",
              scale=None, cross_region_bias=-100.0) -> Swin3dWattnDesc:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    d = Swin3dWattnDesc()
    d.B, d.D, d.H, d.W, d.heads, d.head_dim = B, D, H, W, heads, head_dim
    d.window = (ctypes.c_int32 * 3)(*window)
    d.shift = (ctypes.c_int32 * 3)(*shift)
    d.dtype = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    d.scale = scale
    d.cross_region_bias = cross_region_bias
    return d


class Plan:
    """An immutable plan for one problem shape; run() launches on the current stream."""

    def __init__(self, B, D, H, W, heads, head_dim, window=(2, 6, 12), shift=(0, 0, 0), dtype="bf16",
                 scale=None, cross_region_bias=-100.0):
        self.desc = make_desc(B, D, H, W, heads, head_dim, window, shift, dtype, scale, cross_region_bias)
        self.shape = (B, D, H, W, heads, head_dim)
        rc, h = swin3d_wattn_create(self.desc)
        if rc != SWIN3D_WATTN_OK:
            raise Swin3dWattnError(rc, "swin3d_wattn_create")
        self._h = h
        self._lib = load_library()

    @property
    def handle(self):
        return self._h

    def info(self) -> Swin3dWattnInfo:
        rc, info = swin3d_wattn_get_info(self._h)
        if rc != SWIN3D_WATTN_OK:
            raise Swin3dWattnError(rc, "swin3d_wattn_get_info")
        return info

    def _token_stride(self, t) -> int:
        """Elements between consecutive tokens of a [B, D, H, W, heads, head_dim] view whose
        (heads, head_dim) block is contiguous and whose tokens are evenly spaced in row-major
        [B, D, H, W] order (a contiguous tensor, or e.g. q/k/v slices of a fused QKV buffer)."""
        heads, dh = self.shape[4], self.shape[5]
        st = t.stride()
        if (dh > 1 and st[5] != 1) or (heads > 1 and st[4] != dh):
            raise ValueError("the (heads, head_dim) block of each token must be contiguous")
        ts = None
        span = 1
        for axis in (3, 2, 1, 0):
            if t.shape[axis] > 1:
                if ts is None:
                    ts = st[axis] // span if st[axis] % span == 0 else -1
                if ts < 0 or st[axis] != ts * span:
                    raise ValueError("tokens must be evenly spaced in [B, D, H, W] order")
            span *= t.shape[axis]
        return heads * dh if ts is None else ts

    def run(self, q, k, v, o, stream=None) -> None:
        """O = attention(Q, K, V) on `stream` (default: torch's current stream). Q, K, V, O are
        [B, D, H, W, heads, head_dim] device tensors: contiguous, or token-strided views."""
        import torch

        strides = []
        for t in (q, k, v, o):
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise ValueError("q, k, v, o must be device tensors")
            if tuple(t.shape) != self.shape:
                raise ValueError(f"expected shape {self.shape}, got {tuple(t.shape)}")
            if _dtype_code(t.dtype) != _io_code(self.desc.dtype):
                raise ValueError("tensor dtype does not match the plan")
            strides.append(self._token_stride(t))
        if any(t.device != q.device for t in (k, v, o)):
            raise ValueError("q, k, v, o must be on one device")
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            if stream.device != q.device:
                raise ValueError("the stream must belong to the tensors' device")
            stream = stream.cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr())
        row = self.shape[4] * self.shape[5]
        with torch.cuda.device(q.device):  # the launch goes to the current device
            if all(s == row for s in strides):
                rc = self._lib.swin3d_wattn_run(self._h, *ptrs, stream)
                where = "swin3d_wattn_run"
            else:
                rc = self._lib.swin3d_wattn_run_strided(self._h, *ptrs,
                                                        ctypes.byref(Swin3dWattnStrides(*strides)), stream)
                where = "swin3d_wattn_run_strided"
        if rc != SWIN3D_WATTN_OK:
            raise Swin3dWattnError(rc, where)

    def close(self) -> None:
        if getattr(self, "_h", None):
            swin3d_wattn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def window_attention(q, k, v, window=(2, 6, 12), shift=(0, 0, 0), scale=None, cross_region_bias=-100.0,
                     out=None, precision=None):
    """Swin3D shifted-window attention of grid-layout device tensors [B, D, H, W, heads, head_dim].
    precision: None (the tensors' dtype), or "f32_split" for float32 tensors on the matrix cores."""
    import torch

    B, D, H, W, heads, dh = q.shape
    plan = Plan(B, D, H, W, heads, dh, window, shift, precision or q.dtype, scale, cross_region_bias)
    if out is None:
        out = torch.empty_like(q)
    plan.run(q, k, v, out)
    return out


def adaln_residual(x, res, gamma, beta, eps=1e-5, out=None, out_dtype=None, stream=None):
    """out = res + gamma[b] * LayerNorm(x) + beta[b] for device tensors x, res [B, rows, C]
    (bf16 or float32, contiguous) and gamma, beta [B, C] float32. out defaults to a new tensor of
    out_dtype (default: res's dtype); out may be res itself (in-place residual update)."""
    import torch

    if x.dim() != 3 or res.shape != x.shape or gamma.shape != (x.shape[0], x.shape[2]) or beta.shape != gamma.shape:
        raise ValueError("x, res: [B, rows, C]; gamma, beta: [B, C]")
    for t in (x, res, gamma, beta):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise ValueError("gamma and beta must be float32")
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or res.dtype, device=x.device)
    if out.shape != x.shape or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous [B, rows, C] device tensor")
    if any(t.device != x.device for t in (res, gamma, beta, out)):
        raise ValueError("x, res, gamma, beta, out must be on one device")
    d = Swin3dAdalnDesc(x.shape[1], x.shape[0], x.shape[2], _dtype_code(x.dtype), _dtype_code(res.dtype),
                        _dtype_code(out.dtype), eps)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        if stream.device != x.device:
            raise ValueError("the stream must belong to the tensors' device")
        stream = stream.cuda_stream
    with torch.cuda.device(x.device):  # the launch goes to the current device
        rc = swin3d_adaln_residual(d, x.data_ptr(), res.data_ptr(), gamma.data_ptr(), beta.data_ptr(),
                                   out.data_ptr(), stream)
    if rc != SWIN3D_WATTN_OK:
        raise Swin3dWattnError(rc, "swin3d_adaln_residual")
    return out
