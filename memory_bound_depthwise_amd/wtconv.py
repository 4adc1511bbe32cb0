"""Python binding of libwtconv.so (the C ABI in include/wtconv.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  torch supplies device memory and the current stream.  There is no
CPU path: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwtconv.so")

F32, BF16, F16 = 0, 1, 2
OP_FORWARD, OP_BACKWARD_INPUT, OP_BACKWARD_WEIGHT = 0, 1, 2
MAX_LEVELS = 8

EXPORTED = ["wtconv_workspace_size", "wtconv_forward", "wtconv_backward_input",
            "wtconv_backward_weight", "wtconv_status_string", "wtconv_version",
            "wtconv_profile_begin", "wtconv_profile_end", "wtconv_plan_launches",
            "wtconv_backward_weight_noalloc"]


class Desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("c", ctypes.c_int32), ("h", ctypes.c_int32),
                ("w", ctypes.c_int32), ("k", ctypes.c_int32), ("levels", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("count", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("min_ms", ctypes.c_double),
                ("max_ms", ctypes.c_double)]


class Launch(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("workgroups", ctypes.c_int64),
                ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class WTConvError(RuntimeError):
    pass


_lib = None


def library():
    """Load libwtconv.so (built in-tree by memory_bound_depthwise_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise WTConvError(f"{LIB_PATH} is not built; run `python -m memory_bound_depthwise_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, fp, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        dp = ctypes.POINTER(Desc)
        lib.wtconv_workspace_size.argtypes = [dp, i32, ctypes.POINTER(ctypes.c_size_t)]
        lib.wtconv_forward.argtypes = [dp, vp, fp, fp, fp, fp, fp, vp, vp, ctypes.c_size_t, vp]
        lib.wtconv_backward_input.argtypes = [dp, vp, fp, fp, fp, fp, vp, vp, ctypes.c_size_t, vp]
        lib.wtconv_backward_weight.argtypes = [dp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                               vp, ctypes.c_size_t, vp]
        lib.wtconv_backward_weight_noalloc.argtypes = [dp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, vp]
        lib.wtconv_status_string.argtypes = [i32]
        lib.wtconv_status_string.restype = ctypes.c_char_p
        lib.wtconv_version.argtypes = []
        lib.wtconv_profile_begin.argtypes = []
        lib.wtconv_profile_end.argtypes = [ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)]
        lib.wtconv_plan_launches.argtypes = [dp, i32, ctypes.POINTER(Launch), i32, ctypes.POINTER(i32)]
        for name in EXPORTED:
            if name not in ("wtconv_status_string",):
                getattr(lib, name).restype = i32
        _lib = lib
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = library().wtconv_status_string(rc).decode()
        raise WTConvError(f"{what}: {msg} (status {rc})")


def make_desc(n, c, h, w, k, levels, dtype) -> Desc:
    return Desc(int(n), int(c), int(h), int(w), int(k), int(levels), int(dtype), 0)


def wtconv_plan_launches(desc: Desc, op: int):
    """Kernel launches an operation enqueues for this shape: list of dicts with
    name, workgroups, threads, lds_bytes (host only)."""
    arr = (Launch * 32)()
    n = ctypes.c_int(0)
    _check(library().wtconv_plan_launches(ctypes.byref(desc), int(op), arr, 32, ctypes.byref(n)),
           "wtconv_plan_launches")
    return [{"name": arr[i].name.decode(), "workgroups": arr[i].workgroups, "threads": arr[i].threads,
             "lds_bytes": arr[i].lds_bytes, "variant": arr[i].variant} for i in range(min(n.value, 32))]


def wtconv_workspace_size(desc: Desc, op: int) -> int:
    out = ctypes.c_size_t(0)
    _check(library().wtconv_workspace_size(ctypes.byref(desc), int(op), ctypes.byref(out)),
           "wtconv_workspace_size")
    return int(out.value)


# ---------------------------------------------------------------------------
# torch-facing helpers (torch is imported lazily: the C ABI checks above run
# without it)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise WTConvError(f"activation dtype {t.dtype} is not supported (float32, bfloat16 or float16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(t, name, device, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise WTConvError(f"{name} must live on {device}")
    if not t.is_contiguous():
        raise WTConvError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise WTConvError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise WTConvError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    del torch


def _param_checks(device, C, k, levels, w0, b0, s0, wl, sl):
    torch = _torch()
    f32 = torch.float32
    _check_tensor(w0, "w0", device, f32, (C, k, k))
    _check_tensor(b0, "b0", device, f32, (C,))
    _check_tensor(s0, "s0", device, f32, (C,))
    if levels > 0:
        _check_tensor(wl, "wl", device, f32, (levels, C, 4, k, k))
        _check_tensor(sl, "sl", device, f32, (levels, C, 4))


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise WTConvError(f"workspace too small: need {nbytes} bytes")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def wtconv_forward(x, w0, b0, s0, wl, sl, levels: int, out=None, workspace=None):
    """y = WTConv(x).  x: [n, C, H, W] float32 or bfloat16 on the GPU; parameters
    float32: w0 [C,k,k], b0 [C] or None, s0 [C], wl [L,C,4,k,k], sl [L,C,4]."""
    torch = _torch()
    n, C, H, W = x.shape
    k = w0.shape[-1]
    _check_tensor(x, "x", x.device)
    _param_checks(x.device, C, k, levels, w0, b0, s0, wl, sl)
    desc = make_desc(n, C, H, W, k, levels, _dtype_code(x))
    y = torch.empty_like(x) if out is None else out
    _check_tensor(y, "out", x.device, x.dtype, x.shape)
    ws, wsb = _workspace(wtconv_workspace_size(desc, OP_FORWARD), x.device, workspace)
    rc = library().wtconv_forward(ctypes.byref(desc), _ptr(x), _ptr(w0), _ptr(b0), _ptr(s0),
                                  _ptr(wl if levels else None), _ptr(sl if levels else None),
                                  _ptr(y), _ptr(ws), wsb, _stream(x.device))
    _check(rc, "wtconv_forward")
    return y


def wtconv_backward_input(dy, w0, s0, wl, sl, levels: int, out=None, workspace=None):
    """dx = dL/dx for upstream gradient dy (same layout as x)."""
    torch = _torch()
    n, C, H, W = dy.shape
    k = w0.shape[-1]
    _check_tensor(dy, "dy", dy.device)
    _param_checks(dy.device, C, k, levels, w0, None, s0, wl, sl)
    desc = make_desc(n, C, H, W, k, levels, _dtype_code(dy))
    dx = torch.empty_like(dy) if out is None else out
    _check_tensor(dx, "out", dy.device, dy.dtype, dy.shape)
    ws, wsb = _workspace(wtconv_workspace_size(desc, OP_BACKWARD_INPUT), dy.device, workspace)
    rc = library().wtconv_backward_input(ctypes.byref(desc), _ptr(dy), _ptr(w0), _ptr(s0),
                                         _ptr(wl if levels else None), _ptr(sl if levels else None),
                                         _ptr(dx), _ptr(ws), wsb, _stream(dy.device))
    _check(rc, "wtconv_backward_input")
    return dx


def wtconv_backward_weight(x, dy, w0, b0, s0, wl, sl, levels: int, out=None, workspace=None):
    """Parameter gradients (float32): dict with dw0, db0 (None without bias), ds0, dwl, dsl."""
    torch = _torch()
    n, C, H, W = x.shape
    k = w0.shape[-1]
    _check_tensor(x, "x", x.device)
    _check_tensor(dy, "dy", x.device, x.dtype, x.shape)
    _param_checks(x.device, C, k, levels, w0, b0, s0, wl, sl)
    desc = make_desc(n, C, H, W, k, levels, _dtype_code(x))
    dev, f32 = x.device, torch.float32
    if out is None:
        out = {"dw0": torch.empty((C, k, k), dtype=f32, device=dev),
               "db0": torch.empty((C,), dtype=f32, device=dev) if b0 is not None else None,
               "ds0": torch.empty((C,), dtype=f32, device=dev),
               "dwl": torch.empty((levels, C, 4, k, k), dtype=f32, device=dev),
               "dsl": torch.empty((levels, C, 4), dtype=f32, device=dev)}
    ws, wsb = _workspace(wtconv_workspace_size(desc, OP_BACKWARD_WEIGHT), dev, workspace)
    rc = library().wtconv_backward_weight(
        ctypes.byref(desc), _ptr(x), _ptr(dy), _ptr(w0), _ptr(b0), _ptr(s0),
        _ptr(wl if levels else None), _ptr(sl if levels else None),
        _ptr(out["dw0"]), _ptr(out["db0"]), _ptr(out["ds0"]),
        _ptr(out["dwl"] if levels else None), _ptr(out["dsl"] if levels else None),
        _ptr(ws), wsb, _stream(dev))
    _check(rc, "wtconv_backward_weight")
    return out


def wtconv_backward_weight_noalloc(x, dy, w0, b0, s0, wl, sl, levels: int, out):
    """wtconv_backward_weight through the allocation-free entry point (the library's
    static device scratch instead of a workspace).  `out` holds the preallocated
    float32 gradients (keys as wtconv_backward_weight returns); nothing is allocated."""
    n, C, H, W = x.shape
    k = w0.shape[-1]
    _check_tensor(x, "x", x.device)
    _check_tensor(dy, "dy", x.device, x.dtype, x.shape)
    _param_checks(x.device, C, k, levels, w0, b0, s0, wl, sl)
    desc = make_desc(n, C, H, W, k, levels, _dtype_code(x))
    rc = library().wtconv_backward_weight_noalloc(
        ctypes.byref(desc), _ptr(x), _ptr(dy), _ptr(w0), _ptr(b0), _ptr(s0),
        _ptr(wl if levels else None), _ptr(sl if levels else None),
        _ptr(out["dw0"]), _ptr(out["db0"]), _ptr(out["ds0"]),
        _ptr(out["dwl"] if levels else None), _ptr(out["dsl"] if levels else None), _stream(x.device))
    _check(rc, "wtconv_backward_weight_noalloc")
    return out


STATIC_SCRATCH_BYTES = 16 << 20  # WTCONV_STATIC_SCRATCH_BYTES


def profile_begin():
    _check(library().wtconv_profile_begin(), "wtconv_profile_begin")


def profile_end(max_entries: int = 64):
    arr = (KernelTime * max_entries)()
    n = ctypes.c_int(0)
    _check(library().wtconv_profile_end(arr, max_entries, ctypes.byref(n)), "wtconv_profile_end")
    return [{"name": arr[i].name.decode(), "count": arr[i].count, "total_ms": arr[i].total_ms,
             "min_ms": arr[i].min_ms, "max_ms": arr[i].max_ms} for i in range(n.value)]
