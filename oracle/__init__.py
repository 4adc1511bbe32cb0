"""CPU oracle of the WTConv layer (float64, plain unfused definition).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only users.  The GPU library never
imports, loads or calls anything here, and this package imports nothing from it.

The arithmetic lives in ``wtconv_oracle.c`` (built with gcc by ``oracle/build.py``);
this module only marshals numpy arrays into it.  Source of the definition:
"Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation",
§2.1 Algorithm 1, §2.2 Proposition 1 / Eq. 1, §4.1 Eq. 5, Appendix A Eq. 12.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwtconv_oracle.so")

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        i = ctypes.c_int
        lib.wo_forward.argtypes = [i, i, i, i, i, i] + [_dp] * 8
        lib.wo_forward.restype = i
        lib.wo_backward.argtypes = [i, i, i, i, i, i] + [_dp] * 13
        lib.wo_backward.restype = i
        lib.wo_haar_analysis.argtypes = [i, i, _dp, _dp]
        lib.wo_haar_analysis.restype = None
        lib.wo_haar_synthesis.argtypes = [i, i, _dp, _dp]
        lib.wo_haar_synthesis.restype = None
        lib.wo_threads.argtypes = []
        lib.wo_threads.restype = i
        _lib = lib
    return _lib


def use_library(path: str | None) -> None:
    """Point the wrapper at another build of the oracle source (the mutation test
    builds copies with a planted mistake); None returns to the default build."""
    global _lib, LIB_PATH
    _lib = None
    LIB_PATH = path or os.path.join(_HERE, "libwtconv_oracle.so")


def _in(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=np.float64)
    return arr, arr.ctypes.data_as(_dp)


def _out(shape):
    arr = np.zeros(shape, dtype=np.float64)
    return arr, arr.ctypes.data_as(_dp)


def threads() -> int:
    return int(_load().wo_threads())


def level_sizes(h: int, w: int, levels: int):
    hs, ws = [h], [w]
    for _ in range(levels):
        hs.append((hs[-1] + 1) // 2)
        ws.append((ws[-1] + 1) // 2)
    return hs, ws


def haar_analysis(plane: np.ndarray) -> np.ndarray:
    """One Haar level of an h x w plane (zero pad to even); returns [4, ceil(h/2), ceil(w/2)]."""
    h, w = plane.shape
    x, xp = _in(plane)
    out, op = _out((4, (h + 1) // 2, (w + 1) // 2))
    _load().wo_haar_analysis(h, w, xp, op)
    return out


def haar_synthesis(bands: np.ndarray, h: int, w: int) -> np.ndarray:
    """Inverse of haar_analysis, cropped to h x w."""
    assert bands.shape == (4, (h + 1) // 2, (w + 1) // 2)
    b, bp = _in(bands)
    out, op = _out((h, w))
    _load().wo_haar_synthesis(h, w, bp, op)
    return out


def forward(x: np.ndarray, params: dict, levels: int, k: int, return_coeffs: bool = False):
    """y = WTConv(x).  x: [n, C, H, W]; params: w0 [C,k,k], b0 [C] or None, s0 [C],
    wl [L,C,4,k,k], sl [L,C,4].  With return_coeffs, also returns the list of the
    scaled, filtered level coefficients Z^(l), each [n, C, 4, H_l, W_l]."""
    n, C, H, W = x.shape
    L = levels
    xa, xp = _in(x)
    w0, w0p = _in(params["w0"])
    b0, b0p = _in(params.get("b0"))
    s0, s0p = _in(params["s0"])
    wl, wlp = _in(params["wl"] if L > 0 else np.zeros((1,)))
    sl, slp = _in(params["sl"] if L > 0 else np.zeros((1,)))
    y, yp = _out((n, C, H, W))
    hs, ws = level_sizes(H, W, L)
    zp = None
    if return_coeffs:
        total = sum(n * C * 4 * hs[l] * ws[l] for l in range(1, L + 1))
        z, zp = _out((max(total, 1),))
    rc = _load().wo_forward(n, C, H, W, k, L, xp, w0p, b0p, s0p, wlp, slp, yp, zp)
    if rc != 0:
        raise RuntimeError(f"oracle forward failed: {rc}")
    if not return_coeffs:
        return y
    coeffs, off = [], 0
    for l in range(1, L + 1):
        e = n * C * 4 * hs[l] * ws[l]
        coeffs.append(z[off:off + e].reshape(n, C, 4, hs[l], ws[l]))
        off += e
    return y, coeffs


GRADIENTS = ("dx", "dw0", "db0", "ds0", "dwl", "dsl")


def backward(x: np.ndarray, dy: np.ndarray, params: dict, levels: int, k: int, outputs=GRADIENTS) -> dict:
    """Reverse mode of forward.  Returns dx, dw0, db0, ds0, dwl, dsl (float64);
    `outputs` names the ones to compute (the others are passed to the C code as
    NULL, which skips them, and come back as None)."""
    n, C, H, W = x.shape
    L = levels
    xa, xp = _in(x)
    g, gp = _in(dy)
    w0, w0p = _in(params["w0"])
    b0, b0p = _in(params.get("b0"))
    s0, s0p = _in(params["s0"])
    wl, wlp = _in(params["wl"] if L > 0 else np.zeros((1,)))
    sl, slp = _in(params["sl"] if L > 0 else np.zeros((1,)))
    dx, dxp = _out((n, C, H, W))
    dw0, dw0p = _out((C, k, k))
    db0, db0p = _out((C,))
    ds0, ds0p = _out((C,))
    dwl, dwlp = _out((max(L, 1), C, 4, k, k))
    dsl, dslp = _out((max(L, 1), C, 4))
    want = set(outputs)
    ptrs = {"dx": dxp, "dw0": dw0p, "db0": db0p, "ds0": ds0p, "dwl": dwlp, "dsl": dslp}
    args = [ptrs[name] if name in want else None for name in GRADIENTS]
    rc = _load().wo_backward(n, C, H, W, k, L, xp, gp, w0p, b0p, s0p, wlp, slp, *args)
    if rc != 0:
        raise RuntimeError(f"oracle backward failed: {rc}")
    res = {"dx": dx, "dw0": dw0, "db0": db0, "ds0": ds0, "dwl": dwl[:L], "dsl": dsl[:L]}
    return {name: (res[name] if name in want else None) for name in GRADIENTS}
