"""Host-side checks of libwtconv.so that need no GPU: the library loads, exports
every function include/wtconv.h declares, and rejects bad arguments with the
documented status before anything is enqueued.  Calls here never reach a kernel
launch (each has an argument the checks reject)."""
import ctypes
import os
import re

import pytest

import memory_bound_depthwise_amd as wt
from memory_bound_depthwise_amd import wtconv as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wtconv.h")

OK, E_SHAPE, E_KERNEL, E_LEVELS, E_DTYPE, E_NULL, E_WS, E_ALIGN, E_OP, E_HIP, E_SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wtconv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ["wtconv_forward", "wtconv_backward_input", "wtconv_backward_weight",
                     "wtconv_workspace_size", "wtconv_status_string"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = wt.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(binding.EXPORTED)
    assert lib.wtconv_version() == 1


def test_status_strings():
    lib = wt.library()
    for code in [OK, E_SHAPE, E_KERNEL, E_LEVELS, E_DTYPE, E_NULL, E_WS, E_ALIGN, E_OP, E_HIP, E_SCRATCH]:
        s = lib.wtconv_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.wtconv_status_string(12345).decode() == "unknown status"


def _ws(desc, op):
    out = ctypes.c_size_t(123)
    rc = wt.library().wtconv_workspace_size(ctypes.byref(desc) if desc is not None else None, op,
                                            ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("fields,code", [
    ((1, 8, 16, 16, 4, 2, 0), E_KERNEL), ((1, 8, 16, 16, 9, 2, 0), E_KERNEL),
    ((1, 8, 16, 16, 5, -1, 0), E_LEVELS), ((1, 8, 16, 16, 5, 9, 0), E_LEVELS),
    ((1, 8, 16, 16, 5, 2, 3), E_DTYPE), ((-1, 8, 16, 16, 5, 2, 0), E_SHAPE),
    ((1, 8, -16, 16, 5, 2, 0), E_SHAPE), ((1, 8, 65536, 65536, 5, 2, 0), E_SHAPE),
])
def test_desc_validation(fields, code):
    d = wt.make_desc(*fields)
    assert _ws(d, 0)[0] == code
    d = wt.make_desc(1, 8, 16, 16, 5, 2, 0)
    d.reserved = 1
    assert _ws(d, 0)[0] == E_SHAPE


def test_workspace_query_errors():
    d = wt.make_desc(1, 8, 16, 16, 5, 2, 0)
    assert _ws(None, 0)[0] == E_NULL
    assert _ws(d, 3)[0] == E_OP
    assert wt.library().wtconv_workspace_size(ctypes.byref(d), 0, None) == E_NULL


def test_workspace_sizes():
    # planes up to 64 x 64 stay in LDS: the forward-shaped passes need no workspace
    for dt in (wt.F32, wt.BF16, wt.F16):
        d = wt.make_desc(2, 3, 37, 45, 5, 3, dt)
        assert wt.wtconv_workspace_size(d, wt.OP_FORWARD) == 0
        assert wt.wtconv_workspace_size(d, wt.OP_BACKWARD_INPUT) == 0
    # larger planes, per-level path: Q(l) (4 values per coefficient block) for every
    # level + carriers for l < L; in bfloat16 with k <= 5 the tiled matrix-core kernel
    # takes level 1 and its Q(1) is not stored
    n, c, h, w, L = 2, 3, 137, 45, 3
    for dt, es, k, l0 in [(wt.F32, 4, 5, 1), (wt.BF16, 2, 5, 2), (wt.BF16, 2, 7, 1), (wt.F16, 2, 5, 1)]:
        d = wt.make_desc(n, c, h, w, k, L, dt)
        hs, ws = [h], [w]
        for _ in range(L):
            hs.append((hs[-1] + 1) // 2)
            ws.append((ws[-1] + 1) // 2)
        align = lambda v: (v + 255) // 256 * 256
        want = sum(align(n * c * 4 * hs[l] * ws[l] * es) for l in range(l0, L + 1))
        want += sum(align(n * c * hs[l] * ws[l] * es) for l in range(1, L))
        assert wt.wtconv_workspace_size(d, wt.OP_FORWARD) == want
        assert wt.wtconv_workspace_size(d, wt.OP_BACKWARD_INPUT) == want
        assert wt.wtconv_workspace_size(d, wt.OP_BACKWARD_WEIGHT) > 0
    # levels = 0 forward needs none; empty tensors need none
    assert wt.wtconv_workspace_size(wt.make_desc(2, 3, 16, 16, 5, 0, 0), 0) == 0
    for shape in [(0, 3, 8, 8), (2, 3, 0, 8), (2, 0, 8, 8)]:
        d = wt.make_desc(*shape, 5, 2, 1)
        assert wt.wtconv_workspace_size(d, 0) == 0
        assert wt.wtconv_workspace_size(d, 2) == 0


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# The argument-error tests pass placeholder addresses that are never
# dereferenced because an earlier check fails; they stay off GPU machines.
needs_no_gpu = pytest.mark.skipif(_gpu_present(), reason="placeholder pointers are for GPU-less hosts only")

P = ctypes.c_void_p(0x10000)        # aligned placeholder, never dereferenced
P_ODD = ctypes.c_void_p(0x10001)    # misaligned placeholder


@needs_no_gpu
def test_forward_argument_errors():
    lib = wt.library()
    d = wt.make_desc(2, 3, 16, 16, 5, 2, 0)
    f = lambda desc, x=P, w0=P, b0=P, s0=P, wl=P, sl=P, y=P, ws=P, wsb=0: lib.wtconv_forward(
        ctypes.byref(desc) if desc is not None else None, x, w0, b0, s0, wl, sl, y, ws, wsb, None)
    assert f(None) == E_NULL
    assert f(d, x=None) == E_NULL
    assert f(d, y=None) == E_NULL
    assert f(d, w0=None) == E_NULL
    assert f(d, s0=None) == E_NULL
    assert f(d, wl=None) == E_NULL
    assert f(d, sl=None) == E_NULL
    assert f(d, x=P_ODD) == E_ALIGN
    assert f(d, y=P_ODD) == E_ALIGN
    assert f(d, w0=P_ODD) == E_ALIGN
    # planes up to 64 x 64 need no workspace; a larger plane's too-small one is refused
    big = wt.make_desc(2, 3, 130, 70, 5, 2, 0)
    assert f(big, ws=P, wsb=10) == E_WS
    assert f(big, ws=None, wsb=1 << 30) == E_WS
    bad = wt.make_desc(2, 3, 16, 16, 6, 2, 0)
    assert f(bad) == E_KERNEL
    # empty tensors: nothing to do, success without touching any pointer
    assert f(wt.make_desc(0, 3, 16, 16, 5, 2, 0), x=None, y=None, ws=None) == OK
    # backward_input shares the checks
    g = lambda desc, **kw: lib.wtconv_backward_input(ctypes.byref(desc), kw.get("dy", P), P, P, P, P,
                                                     kw.get("dx", P), kw.get("ws", P), kw.get("wsb", 0), None)
    assert g(d, dy=None) == E_NULL
    assert g(d, dx=P_ODD) == E_ALIGN
    assert g(big, wsb=1) == E_WS


@needs_no_gpu
def test_backward_weight_argument_errors():
    lib = wt.library()
    d = wt.make_desc(2, 3, 16, 16, 5, 2, 1)

    def f(desc, **kw):
        a = dict(x=P, dy=P, w0=P, b0=P, s0=P, wl=P, sl=P, dw0=P, db0=P, ds0=P, dwl=P, dsl=P, ws=P, wsb=0)
        a.update(kw)
        return lib.wtconv_backward_weight(ctypes.byref(desc), a["x"], a["dy"], a["w0"], a["b0"], a["s0"],
                                          a["wl"], a["sl"], a["dw0"], a["db0"], a["ds0"], a["dwl"], a["dsl"],
                                          a["ws"], a["wsb"], None)
    for key in ["x", "dy", "w0", "s0", "wl", "sl", "dw0", "ds0", "dwl", "dsl"]:
        assert f(d, **{key: None}) == E_NULL, key
    for key in ["dy", "dw0", "ds0", "dwl"]:
        assert f(d, **{key: P_ODD}) == E_ALIGN, key
    assert f(d) == E_WS
    assert f(d, ws=P, wsb=16) == E_WS


def test_launch_plan_query():
    # host-only query: the kernels each operation enqueues for a shape
    plan = lambda d, op: [e["name"] for e in wt.wtconv_plan_launches(d, op)]
    d = wt.make_desc(64, 96, 56, 56, 5, 3, wt.BF16)       # plane-resident path, bfloat16 on the matrix cores
    assert plan(d, wt.OP_FORWARD) == ["mma_fwd<5,bf16>"]
    assert plan(d, wt.OP_BACKWARD_INPUT) == ["mma_fwd<5,bf16>"]
    # weight gradients: base and level 1 by the correlation kernel, levels 2..L by the level kernel
    assert plan(d, wt.OP_BACKWARD_WEIGHT) == ["plane_dwc<5,bf16>", "plane_dwd<5,bf16>", "dw_finalize<5,bf16>"]
    d = wt.make_desc(64, 96, 56, 56, 5, 3, wt.F16)        # ... on the vector units for the other dtypes
    assert plan(d, wt.OP_FORWARD) == ["plane_fwd<5,f16>"]
    assert plan(d, wt.OP_BACKWARD_WEIGHT) == ["plane_dwl<5,f16>", "plane_dwb<5,f16>", "dw_finalize<5,f16>"]
    d = wt.make_desc(64, 384, 14, 14, 5, 1, wt.BF16)      # narrow planes side by side on the matrix cores
    assert plan(d, wt.OP_FORWARD) == ["mma_fwd<5,bf16>"]
    d = wt.make_desc(64, 384, 5, 14, 5, 1, wt.BF16)       # ... but under 4 cell rows on the vector units
    assert plan(d, wt.OP_FORWARD) == ["plane_fwd<5,bf16>"]
    d = wt.make_desc(64, 96, 56, 56, 7, 0, wt.BF16)       # levels = 0: the same kernel, base only
    assert plan(d, wt.OP_FORWARD) == ["plane_fwd<7,bf16>"]
    assert plan(d, wt.OP_BACKWARD_WEIGHT) == ["plane_dwc<7,bf16>", "dw_finalize<7,bf16>"]
    d = wt.make_desc(2, 4, 256, 256, 3, 2, wt.F32)         # per-level path (plane past 64x64)
    assert plan(d, wt.OP_FORWARD) == ["level_fwd<3,f32>#1", "level_fwd<3,f32>#2", "synth<3,f32>"]
    assert plan(d, wt.OP_BACKWARD_WEIGHT) == ["dw_level<3,f32>#1", "dw_level<3,f32>#2", "dw_base<3,f32>",
                                              "dw_finalize<3,f32>"]
    for e in wt.wtconv_plan_launches(d, wt.OP_FORWARD):
        assert e["workgroups"] > 0 and e["threads"] == 256 and 0 < e["lds_bytes"] <= 64 * 1024
    # empty input: nothing to launch forward; the weight gradient still writes zeros
    d = wt.make_desc(0, 4, 16, 16, 5, 2, wt.F32)
    assert plan(d, wt.OP_FORWARD) == []
    assert plan(d, wt.OP_BACKWARD_WEIGHT) == ["dw_finalize<5,f32>"]
    n = ctypes.c_int(-1)
    assert wt.library().wtconv_plan_launches(ctypes.byref(d), 7, None, 0, ctypes.byref(n)) == E_OP
    assert wt.library().wtconv_plan_launches(ctypes.byref(d), 0, None, 0, None) == E_NULL


@needs_no_gpu
def test_noalloc_refuses_shapes_beyond_the_static_scratch():
    """The allocation-free weight gradient checks its arguments like the workspace
    variant and refuses a shape whose workspace exceeds the static scratch before
    anything is enqueued (or the scratch address is looked up)."""
    lib = wt.library()
    f = lambda desc, **kw: lib.wtconv_backward_weight_noalloc(
        ctypes.byref(desc), kw.get("x", P), kw.get("dy", P), P, P, P, P, P, P, P, P, P, P, None)
    big = wt.make_desc(8, 128, 256, 256, 5, 3, wt.BF16)  # per-level kernels: carriers of x and dy
    assert wt.wtconv_workspace_size(big, wt.OP_BACKWARD_WEIGHT) > wt.STATIC_SCRATCH_BYTES
    assert f(big) == E_SCRATCH
    small = wt.make_desc(2, 3, 16, 16, 5, 2, wt.BF16)
    assert f(small, x=None) == E_NULL
    assert f(small, dy=P_ODD) == E_ALIGN
    d = wt.make_desc(2, 3, 16, 16, 5, 9, wt.BF16)
    assert f(d) == E_LEVELS
    # every workload of the layer study fits
    from synthetic import baseline_cases
    code = {"f32": wt.F32, "bf16": wt.BF16, "f16": wt.F16}
    for c in baseline_cases().values():
        if c.h <= 64 and c.w <= 64:
            d = wt.make_desc(c.n, c.c, c.h, c.w, c.k, c.levels, code[c.dtype])
            assert wt.wtconv_workspace_size(d, wt.OP_BACKWARD_WEIGHT) <= wt.STATIC_SCRATCH_BYTES, c
