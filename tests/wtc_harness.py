"""Shared helpers of the GPU parity tests: run a synthetic case through the HIP
library (via its C ABI binding) and through the CPU oracle, and compare.

Two measures per output tensor (g: GPU, r: oracle):
  normwise    max_i |g_i - r_i| / max_i |r_i|
  elementwise max_i |g_i - r_i| / |r_i| over the elements with |r_i| >= 1e-3 max|r|
The normwise error is held to the stated bars: 1e-5 for float32 forward outputs,
1e-4 for float32 gradients, 2e-2 for bfloat16 activations (float32 accumulation);
IEEE half activations take the bar derived in `tol`.

On top of that every element is held to a bound derived from the arithmetic of
the path that ran (`elem_bound`), which is far tighter than the 2e-2 bar for
16-bit activations: an error confined to a few elements (a plane border, one
plane of a stacked pass) shows up there even when it is small next to max|r|.
"""
from __future__ import annotations

import json
import os

import numpy as np

TOL = {("f32", "fwd"): 1e-5, ("f32", "grad"): 1e-4, ("bf16", "fwd"): 2e-2, ("bf16", "grad"): 2e-2,
       # IEEE half storage: see tol()
       ("f16", "fwd"): None, ("f16", "grad"): None}

# unit roundoff of the activation storage (half an ulp relative to the value at
# the bottom of a binade): bfloat16 keeps 8 significant bits, IEEE half 11
UNIT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}

ACT_KEYS = ("y", "dx")   # outputs stored in the activation dtype
FLOOR = 1e-3             # elementwise measure: |r_i| >= FLOOR * max|r|


def tol(case, kind):
    """The normwise bar for one output of a case.  For IEEE half activations it
    follows from the arithmetic: every value stored in half is rounded once, by at
    most 2^-11 of its magnitude.  The output is rounded once, and the per-level
    path (planes whose pyramid does not fit in LDS) also stores each level's
    synthesised coefficients and carrier in the activation dtype: at most 2L + 1
    roundings, plus one for float32 accumulation, each bounded by 2^-11 of the
    largest value."""
    if case.dtype == "f16":
        return (2 * case.levels + 2) * 2.0 ** -11
    return TOL[(case.dtype, kind)]


def plan_names(case):
    """Kernel names the library runs for a case, per operation (host only)."""
    import memory_bound_depthwise_amd as wt
    code = {"f32": wt.F32, "bf16": wt.BF16, "f16": wt.F16}[case.dtype]
    desc = wt.make_desc(case.n, case.c, case.h, case.w, case.k, case.levels, code)
    return {op: [e["name"] for e in wt.wtconv_plan_launches(desc, op)]
            for op in (wt.OP_FORWARD, wt.OP_BACKWARD_INPUT, wt.OP_BACKWARD_WEIGHT)}


def path_of(case):
    """(forward path, weight-gradient path): 'plane' when the plane-resident
    kernels run (every intermediate stays on chip in float32; the matrix-core
    forward kernel multiplies the bfloat16 pixels by weights split into two
    bfloat16 halves, ~16 significant bits, with float32 accumulation), 'level' when the
    per-level kernels run (coefficients and carriers pass through the workspace in
    the activation dtype)."""
    import memory_bound_depthwise_amd as wt
    names = plan_names(case)
    fwd = "plane" if any(n.startswith(("plane_fwd", "mma_fwd")) for n in names[wt.OP_FORWARD]) else "level"
    # weight gradients: the per-level kernels (dw_level, dw_base, and the tiled
    # correlation kernel of a level l >= 2, 'dwc_tile...#l', which reads the level-(l-1)
    # carriers) pass carriers through the workspace; the plane-resident ones
    # (plane_dwb, plane_dwl, and for bfloat16 the correlation kernel plane_dwc, whose
    # products of bfloat16 values are exact, beside plane_dwd for levels 2..L) keep
    # everything in float32
    dw = names[wt.OP_BACKWARD_WEIGHT]
    dwp = "level" if any(n.startswith(("dw_level", "dw_base")) or (n.startswith("dwc_tile") and "#" in n)
                         for n in dw) else "plane"
    return fwd, dwp


def elem_bound(case, key, path):
    """(a, b) of the per-element bound |g_i - r_i| <= a |r_i| + b max|r|.

    Activation outputs (y, dx) are rounded once to the activation dtype: a = u,
    the dtype's unit roundoff.  Float32 accumulation of a few hundred products of
    bounded terms adds far less than u max|r| for 16-bit activations; for float32
    activations b is the float32 bar itself.  The per-level path stores 2L
    intermediates (coefficients and carriers) in the activation dtype, each
    rounded by at most u of its magnitude, bounded by max|r| for these inputs:
    b = (2L + 1) u.  The plane-resident path keeps them in float32: b = u.
    Parameter gradients are float32 sums over float32 products of inputs that
    are exact in the activation dtype: on the plane path they are as accurate as
    float32 gradients (b = 1e-4); on the per-level path the level carriers are
    rounded to the activation dtype, b = 2L u."""
    u = UNIT[case.dtype]
    L = case.levels
    if key in ACT_KEYS:
        if case.dtype == "f32":
            return 0.0, TOL[("f32", "fwd" if key == "y" else "grad")]
        return u, (u if path == "plane" else (2 * L + 1) * u)
    if case.dtype == "f32" or path == "plane":
        return 0.0, TOL[("f32", "grad")]
    return 0.0, max(2 * L * u, TOL[("f32", "grad")])


def rel_err(g, r) -> float:
    """Normwise relative error max|g - r| / max|r|."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    denom = float(np.max(np.abs(r)))
    diff = float(np.max(np.abs(g - r)))
    return diff / denom if denom > 0 else diff


def elem_err(g, r, floor=FLOOR) -> float:
    """Elementwise relative error over the elements with |r_i| >= floor max|r|."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.size == 0:
        return 0.0
    ar = np.abs(r)
    m = float(ar.max())
    if m == 0:
        return float(np.max(np.abs(g)))
    sel = ar >= floor * m
    return float(np.max(np.abs(g[sel] - r[sel]) / ar[sel]))


def bound_ratio(g, r, a, b) -> float:
    """max_i |g_i - r_i| / (a |r_i| + b max|r|): at most 1 when the bound holds."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.size == 0:
        return 0.0
    ar = np.abs(r)
    den = a * ar + b * max(float(ar.max()), 1e-300)
    return float(np.max(np.abs(g - r) / den))


def torch_act(a, dtype, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    return t.to(device)


def torch_params(p, device="cuda", bias=True):
    import torch
    out = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device) for k, v in p.items()}
    if not bias:
        out["b0"] = None
    return out


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def gpu_all(case, x, dy, p, bias=True):
    """Forward, input gradient and parameter gradients on the GPU; numpy float64."""
    import torch
    from memory_bound_depthwise_amd import wtconv_backward_input, wtconv_backward_weight, wtconv_forward
    L = case.levels
    tx, tdy = torch_act(x, case.dtype), torch_act(dy, case.dtype)
    tp = torch_params(p, bias=bias)
    y = wtconv_forward(tx, tp["w0"], tp["b0"], tp["s0"], tp["wl"], tp["sl"], L)
    dx = wtconv_backward_input(tdy, tp["w0"], tp["s0"], tp["wl"], tp["sl"], L)
    g = wtconv_backward_weight(tx, tdy, tp["w0"], tp["b0"], tp["s0"], tp["wl"], tp["sl"], L)
    torch.cuda.synchronize()
    out = {"y": to_np(y), "dx": to_np(dx)}
    del y, dx, tx, tdy
    for k, v in g.items():
        out[k] = None if v is None else to_np(v)
    return out


def oracle_all(case, x, dy, p, bias=True):
    import oracle
    q = {k: v.astype(np.float64) for k, v in p.items()}
    if not bias:
        q["b0"] = None
    y = oracle.forward(x.astype(np.float64), q, case.levels, case.k)
    g = oracle.backward(x.astype(np.float64), dy.astype(np.float64), q, case.levels, case.k)
    return {"y": y, "dx": g["dx"], "dw0": g["dw0"], "db0": g["db0"], "ds0": g["ds0"],
            "dwl": g["dwl"], "dsl": g["dsl"]}


def compare(case, got, want, keys=None, bias=True):
    """Return {key: {"norm", "elem", "bound"}}; raises AssertionError with every
    failing key listed.  "norm" must meet the normwise bar (tol), "bound" (the
    ratio of the per-element bound used) must be at most 1."""
    keys = keys or ["y", "dx", "dw0", "db0", "ds0", "dwl", "dsl"]
    fwd_path, dw_path = path_of(case)
    errs, bad = {}, []
    for k in keys:
        if k == "db0" and not bias:
            continue
        if k in ("dwl", "dsl") and case.levels == 0:
            continue
        kind = "fwd" if k == "y" else "grad"
        bar = tol(case, kind)
        a, b = elem_bound(case, k, fwd_path if k in ACT_KEYS else dw_path)
        e = {"norm": rel_err(got[k], want[k]), "elem": elem_err(got[k], want[k]),
             "bound": bound_ratio(got[k], want[k], a, b)}
        errs[k] = e
        if not (e["norm"] <= bar):
            bad.append(f"{k}: normwise rel err {e['norm']:.3e} > {bar:.1e}")
        if not (e["bound"] <= 1.0):
            bad.append(f"{k}: per-element bound {a:.2e}|r| + {b:.2e}max|r| exceeded {e['bound']:.2f}x")
    assert not bad, f"{case}: " + "; ".join(bad)
    return errs


def record(case, errs, path=None):
    """Append one case's achieved errors (JSON line) to the file named by the
    WTC_PARITY_LOG environment variable, if set."""
    dest = os.environ.get("WTC_PARITY_LOG")
    if not dest:
        return
    fwd_path, dw_path = path_of(case)
    rec = {"case": case.name, "shape": [case.n, case.c, case.h, case.w], "k": case.k, "levels": case.levels,
           "dtype": case.dtype, "paths": [fwd_path, dw_path], "errors": errs}
    with open(dest, "a") as f:
        f.write(json.dumps(rec) + "\n")
