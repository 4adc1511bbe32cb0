"""Shared helpers of the GPU parity tests: run a synthetic case through the HIP
library (via its C ABI binding) and through the CPU oracle, and compare.

Tolerance metric (per tensor): max_i |gpu_i - oracle_i| / max_i |oracle_i|.
Bars: 1e-5 for float32 forward outputs, 1e-4 for float32 gradients, 2e-2 for
bfloat16 activations (float32 accumulation).
"""
from __future__ import annotations

import numpy as np

TOL = {("f32", "fwd"): 1e-5, ("f32", "grad"): 1e-4, ("bf16", "fwd"): 2e-2, ("bf16", "grad"): 2e-2,
       # IEEE half storage: see tol()
       ("f16", "fwd"): None, ("f16", "grad"): None}


def tol(case, kind):
    """The bar for one output of a case.  For IEEE half activations it follows from
    the arithmetic: every value stored in half is rounded once, by at most 2^-11 of
    its magnitude.  The output is rounded once, and the per-level path (planes
    above 64 x 64) also stores each level's synthesised coefficients and carrier
    in the activation dtype: at most 2L + 1 roundings, plus one for float32
    accumulation, each bounded by 2^-11 of the largest value."""
    if case.dtype == "f16":
        return (2 * case.levels + 2) * 2.0 ** -11
    return TOL[(case.dtype, kind)]


def rel_err(g, r) -> float:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    denom = float(np.max(np.abs(r)))
    diff = float(np.max(np.abs(g - r)))
    return diff / denom if denom > 0 else diff


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
    """Return {key: rel_err}; raises AssertionError with every failing key listed."""
    keys = keys or ["y", "dx", "dw0", "db0", "ds0", "dwl", "dsl"]
    errs, bad = {}, []
    for k in keys:
        if k == "db0" and not bias:
            continue
        if k in ("dwl", "dsl") and case.levels == 0:
            continue
        kind = "fwd" if k == "y" else "grad"
        bar = tol(case, kind)
        e = rel_err(got[k], want[k])
        errs[k] = e
        if not (e <= bar):
            bad.append(f"{k}: rel err {e:.3e} > {bar:.1e}")
    assert not bad, f"{case}: " + "; ".join(bad)
    return errs
