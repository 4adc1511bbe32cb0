"""The allocation-free weight-gradient entry point, wtconv_backward_weight_noalloc,
called through the C ABI binding: the same kernels as wtconv_backward_weight, with
the library's static device scratch in place of a caller workspace.  Two calls in a
row on one GPU (the second with a smaller input, so the scratch holds the first
call's values when it starts) must each give exactly the outputs of
wtconv_backward_weight, and meet the oracle's bar."""
import numpy as np
import pytest

import memory_bound_depthwise_amd as wt
from synthetic import Case
from wtc_harness import compare, oracle_all, to_np, torch_act, torch_params

pytestmark = pytest.mark.gpu

GRAD_KEYS = ["dw0", "db0", "ds0", "dwl", "dsl"]


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_noalloc_matches_workspace_entry_point_twice():
    torch = _cuda()
    cases = [Case(16, 8, 56, 56, 5, 3, "bf16", seed=21, name="noalloc_big"),   # plane-resident kernels
             Case(2, 3, 70, 66, 5, 2, "bf16", seed=22, name="noalloc_small")]  # per-level kernels (carriers in scratch)
    assert cases[1].numel < cases[0].numel
    for case in cases:
        print(f"case {case}", flush=True)
        L, C, k = case.levels, case.c, case.k
        x, dy, p = case.x(), case.dy(), case.params()
        tx, tdy, tp = torch_act(x, case.dtype), torch_act(dy, case.dtype), torch_params(p)
        desc = wt.make_desc(case.n, C, case.h, case.w, k, L, wt.BF16)
        assert 0 < wt.wtconv_workspace_size(desc, wt.OP_BACKWARD_WEIGHT) <= wt.STATIC_SCRATCH_BYTES
        ref = wt.wtconv_backward_weight(tx, tdy, tp["w0"], tp["b0"], tp["s0"], tp["wl"], tp["sl"], L)
        f32 = torch.float32
        out = {"dw0": torch.full((C, k, k), float("nan"), dtype=f32, device="cuda"),
               "db0": torch.full((C,), float("nan"), dtype=f32, device="cuda"),
               "ds0": torch.full((C,), float("nan"), dtype=f32, device="cuda"),
               "dwl": torch.full((L, C, 4, k, k), float("nan"), dtype=f32, device="cuda"),
               "dsl": torch.full((L, C, 4), float("nan"), dtype=f32, device="cuda")}
        wt.wtconv_backward_weight_noalloc(tx, tdy, tp["w0"], tp["b0"], tp["s0"], tp["wl"], tp["sl"], L, out=out)
        torch.cuda.synchronize()
        for key in GRAD_KEYS:
            assert torch.equal(out[key], ref[key]), (case, key)
        got = {key: to_np(out[key]) for key in GRAD_KEYS}
        want = oracle_all(case, x, dy, p)
        errs = compare(case, got, want, keys=GRAD_KEYS)
        print(f"  ok {errs}", flush=True)
