"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every output element is compared, on small shapes and at the full workload sizes
(run exactly as the benchmark launches them).  The small shapes span several
tiles, ragged tails, odd sizes (pad-to-even), 1x1 planes, levels 0..5, k in
{3, 5, 7}, every compiled variant of the plane-resident kernels and both kernel
families (plane-resident and per-level); tests/test_plan_coverage.py checks that
list against what the library can launch.

Each comparison reports the normwise error (the stated bar) and the elementwise
error, and holds every element to the bound the arithmetic of its path allows
(tests/wtc_harness.py).  With WTC_PARITY_LOG set, the achieved errors are
appended to that file as JSON lines.
"""
import numpy as np
import pytest

from gpu_cases import SMALL, full_cases, small_cases, variant_shapes
from synthetic import Case, baseline_cases
from wtc_harness import TOL, compare, gpu_all, oracle_all, record, to_np, torch_act, torch_params

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _log(msg):
    print(msg, flush=True)


def _fmt(errs):
    return {k: f"norm {v['norm']:.2e} elem {v['elem']:.2e} bound {v['bound']:.2f}" for k, v in errs.items()}


_SMALL = small_cases()


@pytest.mark.parametrize("case", _SMALL, ids=[f"{c.n}x{c.c}x{c.h}x{c.w}-k{c.k}-L{c.levels}-{c.dtype}" for c in _SMALL])
def test_small_shapes_elementwise(case):
    _cuda()
    _log(f"case {case}")
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p)
    want = oracle_all(case, x, dy, p)
    errs = compare(case, got, want)
    record(case, errs)
    _log(f"  errs {_fmt(errs)}")


def test_no_bias_pointer():
    _cuda()
    case = Case(2, 3, 12, 10, 5, 2, "f32", seed=3, name="nobias")
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p, bias=False)
    want = oracle_all(case, x, dy, p, bias=False)
    compare(case, got, want, bias=False)
    assert got["db0"] is None


_FULL = full_cases()


@pytest.mark.parametrize("case", _FULL, ids=[c.name for c in _FULL])
def test_full_size(case):
    """The full workload shapes, every element of every output against the oracle."""
    _cuda()
    _log(f"full-size case {case}")
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p)
    want = oracle_all(case, x, dy, p)
    errs = compare(case, got, want)
    record(case, errs)
    if case.name == "tiny":
        assert errs["y"]["norm"] <= TOL[("f32", "fwd")]
    _log(f"  ok {case.name}: {_fmt(errs)}")


def test_backward_weight_bitwise_deterministic():
    torch = _cuda()
    from memory_bound_depthwise_amd import wtconv_backward_weight
    case = Case(16, 8, 56, 56, 5, 3, "bf16", seed=11, name="det")
    tx, tdy = torch_act(case.x(), "bf16"), torch_act(case.dy(), "bf16")
    tp = torch_params(case.params())
    runs = []
    for _ in range(3):
        g = wtconv_backward_weight(tx, tdy, tp["w0"], tp["b0"], tp["s0"], tp["wl"], tp["sl"], 3)
        torch.cuda.synchronize()
        runs.append({k: v.clone() for k, v in g.items()})
    for r in runs[1:]:
        for k in r:
            assert torch.equal(r[k], runs[0][k]), k


def test_adjoint_on_gpu():
    """<M v, g> = <v, M^T g> for the GPU forward and input-gradient paths (bias 0)."""
    torch = _cuda()
    from memory_bound_depthwise_amd import wtconv_backward_input, wtconv_forward
    case = Case(4, 6, 45, 38, 5, 4, "f32", seed=5, b_std=0.0, name="adj")
    v, g = case.x(), case.dy()
    tp = torch_params(case.params())
    mv = wtconv_forward(torch_act(v, "f32"), tp["w0"], None, tp["s0"], tp["wl"], tp["sl"], 4)
    mtg = wtconv_backward_input(torch_act(g, "f32"), tp["w0"], tp["s0"], tp["wl"], tp["sl"], 4)
    lhs = float(np.sum(to_np(mv) * g))
    rhs = float(np.sum(v * to_np(mtg)))
    assert abs(lhs - rhs) <= 1e-5 * max(1.0, abs(lhs)), (lhs, rhs)
    del torch


def test_empty_inputs_on_gpu():
    torch = _cuda()
    from memory_bound_depthwise_amd import wtconv_backward_weight, wtconv_forward
    C, k, L = 3, 5, 2
    p = torch_params(Case(1, C, 1, 1, k, L, "f32", name="e").params())
    for shape in [(0, C, 8, 8), (2, C, 0, 8), (2, C, 8, 0)]:
        x = torch.zeros(shape, device="cuda")
        y = wtconv_forward(x, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L)
        assert y.shape == x.shape
        out = {"dw0": torch.full((C, k, k), float("nan"), device="cuda"),
               "db0": torch.full((C,), float("nan"), device="cuda"),
               "ds0": torch.full((C,), float("nan"), device="cuda"),
               "dwl": torch.full((L, C, 4, k, k), float("nan"), device="cuda"),
               "dsl": torch.full((L, C, 4), float("nan"), device="cuda")}
        g = wtconv_backward_weight(x, x, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=out)
        torch.cuda.synchronize()
        for key, t in g.items():
            assert torch.count_nonzero(t).item() == 0, (shape, key)


def test_bf16_output_rounding_is_rne():
    """levels = 0, identity kernel, unit scale, zero bias: y = x exactly, and with
    scale 1 + 2^-9 the bf16 result must be the round-to-nearest-even of x*s."""
    torch = _cuda()
    from memory_bound_depthwise_amd import wtconv_forward
    from synthetic import to_bf16_bits
    C, k = 2, 5
    x = Case(2, C, 16, 16, k, 0, "bf16", seed=9, name="rne").x()
    w0 = np.zeros((C, k, k), np.float32)
    w0[:, 2, 2] = 1.0
    s = np.float32(1.0 + 2.0 ** -9)
    p = {"w0": w0, "b0": np.zeros(C, np.float32), "s0": np.full(C, s, np.float32),
         "wl": np.zeros((1, C, 4, k, k), np.float32), "sl": np.zeros((1, C, 4), np.float32)}
    tp = torch_params(p)
    y = wtconv_forward(torch_act(x, "bf16"), tp["w0"], tp["b0"], tp["s0"], None, None, 0)
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    want = to_bf16_bits((x.astype(np.float32) * s).astype(np.float32))
    np.testing.assert_array_equal(got, want)


def test_f16_output_rounding_is_rne():
    """IEEE half activations, levels = 0, identity kernel, zero bias: with scale
    1 + 3 * 2^-12 (x*s is exact in float32 and lies 0.75 to 1.5 half-ulps above x,
    ties included) the half result must be the round-to-nearest-even of x*s
    (numpy's float32 -> float16 conversion rounds the same way)."""
    torch = _cuda()
    from memory_bound_depthwise_amd import wtconv_forward
    C, k = 2, 5
    x = Case(2, C, 16, 16, k, 0, "f16", seed=9, name="rne16").x()
    w0 = np.zeros((C, k, k), np.float32)
    w0[:, 2, 2] = 1.0
    s = np.float32(1.0 + 3.0 * 2.0 ** -12)
    p = {"w0": w0, "b0": np.zeros(C, np.float32), "s0": np.full(C, s, np.float32),
         "wl": np.zeros((1, C, 4, k, k), np.float32), "sl": np.zeros((1, C, 4), np.float32)}
    tp = torch_params(p)
    y = wtconv_forward(torch_act(x, "f16"), tp["w0"], tp["b0"], tp["s0"], None, None, 0)
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    want = (x.astype(np.float32) * s).astype(np.float32).astype(np.float16).view(np.uint16)
    assert not np.array_equal(want, x.astype(np.float16).view(np.uint16))  # the scale does round
    np.testing.assert_array_equal(got, want)


def test_small_list_is_the_shared_one():
    """The parametrised small cases are the ones the coverage test checks."""
    assert len(_SMALL) == 3 * (len(SMALL) + len(variant_shapes()))
    assert set(c.name for c in _FULL) <= set(baseline_cases())
