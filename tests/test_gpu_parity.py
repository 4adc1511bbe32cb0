"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small shapes are compared element by element on every output; they span several
tiles, ragged tails, odd sizes (pad-to-even), 1x1 planes, levels 0..5 and k in
{3, 5, 7}.  The full workload shapes run exactly as the benchmark launches them,
and are compared on sampled (n, c) planes (forward, input gradient: a plane of the
output depends only on the same plane of the input) and sampled channels (weight
gradients: a channel's gradient depends only on that channel of x and dy).
"""
import numpy as np
import pytest

from synthetic import Case, baseline_cases
from wtc_harness import TOL, compare, gpu_all, oracle_all, rel_err, tol, to_np, torch_act, torch_params

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _log(msg):
    print(msg, flush=True)


SMALL = [
    # (n, c, h, w, k, L)
    (2, 3, 16, 16, 5, 2),
    (2, 3, 37, 45, 5, 3),     # odd sizes, ragged strips
    (1, 2, 130, 70, 5, 4),    # several tiles per row / column
    (3, 4, 7, 7, 5, 1),       # 7x7 padded to 8x8
    (2, 3, 1, 1, 5, 3),       # 1x1 planes at every level
    (1, 2, 5, 3, 5, 5),
    (2, 3, 20, 20, 5, 0),     # base path only
    (2, 2, 33, 17, 3, 3),
    (2, 2, 29, 31, 7, 2),
    (5, 6, 9, 14, 5, 4),      # several planes stacked per workgroup
    (1, 1, 256, 9, 5, 5),     # tall and narrow
    (1, 1, 9, 200, 5, 5),     # short and wide
    (1, 2, 9, 255, 7, 2),     # odd width: scalar loads, a staged row wider than a workgroup
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", SMALL, ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}-k{s[4]}-L{s[5]}" for s in SMALL])
def test_small_shapes_elementwise(shape, dtype):
    _cuda()
    n, c, h, w, k, L = shape
    case = Case(n, c, h, w, k, L, dtype, seed=7, w_std=0.1, b_std=0.05, name="small")
    _log(f"case {case}")
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p)
    want = oracle_all(case, x, dy, p)
    errs = compare(case, got, want)
    _log(f"  errs {errs}")


def test_tiny_config_fp32():
    """x[1,8,16,16] fp32, kernels N(0, 0.1), zero bias, L=2, seed 0."""
    _cuda()
    case = baseline_cases()["tiny"]
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p)
    want = oracle_all(case, x, dy, p)
    errs = compare(case, got, want)
    assert errs["y"] <= TOL[("f32", "fwd")]
    _log(f"tiny errs {errs}")


def test_no_bias_pointer():
    _cuda()
    case = Case(2, 3, 12, 10, 5, 2, "f32", seed=3, name="nobias")
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p, bias=False)
    want = oracle_all(case, x, dy, p, bias=False)
    compare(case, got, want, bias=False)
    assert got["db0"] is None


def _sampled_check(case, planes, channels):
    """Full-size GPU run in the benchmark's launch configuration; oracle on samples."""
    import oracle
    torch = _cuda()
    _log(f"full-size case {case}")
    x, dy, p = case.x(), case.dy(), case.params()
    got = gpu_all(case, x, dy, p)
    q = {kk: v.astype(np.float64) for kk, v in p.items()}
    L, k = case.levels, case.k
    # forward / input gradient on sampled planes
    for (nn, cc) in planes:
        qc = {"w0": q["w0"][[cc]], "b0": q["b0"][[cc]], "s0": q["s0"][[cc]],
              "wl": q["wl"][:, [cc]], "sl": q["sl"][:, [cc]]}
        xs = x[nn:nn + 1, cc:cc + 1].astype(np.float64)
        gs = dy[nn:nn + 1, cc:cc + 1].astype(np.float64)
        y = oracle.forward(xs, qc, L, k)
        e = rel_err(got["y"][nn:nn + 1, cc:cc + 1], y)
        assert e <= tol(case, "fwd"), (case, "y", nn, cc, e)
        qr = dict(qc)
        qr["b0"] = None
        dx = oracle.backward(xs, gs, qr, L, k)["dx"]
        e = rel_err(got["dx"][nn:nn + 1, cc:cc + 1], dx)
        assert e <= tol(case, "grad"), (case, "dx", nn, cc, e)
    # weight gradients on sampled channels (all n)
    qc = {"w0": q["w0"][channels], "b0": q["b0"][channels], "s0": q["s0"][channels],
          "wl": q["wl"][:, channels], "sl": q["sl"][:, channels]}
    gw = oracle.backward(x[:, channels].astype(np.float64), dy[:, channels].astype(np.float64), qc, L, k)
    for key, sl in [("dw0", np.s_[channels]), ("db0", np.s_[channels]), ("ds0", np.s_[channels]),
                    ("dwl", np.s_[:, channels]), ("dsl", np.s_[:, channels])]:
        if L == 0 and key in ("dwl", "dsl"):
            continue
        e = rel_err(got[key][sl], gw[key])
        assert e <= tol(case, "grad"), (case, key, e)
    _log(f"  ok {case}")
    del torch


FULL = ["stage1", "stage2", "stage3", "hires_L1", "hires_L2", "hires_L3", "hires_L4", "hires_L5",
        "stack_1", "stack_2", "stack_3", "stack_4", "dw5", "dw7", "stage1_f16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    case = baseline_cases()[name]
    planes = [(0, 0), (case.n - 1, case.c - 1), (case.n // 2, case.c // 3)]
    channels = sorted({0, case.c // 2, case.c - 1})
    _sampled_check(case, planes, channels)


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
