"""The three passes captured in one HIP graph (torch.cuda.graph) and replayed: every
replay must give bit for bit what the same calls give when run eagerly on the same
data.  The library's kernels take fixed-order reductions only, so the two runs
are deterministic and compared exactly.  Between the replays the test does eager
work of its own (other library calls, copies into the captured inputs, device
synchronisations), and each replay runs on fresh input values."""
import numpy as np
import pytest

from synthetic import Case

pytestmark = pytest.mark.gpu

# one case per kernel family: matrix-core forward + correlation weight gradient
# (bfloat16, levels), the plane-resident vector kernels (float32), the per-level
# path (a plane whose pyramid does not fit on chip) and the level-free depthwise
# conv
_CASES = [
    Case(4, 16, 56, 56, 5, 2, "bf16", seed=31, w_std=0.1, b_std=0.05, name="graph-mma"),
    Case(2, 8, 40, 36, 5, 3, "f32", seed=32, w_std=0.1, b_std=0.05, name="graph-plane"),
    Case(1, 2, 224, 224, 5, 2, "bf16", seed=33, w_std=0.1, b_std=0.05, name="graph-levels"),
    Case(2, 8, 28, 28, 7, 0, "bf16", seed=34, w_std=0.1, b_std=0.05, name="graph-nolevels"),
]

_GRADS = ("dw0", "db0", "ds0", "dwl", "dsl")


@pytest.mark.parametrize("case", _CASES, ids=[c.name for c in _CASES])
def test_graph_replays_match_eager(case):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_depthwise_amd as wt
    from wtc_harness import torch_act
    print(f"case {case}", flush=True)
    dev = torch.device("cuda")
    C, k, L = case.c, case.k, case.levels
    p = {name: torch.from_numpy(v).to(dev) for name, v in case.params().items()}
    code = {"f32": wt.F32, "bf16": wt.BF16, "f16": wt.F16}[case.dtype]
    desc = wt.make_desc(case.n, C, case.h, case.w, k, L, code)
    nbytes = max(wt.wtconv_workspace_size(desc, op) for op in range(3))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    # fresh inputs per run: the case's generator with shifted seeds
    def inputs(r):
        c = Case(case.n, C, case.h, case.w, k, L, case.dtype, seed=case.seed + 100 * r, name=case.name)
        return torch_act(c.x(), case.dtype), torch_act(c.dy(), case.dtype)

    x, dy = inputs(0)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    grads = {"dw0": torch.empty((C, k, k), dtype=torch.float32, device=dev),
             "db0": torch.empty((C,), dtype=torch.float32, device=dev),
             "ds0": torch.empty((C,), dtype=torch.float32, device=dev)}
    if L:
        grads["dwl"] = torch.empty((L, C, 4, k, k), dtype=torch.float32, device=dev)
        grads["dsl"] = torch.empty((L, C, 4), dtype=torch.float32, device=dev)

    def step(x, dy, y, dx, grads):
        wt.wtconv_forward(x, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=y, workspace=ws)
        wt.wtconv_backward_input(dy, p["w0"], p["s0"], p["wl"], p["sl"], L, out=dx, workspace=ws)
        wt.wtconv_backward_weight(x, dy, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=grads, workspace=ws)

    def snapshot(y, dx, grads):
        out = {"y": y.float().cpu().numpy(), "dx": dx.float().cpu().numpy()}
        out.update({name: t.cpu().numpy() for name, t in grads.items()})
        return out

    # eager warm-up (plans are built on the first call, outside the capture)
    step(x, dy, y, dx, grads)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x, dy, y, dx, grads)
    torch.cuda.synchronize()

    for r in range(1, 4):
        nx, ndy = inputs(r)
        # eager reference on separate buffers
        ey, edx = torch.empty_like(nx), torch.empty_like(nx)
        eg = {name: torch.empty_like(t) for name, t in grads.items()}
        step(nx, ndy, ey, edx, eg)
        torch.cuda.synchronize()
        want = snapshot(ey, edx, eg)
        # the captured buffers take the new values; stale outputs are overwritten
        x.copy_(nx)
        dy.copy_(ndy)
        y.fill_(float("nan"))
        dx.fill_(float("nan"))
        for t in grads.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(y, dx, grads)
        for name in want:
            same = np.array_equal(got[name], want[name], equal_nan=False)
            assert same, (f"replay {r}: {name} differs from the eager run "
                          f"(max |diff| {np.nanmax(np.abs(got[name] - want[name]))})")
        print(f"  replay {r}: y, dx and {len(grads)} gradients identical to eager", flush=True)
