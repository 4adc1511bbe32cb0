"""Benchmark of the WTConv layer on one MI355X: forward + input gradient + weight
gradients per step, on synthetic WTConvNeXt-shaped tensors.

    python bench.py [--steps K] [--warmup W] [--workload stage1] [--gpus 1]

Prints one JSON line.  `value` is the step's algorithmic HBM bytes (the sum over
its kernel launches, see memory_bound_depthwise_amd/traffic.py) divided by the
measured step time, in GB/s; `ms_per_step` is the time of one forward + backward.
Inputs are resident in device memory before the timed region; `--rotate` buffer
sets (default 3) are cycled so consecutive steps do not find their inputs in the
256 MB last-level cache.

The `roofline` object covers the kernel family with the largest share of the step
time, timed with hipEvents the library records around each launch on its launch
stream; `cpu_baseline` times the float64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WTConv layer fwd+bwd ms and achieved HBM GB/s (% of 8 TB/s), 1 GPU"
HBM_PEAK_GBS = 8000.0
# MI355X's published FP32 vector peak (256 CUs x 2.4 GHz x 256 FLOP per clock).  The
# library issues no packed FP32, but a register-only v_fmac_f32 loop already runs
# above the single-issue figure (78.6), so only the published peak bounds it.
ALU_PEAK_TFLOPS = 157.3

WORKLOADS = {
    "stage1": ["stage1"], "stage2": ["stage2"], "stage3": ["stage3"],
    "hires_L1": ["hires_L1"], "hires_L2": ["hires_L2"], "hires_L3": ["hires_L3"],
    "hires_L4": ["hires_L4"], "hires_L5": ["hires_L5"],
    "stack": ["stack_1", "stack_2", "stack_3", "stack_4"],
    "tiny": ["tiny"],
    # plain depthwise convolutions (levels = 0) on the stage1 shape, for comparison
    "dw5": ["dw5"], "dw7": ["dw7"],
    "stage1_f16": ["stage1_f16"],
}
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2}  # the library's activation dtype codes


def describe(cases):
    parts = [f"x[{c.n},{c.c},{c.h},{c.w}] {c.dtype} k={c.k} L={c.levels}" for c in cases]
    return "; ".join(parts)


def source_digest():
    """Digest of the kernel sources' code (comments and blank lines left out), so that
    a measurement record is recognised as stale exactly when the code changed."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "memory_bound_depthwise_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        code = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
        h.update(name.encode() + "\n".join(line for line in code if line.strip()).encode())
    return h.hexdigest()[:16]


class Layer:
    """Device tensors of one layer: `rotate` sets of (x, dy, y, dx) plus parameters,
    gradient outputs and one workspace, all allocated before timing."""

    def __init__(self, case, rotate, torch, wt):
        from synthetic import normal
        self.case = case
        dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(case.dtype, torch.float32)
        dev = "cuda"
        self.sets = []
        for r in range(rotate):
            if r == 0:
                x, dy = case.x(), case.dy()
            else:  # distinct data per set, same distribution
                x = normal(case.seed + r, f"{case.name}/x", (case.n, case.c, case.h, case.w), case.x_std)
                dy = normal(case.seed + r, f"{case.name}/dy", (case.n, case.c, case.h, case.w), case.dy_std)
            tx = torch.from_numpy(x).to(dev).to(dt)
            tdy = torch.from_numpy(dy).to(dev).to(dt)
            self.sets.append((tx, tdy, torch.empty_like(tx), torch.empty_like(tx)))
        self.p = {k: torch.from_numpy(v).to(dev) for k, v in case.params().items()}
        C, k, L = case.c, case.k, case.levels
        f32 = torch.float32
        self.grads = {"dw0": torch.empty((C, k, k), dtype=f32, device=dev),
                      "db0": torch.empty((C,), dtype=f32, device=dev),
                      "ds0": torch.empty((C,), dtype=f32, device=dev),
                      "dwl": torch.empty((L, C, 4, k, k), dtype=f32, device=dev),
                      "dsl": torch.empty((L, C, 4), dtype=f32, device=dev)}
        desc = wt.make_desc(case.n, case.c, case.h, case.w, k, L, DTYPE_CODE[case.dtype])
        nbytes = max(wt.wtconv_workspace_size(desc, op) for op in range(3))
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def forward(self, i, wt):
        x, _, y, _ = self.sets[i % len(self.sets)]
        p, L = self.p, self.case.levels
        wt.wtconv_forward(x, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=y, workspace=self.ws)

    def backward(self, i, wt):
        x, dy, _, dx = self.sets[i % len(self.sets)]
        p, L = self.p, self.case.levels
        wt.wtconv_backward_input(dy, p["w0"], p["s0"], p["wl"], p["sl"], L, out=dx, workspace=self.ws)
        wt.wtconv_backward_weight(x, dy, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=self.grads,
                                  workspace=self.ws)


def memory_report(layers, torch):
    """Device memory of the step: the allocator's peak over the run (every rotating
    buffer set included) and the footprint of one training step of these layers with
    this library: one set of x, dy, y, dx per layer, the parameters, their gradients
    and the workspace (the forward keeps nothing for the backward)."""
    def nb(t):
        return 0 if t is None else t.numel() * t.element_size()
    step = 0
    for layer in layers:
        step += sum(nb(t) for t in layer.sets[0])
        step += sum(nb(t) for t in layer.p.values()) + sum(nb(t) for t in layer.grads.values()) + nb(layer.ws)
    return {"peak_allocated_bytes": int(torch.cuda.max_memory_allocated()),
            "step_footprint_bytes": int(step),
            "workspace_bytes": int(sum(nb(layer.ws) for layer in layers)),
            "rotate_buffer_sets": len(layers[0].sets)}


def run_step(layers, i, wt):
    for layer in layers:
        layer.forward(i, wt)
    for layer in reversed(layers):
        layer.backward(i, wt)


def cpu_baseline(cases, budget_s, model_bytes_fn):
    """Time the float64 CPU oracle (forward + backward) on a bounded sample of the
    workload: the first planes of each layer's batch (all channels), grown by
    doubling until one pass takes about budget_s / 8 or covers the whole batch,
    then repeated until about budget_s / 2 has run.  Returns the oracle's rate in
    the GPU value's units (algorithmic bytes of the sampled work per second)."""
    import oracle
    from synthetic import Case
    total_s, total_bytes, samples, full_ms = 0.0, 0.0, [], 0.0
    per_layer = budget_s / len(cases)
    for case in cases:
        ns = 1
        while True:
            sub = Case(ns, case.c, case.h, case.w, case.k, case.levels, case.dtype, case.seed,
                       case.x_std, case.dy_std, case.w_std, case.b_std, case.s_low, case.s_high, case.name)
            x, dy, p = sub.x().astype("float64"), sub.dy().astype("float64"), sub.params()
            q = {k: v.astype("float64") for k, v in p.items()}
            t0 = time.perf_counter()
            oracle.forward(x, q, case.levels, case.k)
            oracle.backward(x, dy, q, case.levels, case.k)
            dt = time.perf_counter() - t0
            if dt > per_layer / 8 or ns >= case.n:
                break
            ns = min(case.n, 2 * ns)
        reps, spent = 1, dt
        while spent < per_layer / 2:
            t0 = time.perf_counter()
            oracle.forward(x, q, case.levels, case.k)
            oracle.backward(x, dy, q, case.levels, case.k)
            spent += time.perf_counter() - t0
            reps += 1
        total_s += spent
        total_bytes += reps * model_bytes_fn(sub)
        samples.append(f"{case.name}: n={ns} of {case.n}, {reps} passes")
        full_ms += 1e3 * spent / reps * case.n / ns
    return {
        "value": round(total_bytes / total_s / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": "; ".join(samples) + " (all channels; forward + backward in float64)",
        "ms_per_step_extrapolated": round(full_ms, 1),
        "seconds": round(total_s, 2),
    }


def load_traffic(kernel, workload, digest):
    """HBM bytes per launch of `kernel` ({fetch_bytes, write_bytes, bytes}) from the
    rocprofv3 counter record of this workload, if the counters were taken on this
    kernel source (None otherwise)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("kernels", {}).get(kernel)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="stage1", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds for the oracle leg")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer runs on one GPU; its data-parallel sharding is a design, not code)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 4 * n, "dispatches": 5}), flush=True)
        return

    import memory_bound_depthwise_amd as wt
    from memory_bound_depthwise_amd import traffic
    from synthetic import baseline_cases

    allc = baseline_cases()
    cases = [allc[name] for name in WORKLOADS[args.workload]]
    print(f"# bench: {args.workload}: {describe(cases)}", file=sys.stderr, flush=True)
    layers = [Layer(c, args.rotate, torch, wt) for c in cases]
    es = lambda c: 4 if c.dtype == "f32" else 2

    def case_launches(c):
        # the kernels the library enqueues for this shape, priced by the byte model
        desc = wt.make_desc(c.n, c.c, c.h, c.w, c.k, c.levels, DTYPE_CODE[c.dtype])
        plan = {p: [e["name"] for e in wt.wtconv_plan_launches(desc, op)]
                for p, op in (("forward", wt.OP_FORWARD), ("backward_input", wt.OP_BACKWARD_INPUT),
                              ("backward_weight", wt.OP_BACKWARD_WEIGHT))}
        return traffic.launches_from_plan(c.n, c.c, c.h, c.w, c.k, c.levels, es(c), plan)

    case_ls = {c.name: case_launches(c) for c in cases}
    step_bytes = sum(b for c in cases for _, _, b, _ in case_ls[c.name])
    step_flops = sum(f for c in cases for _, _, _, f in case_ls[c.name])
    # context: the bytes the same step moves when it follows the paper's pass
    # structure (one analysis + conv launch per level, coefficients through HBM,
    # one synthesis pass with the base conv fused in; the per-level kernels here)
    per_level_bytes = sum(b for c in cases
                          for _, _, b, _ in traffic.launches(c.n, c.c, c.h, c.w, c.k, c.levels, es(c)))

    torch.cuda.reset_peak_memory_stats()
    for i in range(args.warmup):
        run_step(layers, i, wt)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        run_step(layers, i, wt)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(wall_ms, gpu_ms) / args.steps
    print(f"# timed {args.steps} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # per-kernel durations: the same steps again with the library's event pairs
    wt.profile_begin()
    for i in range(args.steps):
        run_step(layers, i, wt)
    torch.cuda.synchronize()
    kstats = wt.profile_end()

    # algorithmic bytes / flops per kernel family (summed over layers and passes)
    fam = {}
    for c in cases:
        for key, _pass, b, f in case_ls[c.name]:
            d = fam.setdefault(key, {"bytes": 0, "flops": 0, "launches": 0})
            d["bytes"] += b
            d["flops"] += f
            d["launches"] += 1
    kernels = []
    for s in kstats:
        d = fam.get(s["name"], {"bytes": 0, "flops": 0, "launches": 1})
        per_step_launches = d["launches"]
        avg_ms = s["total_ms"] / s["count"]
        per_launch_bytes = d["bytes"] / per_step_launches
        per_launch_flops = d["flops"] / per_step_launches
        kernels.append({
            "kernel": s["name"], "launches_per_step": per_step_launches,
            "avg_ms": round(avg_ms, 5), "ms_per_step": round(s["total_ms"] / args.steps, 5),
            "bytes_per_launch": per_launch_bytes, "flops_per_launch": per_launch_flops,
            "gbs": round(per_launch_bytes / (avg_ms * 1e-3) / 1e9, 1) if avg_ms > 0 else None,
            "tflops": round(per_launch_flops / (avg_ms * 1e-3) / 1e12, 2) if avg_ms > 0 else None,
        })
    kernels.sort(key=lambda k: -k["ms_per_step"])
    dom = kernels[0]
    t_hbm = dom["bytes_per_launch"] / (HBM_PEAK_GBS * 1e9)
    t_alu = dom["flops_per_launch"] / (ALU_PEAK_TFLOPS * 1e12)
    digest = source_digest()
    if t_hbm >= t_alu:
        roof = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "alu", "achieved": dom["tflops"], "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / ALU_PEAK_TFLOPS, 4)}
    roof["kernel"] = dom["kernel"]
    roof["avg_launch_ms"] = dom["avg_ms"]
    measured = load_traffic(dom["kernel"], args.workload, digest)
    roof["traffic"] = None if measured is None else measured["bytes"]
    if measured is not None:
        roof["traffic_fetch_write"] = [measured["fetch_bytes"], measured["write_bytes"]]
        roof["traffic_vs_algorithmic"] = round(measured["bytes"] / dom["bytes_per_launch"], 3)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cases[0].dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "shapes": describe(cases), "pass": "forward + dx + dW",
                   "rotate_buffer_sets": args.rotate, "step_bytes": step_bytes, "step_flops": step_flops},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "per_level_model": {
            "step_bytes": per_level_bytes,
            "gbs": round(per_level_bytes / (ms_per_step * 1e-3) / 1e9, 1),
            "hbm_frac": round(per_level_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "bytes of the per-level pass structure over the measured step time: the bandwidth "
                    "a per-level implementation would need to match this step; not moved by these kernels",
        },
        "source_digest": digest,
        "kernels": kernels,
        "roofline": roof,
        "memory": memory_report(layers, torch),
    }
    if not args.no_cpu_baseline:
        def sample_bytes(c):
            # the sample runs the full workload's shapes, so its bytes are the step's
            return sum(b for _, _, b, _ in case_ls[c.name])
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cases, args.cpu_budget, sample_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
