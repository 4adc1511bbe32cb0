"""Benchmark of the WTConv layer on one MI355X: forward + input gradient + weight
gradients per step, on synthetic WTConvNeXt-shaped tensors.

    python bench.py [--steps K] [--warmup W] [--workload stack] [--gpus 1]

Prints one JSON line.  The default workload is the four-layer WTConvNeXt-T-shaped
stack at batch 128 (forward of layers 1..4, then the backward of layers 4..1).

* `value`: the step's modeled HBM bytes divided by the measured step time, in GB/s
  (`hbm_frac` = value / 8 TB/s).  The modeled bytes are those of the paper's
  per-level pass structure (memory_bound_depthwise_amd/traffic.py: model_bytes),
  the figure the layer's bandwidth target is stated in.  The bytes the kernels
  this library launches must move (`moved_bytes`; the plane-resident kernels move
  only their inputs and outputs) are reported next to it.
* `ms_per_step`: one forward + backward of the workload's layers; the per-step
  event times also give `ms_per_step_median`, and each pass is timed on its own
  (`per_pass_ms`).  Every launch goes to one stream, in order.  With
  `--two-stream` the layers are scheduled as a chain instead: each layer's weight
  gradients run on a second stream as soon as its dy is in place (the input
  gradient of the layer after it), beside the rest of the input-gradient chain.
  That overlaps only the kernels' tails (every launch fills the GPU), and measured
  slower than one stream: the kernels raise the priority of workgroups with many
  passes left, so a kernel that starts on one stream holds back the tail of the
  one ending on the other.  Launches are eager: the host enqueues the step's kernels
  faster than they run, so the gaps between them are a few microseconds.  With
  `--graph` the step is captured once per buffer set as a HIP graph
  (torch.cuda.graph around the same library calls) and the replays are timed;
  `eager_ms_per_step` then reports eager launches next to them.
Inputs are resident in device memory before the timed region; `--rotate` buffer
sets (default 3) are cycled so consecutive steps do not find their inputs in the
256 MB last-level cache.

The `roofline` object covers the kernel with the largest share of the step time,
timed with hipEvents the library records around each launch on its launch stream,
against the bound that takes longer at peak for its algorithmic bytes and FLOPs:
HBM at 8 TB/s, or the vector ALU at the FP32 FMA rate the kernels can issue (see
VALU_PEAK_TFLOPS).  `cpu_baseline` times the float64 CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WTConv layer fwd+bwd ms and achieved HBM GB/s (% of 8 TB/s), 1 GPU"
HBM_PEAK_GBS = 8000.0
# FP32 FMA peak of MI355X for single-issue vector FMAs: 256 CUs x 4 SIMDs x 16 lanes x
# 2 FLOP x 2.4 GHz = 78.6 TFLOP/s.  The published 157.3 TFLOP/s counts the packed
# dual-FP32 FMA (two FMAs per lane per instruction), which these kernels do not issue
# (packed FP32 instruction selection is switched off in the build).
MFMA_BF16_TFLOPS = 2500.0  # dense bfloat16 matrix-core peak
VALU_PEAK_TFLOPS = 78.6
PUBLISHED_FP32_TFLOPS = 157.3

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
PASSES = ("forward", "backward_input", "backward_weight")


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

    def __init__(self, case, rotate, torch, wt, two_stream=False):
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
        # the weight-gradient pass's own workspace, for when it runs beside the
        # input-gradient pass on a second stream
        self.ws_w = None
        if two_stream:
            nbytes = wt.wtconv_workspace_size(desc, wt.OP_BACKWARD_WEIGHT)
            self.ws_w = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def forward(self, i, wt):
        x, _, y, _ = self.sets[i % len(self.sets)]
        p, L = self.p, self.case.levels
        wt.wtconv_forward(x, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=y, workspace=self.ws)

    def backward_input(self, i, wt):
        _, dy, _, dx = self.sets[i % len(self.sets)]
        p, L = self.p, self.case.levels
        wt.wtconv_backward_input(dy, p["w0"], p["s0"], p["wl"], p["sl"], L, out=dx, workspace=self.ws)

    def backward_weight(self, i, wt, own_workspace=False):
        x, dy, _, _ = self.sets[i % len(self.sets)]
        p, L = self.p, self.case.levels
        wt.wtconv_backward_weight(x, dy, p["w0"], p["b0"], p["s0"], p["wl"], p["sl"], L, out=self.grads,
                                  workspace=self.ws_w if own_workspace else self.ws)

    def backward(self, i, wt):
        self.backward_input(i, wt)
        self.backward_weight(i, wt)


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
        step += sum(nb(t) for t in layer.p.values()) + sum(nb(t) for t in layer.grads.values())
        step += nb(layer.ws) + nb(layer.ws_w)
    return {"peak_allocated_bytes": int(torch.cuda.max_memory_allocated()),
            "step_footprint_bytes": int(step),
            "workspace_bytes": int(sum(nb(layer.ws) + nb(layer.ws_w) for layer in layers)),
            "rotate_buffer_sets": len(layers[0].sets)}


def run_step(layers, i, wt):
    """One step on the current stream: forward of every layer, then the input and
    weight gradients of each layer, last layer first."""
    for layer in layers:
        layer.forward(i, wt)
    for layer in reversed(layers):
        layer.backward(i, wt)


class TwoStreamStep:
    """One step with the weight gradients on a second stream.  The layers are taken
    as a chain, as in a network: layer l's dy is the input gradient of layer l + 1,
    so the weight gradients of layer l wait for that input gradient (the last layer's
    for the end of the forward pass) and then run beside the rest of the input-
    gradient chain; the step ends when both streams have finished.  Each layer's
    weight-gradient pass has a workspace of its own."""

    def __init__(self, layers, torch):
        self.layers = layers
        self.torch = torch
        self.side = torch.cuda.Stream()  # default priority
        self.events = [torch.cuda.Event() for _ in range(len(layers))]

    def __call__(self, i, wt):
        torch = self.torch
        main = torch.cuda.current_stream()
        for layer in self.layers:
            layer.forward(i, wt)
        for j, layer in enumerate(reversed(self.layers)):
            ready = self.events[j]
            ready.record(main)  # this layer's dy and x are in place
            self.side.wait_event(ready)
            with torch.cuda.stream(self.side):
                layer.backward_weight(i, wt, own_workspace=True)
            layer.backward_input(i, wt)
        main.wait_stream(self.side)


def cpu_baseline(cases, budget_s):
    """Time the float64 CPU oracle on a bounded sample of the workload: the first
    images of each layer's batch (all channels), grown by doubling until one
    forward + backward takes about budget_s / 8 or covers the whole batch; then the
    forward, the input gradient and the weight gradients are each repeated until
    about budget_s / 6 has run.  Rates are in the GPU value's units: the sampled
    images' share of the modeled bytes, per second.  The per-pass milliseconds are
    extrapolated to the full batch."""
    import oracle
    from memory_bound_depthwise_amd import traffic
    from synthetic import Case
    total_s, total_bytes, samples = 0.0, 0.0, []
    pass_ms = {p: 0.0 for p in PASSES}
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
        mb = traffic.model_bytes(ns, case.c, case.h, case.w, case.levels, 2 if case.dtype != "f32" else 4)
        runs = {
            "forward": lambda: oracle.forward(x, q, case.levels, case.k),
            "backward_input": lambda: oracle.backward(x, dy, q, case.levels, case.k, outputs=("dx",)),
            "backward_weight": lambda: oracle.backward(x, dy, q, case.levels, case.k,
                                                       outputs=("dw0", "db0", "ds0", "dwl", "dsl")),
        }
        reps_note = []
        for name, fn in runs.items():
            times = []
            while sum(times) < per_layer / 6 or not times:
                t0 = time.perf_counter()
                fn()
                times.append(time.perf_counter() - t0)
            total_s += sum(times)
            total_bytes += len(times) * mb[name]
            pass_ms[name] += 1e3 * statistics.median(times) * case.n / ns
            reps_note.append(f"{name} x{len(times)}")
        samples.append(f"{case.name}: n={ns} of {case.n} ({', '.join(reps_note)})")
    return {
        "value": round(total_bytes / total_s / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.threads(),
        "nproc": os.cpu_count(),
        "kind": "oracle",
        "sample": "; ".join(samples) + " (all channels, float64)",
        "per_pass_ms_extrapolated": {k: round(v, 1) for k, v in pass_ms.items()},
        "ms_per_step_extrapolated": round(sum(pass_ms.values()), 1),
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


def timed(fn, steps, torch):
    """Run fn(i) for i in range(steps) with an event before each step and after the
    last; returns (wall ms, list of per-step ms)."""
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i].record(stream)
        fn(i)
    evs[steps].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return wall_ms, [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stack", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--two-stream", action="store_true",
                    help="run each layer's weight gradients on a second stream, beside the input-gradient chain")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as a HIP graph instead of eager launches")
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
    layers = [Layer(c, args.rotate, torch, wt, args.two_stream) for c in cases]
    es = lambda c: 4 if c.dtype == "f32" else 2

    def case_launches(c):
        # the kernels the library enqueues for this shape, priced by the byte model
        desc = wt.make_desc(c.n, c.c, c.h, c.w, c.k, c.levels, DTYPE_CODE[c.dtype])
        plan = {p: [e["name"] for e in wt.wtconv_plan_launches(desc, op)]
                for p, op in zip(PASSES, (wt.OP_FORWARD, wt.OP_BACKWARD_INPUT, wt.OP_BACKWARD_WEIGHT))}
        return traffic.launches_from_plan(c.n, c.c, c.h, c.w, c.k, c.levels, es(c), plan)

    case_ls = {c.name: case_launches(c) for c in cases}
    moved_bytes = sum(b for c in cases for _, _, b, _ in case_ls[c.name])
    step_flops = sum(f for c in cases for _, _, _, f in case_ls[c.name])
    model = {p: sum(traffic.model_bytes(c.n, c.c, c.h, c.w, c.levels, es(c))[p] for c in cases)
             for p in PASSES + ("step",)}

    step = TwoStreamStep(layers, torch) if args.two_stream else (lambda i, wt: run_step(layers, i, wt))
    torch.cuda.reset_peak_memory_stats()
    for i in range(args.warmup):
        step(i, wt)
    torch.cuda.synchronize()

    # one HIP graph per rotating buffer set, each holding a whole step (every launch
    # of the forward, input-gradient and weight-gradient passes of every layer)
    graphs = []
    if args.graph:
        for r in range(args.rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r, wt)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
    step_fn = (lambda i: graphs[i % len(graphs)].replay()) if graphs else (lambda i: step(i, wt))

    # timed region: exactly `steps` steps, synchronised on both sides
    wall_ms, step_ms = timed(step_fn, args.steps, torch)
    gpu_ms = sum(step_ms)
    ms_per_step = max(wall_ms, gpu_ms) / args.steps
    print(f"# timed {args.steps} steps ({'graph replay' if graphs else 'eager'}): "
          f"{ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)
    eager_ms = None
    if graphs:
        # the same steps as eager launches, for comparison
        ew, es_ms = timed(lambda i: step(i, wt), args.steps, torch)
        eager_ms = max(ew, sum(es_ms)) / args.steps

    # each pass on its own (forward of every layer, then input gradients, then weight gradients)
    per_pass = {}
    for name in PASSES:
        fn = {"forward": lambda i: [l.forward(i, wt) for l in layers],
              "backward_input": lambda i: [l.backward_input(i, wt) for l in reversed(layers)],
              "backward_weight": lambda i: [l.backward_weight(i, wt) for l in reversed(layers)]}[name]
        _, ms = timed(fn, args.steps, torch)
        per_pass[name] = {"mean_ms": round(statistics.mean(ms), 5), "median_ms": round(statistics.median(ms), 5),
                          "model_gbs": round(model[name] / (statistics.mean(ms) * 1e-3) / 1e9, 1)}

    # per-kernel durations: the same steps again with the library's event pairs, on one
    # stream (each launch's pair then times that launch alone)
    wt.profile_begin()
    for i in range(args.steps):
        run_step(layers, i, wt)
    torch.cuda.synchronize()
    kstats = wt.profile_end()

    # algorithmic bytes / flops per kernel name (summed over layers and passes)
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
    on_mfma = dom["kernel"].startswith(("mma_fwd", "mma_tile"))  # level-1 and base products on the matrix cores
    t_alu = dom["flops_per_launch"] / ((MFMA_BF16_TFLOPS if on_mfma else VALU_PEAK_TFLOPS) * 1e12)
    digest = source_digest()
    if t_hbm >= t_alu:
        roof = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4)}
        if on_mfma:
            roof["mfma_tflops"] = dom["tflops"]
            roof["mfma_note"] = ("convolution FLOPs over the launch time; the products run as bfloat16 "
                                 "16x16x32 MFMAs (dense peak 2.5 PFLOP/s), so HBM is the bound")
    else:
        roof = {"bound": "alu", "achieved": dom["tflops"], "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / VALU_PEAK_TFLOPS, 4),
                "frac_of_published_fp32_peak": round(dom["tflops"] / PUBLISHED_FP32_TFLOPS, 4),
                "peak_note": "single-issue FP32 FMA: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz; "
                             "the published 157.3 TFLOP/s needs packed FP32, which the build does not emit"}
    roof["kernel"] = dom["kernel"]
    roof["avg_launch_ms"] = dom["avg_ms"]
    roof["algorithmic_bytes_per_launch"] = dom["bytes_per_launch"]
    roof["algorithmic_flops_per_launch"] = dom["flops_per_launch"]
    measured = load_traffic(dom["kernel"], args.workload, digest)
    roof["traffic"] = None if measured is None else measured["bytes"]
    if measured is not None:
        roof["traffic_fetch_write"] = [measured["fetch_bytes"], measured["write_bytes"]]
        roof["traffic_vs_algorithmic"] = round(measured["bytes"] / dom["bytes_per_launch"], 3)

    value = model["step"] / (ms_per_step * 1e-3) / 1e9
    moved_gbs = moved_bytes / (ms_per_step * 1e-3) / 1e9
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
                   "rotate_buffer_sets": args.rotate, "launch": "hip_graph" if graphs else "eager",
                   "streams": 2 if args.two_stream else 1,
                   "model_step_bytes": model["step"],
                   "moved_step_bytes": moved_bytes, "step_flops": step_flops},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "ms_per_step_median": round(statistics.median(step_ms), 5),
        "eager_ms_per_step": None if eager_ms is None else round(eager_ms, 5),
        "per_pass_ms": per_pass,
        "moved_bytes": {"gbs": round(moved_gbs, 1), "hbm_frac": round(moved_gbs / HBM_PEAK_GBS, 4),
                        "note": "bytes the launched kernels must move (plane-resident kernels: inputs and "
                                "outputs only) over the step time"},
        "valu": {"step_tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
                 "frac": round(step_flops / (ms_per_step * 1e-3) / 1e12 / VALU_PEAK_TFLOPS, 4),
                 "note": "convolution FLOPs of the step over the step time, against the single-issue FP32 FMA peak"},
        "source_digest": digest,
        "kernels": kernels,
        "roofline": roof,
        "memory": memory_report(layers, torch),
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cases, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
