"""Summarise rocprofv3 SQLite output (rocpd) into the short text kept in profiles/.

    python rocprof_summary.py trace <results.db>
        per-kernel calls, average and total duration (the --kernel-trace --stats data)
    python rocprof_summary.py counters <fetch.db> <write.db> <copy_fetch.db> <copy_write.db> <copy_bytes>
        FETCH_SIZE / WRITE_SIZE per dispatch (KiB), scaled by what the same counters
        read for a plain device copy of known size, as bytes per launch
    python rocprof_summary.py traffic <workload> <fetch.db> <write.db> <copy_fetch.db> <copy_write.db> <copy_bytes>
        the same, keyed by the library's kernel names for the workload's launch plan
        (the record bench.py reads from profiles/traffic_<workload>.txt)
    python rocprof_summary.py sq <results.db> ...
        shader-sequencer counters (SQ_*) per kernel, averaged over dispatches; several
        runs (one counter group each) are merged
"""
from __future__ import annotations

import collections
import json
import sqlite3
import sys


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def trace(db: str):
    """Per kernel: dispatches, average / min / max duration in microseconds (from the
    dispatch start and end timestamps, in nanoseconds) and share of kernel time."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select name, start, end from kernels").fetchall()
    agg = collections.defaultdict(list)
    for name, start, end in rows:
        agg[_short(name)].append((end - start) / 1e3)
    total = sum(sum(v) for v in agg.values())
    out = []
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append({"kernel": k, "calls": len(v), "avg_us": round(sum(v) / len(v), 3),
                    "min_us": round(min(v), 3), "max_us": round(max(v), 3),
                    "total_us": round(sum(v), 1), "pct": round(100 * sum(v) / total, 2)})
    return out


def _counter(db: str, with_counts: bool = False):
    """Mean reading per (kernel, counter, grid) over its dispatches (and, with
    with_counts, the number of dispatches)."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select kernel_name, counter_name, value, grid_size from counters_collection").fetchall()
    agg = collections.defaultdict(list)
    for k, c, v, g in rows:
        agg[(_short(k), c, g)].append(v)
    if with_counts:
        return {key: (sum(v) / len(v), len(v)) for key, v in agg.items()}
    return {key: sum(v) / len(v) for key, v in agg.items()}


def counters(fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes):
    cf = _counter(copy_fetch_db)
    cw = _counter(copy_write_db)
    # the copy kernel is the dispatch with the largest reading of each counter
    fetch_ref = max(v for (k, c, g), v in cf.items() if c == "FETCH_SIZE")
    write_ref = max(v for (k, c, g), v in cw.items() if c == "WRITE_SIZE")
    fetch_scale = copy_bytes / (fetch_ref * 1024.0)
    write_scale = copy_bytes / (write_ref * 1024.0)
    f = _counter(fetch_db, with_counts=True)
    w = _counter(write_db)
    kernels = []
    for (k, c, g), (v, n) in sorted(f.items()):
        wv = w.get((k, "WRITE_SIZE", g))
        kernels.append({"kernel": k, "grid": g, "dispatches": n, "fetch_kib": round(v, 1),
                        "write_kib": None if wv is None else round(wv, 1),
                        "fetch_bytes": round(v * 1024 * fetch_scale),
                        "write_bytes": None if wv is None else round(wv * 1024 * write_scale)})
    return {"fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4), "kernels": kernels}


def _family(short: str) -> str:
    """'wtc::plane_fwd_kernel<5, unsigned short, 4, 7, false>' -> 'plane_fwd'."""
    return short.split("<")[0].split("::")[-1].removesuffix("_kernel")


# launch names whose kernel symbol has another family name (the level pass that also
# adds the deeper levels' patterns runs the level kernel)
_SYMBOL_FAMILY = {"level_acc": "level_fwd"}


def _sequence(db: str, counter: str, fam: str, grid):
    """The readings of one counter for the dispatches of one kernel family (of one
    grid size, unless grid is None), in dispatch order."""
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select kernel_name, grid_size, value from counters_collection "
                       "where counter_name = ? order by dispatch_id", (counter,)).fetchall()
    return [v for k, g, v in rows if _family(_short(k)) == fam and (grid is None or g == grid)]


def _by_order(seq, cycle):
    """Mean reading per launch name when several planned launches share one kernel
    family and grid: a layer runs its launches in plan order every time, so the j-th
    dispatch belongs to cycle[j % len(cycle)].  None when the count does not fit."""
    if not seq or len(seq) % len(cycle):
        return None
    acc = collections.defaultdict(list)
    for j, v in enumerate(seq):
        acc[cycle[j % len(cycle)]].append(v)
    return {n: sum(v) / len(v) for n, v in acc.items()}


def traffic(workload, fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes):
    """Measured HBM bytes per launch for every kernel of the workload's launch plan:
    a counter row matches a planned launch by kernel family and grid size (by family
    alone when the family ran with one grid size only)."""
    import os
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import bench
    import memory_bound_depthwise_amd as wt
    from synthetic import baseline_cases

    rec = counters(fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes)
    rows = collections.defaultdict(list)
    for r in rec["kernels"]:
        rows[(_family(r["kernel"]), r["grid"])].append(r)
    out = {}
    got = collections.defaultdict(dict)
    allc = baseline_cases()
    # launches of one family with one grid size (two levels' kernels) share a counter
    # row, which averages them: they are told apart by dispatch order below
    shared = collections.defaultdict(list)
    for name in bench.WORKLOADS[workload]:
        c = allc[name]
        desc = wt.make_desc(c.n, c.c, c.h, c.w, c.k, c.levels, bench.DTYPE_CODE[c.dtype])
        plan = [e for op in (wt.OP_FORWARD, wt.OP_BACKWARD_INPUT, wt.OP_BACKWARD_WEIGHT)
                for e in wt.wtconv_plan_launches(desc, op)]
        names_at = collections.defaultdict(set)
        for e in plan:
            names_at[(e["name"].split("<")[0], e["workgroups"] * e["threads"])].add(e["name"])
        for e in plan:
            fam = e["name"].split("<")[0]
            fam = _SYMBOL_FAMILY.get(fam, fam)
            grid = e["workgroups"] * e["threads"]
            if len(names_at[(e["name"].split("<")[0], grid)]) > 1:
                shared[(fam, grid)].append((name, e["name"]))
                continue
            match = rows.get((fam, grid))
            if not match:
                # A persistent kernel's grid follows the device's occupancy, which
                # the host-side plan does not know: take the family's rows when
                # they all share one grid.
                grids = {g for (f, g) in rows if f == fam}
                if len(grids) == 1:
                    match = rows[(fam, grids.pop())]
            if not match or any(r["write_bytes"] is None for r in match):
                continue
            for r in match:  # every compiled variant the launch matched (one per layer shape)
                got[e["name"]][r["kernel"]] = r
    # a name's record is the mean over its launches (the layers of a stack that run
    # the same kernel family, as bench.py averages their times): the rows weighted by
    # their dispatch counts (layers that run one compiled variant share its row)
    for name, rs in got.items():
        rs = list(rs.values())
        nd = sum(r["dispatches"] for r in rs)
        fb = round(sum(r["fetch_bytes"] * r["dispatches"] for r in rs) / nd)
        wb = round(sum(r["write_bytes"] * r["dispatches"] for r in rs) / nd)
        out[name] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb, "variants": len(rs)}
    for (fam, grid), launches in shared.items():
        # only one layer's launches in the group: another layer's could interleave
        if len({case for case, _ in launches}) > 1:
            continue
        if (fam, grid) not in rows:
            # a persistent kernel (its grid follows the occupancy): the family's one
            # grid, when no other group of the family claims it
            grids = {g for (f, g) in rows if f == fam}
            if len(grids) != 1 or sum(f == fam for f, _ in shared) > 1:
                continue
            grid = grids.pop()
        cycle = [n for _, n in launches]
        fr = _by_order(_sequence(fetch_db, "FETCH_SIZE", fam, grid), cycle)
        wr = _by_order(_sequence(write_db, "WRITE_SIZE", fam, grid), cycle)
        if fr is None or wr is None:
            continue
        for n in fr:
            fb = round(fr[n] * 1024 * rec["fetch_scale"])
            wb = round(wr[n] * 1024 * rec["write_scale"])
            out[n] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb, "variants": 1,
                      "matched_by": "dispatch order"}
    return {"workload": workload, "source_digest": bench.source_digest(),
            "fetch_scale": rec["fetch_scale"], "write_scale": rec["write_scale"], "kernels": out}


def trace_md(rows):
    out = ["| kernel | calls | avg µs | min µs | max µs | total µs | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']} | {r['min_us']} | {r['max_us']} | "
                   f"{r['total_us']} | {r['pct']} |")
    return "\n".join(out)


def counters_md(rec):
    out = ["| kernel | grid (threads) | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch MB | write MB |",
           "|---|---|---|---|---|---|"]
    for r in rec["kernels"]:
        wb = "" if r["write_bytes"] is None else f"{r['write_bytes'] / 1e6:.1f}"
        out.append(f"| `{r['kernel']}` | {r['grid']} | {r['fetch_kib']} | {r['write_kib']} | "
                   f"{r['fetch_bytes'] / 1e6:.1f} | {wb} |")
    return "\n".join(out)


def sq(*dbs):
    """Per kernel (plane-resident and fused kernels of the library): every SQ_ counter
    found in the given runs, averaged over its dispatches."""
    agg = collections.defaultdict(dict)
    for db in dbs:
        for (k, c, _g), v in _counter(db).items():
            if c.startswith("SQ_") and k.startswith("wtc::"):
                agg[k][c] = v
    return agg


def sq_md(agg):
    names = sorted({c for v in agg.values() for c in v})
    out = ["| kernel | " + " | ".join(n.removeprefix("SQ_") for n in names) + " |",
           "|---|" + "---|" * len(names)]
    for k, v in sorted(agg.items()):
        out.append(f"| `{k}` | " + " | ".join(f"{v[n]:.4g}" if n in v else "" for n in names) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    md = "--md" in sys.argv
    if md:
        sys.argv.remove("--md")
    if sys.argv[1] == "trace":
        rows = trace(sys.argv[2])
        print(trace_md(rows) if md else json.dumps(rows, indent=1))
    elif sys.argv[1] == "counters":
        rec = counters(*sys.argv[2:6], float(sys.argv[6]))
        print(counters_md(rec) if md else json.dumps(rec, indent=1))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], *sys.argv[3:7], float(sys.argv[7])), indent=1))
    elif sys.argv[1] == "sq":
        agg = sq(*sys.argv[2:])
        print(sq_md(agg) if md else json.dumps(agg, indent=1))
