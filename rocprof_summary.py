"""Summarise rocprofv3 SQLite output (rocpd) into the short text kept in profiles/.

    python rocprof_summary.py trace <results.db>
        per-kernel calls, average and total duration (the --kernel-trace --stats data)
    python rocprof_summary.py counters <fetch.db> <write.db> <copy_fetch.db> <copy_write.db> <copy_bytes>
        FETCH_SIZE / WRITE_SIZE per dispatch (KiB), scaled by what the same counters
        read for a plain device copy of known size, as bytes per launch
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


def _counter(db: str):
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select kernel_name, counter_name, value, grid_size from counters_collection").fetchall()
    agg = collections.defaultdict(list)
    for k, c, v, g in rows:
        agg[(_short(k), c, g)].append(v)
    return {key: sum(v) / len(v) for key, v in agg.items()}


def counters(fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes):
    cf = _counter(copy_fetch_db)
    cw = _counter(copy_write_db)
    # the copy kernel is the dispatch with the largest reading of each counter
    fetch_ref = max(v for (k, c, g), v in cf.items() if c == "FETCH_SIZE")
    write_ref = max(v for (k, c, g), v in cw.items() if c == "WRITE_SIZE")
    fetch_scale = copy_bytes / (fetch_ref * 1024.0)
    write_scale = copy_bytes / (write_ref * 1024.0)
    f = _counter(fetch_db)
    w = _counter(write_db)
    kernels = []
    for (k, c, g), v in sorted(f.items()):
        wv = w.get((k, "WRITE_SIZE", g))
        kernels.append({"kernel": k, "grid": g, "fetch_kib": round(v, 1),
                        "write_kib": None if wv is None else round(wv, 1),
                        "fetch_bytes": round(v * 1024 * fetch_scale),
                        "write_bytes": None if wv is None else round(wv * 1024 * write_scale)})
    return {"fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4), "kernels": kernels}


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        print(json.dumps(trace(sys.argv[2]), indent=1))
    elif sys.argv[1] == "counters":
        print(json.dumps(counters(*sys.argv[2:6], float(sys.argv[6])), indent=1))
