"""The traffic record's attribution of counter rows to the library's launches.

rocprof_summary.py reads rocprofv3's counter databases (one row per dispatch and
counter) and keys the HBM bytes by the launch names of a workload's plan.  Launches
of one kernel with one grid size (the tiled correlation kernel at levels 1, 2 and
3 of the per-level weight gradients) share a counter row; they are told apart by
dispatch order.  These tests build small databases of the same table layout, with a
distinct reading for every planned launch, and check that each launch gets its own.
"""
import os
import sqlite3
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import memory_bound_depthwise_amd as wt  # noqa: E402
import rocprof_summary as rs  # noqa: E402
from synthetic import baseline_cases  # noqa: E402

PERSISTENT = 262144  # the grid every launch of the persistent kernels runs with
COPY = 1 << 20       # bytes of the calibration copy


def _make_db(path, rows):
    """rows: (dispatch_id, kernel_name, grid_size, counter_name, value)."""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, "
                "grid_size integer, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    return path


def _symbol(name):
    fam = name.split("<")[0]
    fam = rs._SYMBOL_FAMILY.get(fam, fam)
    return f"void wtc::{fam}_kernel<5>(wtc::Args)"


def test_by_order_cycles_and_rejects_misfits():
    assert rs._by_order([10, 20, 30, 12, 22, 32], ["a", "b", "c"]) == {"a": 11, "b": 21, "c": 31}
    assert rs._by_order([1, 2, 3, 4], ["a", "b", "c"]) is None
    assert rs._by_order([], ["a"]) is None
    # a name that runs twice per cycle takes the mean of both positions
    assert rs._by_order([1, 3, 5, 7], ["a", "a"]) == {"a": 4}


def test_family_of_symbols():
    assert rs._family(rs._short("void wtc::plane_fwd_kernel<5, unsigned short, 4, 7, false>(wtc::A)")) == "plane_fwd"
    assert rs._family(rs._short("void wtc::dwc_tile_kernel<5, true>(wtc::DwcTileArgs)")) == "dwc_tile"


@pytest.mark.parametrize("steps", [1, 3])
def test_traffic_gives_each_level_its_own_reading(tmp_path, steps):
    case = baseline_cases()[bench.WORKLOADS["hires_L3"][0]]
    desc = wt.make_desc(case.n, case.c, case.h, case.w, case.k, case.levels, bench.DTYPE_CODE[case.dtype])
    plan = [e for op in (wt.OP_FORWARD, wt.OP_BACKWARD_INPUT, wt.OP_BACKWARD_WEIGHT)
            for e in wt.wtconv_plan_launches(desc, op)]
    tiles = [e["name"] for e in plan if e["name"].startswith("dwc_tile")]
    assert len(tiles) == case.levels  # level 1, then one launch per deeper level
    # a distinct reading per planned name (KiB); the same in every step
    kib = {}
    for e in plan:
        kib.setdefault(e["name"], 1000.0 * (len(kib) + 1))
    fetch, write, d = [], [], 0
    for _ in range(steps):
        for e in plan:
            d += 1
            fam = e["name"].split("<")[0]
            grid = PERSISTENT if fam == "dwc_tile" else e["workgroups"] * e["threads"]
            fetch.append((d, _symbol(e["name"]), grid, "FETCH_SIZE", kib[e["name"]]))
            write.append((d, _symbol(e["name"]), grid, "WRITE_SIZE", kib[e["name"]] / 2))
        # a library-external dispatch between steps (torch's copies) changes nothing
        d += 1
        fetch.append((d, "void at::native::copy_kernel(x)", 4096, "FETCH_SIZE", 7.0))
        write.append((d, "void at::native::copy_kernel(x)", 4096, "WRITE_SIZE", 7.0))
    # calibration: the copy reads FETCH_SIZE x 1024 x 2 and WRITE_SIZE x 1024 bytes
    cf = _make_db(str(tmp_path / "cf.db"), [(1, "copy", 1, "FETCH_SIZE", COPY / 2048)])
    cw = _make_db(str(tmp_path / "cw.db"), [(1, "copy", 1, "WRITE_SIZE", COPY / 1024)])
    fdb = _make_db(str(tmp_path / "f.db"), fetch)
    wdb = _make_db(str(tmp_path / "w.db"), write)
    rec = rs.traffic("hires_L3", fdb, wdb, cf, cw, COPY)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    for name in tiles:
        got = rec["kernels"][name]
        assert got["fetch_bytes"] == round(kib[name] * 1024 * 2), name
        assert got["write_bytes"] == round(kib[name] / 2 * 1024), name
        assert got["matched_by"] == "dispatch order"
    # the other launches are matched by family and grid, each to its own reading
    for e in plan:
        if not e["name"].startswith("dwc_tile"):
            assert rec["kernels"][e["name"]]["fetch_bytes"] == round(kib[e["name"]] * 2048), e["name"]


def test_traffic_drops_a_shared_group_whose_count_does_not_fit(tmp_path):
    case = baseline_cases()[bench.WORKLOADS["hires_L3"][0]]
    desc = wt.make_desc(case.n, case.c, case.h, case.w, case.k, case.levels, bench.DTYPE_CODE[case.dtype])
    plan = wt.wtconv_plan_launches(desc, wt.OP_BACKWARD_WEIGHT)
    rows_f, rows_w = [], []
    for d, e in enumerate(plan + plan[:1]):  # one dispatch too many of the first launch
        grid = PERSISTENT if e["name"].startswith("dwc_tile") else e["workgroups"] * e["threads"]
        rows_f.append((d, _symbol(e["name"]), grid, "FETCH_SIZE", 100.0))
        rows_w.append((d, _symbol(e["name"]), grid, "WRITE_SIZE", 100.0))
    cf = _make_db(str(tmp_path / "cf.db"), [(1, "copy", 1, "FETCH_SIZE", COPY / 1024)])
    cw = _make_db(str(tmp_path / "cw.db"), [(1, "copy", 1, "WRITE_SIZE", COPY / 1024)])
    rec = rs.traffic("hires_L3", _make_db(str(tmp_path / "f.db"), rows_f), _make_db(str(tmp_path / "w.db"), rows_w),
                     cf, cw, COPY)
    assert not any(n.startswith("dwc_tile") for n in rec["kernels"])
