"""The byte/FLOP accounting used by the benchmark against the numbers the paper
prints (§4.4 Table 1 from Eq. 2 and Eq. 10; §3.2 Eq. 3/4), and the per-kernel
model against a direct count on a small odd-sized shape."""
import json
import os

import pytest

from memory_bound_depthwise_amd import traffic


def test_table1_and_eq3(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "table1_traffic.json")))
    for L, qr, qf, ratio in zip(g["levels"], g["q_ref"], g["q_fused"], g["ratio"]):
        assert round(traffic.paper_q_ref(L), 2) == pytest.approx(qr, abs=1e-9)
        assert round(traffic.paper_q_fused(L), 2) == pytest.approx(qf, abs=1e-9)
        assert round(traffic.paper_q_ref(L) / traffic.paper_q_fused(L), 2) == pytest.approx(ratio, abs=1e-9)
    assert traffic.paper_macs(5, 5) == pytest.approx(g["k5_L5_macs_per_n"], abs=0.05)
    assert traffic.paper_macs(5, 1) == pytest.approx(g["k5_L1_macs_per_n"], abs=1e-9)
    assert 2 * traffic.paper_macs(5, 5) == pytest.approx(g["k5_L5_flops_per_n"], abs=0.05)
    assert 4 * traffic.paper_q_ref(5) == pytest.approx(g["k5_L5_ref_bytes_per_n_fp32"], abs=0.05)
    # Eq. 4 divides the printed 137.9N FLOP by 85.3N bytes (= 1.617) and states the
    # result as "about 1.63"; the pin allows for that rounding.
    assert 2 * traffic.paper_macs(5, 5) / (4 * traffic.paper_q_ref(5)) == pytest.approx(
        g["ref_intensity_fp32"], abs=0.015)


def test_launch_model_fused():
    n, c, h, w, k, L, E = 2, 3, 7, 9, 5, 2, 2
    ls = traffic.launches(n, c, h, w, k, L, E, fused_fwd=True, fused_dw=True)
    assert [x[0] for x in ls] == ["fused_fwd", "fused_fwd", "fused_dw", "dw_base", "dw_finalize"]
    N = n * c * h * w
    P = n * c
    # x in, y out; the FLOPs equal the per-level kernels' sum (same arithmetic, no HBM round trips)
    assert ls[0][2] == E * 2 * N
    per_level = traffic.launches(n, c, h, w, k, L, E)
    assert ls[0][3] == sum(f for name, p, _, f in per_level if p == "forward")
    assert ls[2][2] == E * 2 * N
    assert ls[2][3] == P * (20 + 6) * (8 * k * k + 16)
    # parsing of profiled names back to families
    assert traffic.split_name("level_fwd<5,bf16>#2") == ("level_fwd", 2)
    assert traffic.split_name("fused_fwd<7,f32>") == ("fused_fwd", 0)
    plan = {"forward": ["fused_fwd<5,bf16>"], "backward_input": ["fused_fwd<5,bf16>"],
            "backward_weight": ["fused_dw<5,bf16>", "dw_base<5,bf16>", "dw_finalize<5,bf16>"]}
    lp = traffic.launches_from_plan(n, c, h, w, k, L, E, plan)
    assert [x[2:] for x in lp] == [x[2:] for x in ls]


def test_launch_model_counts():
    n, c, h, w, k, L, E = 2, 3, 7, 9, 5, 2, 2
    ls = traffic.launches(n, c, h, w, k, L, E)
    names = [x[0] for x in ls]
    assert names == ["level_fwd#1", "level_fwd#2", "synth"] * 2 + ["dw_level#1", "dw_level#2", "dw_base", "dw_finalize"]
    P = n * c
    # level 1: reads 7x9, coefficient grid 4x5; writes Q 4*4*5 and carrier 4*5
    assert ls[0][2] == E * P * (7 * 9 + 4 * 20 + 20)
    # level 2 (deepest): reads the 4x5 carrier, grid 2x3, Q only
    assert ls[1][2] == E * P * (20 + 4 * 6)
    assert ls[2][2] == E * P * (2 * 63 + 4 * 20 + 4 * 6)
    assert ls[6][2] == E * P * (2 * 63 + 2 * 20)
    assert ls[8][2] == E * P * 2 * 63
