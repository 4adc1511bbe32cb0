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


def test_launch_model_plane_resident():
    n, c, h, w, k, L, E = 2, 3, 7, 9, 5, 2, 2
    ls = traffic.launches(n, c, h, w, k, L, E, plane_fwd=True, plane_dw=True)
    assert [x[0] for x in ls] == ["plane_fwd", "plane_fwd", "plane_dwl", "plane_dwb", "dw_finalize"]
    N = n * c * h * w
    P = n * c
    # x in, y out; the FLOPs equal the per-level kernels' sum (same arithmetic, no HBM round trips)
    assert ls[0][2] == E * 2 * N
    per_level = traffic.launches(n, c, h, w, k, L, E)
    assert ls[0][3] == sum(f for name, p, _, f in per_level if p == "forward")
    assert ls[2][2] == E * 2 * N
    assert ls[2][3] == P * (20 + 6) * 8 * k * k
    # parsing of profiled names back to families
    assert traffic.split_name("level_fwd<5,bf16>#2") == ("level_fwd", 2)
    assert traffic.split_name("plane_fwd<7,f32>") == ("plane_fwd", 0)
    plan = {"forward": ["plane_fwd<5,bf16>"], "backward_input": ["plane_fwd<5,bf16>"],
            "backward_weight": ["plane_dwl<5,bf16>", "plane_dwb<5,bf16>", "dw_finalize<5,bf16>"]}
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


@pytest.mark.parametrize("L", [0, 1, 2, 3, 4, 5])
def test_model_bytes_closed_forms(L):
    """Per-level pass structure, even sizes: Q_F = 2N + (13/3)N(1-4^-L) - N 4^-L per
    forward-shaped pass (the paper's Eq. 10 without its separate 2N base-conv pass,
    which the synthesis pass absorbs) and Q_BW = (10/3)N(1-4^-L) - 2N 4^-L for the
    weight gradient; without levels both are 2N (x in and y out; x and dy in)."""
    n, c, h, w, E = 2, 3, 64, 96, 2
    N = n * c * h * w
    m = traffic.model_bytes(n, c, h, w, L, E)
    qf = (2 * N + 13.0 / 3.0 * N * (1 - 4.0 ** -L) - N * 4.0 ** -L) if L else 2 * N
    qbw = (10.0 / 3.0 * N * (1 - 4.0 ** -L) - 2 * N * 4.0 ** -L) if L else 2 * N
    assert m["forward"] == pytest.approx(E * qf, rel=1e-12)
    assert m["backward_input"] == m["forward"]
    assert m["backward_weight"] == pytest.approx(E * qbw, rel=1e-12)
    # Eq. 10 itself is this forward plus the separate base conv's 2N
    if L:
        assert qf + 2 * N == pytest.approx(N * traffic.paper_q_fused(L), rel=1e-12)


def test_model_bytes_workloads():
    """Modeled step bytes of the bf16 workloads: x[64,96,56,56] L=3 606.9 MB, x[64,192,28,28]
    L=2 289.0 MB, x[64,384,14,14] L=1 115.6 MB, x[8,128,256,256] L=1..5 1610.6 to 2145.4 MB,
    and the four-layer stack at batch 128 (the 7 x 7 layer padded to 8 x 8 inside) 2150.5 MB."""
    mb = lambda *a: round(traffic.model_bytes(*a, 2)["step"] / 1e6, 1)
    assert mb(64, 96, 56, 56, 3) == 606.9
    assert mb(64, 192, 28, 28, 2) == 289.0
    assert mb(64, 384, 14, 14, 1) == 115.6
    assert [mb(8, 128, 256, 256, L) for L in range(1, 6)] == [1610.6, 2013.3, 2113.9, 2139.1, 2145.4]
    stack = sum(traffic.model_bytes(128, c, h, h, L, 2)["step"] for c, h, L in
                [(96, 56, 3), (192, 28, 2), (384, 14, 1), (768, 7, 1)])
    assert round(stack / 1e6, 1) == 2150.5


def test_conv_flops():
    """Convolution FLOPs per direction: 2 k^2 (N + sum_l 4 B_l); for even sizes
    2 N k^2 (1 + (4/3)(1 - 4^-L))."""
    n, c, h, w, k = 2, 3, 64, 96, 5
    N = n * c * h * w
    for L in range(6):
        want = 2 * N * k * k * (1 + 4.0 / 3.0 * (1 - 4.0 ** -L))
        assert traffic.conv_flops(n, c, h, w, k, L) == pytest.approx(want, rel=1e-12)
