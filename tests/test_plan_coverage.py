"""Every kernel the library can launch is reached by a GPU parity case.

The library picks its kernels (plane-resident or per-level families, and the
compiled variant of a plane-resident kernel) from the shape alone.  This CPU test
sweeps descriptors through the library's launch-plan query and checks that each
(kernel family, k, dtype, variant) it can produce also appears in the plan of
some case that the GPU parity tests run, so no reachable kernel ships untested.
"""
import itertools

import pytest

import memory_bound_depthwise_amd as wt
from gpu_cases import all_cases

DT = {"f32": wt.F32, "bf16": wt.BF16, "f16": wt.F16}


def _family(entry):
    # 'level_fwd<5,bf16>#2' -> ('level_fwd<5,bf16>', variant); levels of the
    # per-level kernels run the same code
    return entry["name"].split("#")[0], entry["variant"]


def _plan_keys(n, c, h, w, k, L, dt):
    desc = wt.make_desc(n, c, h, w, k, L, DT[dt])
    keys = set()
    for op in (wt.OP_FORWARD, wt.OP_BACKWARD_INPUT, wt.OP_BACKWARD_WEIGHT):
        keys.update(_family(e) for e in wt.wtconv_plan_launches(desc, op))
    return keys


@pytest.fixture(scope="module")
def covered():
    keys = set()
    for c in all_cases():
        keys |= _plan_keys(c.n, c.c, c.h, c.w, c.k, c.levels, c.dtype)
    return keys


def _sweep():
    sides = [1, 2, 3, 4, 5, 7, 8, 9, 12, 14, 15, 16, 20, 24, 28, 31, 32, 33, 40, 48, 56, 57, 63, 64, 65, 100]
    for h, w in itertools.product(sides, sides):
        for k in (3, 5, 7):
            for L in range(0, 9):
                for n in (1, 8, 64):
                    yield n, 4, h, w, k, L


def test_every_reachable_kernel_has_a_gpu_case(covered):
    # bfloat16 plans differ from float32 plans (the matrix-core kernels are
    # bfloat16 only, and a shape outside their range falls back to the vector
    # kernels); IEEE half plans are those of float32
    reach = {}
    for n, c, h, w, k, L in _sweep():
        for dt, as_dts in (("bf16", ("bf16",)), ("f32", ("f32", "f16"))):
            for name, variant in _plan_keys(n, c, h, w, k, L, dt):
                fam, rest = name.split("<")
                kk = rest.split(",")[0]
                for adt in as_dts:
                    reach.setdefault((f"{fam}<{kk},{adt}>", variant), (n, c, h, w, k, L, dt))
    missing = [(key, example) for key, example in sorted(reach.items()) if key not in covered]
    assert not missing, "kernels without a GPU parity case: " + "; ".join(f"{k} e.g. {e}" for k, e in missing[:20])
