"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign or index, a transposed operand), builds that copy with gcc in a
temporary directory and runs the pins of test_oracle_pins against it.  At least one
pin must fail for every mutant.  Runs on the CPU only; the real oracle is untouched.
"""
import os
import tempfile

import pytest

import oracle
from oracle import build as oracle_build
import test_oracle_pins as pins

# (name, original text, planted mistake)
MUTANTS = [
    ("eq5_lh_sign", "out[1] = 0.5 * (a + b - c - d);", "out[1] = 0.5 * (a - b + c - d);"),
    ("eq5_bands_swapped", "out[2] = 0.5 * (a - b + c - d);\n    out[3] = 0.5 * (a - b - c + d);",
     "out[3] = 0.5 * (a - b + c - d);\n    out[2] = 0.5 * (a - b - c + d);"),
    ("synthesis_no_half", "x[(size_t)y * w + xx] = 0.5 * (", "x[(size_t)y * w + xx] = 1.0 * ("),
    ("synthesis_hx_sign", "double sx = (xx % 2) ? -1.0 : 1.0;", "double sx = (xx % 2) ? 1.0 : -1.0;"),
    ("pad_top_left", "at(x, h, w, 2 * i + 1, 2 * j + 1), o);", "at(x, h, w, 2 * i - 1, 2 * j + 1), o);"),
    ("kernel_transposed", "acc += ker[u * k + v] * at(in, h, w, i + u - p, j + v - p);",
     "acc += ker[v * k + u] * at(in, h, w, i + u - p, j + v - p);"),
    ("kernel_convolution_not_xcorr", "acc += ker[u * k + v] * at(in, h, w, i + u - p, j + v - p);",
     "acc += ker[u * k + v] * at(in, h, w, i - u + p, j - v + p);"),
    ("level_scale_dropped", "s->Z[l][b * pl + e] = sc * s->Zc[l][b * pl + e];",
     "s->Z[l][b * pl + e] = s->Zc[l][b * pl + e];"),
    ("cascade_lowpass_not_added", "for (size_t e = 0; e < pl; ++e) T[e] += R[e];",
     "for (size_t e = 0; e < pl; ++e) T[e] += 0.0 * R[e];"),
    ("carrier_wrong_band", "carrier = s->Y[l]; /* the LL band is the first band */",
     "carrier = s->Y[l] + pl;"),
    ("bias_outside_scale", "yp[e] = s0[c] * (s.base[e] + bias) + (R ? R[e] : 0.0);",
     "yp[e] = s0[c] * s.base[e] + bias + (R ? R[e] : 0.0);"),
    ("weight_index_band", "const double *ker = Wl + ((((size_t)(l - 1) * C + c) * 4 + b) * k * k);",
     "const double *ker = Wl + ((((size_t)(l - 1) * C + c) * 4 + (3 - b)) * k * k);"),
    ("bwd_scale_grad_uses_scaled", "for (size_t e = 0; e < pl; ++e) acc += gZ[e] * s.Zc[l][b * pl + e];",
     "for (size_t e = 0; e < pl; ++e) acc += gZ[e] * s.Z[l][b * pl + e];"),
    ("bwd_adjoint_shift", "int ii = i + u - p, jj = j + v - p;", "int ii = i - u + p, jj = j + v - p;"),
    ("bwd_level_grad_unscaled", "for (size_t e = 0; e < pl; ++e) s.tmp[e] = sc * gZ[e];",
     "for (size_t e = 0; e < pl; ++e) s.tmp[e] = gZ[e];"),
    ("bwd_carrier_grad_dropped", "for (size_t e = 0; e < pl; ++e) s.gy[l][e] += dX[e];",
     "for (size_t e = 0; e < pl; ++e) s.gy[l][e] += 0.0 * dX[e];"),
    ("bwd_bias_grad_unscaled", "for (size_t e = 0; e < P; ++e) acc += s.tmp[e];",
     "for (size_t e = 0; e < P; ++e) acc += gp[e];"),
    ("bwd_ds0_no_bias", "acc += gp[e] * (s.base[e] + bias);", "acc += gp[e] * s.base[e];"),
]


def _run_pins(golden_dir):
    """Run a representative set of pins; return the names of those that failed."""
    failed = []
    checks = [
        ("eq5", lambda: pins.test_eq5_worked_blocks(golden_dir)),
        ("eq13", lambda: pins.test_eq13_sign_table(golden_dir)),
        ("recon", lambda: pins.test_perfect_reconstruction(7, 9)),
        ("levels0", lambda: pins.test_levels0_is_depthwise_conv((2, 3, 9, 7), 5)),
        ("pyramid", lambda: pins.test_identity_kernels_give_block_mean_pyramid(13, 11, 3)),
        ("band", lambda: [pins.test_single_band_wiring(b, golden_dir) for b in range(4)]),
        ("eq7", lambda: pins.test_prop2_closed_form_equals_cascade((1, 2, 13, 11), 3)),
        ("adjoint", lambda: pins.test_adjoint_identity((1, 2, 7, 9), 3, 3)),
        ("fd", lambda: pins.test_parameter_gradients_exact_central_difference((1, 1, 3, 4), 3, 2)),
        ("eq9", lambda: pins.test_eq9_scale_gradient_recovery()),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, golden_dir):
    with open(oracle_build.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    with tempfile.TemporaryDirectory() as tmp:
        msrc = os.path.join(tmp, "mutant.c")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle_build.build(src=msrc, out=os.path.join(tmp, "libmutant.so"))
        oracle.use_library(lib)
        try:
            failed = _run_pins(golden_dir)
        finally:
            oracle.use_library(None)
    assert failed, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_all(golden_dir):
    assert _run_pins(golden_dir) == []
