"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle is the plain unfused definition of
"Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation"
(§2.1 Algorithm 1); these tests tie it to things other than itself:

* printed values: Eq. 5 on worked blocks, the Eq. 13 sign table (golden files);
* closed forms: Proposition 1 (H symmetric, H^2 = I), perfect reconstruction,
  Parseval, the block-mean pyramid for identity kernels, Proposition 2 / Eq. 7;
* a library special case: levels = 0 is a depthwise conv2d (torch, CPU, float64);
* invariants: linearity, the adjoint identity <M v, g> = <v, M^T g>;
* brute force: every parameter gradient against a central difference, which is
  exact here because the layer is affine in each single parameter;
* Eq. 9: the scale gradient recovered from the folded-weight gradient.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synthetic import Case, to_bf16_bits, bf16_bits_to_f32, normal

RNG = np.random.default_rng(1234)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _params(C, k, L, seed=0, bias=True, w_std=0.3):
    c = Case(1, C, 1, 1, k, L, "f32", seed, w_std=w_std, b_std=0.2 if bias else 0.0, name="pins")
    p = {key: v.astype(np.float64) for key, v in c.params().items()}
    return p


def _torch_dwconv(x, w0):
    """Depthwise cross-correlation, zero 'same' padding, via torch CPU conv2d."""
    C, k, _ = w0.shape
    out = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w0)[:, None],
                                     padding=(k - 1) // 2, groups=C)
    return out.numpy()


# --------------------------------------------------------------------------
# Haar step
# --------------------------------------------------------------------------

def test_eq5_worked_blocks(golden_dir):
    g = _load(golden_dir, "haar_eq5_blocks.json")
    for case in g["cases"]:
        bands = oracle.haar_analysis(np.array(case["block"], dtype=np.float64))
        assert bands.shape == (4, 1, 1)
        got = bands[:, 0, 0]
        want = [case["LL"], case["LH"], case["HL"], case["HH"]]
        np.testing.assert_array_equal(got, want)


def test_eq13_sign_table(golden_dir):
    g = _load(golden_dir, "haar_eq13_signs.json")
    for bi, band in enumerate(["LH", "HL", "HH"], start=1):
        unit = np.zeros((4, 1, 1))
        unit[bi] = 2.0  # synthesis halves it: the pixel value is the sign
        px = oracle.haar_synthesis(unit, 2, 2)
        for row in g["rows"]:
            assert px[row["ry"], row["rx"]] == row[band], (band, row)
    unit = np.zeros((4, 1, 1))
    unit[0] = 2.0
    np.testing.assert_array_equal(oracle.haar_synthesis(unit, 2, 2), np.ones((2, 2)))


def test_prop1_symmetric_involutory():
    H = np.zeros((4, 4))
    for col in range(4):
        e = np.zeros(4)
        e[col] = 1.0
        H[:, col] = oracle.haar_analysis(e.reshape(2, 2))[:, 0, 0]
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_allclose(H @ H, np.eye(4), atol=0, rtol=0)


@pytest.mark.parametrize("h,w", [(8, 8), (7, 9), (1, 1), (1, 6), (13, 11), (2, 3)])
def test_perfect_reconstruction(h, w):
    x = RNG.standard_normal((h, w))
    rec = oracle.haar_synthesis(oracle.haar_analysis(x), h, w)
    np.testing.assert_allclose(rec, x, rtol=0, atol=1e-14)


@pytest.mark.parametrize("h,w", [(8, 8), (6, 10)])
def test_parseval_and_inverse_on_even(h, w):
    x = RNG.standard_normal((h, w))
    bands = oracle.haar_analysis(x)
    assert np.isclose(np.sum(bands ** 2), np.sum(x ** 2), rtol=1e-14)
    c = RNG.standard_normal((4, h // 2, w // 2))
    np.testing.assert_allclose(oracle.haar_analysis(oracle.haar_synthesis(c, h, w)), c, atol=1e-14)


def test_constant_input_bands():
    x = np.full((6, 8), 3.0)
    bands = oracle.haar_analysis(x)
    np.testing.assert_array_equal(bands[0], np.full((3, 4), 6.0))
    np.testing.assert_array_equal(bands[1:], 0.0)


# --------------------------------------------------------------------------
# Whole operator
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape,k", [((2, 3, 9, 7), 5), ((1, 4, 16, 16), 3), ((2, 2, 5, 12), 7)])
def test_levels0_is_depthwise_conv(shape, k):
    n, C, H, W = shape
    p = _params(C, k, 0)
    x = RNG.standard_normal(shape)
    y = oracle.forward(x, p, 0, k)
    ref = p["s0"][None, :, None, None] * (_torch_dwconv(x, p["w0"]) + p["b0"][None, :, None, None])
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def _block_mean(plane, j):
    b = 2 ** j
    H, W = plane.shape
    Hp, Wp = -(-H // b) * b, -(-W // b) * b
    xp = np.zeros((Hp, Wp))
    xp[:H, :W] = plane
    s = xp.reshape(Hp // b, b, Wp // b, b).sum(axis=(1, 3)) / (b * b)
    return np.repeat(np.repeat(s, b, 0), b, 1)[:H, :W]


@pytest.mark.parametrize("H,W,L", [(16, 16, 3), (13, 11, 3), (7, 7, 1), (9, 20, 4), (5, 3, 5)])
def test_identity_kernels_give_block_mean_pyramid(H, W, L):
    """Identity level kernels, unit scales, no base path: the wavelet path is
    sum_{j<L} BlockMean_{2^j}(x) (zero-padded blocks), which fixes the 2^-l weights,
    the carried low-pass band and the pad/crop handling independently of the signs."""
    k, C = 5, 2
    p = _params(C, k, L)
    p["w0"][:] = 0.0
    p["b0"][:] = 0.0
    p["wl"][:] = 0.0
    p["wl"][..., k // 2, k // 2] = 1.0
    p["sl"][:] = 1.0
    x = RNG.standard_normal((1, C, H, W))
    y = oracle.forward(x, p, L, k)
    for c in range(C):
        want = sum(_block_mean(x[0, c], j) for j in range(L))
        np.testing.assert_allclose(y[0, c], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("band", [0, 1, 2, 3])
def test_single_band_wiring(band, golden_dir):
    """Only band `band` of level 1 passes (identity kernel, scale s): the output is
    1/2 * sign(ry, rx) * s * Y_band on each block, with the Eq. 13 signs; this pins
    which weight/scale slot multiplies which band."""
    signs = {(r["ry"], r["rx"]): r for r in _load(golden_dir, "haar_eq13_signs.json")["rows"]}
    names = ["LL", "LH", "HL", "HH"]
    k, C, H, W = 3, 1, 6, 7
    p = _params(C, k, 1)
    p["w0"][:] = 0.0
    p["b0"][:] = 0.0
    p["wl"][:] = 0.0
    p["wl"][0, 0, band, 1, 1] = 1.0
    p["sl"][:] = 7.0
    p["sl"][0, 0, band] = 1.5
    x = RNG.standard_normal((1, 1, H, W))
    y = oracle.forward(x, p, 1, k)[0, 0]
    Y = oracle.haar_analysis(x[0, 0])[band]
    for yy in range(H):
        for xx in range(W):
            sgn = 1 if band == 0 else signs[(yy % 2, xx % 2)][names[band]]
            assert np.isclose(y[yy, xx], 0.5 * sgn * 1.5 * Y[yy // 2, xx // 2], rtol=0, atol=1e-14)


@pytest.mark.parametrize("shape,L", [((2, 3, 16, 16), 3), ((1, 2, 13, 11), 3), ((1, 2, 7, 9), 4),
                                     ((1, 1, 32, 8), 5)])
def test_prop2_closed_form_equals_cascade(shape, L):
    """Eq. 7: R(y,x) = sum_l 2^-l (LL + s_y LH + s_x HL + s_y s_x HH) at (y>>l, x>>l),
    s_y = (-1)^bit_{l-1}(y); compared with the cascade's output minus the base path."""
    n, C, H, W = shape
    k = 5
    p = _params(C, k, L)
    x = RNG.standard_normal(shape)
    y, Z = oracle.forward(x, p, L, k, return_coeffs=True)
    base = p["s0"][None, :, None, None] * (_torch_dwconv(x, p["w0"]) + p["b0"][None, :, None, None])
    yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    R = np.zeros(shape)
    for l in range(1, L + 1):
        z = Z[l - 1]
        sy = np.where((yy >> (l - 1)) & 1, -1.0, 1.0)
        sx = np.where((xx >> (l - 1)) & 1, -1.0, 1.0)
        cy, cx = yy >> l, xx >> l
        R += 2.0 ** -l * (z[:, :, 0, cy, cx] + sy * z[:, :, 1, cy, cx] + sx * z[:, :, 2, cy, cx]
                          + sy * sx * z[:, :, 3, cy, cx])
    np.testing.assert_allclose(y - base, R, rtol=0, atol=1e-12)


def test_appendix_a_worked_bits():
    """Appendix A: the level-1 term is selected by (y mod 2, x mod 2) and weighted 1/2,
    the level-2 term by (floor(y/2) mod 2, floor(x/2) mod 2) and weighted 1/4.
    Only the HH band of level 2 is non-zero here (identity kernel), so pixel (y, x)
    must equal 1/4 * (-1)^(b1(y) + b1(x)) * s * HH2[y>>2, x>>2]."""
    k, L, H, W = 3, 2, 8, 8
    p = _params(1, k, L)
    p["w0"][:] = 0.0
    p["b0"][:] = 0.0
    p["wl"][:] = 0.0
    p["wl"][1, 0, 3, 1, 1] = 1.0
    p["sl"][:] = 1.0
    x = RNG.standard_normal((1, 1, H, W))
    y, Z = oracle.forward(x, p, L, k, return_coeffs=True)
    hh2 = Z[1][0, 0, 3]
    for yy in range(H):
        for xx in range(W):
            sgn = (-1) ** (((yy >> 1) & 1) + ((xx >> 1) & 1))
            assert np.isclose(y[0, 0, yy, xx], 0.25 * sgn * hh2[yy >> 2, xx >> 2], atol=1e-14)


def test_linearity_in_x():
    n, C, H, W, k, L = 2, 3, 11, 10, 5, 3
    p = _params(C, k, L, bias=False)
    x1, x2 = RNG.standard_normal((2, n, C, H, W))
    a, b = 0.75, -1.25
    lhs = oracle.forward(a * x1 + b * x2, p, L, k)
    rhs = a * oracle.forward(x1, p, L, k) + b * oracle.forward(x2, p, L, k)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape,k,L", [((2, 3, 12, 12), 5, 2), ((1, 2, 7, 9), 3, 3), ((1, 2, 9, 6), 7, 4),
                                       ((1, 1, 1, 1), 5, 3)])
def test_adjoint_identity(shape, k, L):
    """<M v, g> = <v, M^T g>, with M the linear part of the layer (bias 0) and
    M^T g the input gradient of the oracle's reverse mode."""
    p = _params(shape[1], k, L, bias=False)
    v = RNG.standard_normal(shape)
    g = RNG.standard_normal(shape)
    lhs = np.sum(oracle.forward(v, p, L, k) * g)
    dx = oracle.backward(v, g, p, L, k)["dx"]
    rhs = np.sum(v * dx)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("shape,k,L", [((2, 3, 12, 12), 5, 2), ((1, 2, 7, 9), 3, 3), ((2, 2, 9, 6), 7, 1)])
def test_input_gradient_is_rotated_forward(shape, k, L):
    """Because the Haar matrix is its own transpose (Prop. 1 / Eq. 1), M^T is the
    same layer with every kernel turned by 180 degrees and no bias."""
    p = _params(shape[1], k, L)
    x = RNG.standard_normal(shape)
    g = RNG.standard_normal(shape)
    dx = oracle.backward(x, g, p, L, k)["dx"]
    q = dict(p)
    q["w0"] = p["w0"][:, ::-1, ::-1].copy()
    q["wl"] = p["wl"][..., ::-1, ::-1].copy()
    q["b0"] = np.zeros_like(p["b0"])
    np.testing.assert_allclose(oracle.forward(g, q, L, k), dx, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape,k,L", [((2, 2, 7, 5), 3, 2), ((1, 2, 6, 9), 5, 3), ((1, 1, 3, 4), 3, 2)])
def test_parameter_gradients_exact_central_difference(shape, k, L):
    """f(theta) = <dy, y(theta)> is affine in every single parameter entry (the
    layer is bilinear in (s, W) and linear in b), so a central difference is exact
    up to float64 rounding; brute-force every entry."""
    n, C, H, W = shape
    p = _params(C, k, L)
    x = RNG.standard_normal(shape)
    dy = RNG.standard_normal(shape)
    grads = oracle.backward(x, dy, p, L, k)
    names = {"w0": "dw0", "b0": "db0", "s0": "ds0", "wl": "dwl", "sl": "dsl"}
    h = 0.5
    for key, gkey in names.items():
        arr = p[key]
        for idx in np.ndindex(arr.shape):
            q = {kk: vv.copy() for kk, vv in p.items()}
            q[key][idx] += h
            fp = np.sum(dy * oracle.forward(x, q, L, k))
            q[key][idx] -= 2 * h
            fm = np.sum(dy * oracle.forward(x, q, L, k))
            fd = (fp - fm) / (2 * h)
            got = grads[gkey][idx]
            assert abs(fd - got) <= 1e-10 * max(1.0, abs(fd)), (key, idx, fd, got)


def test_eq9_scale_gradient_recovery():
    """Eq. 9: with W~ = s W and b~ = s b, dL/ds = <dL/dW~, W> + dL/db~ * b, where
    dL/dW~ = (dL/dW) / s and dL/db~ = (dL/db) / s.  The oracle computes ds directly
    from the unscaled convolution output, so this ties the two routes together."""
    n, C, H, W, k, L = 2, 3, 10, 9, 5, 2
    p = _params(C, k, L)
    x = RNG.standard_normal((n, C, H, W))
    dy = RNG.standard_normal((n, C, H, W))
    g = oracle.backward(x, dy, p, L, k)
    dwt0 = g["dw0"] / p["s0"][:, None, None]
    dbt0 = g["db0"] / p["s0"]
    ds0 = np.sum(dwt0 * p["w0"], axis=(1, 2)) + dbt0 * p["b0"]
    np.testing.assert_allclose(ds0, g["ds0"], rtol=1e-12, atol=1e-12)
    dwtl = g["dwl"] / p["sl"][..., None, None]
    dsl = np.sum(dwtl * p["wl"], axis=(3, 4))
    np.testing.assert_allclose(dsl, g["dsl"], rtol=1e-12, atol=1e-12)


def test_empty_inputs():
    p = _params(3, 5, 2)
    for shape in [(0, 3, 8, 8), (2, 3, 0, 8), (2, 3, 8, 0)]:
        x = np.zeros(shape)
        assert oracle.forward(x, p, 2, 5).shape == shape
        g = oracle.backward(x, x, p, 2, 5)
        for key in ["dw0", "db0", "ds0", "dwl", "dsl"]:
            assert not np.any(g[key]), key


# --------------------------------------------------------------------------
# Input generator / storage codec (shared by both sides)
# --------------------------------------------------------------------------

def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 0.0],
                    dtype=np.float32)
    bits = to_bf16_bits(vals)
    np.testing.assert_array_equal(bits, [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000])
    np.testing.assert_array_equal(bf16_bits_to_f32(bits)[[0, 4]], [1.0, -2.5])


def test_generator_is_deterministic_and_normal():
    a = normal(0, "gen", (200000,), 1.0)
    b = normal(0, "gen", (200000,), 1.0)
    np.testing.assert_array_equal(a, b)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1.0) < 0.01
    c = normal(0, "other", (10,), 1.0)
    assert not np.array_equal(a[:10], c)
