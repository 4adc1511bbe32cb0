"""The shapes the GPU parity tests run, in one place: the GPU tests take them from
here, and a CPU test checks that every kernel the library can launch for a plane of
up to 64 x 64 (or a larger one) is reached by at least one of them."""
from synthetic import Case, baseline_cases

# (n, c, h, w, k, L), each run in f32, bf16 and f16 and compared element by element
SMALL = [
    (2, 3, 16, 16, 5, 2),
    (2, 3, 37, 45, 5, 3),     # odd sizes, ragged strips
    (1, 2, 130, 70, 5, 4),    # several tiles per row / column
    (3, 4, 7, 7, 5, 1),       # 7x7 padded to 8x8
    (2, 3, 1, 1, 5, 3),       # 1x1 planes at every level
    (1, 2, 5, 3, 5, 5),
    (2, 3, 20, 20, 5, 0),     # base path only
    (2, 2, 33, 17, 3, 3),
    (2, 2, 29, 31, 7, 2),
    (5, 6, 9, 14, 5, 4),      # several planes stacked per workgroup
    (1, 1, 256, 9, 5, 5),     # tall and narrow
    (1, 1, 9, 200, 5, 5),     # short and wide
    (1, 2, 9, 255, 7, 2),     # odd width: scalar loads, a staged row wider than a workgroup
    (2, 3, 64, 64, 7, 3),     # 64 x 64, k = 7: pyramid beyond the plane-resident LDS budget
    (8, 16, 64, 64, 5, 3),    # 64 x 64 planes: forward plane-resident, level gradients per level
    (1, 3, 57, 63, 5, 5),     # odd 57 x 63, five levels: per-level forward
    (3, 5, 22, 30, 3, 1),     # k = 3 on the plane-resident path with CW = 1
    (4, 7, 12, 24, 7, 0),     # levels = 0 with k = 7
    (6, 4, 8, 8, 5, 2),       # item strips of 4 rows
    (2, 3, 56, 20, 5, 2),     # item strips of 7 rows, CW = 2
    (2, 2, 70, 66, 3, 2),     # k = 3 on the per-level kernels
    (24, 2, 14, 14, 5, 1),    # many planes side by side in one pass (arrays whose size is not a multiple of 4)
    (40, 2, 7, 7, 5, 1),      # the same for 7 x 7 planes
    (12, 2, 28, 28, 5, 2),    # several 28 x 28 planes per pass, two levels
    (1, 2, 80, 70, 5, 0),     # levels = 0 past the plane-resident range (synthesis kernel alone)
    (1, 2, 9, 130, 3, 0),     # ... with k = 3
    (1, 2, 70, 9, 7, 0),      # ... and k = 7
]
DTYPES = ["f32", "bf16", "f16"]


def variant_shapes():
    """One shape per compiled variant of the plane-resident kernels, for every k and
    for levels = 0 and >= 1 (the matrix-core kernel's at the end).  The library picks the variant from the plane alone:
    cell rows per item RH = 7 when ceil(h/2) is a multiple of 7, 4 when ceil(h/2) <= 4,
    8 otherwise; cells per staging item CW = 4 when w % 8 == 0, 2 when w % 4 == 0,
    1 otherwise.  Heights alternate between even and odd (pad-to-even), and three
    images per channel exercise plane stacking with a ragged last group."""
    out = []
    heights = {4: (8, 7), 7: (28, 27), 8: (20, 19)}      # RH -> (even h, odd h)
    widths = {4: 24, 2: 12, 1: 10}                       # CW -> w
    i = 0
    for k in (3, 5, 7):
        for rh, (he, ho) in heights.items():
            for cw, w in widths.items():
                for L in (0, 1 + i % 3):
                    h = he if i % 2 == 0 else ho
                    out.append((3, 2, h, w, k, L))
                    i += 1
    # bfloat16 planes 7..64 on a side with levels run the matrix-core kernel, k = 3 or 5:
    # one shape per commit width CW (w % 8 == 0, w % 4 == 0, odd w), levels 1..3,
    # even and odd heights, three images per channel
    mma = {4: 32, 2: 28, 1: 29}
    for k in (3, 5):
        for cw, w in mma.items():
            h = (30, 33, 40)[i % 3]
            out.append((3, 2, h, w, k, 1 + i % 3))
            i += 1
    # planes under 7 pixels on a side stay on the vector kernel in bfloat16 too (the
    # matrix-core kernel takes the rest): its variants for k = 3 and 5 on such planes
    for k in (3, 5):
        for h, w, L in ((14, 1, 1), (9, 1, 2), (1, 4, 1), (14, 4, 2), (9, 4, 3), (1, 8, 1), (1, 1, 1)):
            out.append((3, 2, h, w, k, L))
    # bfloat16 weight gradients of levels 2..L beside the correlation kernel, for the
    # kernel sizes the rows above leave out at CW = 4
    for k in (3, 7):
        out.append((3, 2, 17, 24, k, 2))
    return out


def small_cases():
    out = []
    for s in SMALL + variant_shapes():
        n, c, h, w, k, L = s
        for dt in DTYPES:
            out.append(Case(n, c, h, w, k, L, dt, seed=7, w_std=0.1, b_std=0.05, name="small"))
    return out


FULL = ["stage1", "stage2", "stage3", "hires_L1", "hires_L2", "hires_L3", "hires_L4", "hires_L5",
        "stack_1", "stack_2", "stack_3", "stack_4", "dw5", "dw7", "stage1_f16", "tiny"]


def full_cases():
    allc = baseline_cases()
    return [allc[name] for name in FULL]


def other_cases():
    """Shapes of the remaining GPU tests (no-bias, determinism, adjoint)."""
    return [Case(2, 3, 12, 10, 5, 2, "f32", seed=3, name="nobias"),
            Case(16, 8, 56, 56, 5, 3, "bf16", seed=11, name="det"),
            Case(4, 6, 45, 38, 5, 4, "f32", seed=5, b_std=0.0, name="adj")]


def all_cases():
    return small_cases() + full_cases() + other_cases()
