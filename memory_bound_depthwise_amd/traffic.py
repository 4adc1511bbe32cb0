"""Algorithmic HBM bytes and FLOPs of the layer and of every kernel launch.

"Algorithmic" means what each pass must move and compute by its design, in the
units the paper's I/O model uses ("Fast and Memory-Efficient Wavelet Convolutions
via I/O-Aware Reformulation", §3.1 Eq. 2 and §4.4 Eq. 10: every tensor a stage
reads or writes crosses HBM once), with exact element counts including the
pad-to-even of odd planes.  Parameters, weight-gradient partials and halo
re-reads are not counted (they are O(C k^2) or cache hits).

Two byte counts are kept apart:
* `model_bytes`: the per-level pass structure of the paper's fused layer, which
  the layer's stated bandwidth figure is measured against.  Forward (and the input
  gradient, the same pipeline on dy): one analysis + filter pass per level (reads
  the carrier, writes the four filtered bands and, above the deepest level, the
  next carrier) and one synthesis pass with the base conv fused in (reads x and
  every level's bands, writes y).  Weight gradient: one pass per level reading the
  carriers of x and dy (level 1: x and dy themselves, the base gradient fused into
  it) and writing the next carriers.  For even sizes this is
  Q_F = 2N + (13/3)N(1-4^-L) - N 4^-L elements per forward-shaped pass and
  Q_BW = (10/3)N(1-4^-L) - 2N 4^-L for the weight gradient (2N when L = 0).
* `kernel_cost`: the bytes of the kernels this library actually launches for a
  shape (the plane-resident kernels move only x in and y out, or x and dy in).

FLOPs are the convolution multiply-adds at 2 FLOP each: per direction (forward,
input gradient, weight gradient) N k^2 for the base conv plus 4 B_l k^2 for level
l; the Haar butterflies and the synthesis add a few N of additions, not counted.

Per launch, with E = element size, P = n*C planes, H_l x W_l the level-l grid,
B_l = P*H_l*W_l coefficient blocks of level l:
  plane_fwd    : read x (N), write y (N).  FLOPs: 2 (N k^2 + sum_l 4 B_l k^2).
  plane_dwl    : read x and dy (2N).  FLOPs: 2 sum_l 4 B_l k^2.
  level_fwd l  : reads the carrier P*H_{l-1}*W_{l-1}; writes Q(l) 4*B_l and,
                 for l < L, the carrier B_l.  FLOPs: 2 * 4 B_l k^2.
  synth        : reads x (N) and every Q(l); writes y (N).  FLOPs: 2 N k^2.
  carrier l    : reads the carrier of level l - 1 (x for l = 1), writes B_l.
                 FLOPs: 0 (adds only).
  level_acc l  : level_fwd without the carrier write, plus a read of the deeper
                 levels' summed patterns 4 B_{l+1} for l < L.
  dwc_tile     : reads x and dy (2N); for L >= 2 writes both level-1 carriers
                 (2 B_1).  FLOPs: 2 (N k^2 + 4 B_1 k^2) (base and level 1).
  mma_tile     : reads x (N) and, for L >= 2, the summed patterns 4 B_2; writes
                 y (N).  FLOPs: 2 (N k^2 + 4 B_1 k^2) (base conv and level 1).
  dw_level l   : reads the x and dy carriers (2*P*H_{l-1}*W_{l-1}); writes both
                 next carriers for l < L.  FLOPs: 2 * 4 B_l k^2.
  dw_base,
  plane_dwb    : read x and dy (2N).  FLOPs: 2 N k^2.
  dw_finalize  : parameter-sized, counted as 0.
backward_input launches the same kernels as forward.  Which path a shape takes
is the library's decision (wtconv_plan_launches); `launches` takes it as flags.
"""
from __future__ import annotations


def level_sizes(h, w, levels):
    hs, ws = [h], [w]
    for _ in range(levels):
        hs.append((hs[-1] + 1) // 2)
        ws.append((ws[-1] + 1) // 2)
    return hs, ws


def kernel_cost(family, level, n, c, h, w, k, levels, elem_bytes):
    """(bytes, flops) of one launch of kernel `family` (level-indexed families take
    `level` >= 1, others ignore it)."""
    P = n * c
    N = P * h * w
    E = elem_bytes
    hs, ws = level_sizes(h, w, levels)
    blocks = [P * hs[l] * ws[l] for l in range(levels + 1)]
    kk = k * k
    lvl_flops = sum(2 * 4 * blocks[l] * kk for l in range(1, levels + 1))
    if family in ("plane_fwd", "mma_fwd"):
        return E * 2 * N, 2 * N * kk + lvl_flops
    if family == "plane_dwl":
        return E * 2 * N, lvl_flops
    if family == "plane_dwc":  # base and level 1
        return E * 2 * N, 2 * N * kk + (2 * 4 * blocks[1] * kk if levels >= 1 else 0)
    if family == "plane_dwd":  # levels 2..L
        return E * 2 * N, sum(2 * 4 * blocks[l] * kk for l in range(2, levels + 1))
    if family == "level_fwd":
        l = level
        elems = blocks[l - 1] + 4 * blocks[l] + (blocks[l] if l < levels else 0)
        return E * elems, 2 * 4 * blocks[l] * kk
    if family == "synth":
        q = sum(4 * blocks[l] for l in range(1, levels + 1))
        return E * (2 * N + q), 2 * N * kk
    if family == "carrier":
        return E * (blocks[level - 1] + blocks[level]), 0
    if family == "level_acc":
        l = level
        elems = blocks[l - 1] + 4 * blocks[l] + (4 * blocks[l + 1] if l < levels else 0)
        return E * elems, 2 * 4 * blocks[l] * kk
    if family == "dwc_tile" and level >= 2:  # level l from the level-(l - 1) carriers
        l = level
        elems = 2 * blocks[l - 1] + (2 * blocks[l] if l < levels else 0)
        return E * elems, 2 * 4 * blocks[l] * kk
    if family == "dwc_tile":
        return E * (2 * N + (2 * blocks[1] if levels >= 2 else 0)), \
            2 * N * kk + (2 * 4 * blocks[1] * kk if levels >= 1 else 0)
    if family == "mma_tile":
        q = 4 * blocks[2] if levels >= 2 else 0
        return E * (2 * N + q), 2 * N * kk + (2 * 4 * blocks[1] * kk if levels >= 1 else 0)
    if family == "dw_level":
        l = level
        elems = 2 * blocks[l - 1] + (2 * blocks[l] if l < levels else 0)
        return E * elems, 2 * 4 * blocks[l] * kk
    if family in ("dw_base", "plane_dwb"):
        return E * 2 * N, 2 * N * kk
    if family == "dw_finalize":
        return 0, 0
    raise ValueError(f"unknown kernel family {family!r}")


def split_name(name):
    """'level_fwd<5,bf16>#2' -> ('level_fwd', 2); 'synth' -> ('synth', 0)."""
    base, _, lvl = name.partition("#")
    return base.partition("<")[0], int(lvl) if lvl else 0


def launches(n, c, h, w, k, levels, elem_bytes, plane_fwd=False, plane_dw=False):
    """List of (name, pass, bytes, flops) for one forward + input-gradient +
    weight-gradient step of one layer, in launch order; per-level kernels are
    named family#level, as the library's profiling records name them.  The flags
    select the plane-resident kernels for the forward-shaped passes and for the
    weight gradients."""
    def one(fam, l, pass_name):
        b, f = kernel_cost(fam, l, n, c, h, w, k, levels, elem_bytes)
        return (f"{fam}#{l}" if l else fam, pass_name, b, f)

    out = []
    for pass_name in ("forward", "backward_input"):
        if plane_fwd:
            out.append(one("plane_fwd", 0, pass_name))
        else:
            out.extend(one("level_fwd", l, pass_name) for l in range(1, levels + 1))
            out.append(one("synth", 0, pass_name))
    if levels > 0:
        if plane_dw:
            out.append(one("plane_dwl", 0, "backward_weight"))
        else:
            out.extend(one("dw_level", l, "backward_weight") for l in range(1, levels + 1))
    out.append(one("plane_dwb" if plane_dw else "dw_base", 0, "backward_weight"))
    out.append(one("dw_finalize", 0, "backward_weight"))
    return out


def launches_from_plan(n, c, h, w, k, levels, elem_bytes, plan):
    """Same as `launches`, for the kernel names a library plan lists per pass:
    `plan` maps 'forward', 'backward_input', 'backward_weight' to name lists."""
    out = []
    for pass_name in ("forward", "backward_input", "backward_weight"):
        for name in plan[pass_name]:
            fam, l = split_name(name)
            b, f = kernel_cost(fam, l, n, c, h, w, k, levels, elem_bytes)
            out.append((name, pass_name, b, f))
    return out


def model_bytes(n, c, h, w, levels, elem_bytes):
    """Bytes of one forward + input-gradient + weight-gradient step of one layer
    in the per-level pass structure of the paper's fused layer (module docstring),
    exact for odd sizes: {"forward", "backward_input", "backward_weight", "step"}."""
    P = n * c
    N = P * h * w
    hs, ws = level_sizes(h, w, levels)
    blocks = [P * hs[l] * ws[l] for l in range(levels + 1)]
    fwd = 0
    for l in range(1, levels + 1):
        fwd += blocks[l - 1] + 4 * blocks[l] + (blocks[l] if l < levels else 0)
    fwd += 2 * N + sum(4 * blocks[l] for l in range(1, levels + 1))
    if levels == 0:
        bw = 2 * N
    else:
        bw = sum(2 * blocks[l - 1] + (2 * blocks[l] if l < levels else 0) for l in range(1, levels + 1))
    out = {"forward": elem_bytes * fwd, "backward_input": elem_bytes * fwd, "backward_weight": elem_bytes * bw}
    out["step"] = out["forward"] + out["backward_input"] + out["backward_weight"]
    return out


def conv_flops(n, c, h, w, k, levels):
    """Convolution FLOPs of one direction (2 per multiply-add): N k^2 + sum_l 4 B_l k^2."""
    P = n * c
    hs, ws = level_sizes(h, w, levels)
    return 2 * k * k * (P * h * w + sum(4 * P * hs[l] * ws[l] for l in range(1, levels + 1)))


def step_totals(n, c, h, w, k, levels, elem_bytes, **flags):
    ls = launches(n, c, h, w, k, levels, elem_bytes, **flags)
    return sum(b for _, _, b, _ in ls), sum(f for _, _, _, f in ls)


def paper_q_ref(levels):
    """Eq. 2: elements per forward pass of the reference chain, in units of N."""
    return 7.0 + 43.0 / 3.0 * (1.0 - 4.0 ** -levels)


def paper_q_fused(levels):
    """Eq. 10: elements per forward pass of the paper's fused layer, in units of N."""
    return 4.0 + 13.0 / 3.0 * (1.0 - 4.0 ** -levels) - 4.0 ** -levels


def paper_macs(k, levels):
    """Eq. 3: multiply-accumulates of the reference per forward pass, in units of N."""
    return k * k + (k * k + 8) * 4.0 / 3.0 * (1.0 - 4.0 ** -levels)
