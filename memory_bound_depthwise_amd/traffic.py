"""Algorithmic HBM bytes and FLOPs of every kernel launch of the layer.

"Algorithmic" means what each kernel must move and compute by its design, in the
units the paper's I/O model uses ("Fast and Memory-Efficient Wavelet Convolutions
via I/O-Aware Reformulation", §3.1 Eq. 2 and §4.4 Eq. 10: every tensor a stage
reads or writes crosses HBM once), with exact element counts including the
pad-to-even of odd planes.  Parameters, weight-gradient partials and halo
re-reads are not counted (they are O(C k^2) or cache hits).

Per launch, with E = element size, P = n*C planes, H_l x W_l the level-l grid,
B_l = P*H_l*W_l coefficient blocks of level l:
  Plane-resident kernels (the whole pyramid of a plane stays in LDS):
  fused_fwd,
  plane_fwd    : read x (N), write y (N).  FLOPs: the per-level kernels' total,
                 sum_l B_l*(8k^2 + 20) + N*(2k^2 + L).
  fused_dw,
  plane_dwl    : read x and dy (2N).  FLOPs: sum_l B_l*(8k^2 + 16).
  Per-level kernels:
  level_fwd l  : reads the carrier P*H_{l-1}*W_{l-1}; writes Q(l) 4*B_l and,
                 for l < L, the carrier B_l.
                 FLOPs: 2*4*k^2 per coefficient block (the conv), 8 (analysis)
                 and 12 (one-step synthesis) per block.
  synth        : reads x (N) and every Q(l); writes y (N).
                 FLOPs: 2*k^2 per pixel (base conv) + L adds.
  dw_level l   : reads the x and dy carriers (2*P*H_{l-1}*W_{l-1}); writes both
                 next carriers for l < L.  FLOPs: 2*4*k^2 + 16 per block.
  Both paths:
  dw_base,
  plane_dwb    : read x and dy (2N).  FLOPs: 2*k^2 + 1 per pixel.
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
    if family in ("fused_fwd", "plane_fwd"):
        fl = sum(blocks[l] * (8 * k * k + 20) for l in range(1, levels + 1)) + N * (2 * k * k + levels)
        return E * 2 * N, fl
    if family in ("fused_dw", "plane_dwl"):
        return E * 2 * N, sum(blocks[l] * (8 * k * k + 16) for l in range(1, levels + 1))
    if family == "level_fwd":
        l = level
        elems = blocks[l - 1] + 4 * blocks[l] + (blocks[l] if l < levels else 0)
        return E * elems, blocks[l] * (8 * k * k + 20)
    if family == "synth":
        q = sum(4 * blocks[l] for l in range(1, levels + 1))
        return E * (2 * N + q), N * (2 * k * k + levels)
    if family == "dw_level":
        l = level
        elems = 2 * blocks[l - 1] + (2 * blocks[l] if l < levels else 0)
        return E * elems, blocks[l] * (8 * k * k + 16)
    if family in ("dw_base", "plane_dwb"):
        return E * 2 * N, N * (2 * k * k + 1)
    if family == "dw_finalize":
        return 0, 0
    raise ValueError(f"unknown kernel family {family!r}")


def split_name(name):
    """'level_fwd<5,bf16>#2' -> ('level_fwd', 2); 'synth' -> ('synth', 0)."""
    base, _, lvl = name.partition("#")
    return base.partition("<")[0], int(lvl) if lvl else 0


def launches(n, c, h, w, k, levels, elem_bytes, fused_fwd=False, fused_dw=False):
    """List of (name, pass, bytes, flops) for one forward + input-gradient +
    weight-gradient step of one layer, in launch order; per-level kernels are
    named family#level, as the library's profiling records name them.  The flags
    select the plane-resident kernels for the forward-shaped passes and for the
    levels' weight gradients."""
    def one(fam, l, pass_name):
        b, f = kernel_cost(fam, l, n, c, h, w, k, levels, elem_bytes)
        return (f"{fam}#{l}" if l else fam, pass_name, b, f)

    out = []
    for pass_name in ("forward", "backward_input"):
        if fused_fwd:
            out.append(one("fused_fwd", 0, pass_name))
        else:
            out.extend(one("level_fwd", l, pass_name) for l in range(1, levels + 1))
            out.append(one("synth", 0, pass_name))
    if levels > 0:
        if fused_dw:
            out.append(one("fused_dw", 0, "backward_weight"))
        else:
            out.extend(one("dw_level", l, "backward_weight") for l in range(1, levels + 1))
    out.append(one("dw_base", 0, "backward_weight"))
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
