"""Algorithmic HBM bytes and FLOPs of every kernel launch of the layer.

"Algorithmic" means what each kernel must move and compute by its design, in the
units the paper's I/O model uses ("Fast and Memory-Efficient Wavelet Convolutions
via I/O-Aware Reformulation", §3.1 Eq. 2 and §4.4 Eq. 10: every tensor a stage
reads or writes crosses HBM once), with exact element counts including the
pad-to-even of odd planes.  Parameters, weight-gradient partials and halo
re-reads are not counted (they are O(C k^2) or cache hits).

Per launch, with E = element size, P = n*C planes, H_l x W_l the level-l grid:
  level_fwd l  : reads the carrier P*H_{l-1}*W_{l-1}; writes Q(l) 4*P*H_l*W_l and,
                 for l < L, the carrier P*H_l*W_l.
                 FLOPs: 2*4*k^2 per coefficient block (the conv), 8 (analysis)
                 and 12 (one-step synthesis) per block.
  synth        : reads x (N) and every Q(l); writes y (N).
                 FLOPs: 2*k^2 per pixel (base conv) + L adds.
  dw_level l   : reads the x and dy carriers (2*P*H_{l-1}*W_{l-1}); writes both
                 next carriers for l < L.  FLOPs: 2*4*k^2 + 16 per block.
  dw_base      : reads x and dy (2N).  FLOPs: 2*k^2 + 1 per pixel.
  dw_finalize  : parameter-sized, counted as 0.
backward_input launches the same kernels as forward.
"""
from __future__ import annotations


def level_sizes(h, w, levels):
    hs, ws = [h], [w]
    for _ in range(levels):
        hs.append((hs[-1] + 1) // 2)
        ws.append((ws[-1] + 1) // 2)
    return hs, ws


def launches(n, c, h, w, k, levels, elem_bytes):
    """List of (name, pass, bytes, flops) for one forward + input-gradient +
    weight-gradient step of one layer, in launch order; per-level kernels are
    named family#level, as the library's profiling records name them."""
    P = n * c
    N = P * h * w
    E = elem_bytes
    hs, ws = level_sizes(h, w, levels)
    out = []
    for pass_name in ("forward", "backward_input"):
        for l in range(1, levels + 1):
            blocks = P * hs[l] * ws[l]
            elems = P * hs[l - 1] * ws[l - 1] + 4 * blocks + (blocks if l < levels else 0)
            out.append((f"level_fwd#{l}", pass_name, E * elems, blocks * (8 * k * k + 20)))
        q = sum(4 * P * hs[l] * ws[l] for l in range(1, levels + 1))
        out.append(("synth", pass_name, E * (2 * N + q), N * (2 * k * k + levels)))
    for l in range(1, levels + 1):
        blocks = P * hs[l] * ws[l]
        elems = 2 * P * hs[l - 1] * ws[l - 1] + (2 * blocks if l < levels else 0)
        out.append((f"dw_level#{l}", "backward_weight", E * elems, blocks * (8 * k * k + 16)))
    out.append(("dw_base", "backward_weight", E * 2 * N, N * (2 * k * k + 1)))
    out.append(("dw_finalize", "backward_weight", 0, 0))
    return out


def step_totals(n, c, h, w, k, levels, elem_bytes):
    ls = launches(n, c, h, w, k, levels, elem_bytes)
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
