// Host side of libwtconv.so: argument checks, launch plans, workspace sizes,
// profiling records and the C ABI declared in include/wtconv.h.  The launch
// sequences themselves are compiled once per kernel size and activation type
// (wtconv_inst.hip, wtconv_run.hpp) and called through wtconv_host.hpp.
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation".  Launch sequence per call:
//   forward / backward_input : the plane-resident kernel, or the level kernel for
//                              l = 1..L (§4.1) and the closed-form synthesis +
//                              base kernel (§4.2-4.4);
//   backward_weight          : level gradient kernel(s), base gradient kernel,
//                              finalize (fixed-order sums + Eq. 9).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "wtconv.h"
#include "wtconv_host.hpp"

namespace wtc {

constexpr size_t kLdsBudget = 64 * 1024;   // bytes of LDS per workgroup of the per-level kernels
constexpr int kDwTargetBlocks = 2048;      // workgroups wanted for the gradient kernels
constexpr int kPlaneMaxSide = 64;          // largest plane side of the plane-resident kernels
constexpr int kPlanCUs = 256;              // compute units the launch plans are sized for
#ifndef WTC_FWD_PB_CAP
#define WTC_FWD_PB_CAP 64
#endif
#ifndef WTC_DW_PB_CAP
#define WTC_DW_PB_CAP 64
#endif
#ifndef WTC_DW_WG_PER_CU
#define WTC_DW_WG_PER_CU 4
#endif
constexpr int kFwdPbCap = WTC_FWD_PB_CAP;  // planes side by side in one pass of the forward kernel
constexpr int kDwPbCap = WTC_DW_PB_CAP;    // ... of the weight-gradient kernels
constexpr int kDwWgPerCu = WTC_DW_WG_PER_CU;  // resident weight-gradient workgroups per CU aimed at

// Reciprocal for udiv16 (exact n / d for n < 2^16, d < 2^15): ceil(2^31 / d).
inline uint32_t magic31_of(int d) { return (uint32_t)(((1ULL << 31) + (uint64_t)d - 1) / (uint64_t)d); }

// ---------------------------------------------------------------------------
// Profiling: hipEvent pairs around each launch, on the launch stream.
// ---------------------------------------------------------------------------

namespace {

struct ProfRecord {
    std::string name;
    hipEvent_t start, stop;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}


}  // namespace

bool prof_events(hipEvent_t &ev0, hipEvent_t &ev1) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_prof_on) return false;
    ev0 = pooled_event();
    ev1 = pooled_event();
    return ev0 && ev1;
}

void prof_record(const char *family, int K, int dtype, int level, hipEvent_t ev0, hipEvent_t ev1) {
    char name[64];
    if (level > 0)
        snprintf(name, sizeof(name), "%s<%d,%s>#%d", family, K, dtype_name(dtype), level);
    else
        snprintf(name, sizeof(name), "%s<%d,%s>", family, K, dtype_name(dtype));
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof.push_back({name, ev0, ev1});
}

namespace {

// ---------------------------------------------------------------------------
// Shapes, tiling and the workspace plan of the per-level kernels
// ---------------------------------------------------------------------------

LevelDims level_dims(const wtconv_desc &d) {
    LevelDims ld;
    ld.H[0] = d.h;
    ld.W[0] = d.w;
    for (int l = 1; l <= d.levels; ++l) {
        ld.H[l] = (ld.H[l - 1] + 1) / 2;
        ld.W[l] = (ld.W[l - 1] + 1) / 2;
    }
    return ld;
}

// Lanes that work on one item stream: a wavefront per band for the level kernels,
// the whole workgroup otherwise.
int lane_group(Kind kind) { return (kind == Kind::LevelFwd || kind == Kind::DwLevel) ? kWave : kThreads; }

// Tile an Ho x Wo output grid.  Tiles are at most one lane group wide (a full row
// for the small planes of the WTConvNeXt stages) and as tall as needed for about 4
// strips per lane group; then as many planes are stacked per pass as give the
// best lane occupancy within the LDS budget, keeping at least ~2 workgroups per
// compute unit when the problem allows.
Tiling pick_tiling(Kind kind, int K, int n, int C, int Ho, int Wo, int VW) {
    Tiling t{};
    t.VW = VW;
    if (n <= 0 || Ho <= 0 || Wo <= 0) {
        t.TY = t.TX = t.SP = t.tiles_x = t.PB = t.NB = 1;
        t.tiles = t.nblk = 0;
        return t;
    }
    const int U = lane_group(kind);
    // A tile is at most as wide as its lane group (a wavefront per band for the
    // level kernels, the workgroup otherwise): wide tiles keep the halo columns and
    // the partly used cache lines at the row ends a small share of what is staged.
    t.tiles_x = cdiv(Wo, U);
    t.TX = cdiv(Wo, t.tiles_x);
    int sp_max = std::max(1, cdiv(4 * U, t.TX));
    for (;;) {
        const int tiles_y = cdiv(Ho, sp_max * kRH);
        t.TY = cdiv(Ho, tiles_y);
        t.SP = cdiv(t.TY, kRH);
        t.tiles = tiles_y * t.tiles_x;
        t.PB = 1;
        if (sp_max == 1 || lds_bytes(kind, K, t) <= kLdsBudget) break;
        sp_max = std::max(1, sp_max / 2);
    }
    // the synthesis kernel reads the deep levels per strip of kRH rows aligned to kRH
    if (kind == Kind::Synth) t.TY = t.SP * kRH;
    // plane stacking: best lane occupancy, then the smaller PB
    const long long min_blocks = 512;
    double best = -1.0;
    int best_pb = 1;
    for (int pb = 1; pb <= std::min(n, 64); ++pb) {
        Tiling c = t;
        c.PB = pb;
        if (lds_bytes(kind, K, c) > kLdsBudget) break;
        if (pb > 1 && (long long)t.tiles * C * cdiv(n, pb) < min_blocks) break;
        const long long items = (long long)pb * t.SP * t.TX;
        const double occ = (double)items / (double)(cdiv(items, U) * (long long)U);
        if (occ > best + 1e-9) {
            best = occ;
            best_pb = pb;
        }
    }
    t.PB = best_pb;
    if (kind == Kind::LevelFwd || kind == Kind::Synth) {
        t.NB = t.PB;
    } else {
        // gradient kernels walk several planes per workgroup to amortise the
        // reduction; keep enough workgroups to fill the chip
        const long long per_nb = (long long)C * t.tiles;
        const int want_nblk = std::max(1, (int)std::min<long long>(n, cdiv(kDwTargetBlocks, std::max(1LL, per_nb))));
        int nb = cdiv(n, want_nblk);
        nb = cdiv(nb, t.PB) * t.PB;
        t.NB = std::max(t.PB, nb);
    }
    t.nblk = cdiv(n, t.NB);
    return t;
}

bool tiling_fits(Kind kind, int K, const Tiling &t) { return lds_bytes(kind, K, t) <= kLdsBudget; }

// ---------------------------------------------------------------------------
// Plane-resident forward on the polyphase grid: layout, stacking, bank-aware strides
// ---------------------------------------------------------------------------

constexpr int kPlaneLdsBudget = 40960;  // four workgroups per compute unit


// Bank cost of cell reads by items (strip s, plane p, column j), item t =
// (s PB + p) W1 + j on lane t, cell s RH sy + p Pw1 + j: gfx950 serves a 16-byte
// read 16 lanes at a time from 64 banks (an 8-byte read 32 lanes at a time), so
// the read is conflict-free when the cells of those lanes are distinct mod 16 (mod
// 32).  Cost: per group of lanes served together the largest number of them
// sharing a slot (1 = conflict-free), summed.
long long cell_bank_cost(int items, int pb, int W1, int pitch, int RH, int sy, int group = 16) {
    long long cost = 0;
    const int per_strip = pb * W1;
    for (int g = 0; g * group < items; ++g) {
        int cnt[32] = {0};
        int worst = 0;
        for (int t = g * group; t < std::min(items, g * group + group); ++t) {
            const int s = t / per_strip, r = t % per_strip, p = r / W1, j = r % W1;
            const int cell = s * RH * sy + p * pitch + j;
            worst = std::max(worst, ++cnt[cell & (group - 1)]);
        }
        cost += worst;
    }
    return cost;
}

// Smallest row stride in [lo, lo + group) with the least bank cost.
int best_stride(int items, int pb, int W1, int pitch, int RH, int lo, int group = 16) {
    long long best = -1;
    int sy = lo;
    for (int cand = lo; cand < lo + group; ++cand) {
        const long long cost = cell_bank_cost(items, pb, W1, pitch, RH, cand, group);
        if (best < 0 || cost < best) {
            best = cost;
            sy = cand;
        }
    }
    return sy;
}

// Layout for pb planes per pass; false when it does not fit.  Grid arrays hold one
// float4 per cell (polyphase components of x, or the four bands of a level).
bool plane_layout(const wtconv_desc &d, const PlaneCfg &cfg, int pb, PlaneArgs &a) {
    const int K = d.k, KK = K * K, R = (K - 1) / 2, L = d.levels, RH = cfg.RH, CW = cfg.CW;
    a = PlaneArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.L = L;
    a.PB = pb;
    a.H1 = (d.h + 1) / 2;
    a.W1 = (d.w + 1) / 2;
    a.S1 = cdiv(a.H1, RH);
    a.Gw = cdiv(a.W1, CW);
    // the level-1 grid is laid out also for L = 0 (cells of 2 x 2 pixels)
    const int Lg = std::max(L, 1);
    int hs[kMaxLevels + 1], ws[kMaxLevels + 1];
    hs[0] = d.h;
    ws[0] = d.w;
    for (int l = 1; l <= Lg; ++l) {
        hs[l] = (hs[l - 1] + 1) / 2;
        ws[l] = (ws[l - 1] + 1) / 2;
    }
    // column pitch between side-by-side planes: at every level the gap is >= R
    if (pb == 1) {
        a.Pw1 = a.W1;
    } else {
        int pwL = 1;
        for (int l = 1; l <= Lg; ++l) pwL = std::max(pwL, cdiv(ws[l] + R, 1LL << (Lg - l)));
        while (((long long)pwL << (Lg - 1)) % CW) ++pwL;
        a.Pw1 = pwL << (Lg - 1);
    }
    const int W1s = pb == 1 ? a.W1 : pb * a.Pw1;
    a.commit_items = pb * a.H1 * a.Gw;
    a.final_items = a.S1 * pb * a.W1;
    // one final item per lane (each keeps its filtered bands across the in-place
    // rebuild of the cells); a single plane of at most 64 x 64 always fits
    if (a.final_items > kFwdThreads || a.commit_items >= 32768) return false;
    if ((long long)pb * d.c * d.h * d.w >= (1LL << 31)) return false;  // 32-bit offsets from a plane base
    // level-1 arrays: the stride (cells) with the fewest bank conflicts in the final pass
    a.sy1 = best_stride(a.final_items, pb, a.W1, a.Pw1, RH, kPlaneCO + W1s + R);
    a.a1 = (a.S1 * RH + 2 * R) * a.sy1;
    long long cells = a.a1;
    int deep = 0;
    for (int l = 2; l <= L; ++l) {
        const int li = l - 2;
        a.hl[li] = hs[l];
        a.wls[li] = pb == 1 ? ws[l] : (pb * a.Pw1) >> (l - 1);
        a.sd[li] = cdiv(hs[l], kPlaneRHd);
        a.syd[li] = kPlaneCO + a.wls[li] + R;
        a.offd[li] = (int)cells;
        cells += (long long)(a.sd[li] * kPlaneRHd + 2 * R) * a.syd[li];
        deep += a.sd[li] * a.wls[li];
        a.dend[li] = deep;
        if ((long long)a.hl[li] * a.wls[li] >= 32768 || deep >= 32768) return false;
    }
    long long fl = 4 * cells;  // floats
    for (int l = 2; l <= L; ++l) {
        const int li = l - 2;
        a.sq[li] = 2 * a.wls[li];
        a.offq[li] = (int)fl;
        fl += ((2LL * hs[l] * a.sq[li]) + 3) & ~3LL;
    }
    a.wt = (int)fl;
    fl += ((4LL * L + 1) * KK + 1 + 3) & ~3LL;  // weights, then the folded bias
    a.zero_floats = (int)fl;
    a.tab = (int)fl;  // deep-level geometry table, filled once per workgroup
    fl += (kPlaneTabFields * std::max(L - 1, 0) + 3) & ~3;
    // the final pass reads the deep patterns of every item row, also of rows past
    // the plane (their outputs are discarded): keep those reads in the allocation
    for (int l = 2; l <= L; ++l) {
        const int li = l - 2;
        const long long end = a.offq[li] + (long long)((a.S1 * RH - 1) >> li) * a.sq[li] + ((W1s - 1) >> li) + 1;
        fl = std::max(fl, (end + 3) & ~3LL);
    }
    a.lds_floats = (int)fl;
    if (fl * 4 > kPlaneLdsBudget) return false;
    a.m_gw = magic31_of(a.Gw);
    a.m_h1 = magic31_of(a.H1);
    a.m_strip = magic31_of(pb * a.W1);
    a.m_w1 = magic31_of(a.W1);
    for (int l = 2; l <= L; ++l) a.m_wls[l - 2] = magic31_of(a.wls[l - 2]);
    return true;
}

// Choose the variant (CW, RH), PB and the planes per workgroup; false when the
// shape is outside the kernel's range.
bool plan_plane(const wtconv_desc &d, PlaneArgs &a, PlaneCfg &cfg) {
    if (d.levels < 0 || d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kPlaneMaxSide || d.w > kPlaneMaxSide) return false;
    const int H1 = (d.h + 1) / 2;
    cfg.RH = H1 % 7 == 0 ? 7 : (H1 <= 4 ? 4 : 8);
    cfg.CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    const int K = d.k;
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, kFwdPbCap); ++pb) {
        PlaneArgs t{};
        if (!plane_layout(d, cfg, pb, t)) {
            if (pb == 1) return false;
            break;
        }
        // wave-instructions per pass: a final item is ~(4 + 4) RH K^2 FMAs plus
        // ~60 RH others, a deep item 4 kPlaneRHd K^2; commit and Haar ~30 per item;
        // ~400 fixed
        const double fin = cdiv(t.final_items, kFwdThreads) * 2.0 * ((d.levels ? 8.0 : 4.0) * cfg.RH * K * K + 60.0 * cfg.RH);
        const int deep_items = d.levels >= 2 ? t.dend[d.levels - 2] : 0;
        const double deep = cdiv(deep_items, kFwdThreads) * 2.0 * (4.0 * kPlaneRHd * K * K + 60.0);
        const double misc = cdiv(t.commit_items, kFwdThreads) * 40.0 + 400.0;
        const double cost = (fin + deep + misc) / pb;
        if (cost < best - 1e-9) {
            best = cost;
            best_pb = pb;
        }
    }
    if (!plane_layout(d, cfg, best_pb, a)) return false;
    a.NG = cdiv(d.n, a.PB);
    const long long units = (long long)d.c * a.NG;
    if (units >= (1LL << 31)) return false;
    a.U = (int)units;
    return true;
}

// ---------------------------------------------------------------------------
// Plane-resident forward kernel on the matrix cores (bfloat16 activations)
// ---------------------------------------------------------------------------

#ifndef WTC_MMA
#define WTC_MMA 1  // 0: bfloat16 forward-shaped passes on the vector kernel (for comparisons)
#endif
constexpr int kMmaLdsBudget = 40960;

// Layout for pb planes per pass; false when it does not fit.  The geometry
// constants follow MmaGeom (wtconv_mma.hpp).
bool mma_layout(const wtconv_desc &d, int CW, int pb, MmaArgs &a) {
    const int K = d.k, KK = K * K, R = (K - 1) / 2, L = d.levels;
    const int ROW0 = 2 * R, COL0 = 2 * R, RROWS = 8 + 4 * R;
    const bool TAIL = K == 5;
    a = MmaArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.L = L;
    a.PB = pb;
    a.H1 = (d.h + 1) / 2;
    a.W1 = (d.w + 1) / 2;
    a.Gw = cdiv(a.W1, CW);
    const int Lg = std::max(L, 1);
    int hs[kMaxLevels + 1], ws[kMaxLevels + 1];
    hs[0] = d.h;
    ws[0] = d.w;
    for (int l = 1; l <= Lg; ++l) {
        hs[l] = (hs[l - 1] + 1) / 2;
        ws[l] = (ws[l - 1] + 1) / 2;
    }
    // column pitch between side-by-side planes: at every level the gap is >= R
    // cells; a multiple of 4 cells (a lane's four output cells share a plane) that
    // holds every commit group
    if (pb == 1) {
        a.Pw1 = (std::max(a.W1, a.Gw * CW) + 3) & ~3;
    } else {
        int pwL = 1;
        for (int l = 1; l <= Lg; ++l) pwL = std::max(pwL, cdiv(ws[l] + R, 1LL << (Lg - l)));
        while (((long long)pwL << (Lg - 1)) % 4) ++pwL;
        a.Pw1 = pwL << (Lg - 1);
    }
    if (a.Pw1 < a.Gw * CW) return false;
    const int Wc = pb == 1 ? a.W1 : (pb - 1) * a.Pw1 + a.W1;  // cells of the side-by-side strip
    const int TY = cdiv(a.H1, 4);
    // A tile's 16 M rows are 16 consecutive strip columns, or (planes at most 16
    // cells wide) whole planes: MW = 4, 8 or 16 rows each, 16 / MW planes a tile and no
    // gap columns; whichever needs fewer tiles
    const int mw = a.W1 <= 4 ? 4 : (a.W1 <= 8 ? 8 : 16);
    const int tx_strip = cdiv(Wc, 16), tx_planes = cdiv(pb, 16 / mw);
    a.aligned = pb > 1 && a.W1 <= 16 && tx_planes < tx_strip ? 1 : 0;
    a.MW = a.aligned ? mw : 16;
    a.TX = a.aligned ? tx_planes : tx_strip;
    // last strip column a tile reads
    const long long cmax = a.aligned ? (long long)(a.TX * (16 / a.MW) - 1) * a.Pw1 + a.MW - 1 : 16LL * a.TX - 1;
    a.tiles = TY * a.TX;
    a.commit_items = pb * a.H1 * a.Gw;
    a.H2 = (a.H1 + 1) / 2;
    a.pair_items = pb * a.H2 * a.Gw;
    if (a.commit_items >= 32768 || a.tiles >= 32768) return false;
    if ((long long)pb * d.c * d.h * d.w >= (1LL << 31)) return false;
    // canvas: bfloat16 pixels, row y of the strip at canvas row ROW0 + y, column x at
    // kMmaCL + x; the row stride (dwords) is 16 mod 32, so that the four lane
    // groups of an A read (four consecutive rows) fall on four distinct bank ranges
    const long long s_min = std::max<long long>(kMmaCL / 2 + (long long)pb * a.Pw1,
                                                (kMmaCL - COL0) / 2 + cmax + 1 + 4 + (TAIL ? 1 : 0));
    long long S = s_min;
    while (S % 32 != 16) ++S;
    a.S = (int)S;
    long long rows = std::max<long long>(ROW0 + 2LL * a.H1, 8LL * (TY - 1) + RROWS);
    if (L >= 2) rows = std::max<long long>(rows, ROW0 + 4LL * hs[2]);
    long long cells = (rows * S + 3) / 4;  // float4 cells after the canvas
    int deep = 0;
    for (int l = 2; l <= L; ++l) {
        const int li = l - 2;
        a.hl[li] = hs[l];
        a.wls[li] = pb == 1 ? ws[l] : (pb * a.Pw1) >> (l - 1);
        a.sd[li] = cdiv(hs[l], kPlaneRHd);
        a.syd[li] = kPlaneCO + a.wls[li] + R;
        a.offd[li] = (int)cells;
        cells += (long long)(a.sd[li] * kPlaneRHd + 2 * R) * a.syd[li];
        deep += a.sd[li] * a.wls[li];
        a.dend[li] = deep;
        if ((long long)a.hl[li] * a.wls[li] >= 32768 || deep >= 32768) return false;
    }
    long long fl = 4 * cells;
    for (int l = 2; l <= L; ++l) {
        const int li = l - 2;
        a.sq[li] = li == 0 ? (2 * a.wls[li] + 3) & ~3 : 2 * a.wls[li];  // level 2: float4 rows
        a.offq[li] = (int)fl;
        fl += ((2LL * hs[l] * a.sq[li]) + 3) & ~3LL;
    }
    a.wt = (int)fl;
    fl += ((4LL * L + 1) * KK + 1 + 3) & ~3LL;
    a.zero_floats = (int)fl;
    a.tab = (int)fl;
    fl += (kPlaneTabFields * std::max(L - 1, 0) + 3) & ~3;
    // the tiles read the deep patterns of every tile cell, also past the plane
    for (int l = 2; l <= L; ++l) {
        const int li = l - 2;
        const long long end = a.offq[li] + (long long)((4 * TY - 1) >> li) * a.sq[li] + (cmax >> li) + 1;
        fl = std::max(fl, (end + 3) & ~3LL);
    }
    // the B table: in the level-2 pattern region when it fits there (the table is
    // read before the deep phase writes the patterns), else after everything
    const int bwords = 4 * (2 * K) * (K == 5 ? 12 : 8);
    if (L >= 2 && 2LL * hs[2] * a.sq[0] >= bwords) {
        a.btab = a.offq[0];
        a.btab_alias = 1;
    } else {
        a.btab = (int)fl;
        a.btab_alias = 0;
        fl += bwords;
    }
    a.lds_floats = (int)fl;
    if (fl * 4 > kMmaLdsBudget) return false;
    a.m_gw = magic31_of(a.Gw);
    a.m_h1 = magic31_of(a.H1);
    a.m_tx = magic31_of(a.TX);
    a.m_pw1 = magic31_of(a.Pw1);
    a.m_h2 = magic31_of(a.H2);
    for (int l = 2; l <= L; ++l) a.m_wls[l - 2] = magic31_of(a.wls[l - 2]);
    return true;
}

// bfloat16 planes 7..64 pixels on a side, levels >= 1, k = 3 or 5.
// Chooses CW and PB; false when the shape is outside the kernel's range.
bool plan_mma(const wtconv_desc &d, MmaArgs &a, int &CW) {
    if (!WTC_MMA || d.dtype != WTCONV_BF16) return false;
    if (d.levels < 1 || d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kPlaneMaxSide || d.w > kPlaneMaxSide || d.k > 5) return false;
    // a tile is 16 x 4 cells: planes under 4 x 4 cells leave most of a tile empty
    // and stay on the vector kernel, and so do planes without levels (measured: the
    // base conv alone is too little work per pass to keep the latency of the
    // products hidden); from 7 x 7 pixels up, planes stacked side by side fill the
    // tiles well enough (measured faster than the vector kernel at 7 x 7 and 14 x 14)
    if ((d.w + 1) / 2 < 4 || (d.h + 1) / 2 < 4) return false;
    CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    const int K = d.k;
    const int nfrag = K == 5 ? 5 : 3;  // B fragments (hi and lo each)
    // Workgroups per compute unit as the registers allow (~167 VGPRs: 3 waves per
    // SIMD); the LDS of a layout may allow fewer.  The kernel is latency-bound, so
    // the choice weighs the resident passes as well as the work per pass, and the
    // rounds of passes a workgroup runs: ceil(units / resident workgroups) (a last,
    // partial round costs a whole one).
    const int wg_regs = 6;
    double best = -1.0;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, kFwdPbCap); ++pb) {
        MmaArgs t{};
        if (!mma_layout(d, CW, pb, t)) {
            if (pb == 1) return false;
            break;
        }
        const int wg = std::max(1, std::min(wg_regs, (int)((160 * 1024) / ((long long)t.lds_floats * 4))));
        // wave-instructions per pass: a tile ~8 per fragment (two 16-cycle products)
        // plus ~20 others; deep items as in the vector kernel; commit ~20 per item;
        // ~300 fixed
        const double tiles = cdiv(t.tiles, kMmaThreads / kWave) * 2.0 * (8.0 * nfrag + 20.0);
        const int deep_items = d.levels >= 2 ? t.dend[d.levels - 2] : 0;
        const double deep = cdiv(deep_items, kMmaThreads) * 2.0 * (4.0 * kPlaneRHd * K * K + 60.0);
        const double misc = cdiv(t.commit_items, kMmaThreads) * 2.0 * 20.0 + 300.0;
        const long long units = (long long)d.c * cdiv(d.n, pb);
        const double rounds = (double)cdiv(units, (long long)kPlanCUs * wg);
        // time per pass grows as fewer passes share a compute unit (latency-bound)
        const double score = 1.0 / (rounds * (tiles + deep + misc) * wg_regs / wg);
        if (score > best * (1 + 1e-9)) {
            best = score;
            best_pb = pb;
        }
    }
    if (!mma_layout(d, CW, best_pb, a)) return false;
    a.NG = cdiv(d.n, a.PB);
    const long long units = (long long)d.c * a.NG;
    if (units >= (1LL << 31)) return false;
    a.U = (int)units;
    return true;
}

// The tiled matrix-core forward for planes past the plane-resident range: bfloat16,
// levels >= 1, k = 3 or 5.  A pass is a tile of UR x UC level-1 cells (at most
// 16 x 64, narrower planes take fewer), its canvas the tile's pixels and the 2R
// halo pixels on each side, staged in chunks of 8 pixels.
bool plan_mma_tile(const wtconv_desc &d, MmaTileArgs &a) {
    if (!WTC_MMA || d.dtype != WTCONV_BF16) return false;
    if (d.levels < 1 || d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0 || d.k > 5) return false;
    const int R = (d.k - 1) / 2, KK = d.k * d.k;
    a = MmaTileArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.L = d.levels;
    const int H1 = (d.h + 1) / 2, W1 = (d.w + 1) / 2;
    a.UR = std::min(16, 4 * cdiv(H1, 4));
    a.UC = std::min(64, 16 * cdiv(W1, 16));
    a.TYu = cdiv(H1, a.UR);
    a.TXu = cdiv(W1, a.UC);
    a.rows = 2 * a.UR + 4 * R;
    a.chunks = 2 + a.UC / 4;  // canvas columns X0 - 8 .. X0 + 2 UC + 7
    a.items = a.rows * a.chunks;
    if (a.items > kTileSlots * kTileThreads) return false;
    int S = 4 * a.chunks;  // dwords; 16 mod 32, as in the plane-resident canvas
    while (S % 32 != 16) ++S;
    a.S = S;
    // the block of D (the deeper levels' patterns summed on the level-1 grid) after
    // the canvas: UR rows of UC cells, as pairs
    a.qbase = a.rows * S;
    a.qitems = d.levels >= 2 ? a.UR * (a.UC / 2) : 0;
    if (a.qitems > kTileQSlots * kTileThreads) return false;
    const LevelDims ld = level_dims(d);
    a.hq = d.levels >= 2 ? 2 * ld.H[2] : 0;
    a.wq = d.levels >= 2 ? 2 * ld.W[2] : 0;
    a.wt = (a.qbase + a.qitems + 3) & ~3;
    a.lds_floats = (a.wt + 5 * KK + 1 + 3) & ~3;
    const long long units = (long long)d.c * d.n * a.TYu * a.TXu;
    if (units >= (1LL << 31)) return false;
    a.U = (int)units;
    a.m_chunks = magic31_of(a.chunks);
    a.m_tx = magic31_of(a.UC / 16);
    a.m_qp = magic31_of(a.UC / 2);
    return true;
}

// ---------------------------------------------------------------------------
// Plane-resident base weight gradient (polyphase cells of x and dy)
// ---------------------------------------------------------------------------

constexpr int kDwbLdsBudget = 40960;  // four workgroups per compute unit

bool dwb_layout(const wtconv_desc &d, const PlaneCfg &cfg, int pb, PlaneDwbArgs &a) {
    const int K = d.k, KK = K * K, R = (K - 1) / 2, RC = (R + 1) / 2, RH = cfg.RH, CW = cfg.CW;
    a = PlaneDwbArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.PB = pb;
    a.H1 = (d.h + 1) / 2;
    a.W1 = (d.w + 1) / 2;
    a.S1 = cdiv(a.H1, RH);
    a.Gw = cdiv(a.W1, CW);
    a.Pw1 = pb == 1 ? a.W1 : cdiv(a.W1 + RC, CW) * CW;
    const int W1s = pb == 1 ? a.W1 : pb * a.Pw1;
    a.commit_items = pb * a.H1 * a.Gw;
    a.final_items = a.S1 * pb * a.W1;
    if (a.final_items >= 32768 || a.commit_items >= 32768) return false;
    if ((long long)pb * d.c * d.h * d.w >= (1LL << 31)) return false;  // 32-bit offsets from a plane base
    a.sx = best_stride(a.final_items, pb, a.W1, a.Pw1, RH, kPlaneCO + W1s + RC);
    a.ax = (a.S1 * RH + 2 * RC) * a.sx;
    a.sd = best_stride(a.final_items, pb, a.W1, a.Pw1, RH, W1s);
    const long long floats = 4LL * (a.ax + (long long)a.S1 * RH * a.sd);
    a.lds_floats = (int)std::max<long long>(floats, (long long)(kDwbThreads / kWave) * (KK + 1));
    a.lds_floats = (a.lds_floats + 3) & ~3;
    if ((long long)a.lds_floats * 4 > kDwbLdsBudget) return false;
    a.m_gw = magic31_of(a.Gw);
    a.m_h1 = magic31_of(a.H1);
    a.m_strip = magic31_of(pb * a.W1);
    a.m_w1 = magic31_of(a.W1);
    return true;
}

// Workgroups per channel for the plane-resident weight gradients: as many as fit
// on the device at once (resident workgroups per compute unit from the LDS size,
// at most four of two wavefronts each, x 256 compute units), at most one per image
// group.
int dw_blocks_per_channel(const wtconv_desc &d, int NG, int lds_floats) {
    const int per_cu = std::max(1, std::min(kDwWgPerCu, (160 * 1024) / std::max(1, lds_floats * 4)));
    return std::max(1, std::min(NG, 256 * per_cu / std::max(1, d.c)));
}

bool plan_dwb(const wtconv_desc &d, PlaneDwbArgs &a, PlaneCfg &cfg) {
    if (d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kPlaneMaxSide || d.w > kPlaneMaxSide) return false;
    const int H1 = (d.h + 1) / 2;
    cfg.RH = H1 % 7 == 0 ? 7 : (H1 <= 4 ? 4 : 8);
    cfg.CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, kDwPbCap); ++pb) {
        PlaneDwbArgs t{};
        if (!dwb_layout(d, cfg, pb, t)) {
            if (pb == 1) return false;
            break;
        }
        // wave-instructions per pass: an item is ~4 RH K^2 FMAs + 30 RH others
        const double cost = (cdiv(t.final_items, kDwbThreads) * 2.0 * (4.0 * cfg.RH * d.k * d.k + 30.0 * cfg.RH) +
                             cdiv(t.commit_items, kDwbThreads) * 60.0 + 200.0) / pb;
        if (cost < best - 1e-9) {
            best = cost;
            best_pb = pb;
        }
    }
    if (!dwb_layout(d, cfg, best_pb, a)) return false;
    a.NG = cdiv(d.n, a.PB);
    a.k = dw_blocks_per_channel(d, a.NG, a.lds_floats);
    return (long long)d.c * a.k < (1LL << 31);
}

// ---------------------------------------------------------------------------
// Plane-resident level weight gradients (band-major pyramids of x and dy)
// ---------------------------------------------------------------------------

constexpr int kDwlLdsBudget = 53248;  // three workgroups per compute unit

// Column stride (floats) >= lo for the column-major band arrays: a multiple of 4 with
// an odd quotient, so that 16 consecutive columns' 16-byte reads hit distinct
// groups of 4 banks (gfx950 serves 16 lanes of a 16-byte read per cycle).
int column_stride(int lo) {
    int s = (lo + 3) & ~3;
    if ((s / 4) % 2 == 0) s += 4;
    return s;
}

// Trips of the busiest wavefront of a lane table (the most items a lane runs: the
// item phase of a pass ends with it).
int dwl_wave_trips(const PlaneDwlArgs &a) {
    int total = 0;
    for (int w = 0; w < kDwlThreads / kWave; ++w) {
        int worst = 0;
        for (int t = w * kWave; t < (w + 1) * kWave; ++t) {
            const uint32_t in = a.lane[t];
            const int M = (in >> 16) & 255, l = (int)(in & 15) - 1;
            if (M) worst = std::max(worst, cdiv(a.ns[l] * a.PB * a.wr[l], M));
        }
        total = std::max(total, worst);
    }
    return total;
}

// Lanes per band of each level lfirst .. L - 1 (0-based) with items: M[l] lanes run
// ceil(items / M[l]) trips each.  For three levels or fewer the trips of each level
// are searched from the fewest its lanes allow (at most 64 lanes a band) to seven
// more, for the table (levels with more trips first) whose busiest wavefront has the
// fewest trips (a pass ends at a barrier), then the fewest wavefront trips in all
// (the issue work), then the fewest lane trips; with more levels, greedily (the
// largest item count of a lane made smallest).
bool dwl_lanes(const PlaneDwlArgs &a, int lfirst, int (&M)[kMaxLevels]) {
    const int L = a.L, nl = L - lfirst;
    constexpr int NWv = kDwlThreads / kWave;
    int items[kMaxLevels];
    for (int l = 0; l < L; ++l) {
        M[l] = 0;
        items[l] = l < lfirst ? 0 : a.ns[l] * a.PB * a.wr[l];
    }
    if (nl <= 0) return true;
    if (nl <= 3) {
        long long best = -1;
        int bestM[3] = {0, 0, 0}, t0[3] = {1, 1, 1}, span[3] = {1, 1, 1};
        for (int k = 0; k < nl; ++k) {
            t0[k] = std::max(1, cdiv(items[lfirst + k], kDwlThreads / 4));
            span[k] = 8;
        }
        int T[3];
        for (T[0] = t0[0]; T[0] < t0[0] + span[0]; ++T[0])
            for (T[1] = t0[1]; T[1] < t0[1] + span[1]; ++T[1])
                for (T[2] = t0[2]; T[2] < t0[2] + span[2]; ++T[2]) {
                    int m[3] = {0, 0, 0}, tr[3] = {0, 0, 0}, lanes = 0;
                    bool ok = true;
                    for (int k = 0; k < nl; ++k) {
                        m[k] = cdiv(items[lfirst + k], T[k]);
                        tr[k] = cdiv(items[lfirst + k], m[k]);
                        ok = ok && m[k] <= 255 && tr[k] == T[k];
                        lanes += 4 * m[k];
                    }
                    if (!ok || lanes > kDwlThreads) continue;
                    // groups by trips, most first: a wavefront's most trips is that of
                    // the group holding its first lane
                    int idx[3] = {0, 1, 2};
                    std::stable_sort(idx, idx + nl, [&](int x, int y) { return tr[x] > tr[y]; });
                    long long waves = 0, sum = 0, most = 0;
                    for (int w = 0; w < NWv; ++w) {
                        int first = w * kWave, c = 0;
                        for (int k = 0; k < nl; ++k) {
                            c += 4 * m[idx[k]];
                            if (first < c) {
                                waves += tr[idx[k]];
                                most = std::max<long long>(most, tr[idx[k]]);
                                break;
                            }
                        }
                    }
                    for (int k = 0; k < nl; ++k) sum += 4LL * m[k] * tr[k];
                    const long long cst = (most * 1000 + waves) * 1000000 + sum;
                    if (best < 0 || cst < best) {
                        best = cst;
                        for (int k = 0; k < nl; ++k) bestM[k] = m[k];
                    }
                }
        if (best < 0) return false;
        for (int k = 0; k < nl; ++k) M[lfirst + k] = bestM[k];
        return true;
    }
    for (int l = lfirst; l < L; ++l) M[l] = 1;
    int used = 4 * nl;
    while (used + 4 <= kDwlThreads) {
        int worst = -1, wl_items = 0;
        for (int l = lfirst; l < L; ++l) {
            const int per = cdiv(items[l], M[l]);
            if (M[l] < std::min(items[l], 255) && per > wl_items) {
                wl_items = per;
                worst = l;
            }
        }
        if (worst < 0) break;
        ++M[worst];
        used += 4;
    }
    return true;
}

bool dwl_layout(const wtconv_desc &d, const PlaneCfg &cfg, int pb, PlaneDwlArgs &a, int lfirst) {
    const int K = d.k, KK = K * K, R = (K - 1) / 2, L = d.levels, RHD = cfg.RH, CW = cfg.CW;
    a = PlaneDwlArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.L = L;
    a.PB = pb;
    a.H1 = (d.h + 1) / 2;
    a.W1 = (d.w + 1) / 2;
    a.Gw = cdiv(a.W1, CW);
    int hs[kMaxLevels + 1], ws[kMaxLevels + 1];
    hs[0] = d.h;
    ws[0] = d.w;
    for (int l = 1; l <= L; ++l) {
        hs[l] = (hs[l - 1] + 1) / 2;
        ws[l] = (ws[l - 1] + 1) / 2;
    }
    if (pb == 1) {
        a.Pw1 = a.W1;
    } else {
        int pwL = 1;
        for (int l = 1; l <= L; ++l) pwL = std::max(pwL, cdiv(ws[l] + R, 1LL << (L - l)));
        while (((long long)pwL << (L - 1)) % CW) ++pwL;
        a.Pw1 = pwL << (L - 1);
    }
    a.commit_items = pb * a.H1 * a.Gw;
    if (a.commit_items >= 32768) return false;
    if ((long long)pb * d.c * d.h * d.w >= (1LL << 31)) return false;
    long long fl = 0;
    const int WQ = (RHD + 2 * R + 3) / 4;
    for (int l = 1; l <= L; ++l) {
        const int li = l - 1;
        a.hl[li] = hs[l];
        a.wl[li] = pb == 1 ? ws[l] : (pb * a.Pw1) >> (l - 1);
        a.ns[li] = cdiv(hs[l], RHD);
        a.wr[li] = ws[l];
        a.pw[li] = pb == 1 ? ws[l] : a.Pw1 >> (l - 1);
        const int items = a.ns[li] * pb * a.wr[li];
        if (items >= 32768 || 2LL * hs[l] * a.wl[li] >= 32768) return false;
        // without level-1 items (lfirst = 1) only level 1's low-pass bands are kept:
        // the level-2 analysis reads nothing else of level 1
        const int nb = li < lfirst ? 1 : 4;
        a.xs[li] = column_stride(std::max((a.ns[li] - 1) * RHD + 4 * WQ, a.ns[li] * RHD + 2 * R));
        a.xb[li] = a.xs[li] * (a.wl[li] + 2 * R);
        a.xo[li] = (int)fl;
        fl += (long long)nb * a.xb[li];
        // dy columns: ns RHD >= hl rows (a multiple of 4, so the pad row an odd hl
        // needs for the next level's butterflies is inside), one pad column if wl
        // is odd
        a.gs[li] = column_stride(a.ns[li] * RHD);
        a.gb[li] = a.gs[li] * (a.wl[li] + (a.wl[li] & 1));
        a.go[li] = (int)fl;
        fl += (long long)nb * a.gb[li];
        a.m_wl[li] = magic31_of(a.wl[li]);
        a.m_row[li] = magic31_of(pb * a.wr[li]);
        a.m_wr[li] = magic31_of(a.wr[li]);
        a.m_hl[li] = magic31_of(a.hl[li]);
    }
    const int TC = KK <= 24 ? KK : (KK + 1) / 2;  // reduction chunk of the kernel
    fl = std::max<long long>(fl, (long long)kDwlThreads * (TC + 1));
    a.lds_floats = (int)((fl + 3) & ~3LL);
    if ((long long)a.lds_floats * 4 > kDwlLdsBudget) return false;
    // lanes per (level, band) of levels lfirst + 1 .. L
    int M[kMaxLevels];
    if (4 * (L - lfirst) > kDwlThreads) return false;
    if (!dwl_lanes(a, lfirst, M)) return false;
    // the table: levels by trips per lane, most first, so that the lanes with the
    // most trips share wavefronts; each level's lanes band by band
    int order[kMaxLevels], no = 0;
    for (int l = lfirst; l < L; ++l) order[no++] = l;
    auto trips = [&](int l) { return cdiv(a.ns[l] * a.PB * a.wr[l], M[l]); };
    std::stable_sort(order, order + no, [&](int x, int y) { return trips(x) > trips(y); });
    int t = 0;
    for (int k = 0; k < no; ++k) {
        const int l = order[k];
        a.lane0[l] = t;
        a.lanes[l] = M[l];
        for (int b = 0; b < 4; ++b)
            for (int m = 0; m < M[l]; ++m, ++t)
                a.lane[t] = (uint32_t)(l + 1) | ((uint32_t)b << 4) | ((uint32_t)m << 8) | ((uint32_t)M[l] << 16);
    }
    for (; t < kDwlThreads; ++t) a.lane[t] = 0;
    a.groups = 4 * (L - lfirst);
    a.lfirst = lfirst;
    a.m_gw = magic31_of(a.Gw);
    a.m_h1 = magic31_of(a.H1);
    return true;
}

// lfirst = 1: levels 2..L only (level 1 runs in the correlation kernel)
bool plan_dwl(const wtconv_desc &d, PlaneDwlArgs &a, PlaneCfg &cfg, int lfirst) {
    if (d.levels < 1 + lfirst || d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kPlaneMaxSide || d.w > kPlaneMaxSide) return false;
    cfg.RH = 4;  // item rows: one 16-byte read of dy per item
    cfg.CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, kDwPbCap); ++pb) {
        PlaneDwlArgs t{};
        if (!dwl_layout(d, cfg, pb, t, lfirst)) {
            if (pb == 1) return false;
            break;
        }
        // wave-instructions per pass: the item trips of the busiest wavefront, of
        // RHD K^2 FMAs + 30 others each; commit and Haar ~60 per item; ~300 fixed
        const double cost = (2.0 * dwl_wave_trips(t) * (cfg.RH * d.k * d.k + 30.0) +
                             cdiv(t.commit_items, kDwlThreads) * 120.0 + 300.0) / pb;
        if (cost < best - 1e-9) {
            best = cost;
            best_pb = pb;
        }
    }
    if (!dwl_layout(d, cfg, best_pb, a, lfirst)) return false;
    a.NG = cdiv(d.n, a.PB);
    // Among the workgroup counts per channel that are all resident at once, the one
    // with the least work on the busiest compute unit: workgroups per CU times image
    // groups per workgroup (ties: more workgroups).  Measured on the stage shapes,
    // e.g. x[64,192,28,28] L=2 takes 4 per channel, not the 5 that fit (46 -> 35 us).
    const int kmax = dw_blocks_per_channel(d, a.NG, a.lds_floats);
    long long best_load = -1;
    for (int k = 1; k <= kmax; ++k) {
        const long long load = cdiv((long long)d.c * k, 256) * cdiv(a.NG, k);
        if (best_load < 0 || load <= best_load) {
            best_load = load;
            a.k = k;
        }
    }
    return (long long)d.c * a.k < (1LL << 31);
}

// ---------------------------------------------------------------------------
// Base and level-1 weight gradients on the matrix cores (bfloat16)
// ---------------------------------------------------------------------------

constexpr int kDwcLdsBudget = 40960;

// Layout for pb planes per pass; false when it does not fit.  The offset range
// follows DwcGeom (wtconv_dwc.hpp).
bool dwc_layout(const wtconv_desc &d, int CW, int pb, PlaneDwcArgs &a, bool lev) {
    const int K = d.k, R = (K - 1) / 2;
    const int T0 = lev ? -R : -((R + 1) / 2), T1 = lev ? R : (R + 1) / 2;
    const int NF = (T1 - T0 + 4) / 4, TYMAX = T0 + 4 * NF - 1;
    a = PlaneDwcArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.PB = pb;
    a.H1 = (d.h + 1) / 2;
    a.W1 = (d.w + 1) / 2;
    a.Gw = cdiv(a.W1, CW);
    // cell pitch between side-by-side planes: a gap of at least R zero cells, every
    // commit group inside, even (patches are written as bfloat16 pairs)
    a.Pw1 = (std::max(pb == 1 ? a.W1 : a.W1 + R, a.Gw * CW) + 1) & ~1;
    const int Wc = (pb - 1) * a.Pw1 + a.W1;
    a.nch = cdiv(Wc, 32);
    a.commit_items = pb * a.H1 * a.Gw;
    a.items = a.H1 * a.nch;
    if (a.commit_items >= 32768 || a.items >= 32768) return false;
    if ((long long)pb * d.c * d.h * d.w >= (1LL << 31)) return false;
    // dy planes: DT zero rows above row 0, -T0 below; the row stride is 16 mod 64
    // dwords and the plane size 4 mod 64, so that the 16 A rows of a lane group
    // (4 components x 4 row shifts) fall on distinct banks
    a.DT = std::max(TYMAX, 0);
    const long long rows_d = a.H1 + a.DT + std::max(-T0, 0);
    long long Sd = std::max<long long>(16LL * a.nch, cdiv((long long)pb * a.Pw1, 2));
    while (Sd % 64 != 16) ++Sd;
    long long pd = rows_d * Sd;
    while (pd % 64 != 4) ++pd;
    // x planes: XL zero cells left of column 0; a lane reads five dwords from the
    // pair holding its first cell
    a.XL = (-T0 + 1) & ~1;
    long long Sx = std::max<long long>((a.XL + 32LL * a.nch + T0 + 4 * NF - 5) / 2 + 5, cdiv(a.XL + (long long)pb * a.Pw1, 2));
    long long px = a.H1 * Sx;
    while (px % 64 != 8) ++px;
    a.Sd = (int)Sd;
    a.pd = (int)pd;
    a.Sx = (int)Sx;
    a.px = (int)px;
    a.xo = (int)(4 * pd);
    const long long planes = 4 * pd + 4 * px;
    const long long NC = (long long)NF * NF * 256;
    const long long red = (kDwcThreads / kWave + 1) * NC + kDwcThreads / kWave;
    const long long fl = std::max(planes, red);
    a.lds_floats = (int)((fl + 3) & ~3LL);
    if ((long long)a.lds_floats * 4 > kDwcLdsBudget) return false;
    a.m_gw = magic31_of(a.Gw);
    a.m_h1 = magic31_of(a.H1);
    a.m_nch = magic31_of(a.nch);
    return true;
}

// bfloat16 planes of at most 64 x 64.  Chooses CW, PB and the workgroups per channel.
// lev: level 1 as well as the base (levels >= 1).
bool plan_dwc(const wtconv_desc &d, PlaneDwcArgs &a, int &CW, bool lev) {
    if (!WTC_MMA || d.dtype != WTCONV_BF16) return false;
    if (d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kPlaneMaxSide || d.w > kPlaneMaxSide) return false;
    CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    const int R = (d.k - 1) / 2;
    const int NF = ((lev ? 2 * R : 2 * ((R + 1) / 2)) + 4) / 4;
    double best = -1.0;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, kDwPbCap); ++pb) {
        PlaneDwcArgs t{};
        if (!dwc_layout(d, CW, pb, t, lev)) {
            if (pb == 1) return false;
            break;
        }
        // wave-instructions per pass: an item ~8 per product (16 cycles) plus ~10
        // per operand read and ~20 others; commit ~40 per item; ~300 fixed.  Eight
        // workgroups per compute unit as the registers allow, fewer as the LDS does.
        // A workgroup's passes run one after another (latency-bound), so the time is
        // the passes of the busiest workgroup, ceil(NG / k), times the cost of one.
        const int wg = std::max(1, std::min(8, (int)((160 * 1024) / ((long long)t.lds_floats * 4))));
        const double cost = cdiv(t.items, kDwcThreads / kWave) * 2.0 * (8.0 * NF * NF + 20.0 * NF + 20.0) +
                            cdiv(t.commit_items, kDwcThreads) * 2.0 * 40.0 + 300.0;
        const int ng = cdiv(d.n, pb), k = std::max(1, std::min(ng, kPlanCUs * wg / d.c));
        const double score = 1.0 / (cdiv(ng, k) * cost);
        if (score > best * (1 + 1e-9)) {
            best = score;
            best_pb = pb;
        }
    }
    if (!dwc_layout(d, CW, best_pb, a, lev)) return false;
    a.NG = cdiv(d.n, a.PB);
    const int wg = std::max(1, std::min(8, (int)((160 * 1024) / ((long long)a.lds_floats * 4))));
    a.k = std::max(1, std::min(a.NG, kPlanCUs * wg / d.c));
    return (long long)d.c * a.k < (1LL << 31);
}

// Workspace of the per-level path: the sign patterns Q_l of every level and the
// carriers of levels 1..L-1 (with the tiled matrix-core kernel, level 1 has no Q).
FwdPlan build_forward_plan(const wtconv_desc &d, bool tile) {
    FwdPlan p{};
    p.ld = level_dims(d);
    const size_t es = elem_size(d.dtype), planes = (size_t)d.n * d.c;
    size_t off = 0;
    for (int l = tile ? 2 : 1; l <= d.levels; ++l) {
        p.q_off[l - 1] = off;
        off = align_up(off + planes * 4 * p.ld.H[l] * p.ld.W[l] * es);
    }
    for (int l = 1; l < d.levels; ++l) {
        p.c_off[l - 1] = off;
        off = align_up(off + planes * p.ld.H[l] * p.ld.W[l] * es);
    }
    for (int l = 1; l <= d.levels; ++l)
        p.lvl[l - 1] = pick_tiling(Kind::LevelFwd, d.k, d.n, d.c, p.ld.H[l], p.ld.W[l], 1);
    p.syn = pick_tiling(Kind::Synth, d.k, d.n, d.c, d.h, d.w, max_vec_width(d.dtype));
    p.bytes = off;
    return p;
}

// The tiled correlation kernel for planes past the plane-resident range (bfloat16):
// tiles of UR x 32 level-1 cells (UR at most 16), the x canvas XR = UR + 4 NF - 1
// rows of XC 4-cell chunks (cells c0 - 4 .. of the offsets' reach), the dy canvas
// UR rows between 4 NF - 1 zero rows above and below, 16 dwords a row.
bool plan_dwc_tile(const wtconv_desc &d, DwcTileArgs &a, bool lev) {
    if (!WTC_MMA || d.dtype != WTCONV_BF16) return false;
    if (d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    const int R = (d.k - 1) / 2;
    const int T0 = lev ? -R : -((R + 1) / 2), T1 = lev ? R : (R + 1) / 2;
    const int NF = (T1 - T0 + 4) / 4;
    a = DwcTileArgs{};
    a.n = d.n;
    a.C = d.c;
    a.H = d.h;
    a.W = d.w;
    a.Ho = (d.h + 1) / 2;
    a.Wo = (d.w + 1) / 2;
    a.UR = std::min(kDwcTileRows, a.Ho);
    a.TYu = cdiv(a.Ho, a.UR);
    a.TXu = cdiv(a.Wo, kDwcTileCols);
    const long long P = (long long)d.n * a.TYu * a.TXu;
    if (P >= (1LL << 31)) return false;
    a.P = (int)P;
    // x canvas rows and 4-cell chunks that the used offsets T0..T1 reach (the
    // products of a family's offsets past T1 land in accumulators nothing reads, so
    // what their lanes read there does not matter): rows T0 .. UR - 1 + T1, and the
    // cells of a lane's five-dword B read at XL + 24 + T1 (XL = 4)
    a.XR = a.UR + T1 - T0;
    a.XC = cdiv(2 * ((kDwcTileCols - 4 + T1) >> 1) + 10, 4);
    if (a.XR * a.XC > kDwcTileXSlots * kDwcThreads || a.UR * kDwcTileCols / 4 > kDwcTileDySlots * kDwcThreads)
        return false;
    // bank spread as in the plane-resident layout: row stride 16 mod 64 dwords and
    // plane size 4 mod 64 for dy, plane size 8 mod 64 for x
    a.Sd = 16;
    long long pd = (long long)(a.UR + 8 * NF - 2) * a.Sd;
    while (pd % 64 != 4) ++pd;
    a.pd = (int)pd;
    a.Sx = std::max(2 * a.XC, (4 + kDwcTileCols + T0 + 4 * NF - 5) / 2 + 5);
    long long px = (long long)a.XR * a.Sx;
    while (px % 64 != 8) ++px;
    a.px = (int)px;
    a.xo = 4 * a.pd;
    const long long planes = 4LL * a.pd + 4LL * a.px;
    const long long NC = (long long)NF * NF * 256;
    const long long red = (kDwcThreads / kWave + 1) * NC + kDwcThreads / kWave;
    a.lds_floats = (int)((std::max(planes, red) + 3) & ~3LL);
    if ((long long)a.lds_floats * 4 > kDwcLdsBudget) return false;
    a.m_xc = magic31_of(a.XC);
    // workgroups per channel: about eight resident per compute unit in all
    a.k = std::max(1, std::min(a.P, kPlanCUs * 8 / d.c));
    return (long long)d.c * a.k < (1LL << 31);
}

DwPlan build_backward_weight_plan(const wtconv_desc &d) {
    DwPlan p{};
    p.ld = level_dims(d);
    // bfloat16: base and level 1 by the correlation kernel, levels 2..L by the level
    // kernel; when the level kernel does not fit, the correlation kernel takes the
    // base alone and the per-level kernels all levels
    p.dwc = plan_dwc(d, p.ca, p.ccw, d.levels >= 1);
    p.dwc_lev = p.dwc && d.levels >= 1;
    if (p.dwc_lev && d.levels >= 2 && !plan_dwl(d, p.la, p.lcfg, 1)) {
        p.dwc = plan_dwc(d, p.ca, p.ccw, false);
        p.dwc_lev = false;
    }
    p.dwl = p.dwc_lev ? d.levels >= 2 : plan_dwl(d, p.la, p.lcfg, 0);
    p.dtile = !p.dwc && !p.dwl && plan_dwc_tile(d, p.ta, d.levels >= 1);
    for (int l = 2; l <= d.levels; ++l) {
        wtconv_desc dl = d;
        dl.h = p.ld.H[l - 1];
        dl.w = p.ld.W[l - 1];
        dl.levels = l < d.levels ? 2 : 1;  // 2: it also writes the carriers for level l + 1
        p.dtl[l - 1] = p.dtile && plan_dwc_tile(dl, p.tal[l - 1], true);
    }
    const size_t es = elem_size(d.dtype), planes = (size_t)d.n * d.c;
    size_t off = 0;
    if (!p.dwl && !p.dwc_lev) {
        for (int l = 1; l < d.levels; ++l) {
            p.xc_off[l - 1] = off;
            off = align_up(off + planes * p.ld.H[l] * p.ld.W[l] * es);
            p.gc_off[l - 1] = off;
            off = align_up(off + planes * p.ld.H[l] * p.ld.W[l] * es);
        }
    }
    p.part_off = off;
    const int KK = d.k * d.k;
    p.base = pick_tiling(Kind::DwBase, d.k, d.n, d.c, d.h, d.w, max_vec_width(d.dtype));
    p.dwb = !p.dwc && plan_dwb(d, p.ba, p.bcfg);
    long long floats = 0;
    p.region[0] = 0;
    if (p.dwc)
        p.G[0] = p.ca.k;
    else if (p.dtile)
        p.G[0] = p.ta.k;
    else if (p.dwb)
        p.G[0] = p.ba.k;
    else
        p.G[0] = (d.n > 0 && d.h > 0 && d.w > 0) ? p.base.nblk * p.base.tiles : 0;
    floats += (long long)d.c * p.G[0] * (KK + 1);
    for (int l = 1; l <= d.levels; ++l) {
        p.lvl[l - 1] = pick_tiling(Kind::DwLevel, d.k, d.n, d.c, p.ld.H[l], p.ld.W[l], 1);
        p.region[l] = floats;
        if (p.dwc_lev && l == 1)
            p.G[l] = p.ca.k;
        else if (p.dtile && l == 1)
            p.G[l] = p.ta.k;
        else if (p.dtl[l - 1])
            p.G[l] = p.tal[l - 1].k;
        else if (p.dwl)
            p.G[l] = p.la.k;
        else
            p.G[l] = (d.n > 0 && d.h > 0 && d.w > 0) ? p.lvl[l - 1].nblk * p.lvl[l - 1].tiles : 0;
        floats += (long long)d.c * p.G[l] * 4 * KK;
    }
    p.trash = floats;
    long long trash_rows = 0;
    for (int l = 2; l <= d.levels; ++l)
        if (p.dtl[l - 1]) trash_rows = std::max<long long>(trash_rows, p.tal[l - 1].k);
    floats += (long long)d.c * trash_rows * (KK + 1);
    p.bytes = align_up(off + (size_t)floats * sizeof(float));
    return p;
}

// ---------------------------------------------------------------------------
// Plans per descriptor, argument checks
// ---------------------------------------------------------------------------

bool same_desc(const wtconv_desc &a, const wtconv_desc &b) {
    return a.n == b.n && a.c == b.c && a.h == b.h && a.w == b.w && a.k == b.k && a.levels == b.levels &&
           a.dtype == b.dtype && a.reserved == b.reserved;
}

std::shared_ptr<const PlanSet> plans_for(const wtconv_desc &d) {
    static std::mutex mu;
    static std::vector<std::shared_ptr<const PlanSet>> cache;  // most recent last
    {
        std::lock_guard<std::mutex> lock(mu);
        for (size_t i = cache.size(); i-- > 0;)
            if (same_desc(cache[i]->d, d)) return cache[i];
    }
    auto ps = std::make_shared<PlanSet>();
    ps->d = d;
    ps->plane = plan_plane(d, ps->pa, ps->pcfg);
    ps->mma = plan_mma(d, ps->ma, ps->mcw);
    ps->mtile = !ps->plane && !ps->mma && plan_mma_tile(d, ps->ta);
    ps->fp = build_forward_plan(d, ps->mtile);
    ps->dp = build_backward_weight_plan(d);
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() >= 64) cache.erase(cache.begin());
    cache.push_back(ps);
    return ps;
}


// Workspace of the forward-shaped passes: none when the plane-resident kernel runs
// (a choice made from the descriptor alone), the per-level coefficients and
// carriers otherwise.
size_t forward_workspace_bytes(const wtconv_desc &d) {
    const auto ps = plans_for(d);
    return ps->plane || ps->mma ? 0 : ps->fp.bytes;
}

int check_desc(const wtconv_desc *d) {
    if (!d) return WTCONV_ERR_NULL;
    if (d->n < 0 || d->c < 0 || d->h < 0 || d->w < 0 || d->reserved != 0) return WTCONV_ERR_SHAPE;
    if (d->k != 3 && d->k != 5 && d->k != 7) return WTCONV_ERR_KERNEL;
    if (d->levels < 0 || d->levels > kMaxLevels) return WTCONV_ERR_LEVELS;
    if (d->dtype != WTCONV_F32 && d->dtype != WTCONV_BF16 && d->dtype != WTCONV_F16) return WTCONV_ERR_DTYPE;
    // every workgroup count must fit a 1-D grid; plane offsets are 64-bit
    const long long planes = (long long)d->n * d->c;
    if ((long long)d->h * d->w > (1LL << 31) - 1) return WTCONV_ERR_SHAPE;
    if (planes > (1LL << 31) - 1) return WTCONV_ERR_SHAPE;
    if (!empty(*d)) {
        const auto ps = plans_for(*d);
        const FwdPlan &fp = ps->fp;
        const DwPlan &dp = ps->dp;
        auto too_big = [&](const Tiling &t) { return grid_of(t, d->c) > (1LL << 31) - 1; };
        if (too_big(fp.syn) || too_big(dp.base)) return WTCONV_ERR_SHAPE;
        if (!tiling_fits(Kind::Synth, d->k, fp.syn) || !tiling_fits(Kind::DwBase, d->k, dp.base))
            return WTCONV_ERR_SHAPE;
        for (int l = 0; l < d->levels; ++l) {
            if (too_big(fp.lvl[l]) || too_big(dp.lvl[l])) return WTCONV_ERR_SHAPE;
            if (!tiling_fits(Kind::LevelFwd, d->k, fp.lvl[l]) || !tiling_fits(Kind::DwLevel, d->k, dp.lvl[l]))
                return WTCONV_ERR_SHAPE;
        }
    }
    return WTCONV_OK;
}

#define WTC_DISPATCH(KVAL, DTYPE, FN, ...)                                   \
    do {                                                                    \
        const int dt_ = (DTYPE);                                            \
        switch (KVAL) {                                                     \
            case 3: return dt_ == WTCONV_BF16 ? FN<3, uint16_t>(__VA_ARGS__) \
                         : dt_ == WTCONV_F16 ? FN<3, wtc_f16>(__VA_ARGS__) : FN<3, float>(__VA_ARGS__); \
            case 5: return dt_ == WTCONV_BF16 ? FN<5, uint16_t>(__VA_ARGS__) \
                         : dt_ == WTCONV_F16 ? FN<5, wtc_f16>(__VA_ARGS__) : FN<5, float>(__VA_ARGS__); \
            case 7: return dt_ == WTCONV_BF16 ? FN<7, uint16_t>(__VA_ARGS__) \
                         : dt_ == WTCONV_F16 ? FN<7, wtc_f16>(__VA_ARGS__) : FN<7, float>(__VA_ARGS__); \
            default: return WTCONV_ERR_KERNEL;                              \
        }                                                                   \
    } while (0)

int plane_grid_for(const PlanSet &ps) { WTC_DISPATCH(ps.d.k, ps.d.dtype, plane_grid, ps); }
int mma_grid_for(const PlanSet &ps) { WTC_DISPATCH(ps.d.k, ps.d.dtype, mma_grid, ps); }
int tile_grid_for(const PlanSet &ps) { WTC_DISPATCH(ps.d.k, ps.d.dtype, tile_grid, ps); }

int fwd_common(const wtconv_desc *desc, const void *in, const float *w0, const float *b0, const float *s0,
               const float *wl, const float *sl, void *out, void *workspace, size_t workspace_bytes, void *stream,
               int rotate) {
    int rc = check_desc(desc);
    if (rc) return rc;
    const wtconv_desc &d = *desc;
    if (empty(d)) return WTCONV_OK;
    if (!in || !out || !w0 || !s0 || (d.levels > 0 && (!wl || !sl))) return WTCONV_ERR_NULL;
    const size_t es = elem_size(d.dtype);
    if (!aligned(in, es) || !aligned(out, es) || !aligned(w0, 4) || !aligned(s0, 4) || (b0 && !aligned(b0, 4)) ||
        (wl && !aligned(wl, 4)) || (sl && !aligned(sl, 4)))
        return WTCONV_ERR_ALIGN;
    const auto ps = plans_for(d);
    const size_t need = ps->plane || ps->mma ? 0 : ps->fp.bytes;
    if (need > 0 && (!workspace || workspace_bytes < need)) return WTCONV_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 16)) return WTCONV_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    WTC_DISPATCH(d.k, d.dtype, run_forward, *ps, in, w0, b0, s0, wl, sl, out, static_cast<char *>(workspace), st,
                 rotate);
}

}  // namespace
}  // namespace wtc

// The allocation-free entry point's workspace (see scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[WTCONV_STATIC_SCRATCH_BYTES];

namespace wtc {
namespace {

// Checks shared by the weight-gradient entry points (everything but the workspace).
int check_backward_weight(const wtconv_desc *desc, const void *x, const void *dy, const float *w0, const float *b0,
                          const float *s0, const float *wl, const float *sl, const float *dw0, const float *db0,
                          const float *ds0, const float *dwl, const float *dsl) {
    int rc = check_desc(desc);
    if (rc) return rc;
    const wtconv_desc &d = *desc;
    if (d.c == 0) return WTCONV_OK;
    if (!w0 || !s0 || !dw0 || !ds0 || (d.levels > 0 && (!wl || !sl || !dwl || !dsl))) return WTCONV_ERR_NULL;
    if (!empty(d) && (!x || !dy)) return WTCONV_ERR_NULL;
    const size_t es = elem_size(d.dtype);
    if ((x && !aligned(x, es)) || (dy && !aligned(dy, es)) || !aligned(w0, 4) || !aligned(s0, 4) ||
        !aligned(dw0, 4) || !aligned(ds0, 4) || (b0 && !aligned(b0, 4)) || (db0 && !aligned(db0, 4)) ||
        (wl && !aligned(wl, 4)) || (sl && !aligned(sl, 4)) || (dwl && !aligned(dwl, 4)) ||
        (dsl && !aligned(dsl, 4)))
        return WTCONV_ERR_ALIGN;
    return WTCONV_OK;
}

// The allocation-free entry point's workspace: one array per device, held until
// the process ends.  Host code never uses `scratch` itself (on the host it names a
// stand-in, not device memory): its device address is taken once per device with
// hipGetSymbolAddress and kept in scratch_ptr.
constexpr size_t kScratchBytes = WTCONV_STATIC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure).
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace wtc

using namespace wtc;

extern "C" {

WTCONV_API int wtconv_version(void) { return WTCONV_VERSION; }

WTCONV_API const char *wtconv_status_string(int status) {
    switch (status) {
        case WTCONV_OK: return "ok";
        case WTCONV_ERR_SHAPE: return "invalid shape (negative extent or tensor too large)";
        case WTCONV_ERR_KERNEL: return "unsupported kernel size (3, 5 or 7)";
        case WTCONV_ERR_LEVELS: return "levels out of range";
        case WTCONV_ERR_DTYPE: return "unsupported activation dtype";
        case WTCONV_ERR_NULL: return "required pointer is NULL";
        case WTCONV_ERR_WORKSPACE: return "workspace missing or too small";
        case WTCONV_ERR_ALIGN: return "misaligned pointer";
        case WTCONV_ERR_OP: return "unknown operation";
        case WTCONV_ERR_HIP: return "HIP kernel launch failed";
        case WTCONV_ERR_SCRATCH: return "shape needs more workspace than the library's static scratch holds";
        default: return "unknown status";
    }
}

WTCONV_API int wtconv_workspace_size(const wtconv_desc *desc, int op, size_t *bytes) {
    if (!bytes) return WTCONV_ERR_NULL;
    *bytes = 0;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (op != WTCONV_OP_FORWARD && op != WTCONV_OP_BACKWARD_INPUT && op != WTCONV_OP_BACKWARD_WEIGHT)
        return WTCONV_ERR_OP;
    if (op == WTCONV_OP_BACKWARD_WEIGHT) {
        *bytes = plans_for(*desc)->dp.bytes;
    } else {
        *bytes = empty(*desc) ? 0 : forward_workspace_bytes(*desc);
    }
    return WTCONV_OK;
}

WTCONV_API int wtconv_forward(const wtconv_desc *desc, const void *x, const float *w0, const float *b0,
                              const float *s0, const float *wl, const float *sl, void *y, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return fwd_common(desc, x, w0, b0, s0, wl, sl, y, workspace, workspace_bytes, stream, 0);
}

WTCONV_API int wtconv_backward_input(const wtconv_desc *desc, const void *dy, const float *w0, const float *s0,
                                     const float *wl, const float *sl, void *dx, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    return fwd_common(desc, dy, w0, nullptr, s0, wl, sl, dx, workspace, workspace_bytes, stream, 1);
}

WTCONV_API int wtconv_backward_weight(const wtconv_desc *desc, const void *x, const void *dy, const float *w0,
                                      const float *b0, const float *s0, const float *wl, const float *sl,
                                      float *dw0, float *db0, float *ds0, float *dwl, float *dsl, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    int rc = check_backward_weight(desc, x, dy, w0, b0, s0, wl, sl, dw0, db0, ds0, dwl, dsl);
    if (rc || desc->c == 0) return rc;
    const wtconv_desc &d = *desc;
    const auto ps = plans_for(d);
    if (ps->dp.bytes > 0 && (!workspace || workspace_bytes < ps->dp.bytes)) return WTCONV_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 16)) return WTCONV_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    WTC_DISPATCH(d.k, d.dtype, run_backward_weight, *ps, x, dy, w0, b0, s0, wl, sl, dw0, db0, ds0, dwl, dsl,
                 static_cast<char *>(workspace), st);
}

WTCONV_API int wtconv_backward_weight_noalloc(const wtconv_desc *desc, const void *x, const void *dy,
                                              const float *w0, const float *b0, const float *s0, const float *wl,
                                              const float *sl, float *dw0, float *db0, float *ds0, float *dwl,
                                              float *dsl, void *stream) {
    int rc = check_backward_weight(desc, x, dy, w0, b0, s0, wl, sl, dw0, db0, ds0, dwl, dsl);
    if (rc || desc->c == 0) return rc;
    const wtconv_desc &d = *desc;
    const auto ps = plans_for(d);
    if (ps->dp.bytes > kScratchBytes) return WTCONV_ERR_SCRATCH;
    char *ws = static_cast<char *>(scratch_ptr());
    if (!ws) return WTCONV_ERR_HIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    WTC_DISPATCH(d.k, d.dtype, run_backward_weight, *ps, x, dy, w0, b0, s0, wl, sl, dw0, db0, ds0, dwl, dsl, ws, st);
}

WTCONV_API int wtconv_plan_launches(const wtconv_desc *desc, int op, wtconv_launch *out, int max_entries,
                                    int *n_entries) {
    if (!n_entries) return WTCONV_ERR_NULL;
    *n_entries = 0;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (op != WTCONV_OP_FORWARD && op != WTCONV_OP_BACKWARD_INPUT && op != WTCONV_OP_BACKWARD_WEIGHT)
        return WTCONV_ERR_OP;
    const wtconv_desc &d = *desc;
    const char *dt = dtype_name(d.dtype);
    std::vector<wtconv_launch> v;
    auto add = [&](const char *fam, int level, long long wg, int thr, size_t lds, int variant = 0) {
        wtconv_launch e{};
        e.variant = variant;
        if (level > 0)
            snprintf(e.name, sizeof(e.name), "%s<%d,%s>#%d", fam, d.k, dt, level);
        else
            snprintf(e.name, sizeof(e.name), "%s<%d,%s>", fam, d.k, dt);
        e.workgroups = wg;
        e.threads = thr;
        e.lds_bytes = (int32_t)lds;
        if (wg > 0) v.push_back(e);
    };
    const void *aligned_ptr = reinterpret_cast<const void *>(uintptr_t(256));
    const auto ps = plans_for(d);
    if (op != WTCONV_OP_BACKWARD_WEIGHT) {
        if (!empty(d)) {
            if (ps->mma) {
                add("mma_fwd", 0, mma_grid_for(*ps), kMmaThreads, (size_t)ps->ma.lds_floats * sizeof(float),
                    ps->mcw);
            } else if (ps->plane) {
                add("plane_fwd", 0, plane_grid_for(*ps), kFwdThreads, (size_t)ps->pa.lds_floats * sizeof(float),
                    16 * ps->pcfg.CW + ps->pcfg.RH + (d.levels == 0 ? 256 : 0));
            } else if (ps->mtile) {
                const FwdPlan &p = ps->fp;
                for (int l = 1; l < d.levels; ++l)
                    add("carrier", l,
                        (long long)cdiv((long long)p.ld.H[l] * cdiv(p.ld.W[l], 4), kThreads) *
                            std::min<long long>((long long)d.n * d.c, 65535),
                        kThreads, 0);
                for (int l = d.levels; l >= 2; --l)
                    add("level_acc", l, grid_of(p.lvl[l - 1], d.c), kThreads, lds_bytes(Kind::LevelFwd, d.k, p.lvl[l - 1]));
                add("mma_tile", 0, tile_grid_for(*ps), kTileThreads, (size_t)ps->ta.lds_floats * sizeof(float));
            } else {
                const FwdPlan &p = ps->fp;
                for (int l = 1; l <= d.levels; ++l)
                    add("level_fwd", l, grid_of(p.lvl[l - 1], d.c), kThreads, lds_bytes(Kind::LevelFwd, d.k, p.lvl[l - 1]));
                Tiling t = p.syn;
                t.VW = vec_width(d.w, d.dtype, aligned_ptr);
                add("synth", 0, grid_of(t, d.c), kThreads, lds_bytes(Kind::Synth, d.k, t));
            }
        }
    } else if (d.c > 0) {
        const DwPlan &p = ps->dp;
        if (p.dwc)
            add("plane_dwc", 0, (long long)d.c * p.ca.k, kDwcThreads, (size_t)p.ca.lds_floats * sizeof(float),
                p.ccw + (p.dwc_lev ? 16 : 0));
        if (p.dwc_lev) {
            if (d.levels >= 2)
                add("plane_dwd", 0, (long long)d.c * p.la.k, kDwlThreads, (size_t)p.la.lds_floats * sizeof(float),
                    16 * p.lcfg.CW + p.lcfg.RH);
        } else if (!empty(d)) {
            if (p.dtile)
                add("dwc_tile", 0, (long long)d.c * p.ta.k, kDwcThreads, (size_t)p.ta.lds_floats * sizeof(float),
                    d.levels >= 1 ? 16 : 0);
            if (p.dwl && d.levels > 0) {
                add("plane_dwl", 0, (long long)d.c * p.la.k, kDwlThreads, (size_t)p.la.lds_floats * sizeof(float),
                    16 * p.lcfg.CW + p.lcfg.RH);
            } else {
                for (int l = p.dtile ? 2 : 1; l <= d.levels; ++l) {
                    if (p.dtl[l - 1])
                        add("dwc_tile", l, (long long)d.c * p.tal[l - 1].k, kDwcThreads,
                            (size_t)p.tal[l - 1].lds_floats * sizeof(float), 16);
                    else
                        add("dw_level", l, grid_of(p.lvl[l - 1], d.c), kThreads,
                            lds_bytes(Kind::DwLevel, d.k, p.lvl[l - 1]));
                }
            }
            if (p.dwc || p.dtile) {
                // the base ran in the correlation kernel
            } else if (p.dwb) {
                add("plane_dwb", 0, (long long)d.c * p.ba.k, kDwbThreads, (size_t)p.ba.lds_floats * sizeof(float),
                    16 * p.bcfg.CW + p.bcfg.RH);
            } else {
                Tiling t = p.base;
                t.VW = vec_width(d.w, d.dtype, aligned_ptr);
                add("dw_base", 0, grid_of(t, d.c), kThreads, lds_bytes(Kind::DwBase, d.k, t));
            }
        }
        add("dw_finalize", 0, (long long)d.c * (d.levels + 1), 128, 0);
    }
    const int n = (int)v.size();
    for (int i = 0; i < n && i < max_entries && out; ++i) out[i] = v[i];
    *n_entries = n;
    return WTCONV_OK;
}
WTCONV_API int wtconv_profile_begin(void) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (auto &r : g_prof) {
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_prof.clear();
    g_prof_on = true;
    return WTCONV_OK;
}

WTCONV_API int wtconv_profile_end(wtconv_kernel_time *out, int max_entries, int *n_entries) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_on = false;
    std::vector<wtconv_kernel_time> agg;
    int rc = WTCONV_OK;
    for (auto &r : g_prof) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
            rc = WTCONV_ERR_HIP;
            continue;
        }
        auto it = std::find_if(agg.begin(), agg.end(),
                               [&](const wtconv_kernel_time &k) { return r.name == k.name; });
        if (it == agg.end()) {
            wtconv_kernel_time k{};
            snprintf(k.name, sizeof(k.name), "%s", r.name.c_str());
            k.min_ms = ms;
            k.max_ms = ms;
            agg.push_back(k);
            it = agg.end() - 1;
        }
        it->count += 1;
        it->total_ms += ms;
        it->min_ms = std::min(it->min_ms, (double)ms);
        it->max_ms = std::max(it->max_ms, (double)ms);
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_prof.clear();
    const int n = std::min<int>((int)agg.size(), std::max(0, max_entries));
    for (int i = 0; i < n && out; ++i) out[i] = agg[i];
    if (n_entries) *n_entries = n;
    return rc;
}

}  // extern "C"
