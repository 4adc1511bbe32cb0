// Host side of libwtconv.so: argument checks, workspace plan, tiling, launches
// and the C ABI declared in include/wtconv.h.
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation".  Launch sequence per call:
//   forward / backward_input : level kernel for l = 1..L (§4.1), then the
//                              closed-form synthesis + base kernel (§4.2-4.4);
//   backward_weight          : level gradient kernel for l = 1..L, base gradient
//                              kernel, finalize (fixed-order sums + Eq. 9).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "wtconv.h"
#include "wtconv_fused.hpp"
#include "wtconv_fused_dw.hpp"
#include "wtconv_plane.hpp"
#include "wtconv_plane_dw.hpp"
#include "wtconv_kernels.hpp"

namespace wtc {
namespace {

constexpr int kThreads = 256;
constexpr size_t kLdsBudget = 64 * 1024;   // bytes of LDS per workgroup we allow
constexpr int kDwTargetBlocks = 2048;      // workgroups wanted for the gradient kernels
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Multiply-high reciprocal for fdiv (divisor and dividends below 2^16); 0 encodes 1.
inline uint32_t magic_of(int d) { return d <= 1 ? 0u : (uint32_t)((0x100000000ULL + (uint64_t)d - 1) / (uint64_t)d); }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
// Reciprocal for udiv16 (exact n / d for n < 2^16, d < 2^15): ceil(2^31 / d).
inline uint32_t magic31_of(int d) { return (uint32_t)(((1ULL << 31) + (uint64_t)d - 1) / (uint64_t)d); }

// ---------------------------------------------------------------------------
// Profiling: hipEvent pairs around each launch, on the launch stream.
// ---------------------------------------------------------------------------

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

// Name of an activation dtype as the launch records and plans spell it.
const char *dtype_name(int dtype) {
    return dtype == WTCONV_BF16 ? "bf16" : (dtype == WTCONV_F16 ? "f16" : "f32");
}
// Activation dtype of a storage type.
template <typename T>
constexpr int dtype_of() {
    return std::is_same<T, uint16_t>::value ? WTCONV_BF16 : (std::is_same<T, wtc_f16>::value ? WTCONV_F16 : WTCONV_F32);
}

template <typename Kern, typename Args>
int launch(const char *family, int K, int dtype, int level, Kern kern, dim3 grid, dim3 block, size_t shmem,
           hipStream_t stream, const Args &args) {
    if (grid.x == 0 || grid.y == 0) return WTCONV_OK;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    bool prof = false;
    {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        if (g_prof_on) {
            ev0 = pooled_event();
            ev1 = pooled_event();
            prof = ev0 && ev1;
        }
    }
    if (prof) (void)hipEventRecord(ev0, stream);
    hipLaunchKernelGGL(kern, grid, block, shmem, stream, args);
    hipError_t err = hipGetLastError();
    if (prof) {
        (void)hipEventRecord(ev1, stream);
        char name[64];
        if (level > 0)
            snprintf(name, sizeof(name), "%s<%d,%s>#%d", family, K, dtype_name(dtype), level);
        else
            snprintf(name, sizeof(name), "%s<%d,%s>", family, K, dtype_name(dtype));
        std::lock_guard<std::mutex> lock(g_prof_mu);
        g_prof.push_back({name, ev0, ev1});
    }
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Shapes, tiling and the workspace plan
// ---------------------------------------------------------------------------

struct LevelDims {
    int H[kMaxLevels + 1], W[kMaxLevels + 1];  // H[0] = h; H[l] = ceil(H[l-1] / 2)
};

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

// Bytes of LDS a kernel needs for a tiling (HY rows staged per 8-row strip set
// plus the K - 1 halo; see the kernels for the layouts).
enum class Kind { LevelFwd, Synth, DwLevel, DwBase };

size_t lds_bytes(Kind kind, int K, const Tiling &t) {
    const int R = (K - 1) / 2, KK = K * K;
    const size_t PB = t.PB, HY = (size_t)t.SP * kRH + K - 1, HXP = t.TX + K - 1, GY = (size_t)t.SP * kRH;
    const size_t HXW = stage_width(t.TX, R, t.VW), GW = stage_width(t.TX, 0, t.VW);
    switch (kind) {
        case Kind::LevelFwd: return (PB * 4 * HY * HXP + 4 * KK) * sizeof(float);  // float4 cells, weight table
        case Kind::Synth: return (PB * HY * HXW) * sizeof(float);
        case Kind::DwLevel: return (PB * 4 * HY * HXP + PB * 4 * GY * t.TX + 4 * KK) * sizeof(float);
        case Kind::DwBase: return (PB * HY * HXW + PB * GY * GW + (kThreads / kWave) * (KK + 1)) * sizeof(float);
    }
    return 0;
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

// Widest vector (elements) for staging rows of length W at pointer p.
int vec_width(int W, int dtype, const void *p) {
    int vw = dtype != WTCONV_F32 ? 8 : 4;
    const size_t es = dtype != WTCONV_F32 ? 2 : 4;
    while (vw > 1 && (W % vw != 0 || ((uintptr_t)p % (vw * es)) != 0)) vw /= 2;
    return vw;
}
int max_vec_width(int dtype) { return dtype != WTCONV_F32 ? 8 : 4; }

long long grid_of(const Tiling &t, int C) { return (long long)t.tiles * C * t.nblk; }

// ---------------------------------------------------------------------------
// Plane-resident forward (small planes): LDS layout and plane stacking
// ---------------------------------------------------------------------------

constexpr int kFusedMaxSide = 64;
constexpr int kFusedTargetBlocks = 768;  // ~3 workgroups per compute unit

// Layout of one plane block; fills everything but PB / NB / nblk / VE.  The weight
// table comes first, then the plane blocks, then a tail so that the synthesis
// reads of rows past the plane (values that are discarded) stay in the allocation.
bool fused_layout(const wtconv_desc &d, FusedArgs &a) {
    const int K = d.k, KK = K * K, KKP = (KK + 3) & ~3;
    if (d.h > kFusedMaxSide || d.w > kFusedMaxSide) return false;
    a.H = d.h;
    a.W = d.w;
    a.L = d.levels;
    a.hl[0] = d.h;
    a.wl_[0] = d.w;
    for (int l = 1; l <= d.levels; ++l) {
        a.hl[l] = (a.hl[l - 1] + 1) / 2;
        a.wl_[l] = (a.wl_[l - 1] + 1) / 2;
    }
    for (int l = 0; l <= d.levels; ++l) a.sp[l] = cdiv(a.hl[l], kRH);
    const int wtab_floats = (d.levels * 4 * KKP + 3) & ~3;
    a.wtab = 0;
    int off = wtab_floats;
    // regions hold the grid plus its halo; the extra rows that the last 8-row strip
    // reads (only for outputs past the grid, which are discarded) fall in the next
    // region or in the tail of the allocation
    a.xoff = off;
    a.xs = d.w + K - 1;
    off += (d.h + K - 1) * a.xs;
    int items = 0;
    for (int l = 0; l < d.levels; ++l) {
        off = (off + 3) & ~3;
        a.yb[l] = off;
        a.sy[l] = a.wl_[l + 1] + K - 1;
        a.bs[l] = (a.hl[l + 1] + K - 1) * a.sy[l];
        off += 4 * a.bs[l];
        items += 4 * a.sp[l + 1] * a.wl_[l + 1];
        a.items_end[l] = items;
    }
    a.conv_items = items;
    off = (off + 3) & ~3;
    a.plane_floats = off - wtab_floats;
    return true;
}

int fused_tail_floats(const FusedArgs &a) {
    // Reads for discarded outputs run past a region by at most 8 rows (the last
    // 8-row strip) or 4 block rows (synthesis); past every region but the last they
    // land in the next region, past the last one in this tail.
    const int last = a.L > 0 ? a.sy[a.L - 1] : a.xs;
    return (kRH + 4) * last + 64;
}

int fused_prefetch_capacity(int dtype, int VE) {
    // prefetch words per thread (8 for 16-bit activations, 16 for f32), 256 threads
    const int es = dtype != WTCONV_F32 ? 2 : 4;
    const int words = dtype != WTCONV_F32 ? 8 : 16;
    const int words_per_vec = (VE * es + 3) / 4;
    return (words / words_per_vec) * kThreads * VE;
}

// Choose PB (planes per pass) and NB (planes per workgroup).  False when the plane
// is too large for the plane-resident kernel.
bool plan_fused(const wtconv_desc &d, int VE, FusedArgs &a) {
    if (d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    FusedArgs base{};
    if (!fused_layout(d, base)) return false;
    const int wtab_floats = base.xoff;
    const int tail = fused_tail_floats(base);
    const long long HW = (long long)d.h * d.w;
    const int fin = base.sp[0] * d.w;
    int haar = 0;
    for (int l = 1; l <= d.levels; ++l) haar += base.hl[l] * base.wl_[l];
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, 64); ++pb) {
        const long long lds = (long long)wtab_floats + (long long)pb * base.plane_floats + tail;
        if (lds * 4 > (long long)kLdsBudget) break;
        if ((long long)pb * base.conv_items > (long long)kFusedMaxItems * kThreads) break;
        if ((long long)pb * fin > (long long)kFusedMaxFinal * kThreads) break;
        if (pb * HW > fused_prefetch_capacity(d.dtype, VE)) break;
        if ((long long)pb * d.c * HW >= (1LL << 30)) break;  // 32-bit offsets from a plane base
        // estimated wave-instructions per pass: a conv or final item is 8 K^2 FMAs
        // (+ synthesis for the final ones), Haar / combine ~15 per position, ~300 fixed
        const double per_item = 8.0 * d.k * d.k;
        const double cost = cdiv((long long)pb * base.conv_items, kThreads) * per_item +
                            cdiv((long long)pb * fin, kThreads) * (per_item + 10.0 * d.levels + 20.0) +
                            2.0 * cdiv((long long)pb * haar, kThreads) * 15.0 + 300.0;
        if (cost / pb < best - 1e-9) {
            best = cost / pb;
            best_pb = pb;
        }
    }
    if (best_pb == 0) return false;
    a = base;
    a.PB = best_pb;
    a.lds_floats = wtab_floats + best_pb * base.plane_floats + tail;
    a.VE = VE;
    // planes per workgroup: a multiple of PB, about kFusedTargetBlocks workgroups
    const long long passes = cdiv(d.n, a.PB);
    const long long want_per_chan = std::max<long long>(1, cdiv(kFusedTargetBlocks, d.c));
    const long long passes_per_wg = std::max<long long>(1, cdiv(passes, want_per_chan));
    a.NB = (int)(passes_per_wg * a.PB);
    a.nblk = cdiv(d.n, a.NB);
    a.n = d.n;
    a.C = d.c;
    a.m_hw = magic_of((int)HW);
    a.m_w = magic_of(d.w);
    a.m_conv = magic_of(std::max(1, a.conv_items));
    a.m_fin = magic_of(fin);
    for (int l = 0; l < d.levels; ++l) {
        a.m_per[l] = magic_of(a.hl[l + 1] * a.wl_[l + 1]);
        a.m_wl[l] = magic_of(a.wl_[l + 1]);
    }
    return true;
}



// ---------------------------------------------------------------------------
// Plane-resident forward on the polyphase grid: layout, stacking, bank-aware strides
// ---------------------------------------------------------------------------

constexpr int kPlaneLdsBudget = 40960;  // four workgroups per compute unit

struct PlaneCfg {
    int CW = 1, RH = 8;
};

// Bank cost of 16-byte cell reads by items (strip s, plane p, column j), item t =
// (s PB + p) W1 + j on lane t, cell s RH sy + p Pw1 + j: gfx950 serves a 16-byte
// read 16 lanes at a time from 64 banks, conflict-free when the 16 cells are
// distinct mod 16.  Cost: per group of 16 lanes the largest number of lanes sharing
// a cell slot mod 16 (1 = conflict-free), summed.
long long cell_bank_cost(int items, int pb, int W1, int pitch, int RH, int sy) {
    long long cost = 0;
    const int per_strip = pb * W1;
    for (int g = 0; g * 16 < items; ++g) {
        int cnt[16] = {0};
        int worst = 0;
        for (int t = g * 16; t < std::min(items, g * 16 + 16); ++t) {
            const int s = t / per_strip, r = t % per_strip, p = r / W1, j = r % W1;
            const int cell = s * RH * sy + p * pitch + j;
            worst = std::max(worst, ++cnt[cell & 15]);
        }
        cost += worst;
    }
    return cost;
}

// Smallest row stride in [lo, lo + 16) with the least bank cost.
int best_stride(int items, int pb, int W1, int pitch, int RH, int lo) {
    long long best = -1;
    int sy = lo;
    for (int cand = lo; cand < lo + 16; ++cand) {
        const long long cost = cell_bank_cost(items, pb, W1, pitch, RH, cand);
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
    if (a.final_items >= 32768 || a.commit_items >= 32768) return false;
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
    if (d.h > kFusedMaxSide || d.w > kFusedMaxSide) return false;
    const int H1 = (d.h + 1) / 2;
    cfg.RH = H1 % 7 == 0 ? 7 : (H1 <= 4 ? 4 : 8);
    cfg.CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    const int K = d.k;
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, 64); ++pb) {
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
    a.lds_floats = (int)std::max<long long>(floats, (long long)kDwbThreads * (KK + 2));
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
    const int per_cu = std::max(1, std::min(4, (160 * 1024) / std::max(1, lds_floats * 4)));
    return std::max(1, std::min(NG, 256 * per_cu / std::max(1, d.c)));
}

bool plan_dwb(const wtconv_desc &d, PlaneDwbArgs &a, PlaneCfg &cfg) {
    if (d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kFusedMaxSide || d.w > kFusedMaxSide) return false;
    const int H1 = (d.h + 1) / 2;
    cfg.RH = H1 % 7 == 0 ? 7 : (H1 <= 4 ? 4 : 8);
    cfg.CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, 64); ++pb) {
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

bool dwl_layout(const wtconv_desc &d, const PlaneCfg &cfg, int pb, PlaneDwlArgs &a) {
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
        const int items = a.ns[li] * a.wl[li];
        if (items >= 32768 || 2LL * hs[l] * a.wl[li] >= 32768) return false;
        a.xs[li] = column_stride(std::max((a.ns[li] - 1) * RHD + 4 * WQ, a.ns[li] * RHD + 2 * R));
        a.xb[li] = a.xs[li] * (a.wl[li] + 2 * R);
        a.xo[li] = (int)fl;
        fl += 4LL * a.xb[li];
        // dy columns: ns RHD >= hl rows (a multiple of 4, so the pad row an odd hl
        // needs for the next level's butterflies is inside), one pad column if wl
        // is odd
        a.gs[li] = column_stride(a.ns[li] * RHD);
        a.gb[li] = a.gs[li] * (a.wl[li] + (a.wl[li] & 1));
        a.go[li] = (int)fl;
        fl += 4LL * a.gb[li];
        a.m_wl[li] = magic31_of(a.wl[li]);
        a.m_hl[li] = magic31_of(a.hl[li]);
    }
    const int TC = KK <= 24 ? KK : (KK + 1) / 2;  // reduction chunk of the kernel
    fl = std::max<long long>(fl, (long long)kDwlThreads * (TC + 1));
    a.lds_floats = (int)((fl + 3) & ~3LL);
    if ((long long)a.lds_floats * 4 > kDwlLdsBudget) return false;
    // lanes per (level, band): greedy, to minimise the largest item count of a lane
    int M[kMaxLevels];
    for (int l = 0; l < L; ++l) M[l] = 1;
    if (4 * L > kDwlThreads) return false;
    int used = 4 * L;
    while (used + 4 <= kDwlThreads) {
        int worst = -1, wl_items = 0;
        for (int l = 0; l < L; ++l) {
            const int items = a.ns[l] * a.wl[l], per = cdiv(items, M[l]);
            if (M[l] < std::min(items, 255) && per > wl_items) {
                wl_items = per;
                worst = l;
            }
        }
        if (worst < 0) break;
        ++M[worst];
        used += 4;
    }
    int t = 0;
    for (int l = 0; l < L; ++l) {
        a.lane0[l] = t;
        a.lanes[l] = M[l];
        for (int b = 0; b < 4; ++b)
            for (int m = 0; m < M[l]; ++m, ++t)
                a.lane[t] = (uint32_t)(l + 1) | ((uint32_t)b << 4) | ((uint32_t)m << 8) | ((uint32_t)M[l] << 16);
    }
    for (; t < kDwlThreads; ++t) a.lane[t] = 0;
    a.groups = 4 * L;
    a.m_gw = magic31_of(a.Gw);
    a.m_h1 = magic31_of(a.H1);
    return true;
}

// Largest item count of a lane (the pass time) for a layout.
int dwl_lane_items(const PlaneDwlArgs &a) {
    int worst = 0;
    for (int t = 0; t < kDwlThreads; ++t) {
        const uint32_t in = a.lane[t];
        const int M = (in >> 16) & 255, l = (int)(in & 15) - 1;
        if (M) worst = std::max(worst, cdiv(a.ns[l] * a.wl[l], M));
    }
    return worst;
}

bool plan_dwl(const wtconv_desc &d, PlaneDwlArgs &a, PlaneCfg &cfg) {
    if (d.levels < 1 || d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kFusedMaxSide || d.w > kFusedMaxSide) return false;
    cfg.RH = 4;  // item rows: one 16-byte read of dy per item
    cfg.CW = d.w % 8 == 0 ? 4 : (d.w % 4 == 0 ? 2 : 1);
    double best = 1e30;
    int best_pb = 0;
    for (int pb = 1; pb <= std::min(d.n, 64); ++pb) {
        PlaneDwlArgs t{};
        if (!dwl_layout(d, cfg, pb, t)) {
            if (pb == 1) return false;
            break;
        }
        // wave-instructions per pass: a lane's items of RHD K^2 FMAs + 30 others;
        // commit and Haar ~60 per item; ~300 fixed
        const double cost = (2.0 * dwl_lane_items(t) * (cfg.RH * d.k * d.k + 30.0) +
                             cdiv(t.commit_items, kDwlThreads) * 120.0 + 300.0) / pb;
        if (cost < best - 1e-9) {
            best = cost;
            best_pb = pb;
        }
    }
    if (!dwl_layout(d, cfg, best_pb, a)) return false;
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
// Plane-resident weight gradient of the levels (small planes)
// ---------------------------------------------------------------------------

constexpr int kFusedDwTargetBlocks = 1024;

// Layout and lane allocation from the shape alone (the prefetch capacity does not
// depend on the vector width), so that the workspace size is shape-determined.
bool plan_fused_dw(const wtconv_desc &d, FusedDwArgs &a) {
    if (d.levels < 1 || d.n <= 0 || d.c <= 0 || d.h <= 0 || d.w <= 0) return false;
    if (d.h > kFusedMaxSide || d.w > kFusedMaxSide) return false;
    const int K = d.k, L = d.levels;
    FusedDwArgs b{};
    b.H = d.h;
    b.W = d.w;
    b.L = L;
    b.hl[0] = d.h;
    b.wl_[0] = d.w;
    for (int l = 1; l <= L; ++l) {
        b.hl[l] = (b.hl[l - 1] + 1) / 2;
        b.wl_[l] = (b.wl_[l - 1] + 1) / 2;
    }
    for (int l = 0; l <= L; ++l) b.sp[l] = cdiv(b.hl[l], kRH);
    // regions: x pyramid (halo R, rows trimmed to the grid), then dy pyramid (centre)
    int off = 0;
    for (int l = 0; l < L; ++l) {
        off = (off + 3) & ~3;
        b.yb[l] = off;
        b.ys[l] = b.wl_[l + 1] + K - 1;
        b.ybs[l] = (b.hl[l + 1] + K - 1) * b.ys[l];
        off += 4 * b.ybs[l];
    }
    for (int l = 0; l < L; ++l) {
        off = (off + 3) & ~3;
        b.gb[l] = off;
        b.gbs[l] = b.hl[l + 1] * b.wl_[l + 1];
        off += 4 * b.gbs[l];
    }
    b.plane_floats = (off + 3) & ~3;
    // reads for discarded rows run up to 8 (+4) rows past the last region
    const int tail = (kRH + 4) * std::max(b.wl_[L], b.ys[L - 1]) + 64;
    b.blocks = b.hl[1] * b.wl_[1];
    const int capacity = d.dtype != WTCONV_F32 ? 2048 : 1024;  // level-1 blocks prefetched per pass
    long long per_pair[kMaxLevels];
    for (int l = 0; l < L; ++l) per_pair[l] = (long long)b.sp[l + 1] * b.wl_[l + 1];
    const int KK = K * K;
    double best = 1e30;
    int best_pb = 0, best_r = 0;
    for (int pb = 1; pb <= std::min(d.n, 16); ++pb) {
        const long long lds = std::max<long long>((long long)pb * b.plane_floats + tail, 256LL * 9);
        if (lds * 4 > (long long)kLdsBudget) break;
        if ((long long)pb * b.blocks > capacity) break;
        if ((long long)pb * d.c * d.h * d.w >= (1LL << 30)) break;
        int r = 1;
        for (; r <= kDwMaxRounds; ++r) {
            long long lanes = 0;
            for (int l = 0; l < L; ++l) lanes += 4 * cdiv(pb * per_pair[l], r);
            if (lanes <= kThreads) break;
        }
        if (r > kDwMaxRounds) continue;
        // wave-instructions per pass: r rounds of 8 K^2 FMAs (+ ~40), Haar ~300, fixed ~300
        const double cost = r * (8.0 * KK + 40.0) + 300.0 + 300.0;
        if (cost / pb < best - 1e-9) {
            best = cost / pb;
            best_pb = pb;
            best_r = r;
        }
    }
    if (best_pb == 0) return false;
    a = b;
    a.PB = best_pb;
    a.rounds = best_r;
    int lane = 0;
    for (int l = 0; l < L; ++l)
        for (int bd = 0; bd < 4; ++bd) {
            a.lane0[4 * l + bd] = lane;
            a.lanes[4 * l + bd] = cdiv(best_pb * per_pair[l], best_r);
            lane += a.lanes[4 * l + bd];
        }
    a.lds_floats = (int)std::max<long long>((long long)best_pb * b.plane_floats + tail, 256LL * 9);
    const long long passes = cdiv(d.n, a.PB);
    const long long want_per_chan = std::max<long long>(1, cdiv(kFusedDwTargetBlocks, d.c));
    const long long passes_per_wg = std::max<long long>(1, cdiv(passes, want_per_chan));
    a.NB = (int)(passes_per_wg * a.PB);
    a.nblk = cdiv(d.n, a.NB);
    a.n = d.n;
    a.C = d.c;
    a.m_w1 = magic_of(a.wl_[1]);
    a.m_blocks = magic_of(a.blocks);
    for (int l = 0; l < L; ++l) {
        a.m_per[l] = magic_of(a.hl[l + 1] * a.wl_[l + 1]);
        a.m_wl[l] = magic_of(a.wl_[l + 1]);
    }
    return true;
}

struct FwdPlan {
    LevelDims ld;
    size_t q_off[kMaxLevels], c_off[kMaxLevels];  // byte offsets into the workspace
    Tiling lvl[kMaxLevels], syn;
    size_t bytes;
};

struct DwPlan {
    bool fused;          // levels by the plane-resident kernel (no carriers)
    FusedDwArgs fa;
    bool dwb;            // base by the plane-resident kernel
    PlaneDwbArgs ba;
    PlaneCfg bcfg;
    bool dwl;            // levels by the band-major plane-resident kernel
    PlaneDwlArgs la;
    PlaneCfg lcfg;
    LevelDims ld;
    size_t xc_off[kMaxLevels], gc_off[kMaxLevels];
    size_t part_off;                 // byte offset of the partials
    long long region[kMaxLevels + 1];  // float offsets within the partials
    int G[kMaxLevels + 1];
    Tiling lvl[kMaxLevels], base;
    size_t bytes;
};

size_t elem_size(int dtype) { return dtype != WTCONV_F32 ? 2 : 4; }

FwdPlan build_forward_plan(const wtconv_desc &d) {
    FwdPlan p{};
    p.ld = level_dims(d);
    const size_t es = elem_size(d.dtype), planes = (size_t)d.n * d.c;
    size_t off = 0;
    for (int l = 1; l <= d.levels; ++l) {
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

DwPlan build_backward_weight_plan(const wtconv_desc &d) {
    DwPlan p{};
    p.ld = level_dims(d);
    p.dwl = plan_dwl(d, p.la, p.lcfg);
    p.fused = !p.dwl && plan_fused_dw(d, p.fa);
    const size_t es = elem_size(d.dtype), planes = (size_t)d.n * d.c;
    size_t off = 0;
    if (!p.fused && !p.dwl) {
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
    p.dwb = plan_dwb(d, p.ba, p.bcfg);
    long long floats = 0;
    p.region[0] = 0;
    if (p.dwb)
        p.G[0] = p.ba.k;
    else
        p.G[0] = (d.n > 0 && d.h > 0 && d.w > 0) ? p.base.nblk * p.base.tiles : 0;
    floats += (long long)d.c * p.G[0] * (KK + 1);
    for (int l = 1; l <= d.levels; ++l) {
        p.lvl[l - 1] = pick_tiling(Kind::DwLevel, d.k, d.n, d.c, p.ld.H[l], p.ld.W[l], 1);
        p.region[l] = floats;
        if (p.dwl)
            p.G[l] = p.la.k;
        else if (p.fused)
            p.G[l] = p.fa.nblk;
        else
            p.G[l] = (d.n > 0 && d.h > 0 && d.w > 0) ? p.lvl[l - 1].nblk * p.lvl[l - 1].tiles : 0;
        floats += (long long)d.c * p.G[l] * 4 * KK;
    }
    p.bytes = align_up(off + (size_t)floats * sizeof(float));
    return p;
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------

bool empty(const wtconv_desc &d) { return d.n == 0 || d.c == 0 || d.h == 0 || d.w == 0; }

// Plans depend on the descriptor only; they are built once per descriptor and
// kept (a call's host cost is then a lookup, not the layout searches).
struct PlanSet {
    wtconv_desc d;
    FwdPlan fp;
    DwPlan dp;
    bool plane;  // forward by the plane-resident kernel
    PlaneArgs pa;
    PlaneCfg pcfg;
};

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
    ps->fp = build_forward_plan(d);
    ps->dp = build_backward_weight_plan(d);
    ps->plane = plan_plane(d, ps->pa, ps->pcfg);
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() >= 64) cache.erase(cache.begin());
    cache.push_back(ps);
    return ps;
}

FwdPlan plan_forward(const wtconv_desc &d) { return plans_for(d)->fp; }
DwPlan plan_backward_weight(const wtconv_desc &d) { return plans_for(d)->dp; }

// Workspace of the forward-shaped passes: none when the plane-resident kernel runs
// (a choice made from the descriptor alone), the per-level coefficients and
// carriers otherwise.
size_t forward_workspace_bytes(const wtconv_desc &d) { return plans_for(d)->plane ? 0 : plan_forward(d).bytes; }

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
        const FwdPlan fp = plan_forward(*d);
        const DwPlan dp = plan_backward_weight(*d);
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

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------------------
// Launch sequences, templated on kernel size K and activation storage T
// ---------------------------------------------------------------------------

template <int K, typename T>
int run_fused_forward(const wtconv_desc &d, FusedArgs a, const void *x, const float *w0, const float *b0,
                      const float *s0, const float *wl, const float *sl, void *y, hipStream_t st, int rotate) {
    const int bf = dtype_of<T>();  // dtype code, for the launch records
    a.x = x;
    a.y = y;
    a.w0 = w0;
    a.b0 = b0;
    a.s0 = s0;
    a.wl = wl;
    a.sl = sl;
    a.rotate = rotate;
    const dim3 grid((unsigned)((long long)d.c * a.nblk)), block(kThreads);
    const size_t shm = (size_t)a.lds_floats * sizeof(float);
    switch (a.VE) {
        case 8:
            if constexpr (sizeof(T) == 2)
                return launch("fused_fwd", K, bf, 0, fused_fwd_kernel<K, T, 8>, grid, block, shm, st, a);
            return WTCONV_ERR_HIP;
        case 4: return launch("fused_fwd", K, bf, 0, fused_fwd_kernel<K, T, 4>, grid, block, shm, st, a);
        case 2: return launch("fused_fwd", K, bf, 0, fused_fwd_kernel<K, T, 2>, grid, block, shm, st, a);
        default: return launch("fused_fwd", K, bf, 0, fused_fwd_kernel<K, T, 1>, grid, block, shm, st, a);
    }
}

template <int K, typename T, int CW>
const void *plane_kernel_rh(int RH, bool base) {
#define WTC_PKR(RH_) base ? reinterpret_cast<const void *>(plane_fwd_kernel<K, T, CW, RH_, true>) \
                          : reinterpret_cast<const void *>(plane_fwd_kernel<K, T, CW, RH_, false>)
    switch (RH) {
        case 7: return WTC_PKR(7);
        case 4: return WTC_PKR(4);
        default: return WTC_PKR(8);
    }
#undef WTC_PKR
}

template <int K, typename T>
const void *plane_kernel(const PlaneCfg &cfg, bool base) {
    switch (cfg.CW) {
        case 4: return plane_kernel_rh<K, T, 4>(cfg.RH, base);
        case 2: return plane_kernel_rh<K, T, 2>(cfg.RH, base);
        default: return plane_kernel_rh<K, T, 1>(cfg.RH, base);
    }
}

const void *plane_kernel_for(const wtconv_desc &d, const PlaneCfg &cfg) {
    const bool base = d.levels == 0;
#define WTC_PK(KV) \
    (d.dtype == WTCONV_BF16 ? plane_kernel<KV, uint16_t>(cfg, base) \
                            : d.dtype == WTCONV_F16 ? plane_kernel<KV, wtc_f16>(cfg, base) : plane_kernel<KV, float>(cfg, base))
    switch (d.k) {
        case 3: return WTC_PK(3);
        case 5: return WTC_PK(5);
        default: return WTC_PK(7);
    }
#undef WTC_PK
}

// Persistent grid: as many workgroups as can be resident at once on the current
// device (they stride over the units), never more than the units.
int plane_grid(const wtconv_desc &d, const PlaneArgs &a, const PlaneCfg &cfg) {
    int dev = 0, cus = 0, per_cu = 0;
    const size_t shm = (size_t)a.lds_floats * sizeof(float);
    const void *kern = plane_kernel_for(d, cfg);
    static std::mutex mu;
    struct Entry {
        int dev;
        const void *kern;
        size_t shm;
        int slots;
    };
    static std::vector<Entry> seen;
    if (hipGetDevice(&dev) == hipSuccess) {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : seen)
            if (e.dev == dev && e.kern == kern && e.shm == shm) return (int)std::min<long long>(a.U, e.slots);
    }
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFwdThreads, shm) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        cus = 256;
        per_cu = std::max(1, std::min(4, (int)((160 * 1024) / std::max<size_t>(shm, 1))));
    } else {
        std::lock_guard<std::mutex> lock(mu);
        seen.push_back(Entry{dev, kern, shm, cus * per_cu});
    }
    return (int)std::min<long long>(a.U, (long long)cus * per_cu);
}

template <int K, typename T>
int run_plane_forward(const wtconv_desc &d, PlaneArgs a, const PlaneCfg &cfg, const void *x, const float *w0,
                      const float *b0, const float *s0, const float *wl, const float *sl, void *y, hipStream_t st,
                      int rotate) {
    a.x = x;
    a.y = y;
    a.w0 = w0;
    a.b0 = b0;
    a.s0 = s0;
    a.wl = wl;
    a.sl = sl;
    a.rotate = rotate;
    a.vec = d.w % (2 * cfg.CW) == 0 && aligned(x, 2 * cfg.CW * sizeof(T)) ? 1 : 0;
    a.pair_store = d.w % 2 == 0 && aligned(y, 2 * sizeof(T)) ? 1 : 0;
    const dim3 grid((unsigned)plane_grid(d, a, cfg));
    const size_t shm = (size_t)a.lds_floats * sizeof(float);
    const int bf = dtype_of<T>();  // dtype code, for the launch records
#define WTC_PLANE_LAUNCH(CW_, RH_)                                                                                \
    (d.levels == 0                                                                                               \
         ? launch("plane_fwd", K, bf, 0, plane_fwd_kernel<K, T, CW_, RH_, true>, grid, dim3(kFwdThreads), shm, st, a) \
         : launch("plane_fwd", K, bf, 0, plane_fwd_kernel<K, T, CW_, RH_, false>, grid, dim3(kFwdThreads), shm, st, a))
    switch (cfg.CW * 16 + cfg.RH) {
        case 4 * 16 + 7: return WTC_PLANE_LAUNCH(4, 7);
        case 4 * 16 + 4: return WTC_PLANE_LAUNCH(4, 4);
        case 4 * 16 + 8: return WTC_PLANE_LAUNCH(4, 8);
        case 2 * 16 + 7: return WTC_PLANE_LAUNCH(2, 7);
        case 2 * 16 + 4: return WTC_PLANE_LAUNCH(2, 4);
        case 2 * 16 + 8: return WTC_PLANE_LAUNCH(2, 8);
        case 1 * 16 + 7: return WTC_PLANE_LAUNCH(1, 7);
        case 1 * 16 + 4: return WTC_PLANE_LAUNCH(1, 4);
        default: return WTC_PLANE_LAUNCH(1, 8);
    }
#undef WTC_PLANE_LAUNCH
}

template <int K, typename T>
int run_plane_dwb(const wtconv_desc &d, PlaneDwbArgs a, const PlaneCfg &cfg, const void *x, const void *dy,
                  float *partial, hipStream_t st) {
    a.x = x;
    a.dy = dy;
    a.partial = partial;
    a.vec = d.w % (2 * cfg.CW) == 0 && aligned(x, 2 * cfg.CW * sizeof(T)) && aligned(dy, 2 * cfg.CW * sizeof(T)) ? 1 : 0;
    const dim3 grid((unsigned)((long long)d.c * a.k));
    const size_t shm = (size_t)a.lds_floats * sizeof(float);
    const int bf = dtype_of<T>();  // dtype code, for the launch records
#define WTC_DWB_LAUNCH(CW_, RH_) \
    launch("plane_dwb", K, bf, 0, plane_dwb_kernel<K, T, CW_, RH_>, grid, dim3(kDwbThreads), shm, st, a)
    switch (cfg.CW * 16 + cfg.RH) {
        case 4 * 16 + 7: return WTC_DWB_LAUNCH(4, 7);
        case 4 * 16 + 4: return WTC_DWB_LAUNCH(4, 4);
        case 4 * 16 + 8: return WTC_DWB_LAUNCH(4, 8);
        case 2 * 16 + 7: return WTC_DWB_LAUNCH(2, 7);
        case 2 * 16 + 4: return WTC_DWB_LAUNCH(2, 4);
        case 2 * 16 + 8: return WTC_DWB_LAUNCH(2, 8);
        case 1 * 16 + 7: return WTC_DWB_LAUNCH(1, 7);
        case 1 * 16 + 4: return WTC_DWB_LAUNCH(1, 4);
        default: return WTC_DWB_LAUNCH(1, 8);
    }
#undef WTC_DWB_LAUNCH
}

template <int K, typename T>
int run_plane_dwl(const wtconv_desc &d, const DwPlan &p, const void *x, const void *dy, float *partial,
                  hipStream_t st) {
    PlaneDwlArgs a = p.la;
    const PlaneCfg &cfg = p.lcfg;
    a.x = x;
    a.dy = dy;
    a.partial = partial;
    for (int l = 0; l < d.levels; ++l) a.off[l] = p.region[l + 1];
    a.vec = d.w % (2 * cfg.CW) == 0 && aligned(x, 2 * cfg.CW * sizeof(T)) && aligned(dy, 2 * cfg.CW * sizeof(T)) ? 1 : 0;
    const dim3 grid((unsigned)((long long)d.c * a.k));
    const size_t shm = (size_t)a.lds_floats * sizeof(float);
    const int bf = dtype_of<T>();  // dtype code, for the launch records
#define WTC_DWL_LAUNCH(CW_, RH_) \
    launch("plane_dwl", K, bf, 0, plane_dwl_kernel<K, T, CW_, RH_>, grid, dim3(kDwlThreads), shm, st, a)
    switch (cfg.CW) {
        case 4: return WTC_DWL_LAUNCH(4, 4);
        case 2: return WTC_DWL_LAUNCH(2, 4);
        default: return WTC_DWL_LAUNCH(1, 4);
    }
#undef WTC_DWL_LAUNCH
}

template <int K, typename T>
int run_forward(const wtconv_desc &d, const void *x, const float *w0, const float *b0, const float *s0,
                const float *wl, const float *sl, void *y, char *ws, hipStream_t st, int rotate) {
    {
        const auto ps = plans_for(d);
        if (ps->plane) return run_plane_forward<K, T>(d, ps->pa, ps->pcfg, x, w0, b0, s0, wl, sl, y, st, rotate);
    }
    {
        FusedArgs fa{};
        if (plan_fused(d, vec_width(d.w, d.dtype, x), fa))
            return run_fused_forward<K, T>(d, fa, x, w0, b0, s0, wl, sl, y, st, rotate);
    }
    const FwdPlan p = plan_forward(d);
    const int bf = dtype_of<T>();  // dtype code, for the launch records

    const int L = d.levels;
    for (int l = 1; l <= L; ++l) {
        LevelArgs a{};
        a.in = l == 1 ? x : (const void *)(ws + p.c_off[l - 2]);
        a.qout = ws + p.q_off[l - 1];
        a.cout = l < L ? (void *)(ws + p.c_off[l - 1]) : nullptr;
        a.wl = wl + (size_t)(l - 1) * d.c * 4 * K * K;
        a.sl = sl + (size_t)(l - 1) * d.c * 4;
        a.n = d.n;
        a.C = d.c;
        a.Hi = p.ld.H[l - 1];
        a.Wi = p.ld.W[l - 1];
        a.Ho = p.ld.H[l];
        a.Wo = p.ld.W[l];
        a.wscale = std::ldexp(1.0f, -(l + 1));
        a.rotate = rotate;
        a.pairs = (a.Wi % 2 == 0) && ((uintptr_t)a.in % (2 * sizeof(T)) == 0);
        a.t = p.lvl[l - 1];
        const size_t shm = lds_bytes(Kind::LevelFwd, K, a.t);
        int rc = launch("level_fwd", K, bf, l, level_fwd_kernel<K, T>, dim3((unsigned)grid_of(a.t, d.c)),
                        dim3(kThreads), shm, st, a);
        if (rc) return rc;
    }
    SynthArgs s{};
    s.x = x;
    s.y = y;
    s.w0 = w0;
    s.b0 = b0;
    s.s0 = s0;
    for (int l = 1; l <= L; ++l) {
        s.q[l - 1] = ws + p.q_off[l - 1];
        s.wq[l - 1] = 2 * p.ld.W[l];
        s.qplane[l - 1] = 4LL * p.ld.H[l] * p.ld.W[l];
    }
    s.n = d.n;
    s.C = d.c;
    s.H = d.h;
    s.W = d.w;
    s.L = L;
    s.rotate = rotate;
    s.t = p.syn;
    s.t.VW = vec_width(d.w, d.dtype, x);
    const size_t shm = lds_bytes(Kind::Synth, K, s.t);
    return launch("synth", K, bf, 0, synth_kernel<K, T>, dim3((unsigned)grid_of(s.t, d.c)), dim3(kThreads), shm, st,
                  s);
}

template <int K, typename T>
int run_backward_weight(const wtconv_desc &d, const void *x, const void *dy, const float *w0, const float *b0,
                        const float *s0, const float *wl, const float *sl, float *dw0, float *db0, float *ds0,
                        float *dwl, float *dsl, char *ws, hipStream_t st) {
    const DwPlan p = plan_backward_weight(d);
    const int bf = dtype_of<T>();  // dtype code, for the launch records
    const int L = d.levels;
    float *partial = reinterpret_cast<float *>(ws + p.part_off);
    if (!empty(d) && p.dwl && L > 0) {
        int rc = run_plane_dwl<K, T>(d, p, x, dy, partial, st);
        if (rc) return rc;
    }
    if (!empty(d) && p.fused && L > 0) {
        FusedDwArgs a = p.fa;
        a.x = x;
        a.dy = dy;
        a.partial = partial;
        for (int l = 0; l < L; ++l) a.off[l] = p.region[l + 1];
        const int ve = std::min(vec_width(d.w, d.dtype, x), vec_width(d.w, d.dtype, dy));
        a.VE = ve >= 2 ? ve : 1;
        const dim3 grid((unsigned)((long long)d.c * a.nblk)), block(kThreads);
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        int rc;
        switch (a.VE) {
            case 8:
                if constexpr (sizeof(T) == 2) {
                    rc = launch("fused_dw", K, bf, 0, fused_dw_kernel<K, T, 8>, grid, block, shm, st, a);
                    break;
                }
                return WTCONV_ERR_HIP;
            case 4: rc = launch("fused_dw", K, bf, 0, fused_dw_kernel<K, T, 4>, grid, block, shm, st, a); break;
            case 2: rc = launch("fused_dw", K, bf, 0, fused_dw_kernel<K, T, 2>, grid, block, shm, st, a); break;
            default: rc = launch("fused_dw", K, bf, 0, fused_dw_kernel<K, T, 1>, grid, block, shm, st, a); break;
        }
        if (rc) return rc;
    }
    if (!empty(d)) {
        for (int l = 1; l <= L && !p.fused && !p.dwl; ++l) {
            DwLevelArgs a{};
            a.xin = l == 1 ? x : (const void *)(ws + p.xc_off[l - 2]);
            a.gin = l == 1 ? dy : (const void *)(ws + p.gc_off[l - 2]);
            a.xc = l < L ? (void *)(ws + p.xc_off[l - 1]) : nullptr;
            a.gc = l < L ? (void *)(ws + p.gc_off[l - 1]) : nullptr;
            a.partial = partial + p.region[l];
            a.n = d.n;
            a.C = d.c;
            a.Hi = p.ld.H[l - 1];
            a.Wi = p.ld.W[l - 1];
            a.Ho = p.ld.H[l];
            a.Wo = p.ld.W[l];
            a.pairs = (a.Wi % 2 == 0) && ((uintptr_t)a.xin % (2 * sizeof(T)) == 0) &&
                      ((uintptr_t)a.gin % (2 * sizeof(T)) == 0);
            a.t = p.lvl[l - 1];
            const size_t shm = lds_bytes(Kind::DwLevel, K, a.t);
            int rc = launch("dw_level", K, bf, l, dw_level_kernel<K, T>, dim3((unsigned)grid_of(a.t, d.c)),
                            dim3(kThreads), shm, st, a);
            if (rc) return rc;
        }
        if (p.dwb) {
            int rc = run_plane_dwb<K, T>(d, p.ba, p.bcfg, x, dy, partial + p.region[0], st);
            if (rc) return rc;
        }
        DwBaseArgs b{};
        b.x = x;
        b.dy = dy;
        b.partial = partial + p.region[0];
        b.n = d.n;
        b.C = d.c;
        b.H = d.h;
        b.W = d.w;
        b.t = p.base;
        b.t.VW = std::min(vec_width(d.w, d.dtype, x), vec_width(d.w, d.dtype, dy));
        const size_t shm = lds_bytes(Kind::DwBase, K, b.t);
        int rc = p.dwb ? 0
                       : launch("dw_base", K, bf, 0, dw_base_kernel<K, T>, dim3((unsigned)grid_of(b.t, d.c)),
                                dim3(kThreads), shm, st, b);
        if (rc) return rc;
    }
    FinalizeArgs f{};
    f.partial = partial;
    for (int r = 0; r <= L; ++r) {
        f.off[r] = p.region[r];
        f.G[r] = p.G[r];
    }
    f.C = d.c;
    f.L = L;
    f.w0 = w0;
    f.b0 = b0;
    f.s0 = s0;
    f.wl = wl;
    f.sl = sl;
    f.dw0 = dw0;
    f.db0 = db0;
    f.ds0 = ds0;
    f.dwl = dwl;
    f.dsl = dsl;
    return launch("dw_finalize", K, bf, 0, dw_finalize_kernel<K>, dim3((unsigned)d.c, (unsigned)(L + 1)), dim3(128), 0,
                  st, f);
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
    const size_t need = forward_workspace_bytes(d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return WTCONV_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 16)) return WTCONV_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    WTC_DISPATCH(d.k, d.dtype, run_forward, d, in, w0, b0, s0, wl, sl, out, static_cast<char *>(workspace), st,
                 rotate);
}

}  // namespace
}  // namespace wtc

using namespace wtc;

extern "C" {

int wtconv_version(void) { return WTCONV_VERSION; }

const char *wtconv_status_string(int status) {
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
        default: return "unknown status";
    }
}

int wtconv_workspace_size(const wtconv_desc *desc, int op, size_t *bytes) {
    if (!bytes) return WTCONV_ERR_NULL;
    *bytes = 0;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (op != WTCONV_OP_FORWARD && op != WTCONV_OP_BACKWARD_INPUT && op != WTCONV_OP_BACKWARD_WEIGHT)
        return WTCONV_ERR_OP;
    if (op == WTCONV_OP_BACKWARD_WEIGHT) {
        *bytes = plan_backward_weight(*desc).bytes;
    } else {
        *bytes = empty(*desc) ? 0 : forward_workspace_bytes(*desc);
    }
    return WTCONV_OK;
}

int wtconv_forward(const wtconv_desc *desc, const void *x, const float *w0, const float *b0, const float *s0,
                   const float *wl, const float *sl, void *y, void *workspace, size_t workspace_bytes,
                   void *stream) {
    return fwd_common(desc, x, w0, b0, s0, wl, sl, y, workspace, workspace_bytes, stream, 0);
}

int wtconv_backward_input(const wtconv_desc *desc, const void *dy, const float *w0, const float *s0,
                          const float *wl, const float *sl, void *dx, void *workspace, size_t workspace_bytes,
                          void *stream) {
    return fwd_common(desc, dy, w0, nullptr, s0, wl, sl, dx, workspace, workspace_bytes, stream, 1);
}

int wtconv_backward_weight(const wtconv_desc *desc, const void *x, const void *dy, const float *w0,
                           const float *b0, const float *s0, const float *wl, const float *sl, float *dw0,
                           float *db0, float *ds0, float *dwl, float *dsl, void *workspace, size_t workspace_bytes,
                           void *stream) {
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
    const DwPlan p = plan_backward_weight(d);
    if (p.bytes > 0 && (!workspace || workspace_bytes < p.bytes)) return WTCONV_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 16)) return WTCONV_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    WTC_DISPATCH(d.k, d.dtype, run_backward_weight, d, x, dy, w0, b0, s0, wl, sl, dw0, db0, ds0, dwl, dsl,
                 static_cast<char *>(workspace), st);
}

int wtconv_plan_launches(const wtconv_desc *desc, int op, wtconv_launch *out, int max_entries, int *n_entries) {
    if (!n_entries) return WTCONV_ERR_NULL;
    *n_entries = 0;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (op != WTCONV_OP_FORWARD && op != WTCONV_OP_BACKWARD_INPUT && op != WTCONV_OP_BACKWARD_WEIGHT)
        return WTCONV_ERR_OP;
    const wtconv_desc &d = *desc;
    const char *dt = dtype_name(d.dtype);
    const size_t es = elem_size(d.dtype);
    std::vector<wtconv_launch> v;
    auto add = [&](const char *fam, int level, long long wg, int thr, size_t lds) {
        wtconv_launch e{};
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
    if (op != WTCONV_OP_BACKWARD_WEIGHT) {
        if (!empty(d)) {
            FusedArgs fa{};
            const auto ps = plans_for(d);
            if (ps->plane) {
                add("plane_fwd", 0, plane_grid(d, ps->pa, ps->pcfg), kFwdThreads,
                    (size_t)ps->pa.lds_floats * sizeof(float));
            } else if (plan_fused(d, vec_width(d.w, d.dtype, aligned_ptr), fa)) {
                add("fused_fwd", 0, (long long)d.c * fa.nblk, kThreads, (size_t)fa.lds_floats * sizeof(float));
            } else {
                const FwdPlan p = plan_forward(d);
                for (int l = 1; l <= d.levels; ++l)
                    add("level_fwd", l, grid_of(p.lvl[l - 1], d.c), kThreads, lds_bytes(Kind::LevelFwd, d.k, p.lvl[l - 1]));
                Tiling t = p.syn;
                t.VW = vec_width(d.w, d.dtype, aligned_ptr);
                add("synth", 0, grid_of(t, d.c), kThreads, lds_bytes(Kind::Synth, d.k, t));
            }
        }
    } else if (d.c > 0) {
        const DwPlan p = plan_backward_weight(d);
        if (!empty(d)) {
            if (p.dwl && d.levels > 0) {
                add("plane_dwl", 0, (long long)d.c * p.la.k, kDwlThreads, (size_t)p.la.lds_floats * sizeof(float));
            } else if (p.fused && d.levels > 0) {
                add("fused_dw", 0, (long long)d.c * p.fa.nblk, kThreads, (size_t)p.fa.lds_floats * sizeof(float));
            } else {
                for (int l = 1; l <= d.levels; ++l)
                    add("dw_level", l, grid_of(p.lvl[l - 1], d.c), kThreads, lds_bytes(Kind::DwLevel, d.k, p.lvl[l - 1]));
            }
            if (p.dwb) {
                add("plane_dwb", 0, (long long)d.c * p.ba.k, kDwbThreads, (size_t)p.ba.lds_floats * sizeof(float));
            } else {
                Tiling t = p.base;
                t.VW = vec_width(d.w, d.dtype, aligned_ptr);
                add("dw_base", 0, grid_of(t, d.c), kThreads, lds_bytes(Kind::DwBase, d.k, t));
            }
        }
        add("dw_finalize", 0, (long long)d.c * (d.levels + 1), 128, 0);
    }
    (void)es;
    const int n = (int)v.size();
    for (int i = 0; i < n && i < max_entries && out; ++i) out[i] = v[i];
    *n_entries = n;
    return WTCONV_OK;
}

int wtconv_profile_begin(void) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (auto &r : g_prof) {
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_prof.clear();
    g_prof_on = true;
    return WTCONV_OK;
}

int wtconv_profile_end(wtconv_kernel_time *out, int max_entries, int *n_entries) {
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
