// Host-side declarations shared by the C ABI (wtconv_api.hip) and the launch
// code compiled once per kernel size and activation type (wtconv_inst.hip).
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation".  A call runs one of two kernel families:
//   * plane-resident kernels (planes whose whole Haar pyramid fits in LDS): one
//     launch per forward-shaped pass (on the matrix cores for bfloat16), two
//     gradient launches and the finalize;
//   * per-level kernels (larger planes): one analysis + filter launch per level
//     and one closed-form synthesis launch per forward-shaped pass (§4.1-4.4), one
//     gradient launch per level, the base gradient and the finalize; for bfloat16
//     the level-1 carrier, the levels 2..L and one tiled matrix-core launch that
//     takes level 1, the base conv and the synthesis per forward-shaped pass.
// Plans (layouts, tilings, launch sizes) depend on the descriptor only and are
// built once per descriptor in wtconv_api.hip.

#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "wtconv.h"
#include "wtconv_kernels.hpp"
#include "wtconv_plane.hpp"
#include "wtconv_plane_dw.hpp"
#include "wtconv_mma.hpp"
#include "wtconv_dwc.hpp"
#include "wtconv_mma_tile.hpp"
#include "wtconv_dwc_tile.hpp"

namespace wtc {

constexpr int kThreads = 256;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
inline size_t elem_size(int dtype) { return dtype != WTCONV_F32 ? 2 : 4; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline bool empty(const wtconv_desc &d) { return d.n == 0 || d.c == 0 || d.h == 0 || d.w == 0; }

// Name of an activation dtype as the launch records and plans spell it.
inline const char *dtype_name(int dtype) {
    return dtype == WTCONV_BF16 ? "bf16" : (dtype == WTCONV_F16 ? "f16" : "f32");
}
// Activation dtype of a storage type.
template <typename T>
constexpr int dtype_of() {
    return std::is_same<T, uint16_t>::value ? WTCONV_BF16 : (std::is_same<T, wtc_f16>::value ? WTCONV_F16 : WTCONV_F32);
}

// Widest vector (elements) for staging rows of length W at pointer p.
inline int vec_width(int W, int dtype, const void *p) {
    int vw = dtype != WTCONV_F32 ? 8 : 4;
    const size_t es = elem_size(dtype);
    while (vw > 1 && (W % vw != 0 || ((uintptr_t)p % (vw * es)) != 0)) vw /= 2;
    return vw;
}
inline int max_vec_width(int dtype) { return dtype != WTCONV_F32 ? 8 : 4; }

// Bytes of LDS a per-level kernel needs for a tiling (HY rows staged per 8-row
// strip set plus the K - 1 halo; see the kernels for the layouts).
enum class Kind { LevelFwd, Synth, DwLevel, DwBase };

inline size_t lds_bytes(Kind kind, int K, const Tiling &t) {
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

inline long long grid_of(const Tiling &t, int C) { return (long long)t.tiles * C * t.nblk; }

struct LevelDims {
    int H[kMaxLevels + 1], W[kMaxLevels + 1];  // H[0] = h; H[l] = ceil(H[l-1] / 2)
};

// Variant of a plane-resident kernel: CW cells per commit item, RH cell rows per item.
struct PlaneCfg {
    int CW = 1, RH = 8;
};

struct FwdPlan {
    LevelDims ld;
    size_t q_off[kMaxLevels], c_off[kMaxLevels];  // byte offsets into the workspace
    Tiling lvl[kMaxLevels], syn;
    size_t bytes;
};

struct DwPlan {
    bool dwc;            // base by the matrix-core correlation kernel (bfloat16) ...
    bool dwc_lev;        // ... and level 1 too; the level kernel then takes levels 2..L only
    PlaneDwcArgs ca;
    int ccw;             // its commit width
    bool dwb;            // base by the plane-resident kernel
    PlaneDwbArgs ba;
    PlaneCfg bcfg;
    bool dtile;          // base and level 1 by the tiled correlation kernel (bfloat16, planes
    DwcTileArgs ta;      // past the plane-resident range), levels 2..L by the per-level kernels
    bool dwl;            // levels by the plane-resident kernel
    PlaneDwlArgs la;
    // with dtile, level l >= 2 (index l - 1) by the tiled correlation kernel too, on the
    // level-(l - 1) carriers: their level-1 bands are level l's, and its level-1 raw
    // sums are level l's (the carrier's 1/2 and the 4^-l cancel); its base sums go
    // to a region nothing reads
    bool dtl[kMaxLevels];
    DwcTileArgs tal[kMaxLevels];
    long long trash;     // float offset of that region within the partials
    PlaneCfg lcfg;
    LevelDims ld;
    size_t xc_off[kMaxLevels], gc_off[kMaxLevels];  // carriers of the per-level kernels
    size_t part_off;                   // byte offset of the partials
    long long region[kMaxLevels + 1];  // float offsets within the partials
    int G[kMaxLevels + 1];             // partial rows per channel of each region
    Tiling lvl[kMaxLevels], base;
    size_t bytes;
};

// Everything a call needs that depends on the descriptor alone.
struct PlanSet {
    wtconv_desc d;
    FwdPlan fp;
    DwPlan dp;
    bool plane;  // forward-shaped passes by the plane-resident kernel
    PlaneArgs pa;
    PlaneCfg pcfg;
    bool mma = false;  // ... by the plane-resident kernel on the matrix cores (bfloat16)
    MmaArgs ma{};
    int mcw = 1;       // its commit width (cells per item)
    bool mtile = false;  // per-level path: levels 2..L by the level kernels, the rest by
    MmaTileArgs ta{};    // the tiled matrix-core kernel (bfloat16)
};

// ---- Profiling hooks (wtconv_api.hip) ------------------------------------
// prof_events: while profiling is on, hands out two events for one launch.
// prof_record: files the pair under the launch's name.
bool prof_events(hipEvent_t &ev0, hipEvent_t &ev1);
void prof_record(const char *family, int K, int dtype, int level, hipEvent_t ev0, hipEvent_t ev1);

// ---- Launch sequences (wtconv_run.hpp, one instantiation per K and T) -------
template <int K, typename T>
int run_forward(const PlanSet &ps, const void *x, const float *w0, const float *b0, const float *s0,
                const float *wl, const float *sl, void *y, char *ws, hipStream_t st, int rotate);
template <int K, typename T>
int run_backward_weight(const PlanSet &ps, const void *x, const void *dy, const float *w0, const float *b0,
                        const float *s0, const float *wl, const float *sl, float *dw0, float *db0, float *ds0,
                        float *dwl, float *dsl, char *ws, hipStream_t st);
// Workgroups of the persistent plane-resident forward kernel: as many as are
// resident at once on the current device, at most one per unit.
template <int K, typename T>
int plane_grid(const PlanSet &ps);
// ... of the matrix-core forward kernel (one contiguous range of units each).
template <int K, typename T>
int mma_grid(const PlanSet &ps);
// ... of the tiled matrix-core forward kernel.
template <int K, typename T>
int tile_grid(const PlanSet &ps);

}  // namespace wtc
