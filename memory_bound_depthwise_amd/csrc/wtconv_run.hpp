// Launch sequences of the WTConv layer for one kernel size K and activation
// storage type T.  wtconv_inst.hip compiles this once per (K, T), so that the
// kernel instances of the library build in parallel.
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation".  Per call:
//   forward / backward_input : the plane-resident kernel (one launch), or the
//                              level kernel for l = 1..L (§4.1) followed by the
//                              closed-form synthesis + base kernel (§4.2-4.4);
//   backward_weight          : level gradients (one plane-resident launch, or one
//                              launch per level), base gradient, finalize
//                              (fixed-order sums + Eq. 9).

#pragma once

#include <cmath>
#include <mutex>
#include <vector>

#include "wtconv_host.hpp"

namespace wtc {

template <typename Kern, typename Args>
int launch(const char *family, int K, int dtype, int level, Kern kern, dim3 grid, dim3 block, size_t shmem,
           hipStream_t stream, const Args &args) {
    if (grid.x == 0 || grid.y == 0) return WTCONV_OK;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    const bool prof = prof_events(ev0, ev1);
    if (prof) (void)hipEventRecord(ev0, stream);
    hipLaunchKernelGGL(kern, grid, block, shmem, stream, args);
    hipError_t err = hipGetLastError();
    if (prof) {
        (void)hipEventRecord(ev1, stream);
        prof_record(family, K, dtype, level, ev0, ev1);
    }
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
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

template <int K, typename T>
int plane_grid(const PlanSet &ps) {
    const wtconv_desc &d = ps.d;
    const PlaneArgs &a = ps.pa;
    int dev = 0, cus = 0, per_cu = 0;
    const size_t shm = (size_t)a.lds_floats * sizeof(float);
    const void *kern = plane_kernel<K, T>(ps.pcfg, d.levels == 0);
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
int run_plane_forward(const PlanSet &ps, const void *x, const float *w0, const float *b0, const float *s0,
                      const float *wl, const float *sl, void *y, hipStream_t st, int rotate) {
    const wtconv_desc &d = ps.d;
    const PlaneCfg &cfg = ps.pcfg;
    PlaneArgs a = ps.pa;
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
    const dim3 grid((unsigned)plane_grid<K, T>(ps));
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
int run_plane_dwb(const PlanSet &ps, const void *x, const void *dy, float *partial, hipStream_t st) {
    const wtconv_desc &d = ps.d;
    const PlaneCfg &cfg = ps.dp.bcfg;
    PlaneDwbArgs a = ps.dp.ba;
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
int run_plane_dwc(const PlanSet &ps, const void *x, const void *dy, float *partial, hipStream_t st) {
    if constexpr (!std::is_same<T, uint16_t>::value) {
        return WTCONV_ERR_DTYPE;  // not planned: bfloat16 only
    } else {
        const wtconv_desc &d = ps.d;
        const DwPlan &p = ps.dp;
        PlaneDwcArgs a = p.ca;
        const int CW = p.ccw;
        a.x = x;
        a.dy = dy;
        a.pbase = partial + p.region[0];
        a.plev = p.dwc_lev ? partial + p.region[1] : nullptr;
        a.vec = d.w % (2 * CW) == 0 && aligned(x, 2 * CW * sizeof(T)) && aligned(dy, 2 * CW * sizeof(T)) ? 1 : 0;
        const dim3 grid((unsigned)((long long)d.c * a.k));
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        const int bf = dtype_of<T>();
#define WTC_DWC_LAUNCH(CW_, LEV_) \
    launch("plane_dwc", K, bf, 0, plane_dwc_kernel<K, CW_, LEV_>, grid, dim3(kDwcThreads), shm, st, a)
        if (p.dwc_lev) {
            switch (CW) {
                case 4: return WTC_DWC_LAUNCH(4, true);
                case 2: return WTC_DWC_LAUNCH(2, true);
                default: return WTC_DWC_LAUNCH(1, true);
            }
        }
        switch (CW) {
            case 4: return WTC_DWC_LAUNCH(4, false);
            case 2: return WTC_DWC_LAUNCH(2, false);
            default: return WTC_DWC_LAUNCH(1, false);
        }
#undef WTC_DWC_LAUNCH
    }
}

template <int K, typename T>
int run_plane_dwl(const PlanSet &ps, const void *x, const void *dy, float *partial, hipStream_t st) {
    const wtconv_desc &d = ps.d;
    const DwPlan &p = ps.dp;
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
    // with the correlation kernel taking level 1, this launch covers levels 2..L
#define WTC_DWL_LAUNCH(CW_, RH_)                                                                                 \
    (a.lfirst ? launch("plane_dwd", K, bf, 0, plane_dwd_kernel<K, T, CW_, RH_>, grid, dim3(kDwlThreads), shm, st, a) \
              : launch("plane_dwl", K, bf, 0, plane_dwl_kernel<K, T, CW_, RH_>, grid, dim3(kDwlThreads), shm, st, a))
    switch (cfg.CW) {
        case 4: return WTC_DWL_LAUNCH(4, 4);
        case 2: return WTC_DWL_LAUNCH(2, 4);
        default: return WTC_DWL_LAUNCH(1, 4);
    }
#undef WTC_DWL_LAUNCH
}

// Resident workgroups of a kernel on the current device (cached per device, kernel
// and LDS size); a conservative estimate when the occupancy query fails.
inline long long resident_slots(const void *kern, int threads, size_t shm) {
    static std::mutex mu;
    struct Entry {
        int dev;
        const void *kern;
        size_t shm;
        long long slots;
    };
    static std::vector<Entry> seen;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : seen)
            if (e.dev == dev && e.kern == kern && e.shm == shm) return e.slots;
    }
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, shm) != hipSuccess || cus <= 0 || per_cu <= 0) {
        (void)hipGetLastError();
        return 256LL * std::max(1, std::min(4, (int)((160 * 1024) / std::max<size_t>(shm, 1))));
    }
    std::lock_guard<std::mutex> lock(mu);
    seen.push_back(Entry{dev, kern, shm, (long long)cus * per_cu});
    return (long long)cus * per_cu;
}

template <int K, typename T>
int mma_grid(const PlanSet &ps) {
    if constexpr (K > 5) {
        return 0;  // not planned: the matrix-core kernel takes K = 3 or 5
    } else {
        const MmaArgs &a = ps.ma;
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        const void *kern = ps.mcw == 4   ? reinterpret_cast<const void *>(mma_fwd_kernel<K, 4>)
                           : ps.mcw == 2 ? reinterpret_cast<const void *>(mma_fwd_kernel<K, 2>)
                                         : reinterpret_cast<const void *>(mma_fwd_kernel<K, 1>);
        return (int)std::min<long long>(a.U, resident_slots(kern, kMmaThreads, shm));
    }
}

template <int K, typename T>
int run_mma_forward(const PlanSet &ps, const void *x, const float *w0, const float *b0, const float *s0,
                    const float *wl, const float *sl, void *y, hipStream_t st, int rotate) {
    if constexpr (!std::is_same<T, uint16_t>::value || K > 5) {
        return WTCONV_ERR_DTYPE;  // not planned: bfloat16 with K = 3 or 5 only
    } else {
        const wtconv_desc &d = ps.d;
        const int CW = ps.mcw;
        MmaArgs a = ps.ma;
        a.x = x;
        a.y = y;
        a.w0 = w0;
        a.b0 = b0;
        a.s0 = s0;
        a.wl = wl;
        a.sl = sl;
        a.rotate = rotate;
        a.vec = d.w % (2 * CW) == 0 && aligned(x, 2 * CW * sizeof(T)) ? 1 : 0;
        a.store_mode = d.w % 4 == 0 && aligned(y, 4 * sizeof(T)) ? 2 : (d.w % 2 == 0 && aligned(y, 2 * sizeof(T)) ? 1 : 0);
        const dim3 grid((unsigned)mma_grid<K, T>(ps));
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        const int bf = dtype_of<T>();
        switch (CW) {
            case 4: return launch("mma_fwd", K, bf, 0, mma_fwd_kernel<K, 4>, grid, dim3(kMmaThreads), shm, st, a);
            case 2: return launch("mma_fwd", K, bf, 0, mma_fwd_kernel<K, 2>, grid, dim3(kMmaThreads), shm, st, a);
            default: return launch("mma_fwd", K, bf, 0, mma_fwd_kernel<K, 1>, grid, dim3(kMmaThreads), shm, st, a);
        }
    }
}

// Level kernel of level l: analysis of the carrier `in` of the level above, the
// four-band conv and the sign patterns Q_l, and (with `carry`) the carrier of
// level l for the next; with `deeper`, the deeper levels' summed patterns are added.
template <int K, typename T>
int run_level_fwd(const PlanSet &ps, const char *family, int l, const void *in, const void *deeper, bool carry,
                  const float *wl, const float *sl, char *ws, hipStream_t st, int rotate) {
    const wtconv_desc &d = ps.d;
    const FwdPlan &p = ps.fp;
    LevelArgs a{};
    a.in = in;
    a.deeper = deeper;
    a.qout = ws + p.q_off[l - 1];
    a.cout = carry && l < d.levels ? (void *)(ws + p.c_off[l - 1]) : nullptr;
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
    return launch(family, K, dtype_of<T>(), l, level_fwd_kernel<K, T>, dim3((unsigned)grid_of(a.t, d.c)),
                  dim3(kThreads), shm, st, a);
}

template <int K, typename T>
int tile_grid(const PlanSet &ps) {
    if constexpr (K > 5) {
        return 0;  // not planned: the matrix-core kernels take K = 3 or 5
    } else {
        const MmaTileArgs &a = ps.ta;
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        return (int)std::min<long long>(
            a.U, resident_slots(reinterpret_cast<const void *>(mma_tile_kernel<K>), kTileThreads, shm));
    }
}

// The per-level path with the tiled matrix-core kernel: the carriers of levels
// 1..L-1, then the level kernels from the deepest level up, each adding the summed
// patterns of the levels below it to its own (level 2 leaves sum_{l >= 2} Q_l on
// the level-1 grid), then the tiles.
template <int K, typename T>
int run_tile_forward(const PlanSet &ps, const void *x, const float *w0, const float *b0, const float *s0,
                     const float *wl, const float *sl, void *y, char *ws, hipStream_t st, int rotate) {
    if constexpr (!std::is_same<T, uint16_t>::value || K > 5) {
        return WTCONV_ERR_DTYPE;  // not planned: bfloat16 with K = 3 or 5 only
    } else {
        const wtconv_desc &d = ps.d;
        const FwdPlan &p = ps.fp;
        const int bf = dtype_of<T>();
        const int L = d.levels;
        for (int l = 1; l < L; ++l) {
            CarrierArgs c{};
            c.in = l == 1 ? x : (const void *)(ws + p.c_off[l - 2]);
            c.out = ws + p.c_off[l - 1];
            c.planes = d.n * d.c;
            c.Hi = p.ld.H[l - 1];
            c.Wi = p.ld.W[l - 1];
            c.Ho = p.ld.H[l];
            c.Wo = p.ld.W[l];
            c.groups = cdiv(c.Wo, 4);
            c.vec = c.Wi % 8 == 0 && aligned(c.in, 16) ? 1 : 0;
            const dim3 grid((unsigned)cdiv((long long)c.Ho * c.groups, kThreads),
                            (unsigned)std::min(c.planes, 65535));
            int rc = launch("carrier", K, bf, l, carrier_kernel<T>, grid, dim3(kThreads), 0, st, c);
            if (rc) return rc;
        }
        for (int l = L; l >= 2; --l) {
            int rc = run_level_fwd<K, T>(ps, "level_acc", l, ws + p.c_off[l - 2],
                                         l < L ? (const void *)(ws + p.q_off[l]) : nullptr, false, wl, sl, ws, st,
                                         rotate);
            if (rc) return rc;
        }
        MmaTileArgs a = ps.ta;
        a.x = x;
        a.y = y;
        a.w0 = w0;
        a.b0 = b0;
        a.s0 = s0;
        a.wl = wl;
        a.sl = sl;
        a.rotate = rotate;
        a.q = L >= 2 ? (const void *)(ws + p.q_off[1]) : nullptr;
        a.vec = d.w % 8 == 0 && aligned(x, 16) ? 1 : 0;
        a.pairs = d.w % 2 == 0 && aligned(y, 2 * sizeof(T)) ? 1 : 0;
        const dim3 grid((unsigned)tile_grid<K, T>(ps));
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        return launch("mma_tile", K, bf, 0, mma_tile_kernel<K>, grid, dim3(kTileThreads), shm, st, a);
    }
}

template <int K, typename T>
int run_forward(const PlanSet &ps, const void *x, const float *w0, const float *b0, const float *s0,
                const float *wl, const float *sl, void *y, char *ws, hipStream_t st, int rotate) {
    if (ps.mma) return run_mma_forward<K, T>(ps, x, w0, b0, s0, wl, sl, y, st, rotate);
    if (ps.plane) return run_plane_forward<K, T>(ps, x, w0, b0, s0, wl, sl, y, st, rotate);
    if (ps.mtile) return run_tile_forward<K, T>(ps, x, w0, b0, s0, wl, sl, y, ws, st, rotate);
    const wtconv_desc &d = ps.d;
    const FwdPlan &p = ps.fp;
    const int L = d.levels;
    for (int l = 1; l <= L; ++l) {
        int rc = run_level_fwd<K, T>(ps, "level_fwd", l, l == 1 ? x : (const void *)(ws + p.c_off[l - 2]), nullptr,
                                     true, wl, sl, ws, st, rotate);
        if (rc) return rc;
    }
    const int bf = dtype_of<T>();  // dtype code, for the launch records
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

// Base and level-1 weight gradients by the tiled correlation kernel; with levels
// >= 2 it also writes the level-1 carriers of x and dy.
template <int K, typename T>
int run_dwc_tile(const PlanSet &ps, const void *x, const void *dy, float *partial, char *ws, hipStream_t st) {
    if constexpr (!std::is_same<T, uint16_t>::value) {
        return WTCONV_ERR_DTYPE;  // not planned: bfloat16 only
    } else {
        const wtconv_desc &d = ps.d;
        const DwPlan &p = ps.dp;
        DwcTileArgs a = p.ta;
        a.x = x;
        a.dy = dy;
        a.pbase = partial + p.region[0];
        a.plev = d.levels >= 1 ? partial + p.region[1] : nullptr;
        a.xc = d.levels >= 2 ? (void *)(ws + p.xc_off[0]) : nullptr;
        a.gc = d.levels >= 2 ? (void *)(ws + p.gc_off[0]) : nullptr;
        a.vec = d.w % 8 == 0 && aligned(x, 16) && aligned(dy, 16) ? 1 : 0;
        const dim3 grid((unsigned)((long long)d.c * a.k));
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        const int bf = dtype_of<T>();
        if (d.levels >= 1)
            return launch("dwc_tile", K, bf, 0, dwc_tile_kernel<K, true>, grid, dim3(kDwcThreads), shm, st, a);
        return launch("dwc_tile", K, bf, 0, dwc_tile_kernel<K, false>, grid, dim3(kDwcThreads), shm, st, a);
    }
}

// Level l >= 2 by the tiled correlation kernel on the level-(l - 1) carriers of x and
// dy (their level-1 raw sums are level l's); it writes the level-l carriers for the
// next level, and its base sums to a region nothing reads.
template <int K, typename T>
int run_dwc_tile_level(const PlanSet &ps, int l, float *partial, char *ws, hipStream_t st) {
    if constexpr (!std::is_same<T, uint16_t>::value) {
        return WTCONV_ERR_DTYPE;  // not planned: bfloat16 only
    } else {
        const wtconv_desc &d = ps.d;
        const DwPlan &p = ps.dp;
        DwcTileArgs a = p.tal[l - 1];
        a.x = ws + p.xc_off[l - 2];
        a.dy = ws + p.gc_off[l - 2];
        a.pbase = partial + p.trash;
        a.plev = partial + p.region[l];
        a.xc = l < d.levels ? (void *)(ws + p.xc_off[l - 1]) : nullptr;
        a.gc = l < d.levels ? (void *)(ws + p.gc_off[l - 1]) : nullptr;
        a.vec = a.W % 8 == 0 && aligned(a.x, 16) && aligned(a.dy, 16) ? 1 : 0;
        const dim3 grid((unsigned)((long long)d.c * a.k));
        const size_t shm = (size_t)a.lds_floats * sizeof(float);
        return launch("dwc_tile", K, dtype_of<T>(), l, dwc_tile_kernel<K, true>, grid, dim3(kDwcThreads), shm, st, a);
    }
}

template <int K, typename T>
int run_backward_weight(const PlanSet &ps, const void *x, const void *dy, const float *w0, const float *b0,
                        const float *s0, const float *wl, const float *sl, float *dw0, float *db0, float *ds0,
                        float *dwl, float *dsl, char *ws, hipStream_t st) {
    const wtconv_desc &d = ps.d;
    const DwPlan &p = ps.dp;
    const int bf = dtype_of<T>();  // dtype code, for the launch records
    const int L = d.levels;
    float *partial = reinterpret_cast<float *>(ws + p.part_off);
    if (!empty(d) && p.dwc) {
        int rc = run_plane_dwc<K, T>(ps, x, dy, partial, st);
        if (rc) return rc;
    }
    if (!empty(d) && p.dwc_lev) {
        if (L >= 2) {
            int rc = run_plane_dwl<K, T>(ps, x, dy, partial, st);
            if (rc) return rc;
        }
    } else if (!empty(d)) {
        if (p.dwl && L > 0) {
            int rc = run_plane_dwl<K, T>(ps, x, dy, partial, st);
            if (rc) return rc;
        }
        if (p.dtile) {
            int rc = run_dwc_tile<K, T>(ps, x, dy, partial, ws, st);
            if (rc) return rc;
        }
        for (int l = p.dtile ? 2 : 1; l <= L && !p.dwl; ++l) {
            if (p.dtl[l - 1]) {
                int rc = run_dwc_tile_level<K, T>(ps, l, partial, ws, st);
                if (rc) return rc;
                continue;
            }
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
        if (p.dwc || p.dtile) {
            // the base ran in the correlation kernel
        } else if (p.dwb) {
            int rc = run_plane_dwb<K, T>(ps, x, dy, partial + p.region[0], st);
            if (rc) return rc;
        } else {
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
            int rc = launch("dw_base", K, bf, 0, dw_base_kernel<K, T>, dim3((unsigned)grid_of(b.t, d.c)),
                            dim3(kThreads), shm, st, b);
            if (rc) return rc;
        }
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

}  // namespace wtc
