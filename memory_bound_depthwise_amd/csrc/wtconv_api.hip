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
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "wtconv.h"
#include "wtconv_kernels.hpp"

namespace wtc {
namespace {

constexpr int kThreads = 256;
constexpr size_t kLdsBudget = 64 * 1024;   // bytes of LDS per workgroup we allow
constexpr int kTargetItems = 256;          // strips per workgroup pass
constexpr int kDwTargetBlocks = 2048;      // workgroups wanted for the gradient kernels
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

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

template <typename Kern, typename Args>
int launch(const char *family, int K, int is_bf16, Kern kern, dim3 grid, dim3 block, size_t shmem,
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
        snprintf(name, sizeof(name), "%s<%d,%s>", family, K, is_bf16 ? "bf16" : "f32");
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

// Bytes of LDS a kernel needs for a tiling, as a function of (PB, TY, SP).
enum class Kind { LevelFwd, Synth, DwLevel, DwBase };

int strip_of(Kind k) { return k == Kind::LevelFwd ? 4 : 8; }

size_t lds_bytes(Kind kind, int K, int PB, int TY, int SP) {
    const int S = strip_of(kind), KK = K * K;
    const size_t HY = TY + K - 1, HXP = (size_t)SP * S + K - 1, GW = (size_t)SP * S;
    switch (kind) {
        case Kind::LevelFwd: return (4 * KK + (size_t)PB * 4 * HY * HXP) * sizeof(float);
        case Kind::Synth: return (KK + (size_t)PB * HY * HXP) * sizeof(float);
        case Kind::DwLevel:
            return ((size_t)PB * 4 * HY * HXP + (size_t)PB * 4 * TY * GW + (kThreads / 256) * 4 * KK) * sizeof(float);
        case Kind::DwBase:
            return ((size_t)PB * HY * HXP + (size_t)PB * TY * GW + (kThreads / 64) * (KK + 1)) * sizeof(float);
    }
    return 0;
}

// Tile an Ho x Wo output grid: rows of at most 64 columns, about kTargetItems
// strips per pass, as many planes stacked per pass as that leaves room for (small
// planes), within the LDS budget.
Tiling pick_tiling(Kind kind, int K, int n, int C, int Ho, int Wo) {
    const int S = strip_of(kind);
    Tiling t{};
    if (n <= 0 || Ho <= 0 || Wo <= 0) {
        t.TY = t.TX = t.SP = t.tiles_x = t.PB = t.NB = 1;
        t.tiles = t.nblk = 0;
        return t;
    }
    t.tiles_x = cdiv(Wo, 64);
    t.TX = cdiv(Wo, t.tiles_x);
    t.SP = cdiv(t.TX, S);
    int ty_max = std::max(1, kTargetItems / t.SP);
    for (;;) {
        const int tiles_y = cdiv(Ho, ty_max);
        t.TY = cdiv(Ho, tiles_y);
        t.tiles = tiles_y * t.tiles_x;
        t.PB = std::max(1, std::min(n, kTargetItems / std::max(1, t.TY * t.SP)));
        while (t.PB > 1 && lds_bytes(kind, K, t.PB, t.TY, t.SP) > kLdsBudget) --t.PB;
        if (ty_max == 1 || lds_bytes(kind, K, t.PB, t.TY, t.SP) <= kLdsBudget) break;
        ty_max = std::max(1, ty_max / 2);  // one plane's tile is still too tall
    }
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

bool tiling_fits(Kind kind, int K, const Tiling &t) {
    return lds_bytes(kind, K, t.PB, t.TY, t.SP) <= kLdsBudget;
}

long long grid_of(const Tiling &t, int C) { return (long long)t.tiles * C * t.nblk; }

struct FwdPlan {
    LevelDims ld;
    size_t q_off[kMaxLevels], c_off[kMaxLevels];  // byte offsets into the workspace
    Tiling lvl[kMaxLevels], syn;
    size_t bytes;
};

struct DwPlan {
    LevelDims ld;
    size_t xc_off[kMaxLevels], gc_off[kMaxLevels];
    size_t part_off;                 // byte offset of the partials
    long long region[kMaxLevels + 1];  // float offsets within the partials
    int G[kMaxLevels + 1];
    Tiling lvl[kMaxLevels], base;
    size_t bytes;
};

size_t elem_size(int dtype) { return dtype == WTCONV_BF16 ? 2 : 4; }

FwdPlan plan_forward(const wtconv_desc &d) {
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
    for (int l = 1; l <= d.levels; ++l) p.lvl[l - 1] = pick_tiling(Kind::LevelFwd, d.k, d.n, d.c, p.ld.H[l], p.ld.W[l]);
    p.syn = pick_tiling(Kind::Synth, d.k, d.n, d.c, d.h, d.w);
    p.bytes = off;
    return p;
}

DwPlan plan_backward_weight(const wtconv_desc &d) {
    DwPlan p{};
    p.ld = level_dims(d);
    const size_t es = elem_size(d.dtype), planes = (size_t)d.n * d.c;
    size_t off = 0;
    for (int l = 1; l < d.levels; ++l) {
        p.xc_off[l - 1] = off;
        off = align_up(off + planes * p.ld.H[l] * p.ld.W[l] * es);
        p.gc_off[l - 1] = off;
        off = align_up(off + planes * p.ld.H[l] * p.ld.W[l] * es);
    }
    p.part_off = off;
    const int KK = d.k * d.k;
    p.base = pick_tiling(Kind::DwBase, d.k, d.n, d.c, d.h, d.w);
    long long floats = 0;
    p.region[0] = 0;
    p.G[0] = (d.n > 0 && d.h > 0 && d.w > 0) ? p.base.nblk * p.base.tiles : 0;
    floats += (long long)d.c * p.G[0] * (KK + 1);
    for (int l = 1; l <= d.levels; ++l) {
        p.lvl[l - 1] = pick_tiling(Kind::DwLevel, d.k, d.n, d.c, p.ld.H[l], p.ld.W[l]);
        p.region[l] = floats;
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

int check_desc(const wtconv_desc *d) {
    if (!d) return WTCONV_ERR_NULL;
    if (d->n < 0 || d->c < 0 || d->h < 0 || d->w < 0 || d->reserved != 0) return WTCONV_ERR_SHAPE;
    if (d->k != 3 && d->k != 5 && d->k != 7) return WTCONV_ERR_KERNEL;
    if (d->levels < 0 || d->levels > kMaxLevels) return WTCONV_ERR_LEVELS;
    if (d->dtype != WTCONV_F32 && d->dtype != WTCONV_BF16) return WTCONV_ERR_DTYPE;
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
int run_forward(const wtconv_desc &d, const void *x, const float *w0, const float *b0, const float *s0,
                const float *wl, const float *sl, void *y, char *ws, hipStream_t st, int rotate) {
    const FwdPlan p = plan_forward(d);
    const int bf = std::is_same<T, uint16_t>::value;
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
        a.t = p.lvl[l - 1];
        const size_t shm = lds_bytes(Kind::LevelFwd, K, a.t.PB, a.t.TY, a.t.SP);
        int rc = launch("level_fwd", K, bf, level_fwd_kernel<K, T>, dim3((unsigned)grid_of(a.t, d.c)),
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
    const size_t shm = lds_bytes(Kind::Synth, K, s.t.PB, s.t.TY, s.t.SP);
    return launch("synth", K, bf, synth_kernel<K, T>, dim3((unsigned)grid_of(s.t, d.c)), dim3(kThreads), shm, st,
                  s);
}

template <int K, typename T>
int run_backward_weight(const wtconv_desc &d, const void *x, const void *dy, const float *w0, const float *b0,
                        const float *s0, const float *wl, const float *sl, float *dw0, float *db0, float *ds0,
                        float *dwl, float *dsl, char *ws, hipStream_t st) {
    const DwPlan p = plan_backward_weight(d);
    const int bf = std::is_same<T, uint16_t>::value;
    const int L = d.levels;
    float *partial = reinterpret_cast<float *>(ws + p.part_off);
    if (!empty(d)) {
        for (int l = 1; l <= L; ++l) {
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
            a.t = p.lvl[l - 1];
            const size_t shm = lds_bytes(Kind::DwLevel, K, a.t.PB, a.t.TY, a.t.SP);
            int rc = launch("dw_level", K, bf, dw_level_kernel<K, T>, dim3((unsigned)grid_of(a.t, d.c)),
                            dim3(kThreads), shm, st, a);
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
        const size_t shm = lds_bytes(Kind::DwBase, K, b.t.PB, b.t.TY, b.t.SP);
        int rc = launch("dw_base", K, bf, dw_base_kernel<K, T>, dim3((unsigned)grid_of(b.t, d.c)), dim3(kThreads),
                        shm, st, b);
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
    return launch("dw_finalize", K, bf, dw_finalize_kernel<K>, dim3((unsigned)d.c, (unsigned)(L + 1)), dim3(128), 0,
                  st, f);
}

#define WTC_DISPATCH(KVAL, DTYPE, FN, ...)                                   \
    do {                                                                    \
        const bool bf16_ = (DTYPE) == WTCONV_BF16;                          \
        switch (KVAL) {                                                     \
            case 3: return bf16_ ? FN<3, uint16_t>(__VA_ARGS__) : FN<3, float>(__VA_ARGS__); \
            case 5: return bf16_ ? FN<5, uint16_t>(__VA_ARGS__) : FN<5, float>(__VA_ARGS__); \
            case 7: return bf16_ ? FN<7, uint16_t>(__VA_ARGS__) : FN<7, float>(__VA_ARGS__); \
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
    const FwdPlan p = plan_forward(d);
    if (p.bytes > 0 && (!workspace || workspace_bytes < p.bytes)) return WTCONV_ERR_WORKSPACE;
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
        *bytes = empty(*desc) ? 0 : plan_forward(*desc).bytes;
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
