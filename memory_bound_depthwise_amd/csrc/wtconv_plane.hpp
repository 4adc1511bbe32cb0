// Plane-resident forward kernel of the WTConv layer on the polyphase grid.
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §4.  The layer output is the base conv plus, for every level,
// the level's filtered coefficients mapped back to pixels by the closed-form
// synthesis (§4.2, Prop. 2 / Eq. 7): pixel (y, x) takes from level l the sign
// pattern of the block at (y >> l, x >> l) selected by bit l-1 of y and of x.
// The kernel keeps a whole plane and its pyramid in LDS and moves only x in and y
// out (2N elements per pass).
//
// Layout.  Everything lives on the level-1 grid (one cell per 2 x 2 pixel block).
// LDS holds, per cell, the four unscaled level-1 Haar bands S1 = (LL, LH, HL, HH)
// as one float4 (Eq. 5 without its factor 1/2, so S_l = 2^l Y_l); x itself is not
// kept: the base conv rebuilds the four pixels of a cell from its bands with the
// inverse butterfly (Prop. 1: H^2 = I, so the synthesis is the same butterfly; its
// factor 1/4 is folded into the base weights).  Deeper levels l >= 2 keep their
// bands S_l (float4 per cell) and, after filtering, their sign patterns Q_l (four
// per block, at level l-1 resolution: Q_l[2a+ry][2b+rx]).  Each array has a zero
// halo of R = (K-1)/2 cells and a row stride chosen so that the lanes of a
// wavefront, which take consecutive items, hit distinct banks.  Small planes are
// placed side by side, PB per pass, with zero columns between them at least R wide
// at every level, so that each pass fills the workgroup.
//
// One workgroup (128 threads) owns one channel and walks a range of its planes:
//   1. commit: the prefetched 2 x 2CW pixel patches become S1 (the level-1
//      butterflies are done in registers); the loads of the next pass are issued;
//   2. Haar analysis of levels 2..L from the low-pass band of the level above;
//   3. deep levels: one item is one column x 2 rows of all four bands of one level;
//      the filtered bands (weights folded with s(l) 4^-l: the scale of Eq. 8, the
//      2^-l of S_l and the 2^-l synthesis weight of Eq. 7) give the four sign
//      patterns of each block (Eq. 12/13), written to Q_l;
//   4. final: one item is one level-1 column x RH level-1 rows, i.e. a 2-pixel x
//      2RH-pixel tile.  Walking the K columns of the level-1 window, the lane
//      filters the four level-1 bands and, on the columns the base conv needs,
//      rebuilds x and runs the base conv over its polyphase components; then it adds
//      the deeper levels' patterns and the bias to the low-pass band (it enters all
//      four sign patterns with a plus sign), forms the level-1 patterns (the
//      level-1 synthesis) and stores y = s0 (W0 * x) + patterns, two adjacent
//      pixels per store.
// With rotate = 1 (and no bias) the same kernel computes the input gradient
// (each kernel turned by 180 degrees, Prop. 1 / Eq. 1).

#pragma once

#include "wtconv_kernels.hpp"

namespace wtc {

constexpr int kFwdThreads = 128;  // threads of a forward workgroup
constexpr int kPlaneCO = 4;         // first data cell of every grid row (left halo)
constexpr int kPlaneRHd = 2;        // level rows of a deep-level item
constexpr int kPlaneMaxWords = 16;  // prefetch registers per thread
constexpr int kPlaneTabFields = 8;  // per deep level: dend, width, 1/width, band stride, band offset,
                                    // pattern stride, pattern offset, rows

// Exact n / d for 0 <= n < 2^16 and 1 <= d < 2^15 with m = ceil(2^31 / d): one
// multiply-high and no special case for d = 1 (checked exhaustively on the host).
__device__ __forceinline__ int udiv16(int n, uint32_t m) { return (int)__umulhi((uint32_t)n << 1, m); }

struct PlaneArgs {
    const void *x;
    void *y;
    const float *w0, *b0, *s0, *wl, *sl;
    int n, C, H, W, L;
    int rotate;
    int vec;               // x rows are read with vector loads (W % 2CW == 0, aligned)
    int pair_store;        // y is written two pixels per store (W even, aligned)
    int PB, Pw1;           // planes per pass (side by side), level-1 column pitch between them
    int NG, U;             // image groups of PB per channel, units (C NG; a unit is one pass)
    int H1, W1;            // level-1 grid of one plane
    int S1;                // level-1 strips of RH rows
    int sy1, a1;           // level-1 bands: row stride and size in cells (from cell 0)
    int Gw;                // commit column groups of CW cells per level-1 row
    int commit_items;      // PB * H1 * Gw
    int final_items;       // S1 * PB * W1
    // deep levels l = 2..L at index l - 2
    int hl[kMaxLevels], wls[kMaxLevels];   // grid rows, width of the side-by-side row
    int sd[kMaxLevels];                    // strips of kPlaneRHd rows
    int syd[kMaxLevels], offd[kMaxLevels];  // bands: row stride (cells), offset (cells)
    int sq[kMaxLevels], offq[kMaxLevels];  // sign patterns: row stride (floats), offset (floats)
    int dend[kMaxLevels];                  // cumulative deep items (strips x width) by level
    int wt;                                // weight table (floats)
    int zero_floats;                       // floats cleared at the start (bands, patterns, weights)
    int tab;                               // deep-level geometry table (kPlaneTabFields ints per level)
    int lds_floats;
    uint32_t m_gw, m_h1, m_strip, m_w1;    // udiv16 reciprocals of Gw, H1, PB*W1, W1
    uint32_t m_wls[kMaxLevels];            // ... of the deep widths
};

// Raw words of one commit item: two pixel rows of 2CW elements.
template <typename T, int CW>
struct PatchIO {
    static constexpr int kWords = sizeof(T) == 2 ? CW : 2 * CW;  // per row

    __device__ __forceinline__ static void load_row(uint32_t *r, const T *src, bool vec, int col0, int W) {
        if (vec) {
            if constexpr (sizeof(T) * 2 * CW == 32) {
                const uint4 q0 = reinterpret_cast<const uint4 *>(src)[0];
                const uint4 q1 = reinterpret_cast<const uint4 *>(src)[1];
                r[0] = q0.x; r[1] = q0.y; r[2] = q0.z; r[3] = q0.w;
                r[4] = q1.x; r[5] = q1.y; r[6] = q1.z; r[7] = q1.w;
            } else if constexpr (sizeof(T) * 2 * CW == 16) {
                const uint4 q = *reinterpret_cast<const uint4 *>(src);
                r[0] = q.x; r[1] = q.y; r[2] = q.z; r[3] = q.w;
            } else if constexpr (sizeof(T) * 2 * CW == 8) {
                const uint2 q = *reinterpret_cast<const uint2 *>(src);
                r[0] = q.x; r[1] = q.y;
            } else {
                r[0] = *reinterpret_cast<const uint32_t *>(src);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 2 * CW; ++e) {
                uint32_t v = 0;
                if (col0 + e < W) {
                    if constexpr (sizeof(T) == 2) v = reinterpret_cast<const uint16_t *>(src)[e];
                    else v = reinterpret_cast<const uint32_t *>(src)[e];
                }
                if constexpr (sizeof(T) == 2) {
                    if (e & 1) r[e >> 1] |= v << 16;
                    else r[e >> 1] = v;
                } else {
                    r[e] = v;
                }
            }
        }
    }

    __device__ __forceinline__ static float elem(const uint32_t *r, int e) {
        if constexpr (kHalf<T>) {
            const uint32_t wv = r[e >> 1];
            return (e & 1) ? Act<T>::hi(wv) : Act<T>::lo(wv);
        } else {
            return __uint_as_float(r[e]);
        }
    }
};

// Loads of a prefetched patch (rows 2i, 2i + 1 of plane p, elements [2CW m, 2CW m +
// 2CW)) from addresses clamped into the images, with no register cleared first;
// mask_patch zeroes what lies outside once the data is used.  A register that is
// cleared and then maybe loaded makes the compiler wait for every load in flight
// before it clears that register again, which would serialize the prefetch.
template <typename T, int CW>
using PatchRegs = uint32_t[2][PatchIO<T, CW>::kWords];
template <typename T, int CW>
__device__ __forceinline__ void load_patch_clamped(PatchRegs<T, CW> &r, const T *base, int p, int i, int m, int live,
                                                   int CHW, int H, int W, bool vec) {
    p = min(p, live - 1);
    const int col0 = 2 * CW * m;
    const T *src = base + (p * CHW + (2 * i) * W + col0);
    PatchIO<T, CW>::load_row(r[0], src, vec, col0, W);
    PatchIO<T, CW>::load_row(r[1], src + (2 * i + 1 < H ? W : 0), vec, col0, W);
}
template <typename T, int CW>
__device__ __forceinline__ void mask_patch(PatchRegs<T, CW> &r, int p, int i, int live, int H, bool full = false) {
    if (full) return;  // wave-uniform: every plane of the pass is live and H is even
#pragma unroll
    for (int w = 0; w < PatchIO<T, CW>::kWords; ++w) {
        if (p >= live) r[0][w] = 0;
        if (p >= live || 2 * i + 1 >= H) r[1][w] = 0;
    }
}

// One commit item: patch rows 2i, 2i+1 of plane p, level-1 cells [CW m, CW m + CW):
// the level-1 butterflies of each cell (kBase: the four pixels themselves).
template <int K, typename T, int CW, bool kBase>
__device__ __forceinline__ void commit_patch(float4 *s4, int sy1, int pw1,
                                             const uint32_t (&raw)[2][PatchIO<T, CW>::kWords], int p, int i, int m) {
    constexpr int R = (K - 1) / 2;
    using IO = PatchIO<T, CW>;
    float4 *d = s4 + (i + R) * sy1 + kPlaneCO + p * pw1 + m * CW;
#pragma unroll
    for (int q = 0; q < CW; ++q) {
        const float x00 = IO::elem(raw[0], 2 * q), x01 = IO::elem(raw[0], 2 * q + 1);
        const float x10 = IO::elem(raw[1], 2 * q), x11 = IO::elem(raw[1], 2 * q + 1);
        if constexpr (kBase) {
            d[q] = make_float4(x00, x01, x10, x11);
        } else {
            const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
            d[q] = make_float4(s0 + s1, s0 - s1, d0 + d1, d0 - d1);
        }
    }
}

// Workgroup index with the workgroups of one XCD numbered consecutively.  The
// command processor deals the workgroups of a launch to the eight XCDs in turn
// (workgroup w to XCD w mod 8), and each XCD has an L2 of its own; numbered this
// way, the workgroups that take neighbouring units (neighbouring channels, whose
// planes share cache lines at their ends) sit behind the same L2.  A bijection of
// [0, G) for any G.
__device__ __forceinline__ int xcd_block(int w, int G) {
    const int x = w & 7, q = G >> 3, r = G & 7;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + (w >> 3);
}

// Wave priority of a workgroup that walks a fixed range of passes, from the passes
// it has left (rem of total; wave-uniform).  The instruction arbiter favours older
// waves, so of the workgroups that share a compute unit the last dispatched fall
// behind and finish last, with equal work.  Lowering the priority of workgroups as
// they near the end of their range lets the others catch up, and the launch ends
// sooner (measured with per-workgroup timestamps: the finish times of the six
// workgroups of a compute unit moved from 61..79 us to 66..75 us).
__device__ __forceinline__ void balance_priority(int rem, int total) {
    const int p = total >= 8 ? rem >> 1 : rem - 1;
    if (p >= 3) {
        __builtin_amdgcn_s_setprio(3);
    } else if (p == 2) {
        __builtin_amdgcn_s_setprio(2);
    } else if (p == 1) {
        __builtin_amdgcn_s_setprio(1);
    } else {
        __builtin_amdgcn_s_setprio(0);
    }
}

// Wave-uniform value made opaque to the optimizer: what is computed from it is
// computed after this point, inside the current phase, instead of being held in
// scalar registers from the top of the kernel.
__device__ __forceinline__ int opaque(int v) {
    v = __builtin_amdgcn_readfirstlane(v);
    asm volatile("" : "+s"(v));
    return v;
}
// A wave-uniform pointer to global memory held in scalar registers (in the global
// address space, so that loads through it are global, not flat, loads).
typedef const __attribute__((address_space(1))) float gfloat;
__device__ __forceinline__ gfloat *opaque_ptr(const float *p) {
    uint64_t v = reinterpret_cast<uint64_t>(p);
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    asm volatile("" : "+s"(lo), "+s"(hi));
    return reinterpret_cast<gfloat *>(((uint64_t)hi << 32) | lo);
}

// z[b][i] += sum_{u,v} wt[v][u].b * win[(i + u) * stride + v].b for the four bands b.
// The tap-column loop stays rolled: unrolled, the compiler issues the reads of every
// column up front and runs out of registers.
template <int K, int RH>
__device__ __forceinline__ void conv_bands(const float4 *win, int stride, const float4 *wt, float (&z)[4][RH]) {
#pragma unroll 1
    for (int v = 0; v < K; ++v) {
        float4 wb[K];
#pragma unroll
        for (int u = 0; u < K; ++u) wb[u] = wt[v * K + u];
        float4 cl[RH + K - 1];
#pragma unroll
        for (int t = 0; t < RH + K - 1; ++t) cl[t] = win[t * stride + v];
#pragma unroll
        for (int u = 0; u < K; ++u)
#pragma unroll
            for (int i = 0; i < RH; ++i) {
                z[0][i] = fmaf(wb[u].x, cl[i + u].x, z[0][i]);
                z[1][i] = fmaf(wb[u].y, cl[i + u].y, z[1][i]);
                z[2][i] = fmaf(wb[u].z, cl[i + u].z, z[2][i]);
                z[3][i] = fmaf(wb[u].w, cl[i + u].w, z[3][i]);
            }
    }
}

// Haar analysis of levels l0..L of a plane-resident pass (unscaled butterflies of
// the low-pass band of the level above; level 1 is the first grid's .x band).
template <int K, typename Args>
__device__ __forceinline__ void haar_levels(const Args &a, float4 *s4, int l0, int tid, int NT) {
    constexpr int R = (K - 1) / 2;
    for (int l = l0; l <= a.L; ++l) {
        const int li = l - 2, Wls = a.wls[li];
        const float4 *src = s4 + (l == 2 ? 0 : a.offd[li - 1]);
        const int ss = l == 2 ? a.sy1 : a.syd[li - 1];
        float4 *dst = s4 + a.offd[li];
        const int ds = a.syd[li];
        for (int q = tid; q < a.hl[li] * Wls; q += NT) {
            const int i = udiv16(q, a.m_wls[li]), j = q - i * Wls;
            const float4 *sp = src + (2 * i + R) * ss + 2 * j + kPlaneCO;
            const float x00 = sp[0].x, x01 = sp[1].x, x10 = sp[ss].x, x11 = sp[ss + 1].x;
            const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
            dst[(i + R) * ds + j + kPlaneCO] = make_float4(s0 + s1, s0 - s1, d0 + d1, d0 - d1);
        }
        __syncthreads();
    }
}

// Deep levels l >= 2 of a plane-resident pass: the filtered bands of each level
// (weights folded with s(l) 4^-l: the scale of Eq. 8, the 2^-l of S_l and the 2^-l
// synthesis weight of Eq. 7) give the four sign patterns of each block (Eq. 12/13),
// written to Q_l.  One item is one column x kPlaneRHd rows of all four bands of one
// level; items of all levels are spread over all lanes.
template <int K, typename Args>
__device__ __forceinline__ void deep_patterns(const Args &a, float4 *s4, float *smem, const int *tab, int tid,
                                              int NT) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    const int L = a.L;
    if (L < 2) return;
    for (int it = tid; it < a.dend[L - 2]; it += NT) {
        // the item's level from comparisons with the (wave-uniform) level ends,
        // then its geometry from the LDS table in one round of independent reads
        int li = 0;
        for (int k = 0; k < L - 2; ++k) li += it >= a.dend[k] ? 1 : 0;
        const int *tl = tab + li * kPlaneTabFields;
        const int loc = it - (li ? tl[-kPlaneTabFields] : 0), Wls = tl[1];
        const int s = udiv16(loc, (uint32_t)tl[2]), j = loc - s * Wls;
        const int syd = tl[3];
        float z[4][kPlaneRHd];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < kPlaneRHd; ++i) z[b][i] = 0.f;
        conv_bands<K, kPlaneRHd>(s4 + tl[4] + (s * kPlaneRHd) * syd + j + kPlaneCO - R, syd,
                                 s4 + (opaque(a.wt) >> 2) + (li + 1) * KK, z);
        const int sq = tl[5], hl = tl[7];
        float *q = smem + tl[6] + 2 * j;
#pragma unroll
        for (int i = 0; i < kPlaneRHd; ++i) {
            const int row = s * kPlaneRHd + i;
            if (row >= hl) break;
            const float a0v = z[0][i] + z[1][i], a1v = z[0][i] - z[1][i];
            const float b0 = z[2][i] + z[3][i], b1 = z[2][i] - z[3][i];
            *reinterpret_cast<float2 *>(q + (2 * row) * sq) = make_float2(a0v + b0, a0v - b0);
            *reinterpret_cast<float2 *>(q + (2 * row + 1) * sq) = make_float2(a1v + b1, a1v - b1);
        }
    }
    __syncthreads();
}

// kBase: levels = 0 (a plain depthwise conv); cells hold the four pixels of each
// 2 x 2 block as loaded, and there is no level to filter.
template <int K, typename T, int CW, int RH, bool kBase>
__device__ __forceinline__ void plane_fwd_body(const PlaneArgs &args) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    constexpr int RC = (R + 1) / 2;  // cells a pixel tap reaches beyond its own cell
    constexpr int NT = kFwdThreads;
    using IO = PatchIO<T, CW>;
    constexpr int SLOTS = kPlaneMaxWords / (2 * IO::kWords) > 0 ? kPlaneMaxWords / (2 * IO::kWords) : 1;
    extern __shared__ float smem[];
    float4 *s4 = reinterpret_cast<float4 *>(smem);
    const PlaneArgs &a0 = args;
    const int tid = threadIdx.x;
    const int HW = a0.H * a0.W, CHW = a0.C * HW, PB = a0.PB;
    constexpr int WSLOTS = 3;  // weight-table entries per thread carried in registers

    for (int i = tid * 4; i < a0.zero_floats; i += NT * 4)
        *reinterpret_cast<float4 *>(smem + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    // Geometry of the deep levels, for the deep phase, whose lanes take items of
    // different levels: read from LDS there, it costs no vector-memory wait (which
    // would also wait for the prefetch in flight).  Visible after the first barrier.
    int *tab = reinterpret_cast<int *>(smem + a0.tab);
    if (tid < a0.L - 1) {
        int *t = tab + tid * kPlaneTabFields;
        t[0] = a0.dend[tid];
        t[1] = a0.wls[tid];
        t[2] = (int)a0.m_wls[tid];
        t[3] = a0.syd[tid];
        t[4] = a0.offd[tid];
        t[5] = a0.sq[tid];
        t[6] = a0.offq[tid];
        t[7] = a0.hl[tid];
    }

    // A unit is PB images of one channel: unit u = (channel u % C, images
    // [(u / C) PB, ...)).  Workgroup w takes units w, w + G, w + 2G, ...; workgroups
    // running side by side take neighbouring channels of the same images, whose
    // planes are adjacent in memory (small planes share cache lines).
    auto unit_of = [&](const auto &A, int u, int &c, int &n0) {
        const int g = u / A.C;
        c = u - g * A.C;
        n0 = g * A.PB;
    };
    // Patch (p, i, m) of commit item g: plane p, level-1 row i, cell group m.
    auto patch_of = [&](const auto &A, int g, int &p, int &i, int &m) {
        const int q = udiv16(g, A.m_gw);
        m = g - q * A.Gw;
        p = udiv16(q, A.m_h1);
        i = q - p * A.H1;
    };
    // lanes past the last item load the last item again (their registers are not
    // used): all loads unconditional measured faster here than skipping them
    auto load_patch = [&](const auto &A, uint32_t (&r)[2][IO::kWords], const T *xb, int live, int g) {
        int p, i, m;
        patch_of(A, min(g, A.commit_items - 1), p, i, m);
        load_patch_clamped<T, CW>(r, xb, p, i, m, live, CHW, A.H, A.W, A.vec);
    };
    // Weight-table entry e of channel c: the two raw factors of its folded value
    // (loaded here, folded by fold_weight).  Level l, band b: s(l,b) 4^-l W(l,b)
    // (Eq. 8 scale, the 2^-l of the unscaled pyramid and the 2^-l synthesis
    // weight), as [l][v][u] float4 over b; base: s0 W0 / 4 as [v][u] (the base conv
    // runs on 4x, rebuilt from S1).  Kernels are turned by 180 degrees for the input
    // gradient.  The parameter pointers are taken as wave-uniform values, so each
    // lane loads through its own address and nothing waits for the loads here.
    // Entry (4L + 1) K^2, after the weights, is the folded bias s0 b.
    auto weight_factors = [&](const auto &A, int c, int e, float &f0, float &f1) {
        const gfloat *sl = opaque_ptr(A.sl), *wl = opaque_ptr(A.wl);
        const gfloat *s0 = opaque_ptr(A.s0), *w0 = opaque_ptr(A.w0), *b0 = opaque_ptr(A.b0);
        const int nl = 4 * A.L;
        const int lb = e / KK, tap = e - lb * KK;  // tap = v K + u (column-major)
        const int v = tap / K, u = tap - v * K;
        const int src = A.rotate ? (K - 1 - u) * K + (K - 1 - v) : u * K + v;
        const size_t pc = lb < nl ? (size_t)((lb >> 2) * A.C + c) * 4 + (lb & 3) : 0;
        const gfloat *p0 = lb < nl ? sl + pc : s0 + c;
        const gfloat *p1 = lb < nl ? wl + pc * KK + src : (lb == nl ? w0 + (size_t)c * KK + src : (b0 ? b0 : s0) + c);
        f0 = *p0;
        f1 = *p1;
    };
    auto fold_weight = [&](const auto &A, int e, float f0, float f1) {
        const int lb = e / KK, nl = 4 * A.L;
        return lb < nl ? ldexpf(f0, -2 * ((lb >> 2) + 1)) * f1
                       : (lb == nl ? (kBase ? 1.f : 0.25f) * f0 * f1 : (A.b0 ? f0 * f1 : 0.f));
    };
    auto weight_slot = [&](const auto &A, int e) {  // LDS float index of entry e
        const int lb = e / KK, tap = e - lb * KK;
        return lb < 4 * A.L ? A.wt + ((lb >> 2) * KK + tap) * 4 + (lb & 3) : A.wt + 4 * A.L * KK + (lb - 4 * A.L) * KK + tap;
    };

    uint32_t raw[SLOTS][2][IO::kWords];
    float wf0[WSLOTS], wf1[WSLOTS];
    auto prefetch = [&](const auto &A, int u) {
        int c, n0;
        unit_of(A, u, c, n0);
        const int live = min(A.PB, A.n - n0);
        const T *xb = static_cast<const T *>(A.x) + ((size_t)n0 * A.C + c) * HW;
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) load_patch(A, raw[k], xb, live, tid + k * NT);
#pragma unroll
        for (int k = 0; k < WSLOTS; ++k) weight_factors(A, c, min(tid + k * NT, (4 * A.L + 1) * KK), wf0[k], wf1[k]);
    };
    // (numbered as launched: renumbering per XCD measured 11 % slower for this kernel's
    // strided unit order)
    const int wb = blockIdx.x;
    if (wb < a0.U) prefetch(args, wb);

    const int own = wb < a0.U ? (a0.U - 1 - wb) / (int)gridDim.x + 1 : 0;
    for (int u = wb; u < a0.U; u += gridDim.x) {
        balance_priority(own - (u - wb) / (int)gridDim.x, own);
        // Every argument below is read through a pointer made opaque per pass, so
        // that nothing derived from the arguments is held in registers across passes.
        // (The argument block is the kernel's only argument: offset 0 of its segment.)
        const __attribute__((address_space(4))) PlaneArgs *ap =
            (const __attribute__((address_space(4))) PlaneArgs *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const auto &a = *ap;
        int c, n0;
        unit_of(a, u, c, n0);
        const int live = min(PB, a.n - n0);
        const int H = a.H, W = a.W, L = a.L;
        const bool full = live == PB && !(H & 1);  // nothing of the pass's patches needs masking
        __syncthreads();  // the previous pass is done with every array
        // 1. commit: this unit's weight table and level-1 bands
        {
            const int nw = (4 * L + 1) * KK + 1;  // weights and the bias
#pragma unroll
            for (int k = 0; k < WSLOTS; ++k) {
                const int e = tid + k * NT;
                if (e < nw) smem[weight_slot(a, e)] = fold_weight(a, e, wf0[k], wf1[k]);
            }
            for (int e = tid + WSLOTS * NT; e < nw; e += NT) {  // beyond the registers
                float f0, f1;
                weight_factors(a, c, e, f0, f1);
                smem[weight_slot(a, e)] = fold_weight(a, e, f0, f1);
            }
            const int sy1 = opaque(a.sy1), pw1 = opaque(a.Pw1);
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int g = tid + k * NT;
                if (g >= a.commit_items) continue;
                int p, i, m;
                patch_of(a, g, p, i, m);
                mask_patch<T, CW>(raw[k], p, i, live, H, full);
                commit_patch<K, T, CW, kBase>(s4, sy1, pw1, raw[k], p, i, m);
            }
            const T *xb = static_cast<const T *>(a.x) + ((size_t)n0 * a.C + c) * HW;
            for (int g = tid + SLOTS * NT; g < a.commit_items; g += NT) {  // beyond the registers
                uint32_t r[2][IO::kWords];
                load_patch(a, r, xb, live, g);
                int p, i, m;
                patch_of(a, g, p, i, m);
                mask_patch<T, CW>(r, p, i, live, H, full);
                commit_patch<K, T, CW, kBase>(s4, sy1, pw1, r, p, i, m);
            }
        }
        __syncthreads();

        // 2. Haar analysis of levels 2..L (unscaled butterflies of the low-pass band)
        haar_levels<K>(a, s4, 2, tid, NT);
        // 3. deep levels: filtered bands -> sign patterns Q_l
        deep_patterns<K>(a, s4, smem, tab, tid, NT);

        // The next unit's loads are issued only now, while no phase of this pass
        // waits for vector memory any more: a wait for anything loaded after them
        // (or for a register that one of them fills) would wait for all of them.
        if (u + (int)gridDim.x < a.U) prefetch(a, u + gridDim.x);
        T *yb = static_cast<T *>(a.y) + ((size_t)n0 * a.C + c) * HW;

        // 4. level 1 + base conv + deeper patterns, one store per pixel pair.  Every
        //    lane owns at most one item (the plan keeps final_items <= kFwdThreads).
        //    4a filters the four level-1 bands of the item's window into registers;
        //    once every item has read its window, 4b rewrites the item's own cells in
        //    place as their pixels (the inverse butterfly, once per cell; 4x, the 1/4
        //    is in the base weights); 4c runs the base conv on those pixels, adds the
        //    deeper levels' patterns and the bias, forms the level-1 patterns and
        //    stores.  Without levels the cells already hold the pixels: only 4c runs.
        //    Lanes past the last item of a wavefront that has items repeat that item
        //    (nothing of theirs is written), so that the branches stay uniform.
        {
            const bool has = tid < a.final_items;
            const int wave_has = __builtin_amdgcn_readfirstlane((tid & ~(kWave - 1)) < a.final_items ? 1 : 0);
            const int t = min(tid, a.final_items - 1);
            const int sy1 = opaque(a.sy1), wt = opaque(a.wt);
            const int s = udiv16(t, a.m_strip), r = t - s * (PB * a.W1);
            const int p = udiv16(r, a.m_w1), j = r - p * a.W1;
            const int col = p * a.Pw1 + j, row0 = s * RH;
            float z[4][RH];
            if constexpr (!kBase) {
                if (wave_has) {
                    // window cell (t, v) is level-1 cell (row0 - R + t, col - R + v)
                    const float4 *win = s4 + row0 * sy1 + col + kPlaneCO - R;
                    const float4 *wt1 = s4 + (wt >> 2);
                    {  // tap column 0 starts the sums (no cleared accumulators)
                        float4 wb[K];
#pragma unroll
                        for (int u = 0; u < K; ++u) wb[u] = wt1[u];
                        float4 cl[RH + K - 1];
#pragma unroll
                        for (int tt = 0; tt < RH + K - 1; ++tt) cl[tt] = win[tt * sy1];
#pragma unroll
                        for (int i = 0; i < RH; ++i) {
                            z[0][i] = wb[0].x * cl[i].x;
                            z[1][i] = wb[0].y * cl[i].y;
                            z[2][i] = wb[0].z * cl[i].z;
                            z[3][i] = wb[0].w * cl[i].w;
                        }
#pragma unroll
                        for (int u = 1; u < K; ++u)
#pragma unroll
                            for (int i = 0; i < RH; ++i) {
                                z[0][i] = fmaf(wb[u].x, cl[i + u].x, z[0][i]);
                                z[1][i] = fmaf(wb[u].y, cl[i + u].y, z[1][i]);
                                z[2][i] = fmaf(wb[u].z, cl[i + u].z, z[2][i]);
                                z[3][i] = fmaf(wb[u].w, cl[i + u].w, z[3][i]);
                            }
                    }
#pragma unroll 1
                    for (int v = 1; v < K; ++v) {  // rolled: see conv_bands
                        float4 wb[K];
#pragma unroll
                        for (int u = 0; u < K; ++u) wb[u] = wt1[v * K + u];
                        float4 cl[RH + K - 1];
#pragma unroll
                        for (int tt = 0; tt < RH + K - 1; ++tt) cl[tt] = win[tt * sy1 + v];
#pragma unroll
                        for (int u = 0; u < K; ++u)
#pragma unroll
                            for (int i = 0; i < RH; ++i) {
                                z[0][i] = fmaf(wb[u].x, cl[i + u].x, z[0][i]);
                                z[1][i] = fmaf(wb[u].y, cl[i + u].y, z[1][i]);
                                z[2][i] = fmaf(wb[u].z, cl[i + u].z, z[2][i]);
                                z[3][i] = fmaf(wb[u].w, cl[i + u].w, z[3][i]);
                            }
                    }
                }
                __syncthreads();  // every window is read: the bands may be overwritten
                if (has) {
                    float4 *own = s4 + (row0 + R) * sy1 + col + kPlaneCO;
#pragma unroll
                    for (int i = 0; i < RH; ++i) {
                        const float4 c4 = own[i * sy1];
                        const float A = c4.x + c4.y, B = c4.x - c4.y, C = c4.z + c4.w, D = c4.z - c4.w;
                        own[i * sy1] = make_float4(A + C, A - C, B + D, B - D);
                    }
                }
                __syncthreads();  // every cell holds its pixels
            }
            const float bias = smem[a.wt + (4 * L + 1) * KK];
            if (wave_has) {
                float P[2][2][RH];
                if constexpr (kBase) {
#pragma unroll
                    for (int i = 0; i < RH; ++i) {
                        P[0][0][i] = P[0][1][i] = P[1][0][i] = P[1][1][i] = bias;
                    }
                } else {
                    // deeper levels' patterns and the bias enter through the low-pass
                    // band; rows past the plane read padding (their outputs are not stored)
                    // (summed apart from z, so that the level loop carries only them)
                    float dz[RH];
#pragma unroll
                    for (int i = 0; i < RH; ++i) dz[i] = bias;
                    for (int l = 2; l <= L; ++l) {
                        const int sh = l - 2, sq = a.sq[sh];
                        const float *qc = smem + a.offq[sh] + (col >> sh);
#pragma unroll
                        for (int i = 0; i < RH; ++i) dz[i] += qc[__umul24((row0 + i) >> sh, sq)];
                    }
#pragma unroll
                    for (int i = 0; i < RH; ++i) z[0][i] += dz[i];
                    // level-1 synthesis: slot (ry, rx) = LL +- LH +- HL +- HH
#pragma unroll
                    for (int i = 0; i < RH; ++i) {
                        const float a0v = z[0][i] + z[1][i], a1v = z[0][i] - z[1][i];
                        const float b0 = z[2][i] + z[3][i], b1 = z[2][i] - z[3][i];
                        P[0][0][i] = a0v + b0;
                        P[0][1][i] = a0v - b0;
                        P[1][0][i] = a1v + b1;
                        P[1][1][i] = a1v - b1;
                    }
                }
                // base conv onto the patterns: output (2i+ry, 2j+rx), tap (u, w) reads
                // pixel (2i+ry+u-R, 2j+rx+w-R), i.e. component (py, px) of cell
                // (i + di, j + dj)
                const float4 *xwin = s4 + (row0 + R - RC) * sy1 + col + kPlaneCO;
                const float *w0 = smem + wt + 4 * L * KK;
#pragma unroll 1
                for (int dj = -RC; dj <= RC; ++dj) {  // rolled: see conv_bands
                    float4 xq[RH + 2 * RC];  // (x00, x01, x10, x11) of each cell
#pragma unroll
                    for (int tt = 0; tt < RH + 2 * RC; ++tt) xq[tt] = xwin[tt * sy1 + dj];
#pragma unroll
                    for (int px = 0; px < 2; ++px)
#pragma unroll
                        for (int rx = 0; rx < 2; ++rx) {
                            const int w = 2 * dj + px - rx + R;
                            if (w < 0 || w >= K) continue;
                            float wv[K];
#pragma unroll
                            for (int u = 0; u < K; ++u) wv[u] = w0[w * K + u];
#pragma unroll
                            for (int py = 0; py < 2; ++py)
#pragma unroll
                                for (int ry = 0; ry < 2; ++ry)
#pragma unroll
                                    for (int u = 0; u < K; ++u) {
                                        const int e = ry + u - R;
                                        if ((e & 1) != py) continue;
                                        const int di = (e - py) / 2;
#pragma unroll
                                        for (int i = 0; i < RH; ++i) {
                                            const float4 q = xq[i + di + RC];
                                            const float xv = py == 0 ? (px == 0 ? q.x : q.y) : (px == 0 ? q.z : q.w);
                                            P[ry][rx][i] = fmaf(wv[u], xv, P[ry][rx][i]);
                                        }
                                    }
                        }
                }
                if (has && p < live) {
                    const int nr = H - 2 * row0;  // pixel rows of the item inside the plane
                    T *dst = yb + (p * CHW + 2 * row0 * W + 2 * j);
#pragma unroll
                    for (int i = 0; i < RH; ++i) {
#pragma unroll
                        for (int ry = 0; ry < 2; ++ry, dst += W) {
                            if (2 * i + ry >= nr) break;
                            if (a.pair_store) {
                                if constexpr (kHalf<T>)
                                    *reinterpret_cast<uint32_t *>(dst) = Act<T>::pack(P[ry][0][i], P[ry][1][i]);
                                else
                                    *reinterpret_cast<float2 *>(dst) = make_float2(P[ry][0][i], P[ry][1][i]);
                            } else {
                                act_store(dst, 0, P[ry][0][i]);
                                if (2 * j + 1 < W) act_store(dst, 1, P[ry][1][i]);
                            }
                        }
                    }
                }
            }
        }
    }
}

template <int K, typename T, int CW, int RH, bool kBase>
__global__ __launch_bounds__(kFwdThreads, 3) void plane_fwd_kernel(PlaneArgs a) {
    plane_fwd_body<K, T, CW, RH, kBase>(a);
}

}  // namespace wtc
