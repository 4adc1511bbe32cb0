// Plane-resident forward kernel of the WTConv layer on the matrix cores (bfloat16
// activations).
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §4.  The layer output is the base conv plus, per level, the
// level's filtered Haar coefficients mapped back to pixels by the closed-form
// synthesis (§4.2, Prop. 2 / Eq. 7).  As in the vector kernel (wtconv_plane.hpp), a
// workgroup keeps whole planes and their pyramid in LDS and moves only x in and y
// out.  The difference is the level-1 filter and the base conv, which are
// nine-tenths of the arithmetic: both are read straight off the pixels by MFMA
// instructions.
//
// Level 1 as a stride-2 convolution of x.  Band b of cell (i, j) is
//   z_b(i, j) = sum_{u,v} w_b[u][v] S_b(i + u - R, j + v - R),
//   S_b(i, j) = sum_{py,px} h_b(py, px) x(2i + py, 2j + px)      (Eq. 5, unscaled)
// with the Haar signs h_b = +1 (LL), -1 on the odd row (LH), on the odd column
// (HL), off the diagonal (HH); so z_b(i, j) = sum over the 2K x 2K pixel window at
// (2i - 2R, 2j - 2R) of w_b[u][v] h_b(py, px) x.  The base conv of each pixel reads a
// K x K window inside the same pixel window.
//
// One MFMA tile is 16 cell columns (the M dimension, one A row per cell column) by
// four cell rows: 64 cells, 256 pixels.  K runs over the window of one cell column
// and four cell rows, (8 + 4R) pixel rows x (4R + 2) pixel columns, cut into groups
// of 8 pixels (one A fragment of a lane: 4 dwords of bfloat16 pairs).  The N
// dimension holds the four pixels of each of the four cell rows, n = 4 r + 2 rx + ry.
// The level-1 synthesis is linear (pixel (ry, rx) of a block takes band b with the
// sign h_b(ry, rx)), so it folds into B together with the base conv: column n of B
// is, at window pixel (py, px) of a level-1 tap (u, v),
//   sum_b h_b(ry, rx) h_b(py, px) w_b[u][v] = sum_b h_b(ry ^ py, rx ^ px) w_b[u][v],
// plus the base weight of that pixel.  One product then gives the level-1 and base
// part of every output pixel.  B is a banded (Toeplitz) matrix that depends on the
// channel only and stays in registers.  Each entry w is split as hi + lo with
// hi = bf16(w), lo = bf16(w - hi), and both halves are multiplied (the products of
// bfloat16 x with hi and lo are exact in the fp32 accumulation), so the weights
// carry ~16 significant bits.
//
// The product is taken transposed (B as the left operand), so that a lane receives
// the four pixels of one cell; the deeper levels' patterns and the bias enter every
// pixel of a cell with a plus sign (they come in through the LL band), so a lane adds
// one value to its four pixels and stores them as two pixel pairs.
//
// Deeper levels (l >= 2) stay on the vector units, as in wtconv_plane.hpp: level 2
// is analysed from the pixels (its cells are 4 x 4 pixel blocks), levels 3..L from
// the low-pass band above, and each level's sign patterns Q_l go to LDS.
//
// Workgroup w takes a contiguous range of units in channel-major order, so its
// channel (and with it the B fragments) changes at most a few times.  With
// rotate = 1 (and no bias) the same kernel computes the input gradient (each kernel
// turned by 180 degrees, Prop. 1 / Eq. 1).

#pragma once

#include "wtconv_plane.hpp"

namespace wtc {

constexpr int kMmaThreads = 128;  // two wavefronts
constexpr int kMmaCL = 8;         // canvas columns left of pixel column 0 (16 bytes)

typedef __bf16 wtc_bf16x8 __attribute__((ext_vector_type(8)));
typedef float wtc_f32x4 __attribute__((ext_vector_type(4)));

// Window geometry of the products for kernel size K (3 or 5).
template <int K>
struct MmaGeom {
    static_assert(K == 3 || K == 5, "the matrix-core kernel takes K = 3 or 5");
    static constexpr int R = (K - 1) / 2;
    // window row 0 is pixel row 2 i0 - 2R; window column 0 of cell column j is pixel
    // column 2 j - 2R (even: the A reads are dword aligned)
    static constexpr int ROW0 = 2 * R;
    static constexpr int COL0 = 2 * R;
    static constexpr int WR = 8 + 4 * R;     // window rows
    static constexpr int NSF = WR / 4;       // steps of full-row groups (one group of 8 columns per row)
    static constexpr int RROWS = NSF * 4;    // window rows the full steps read
    // K = 5: window columns 8 and 9 of all 16 rows form one more step (lane group g
    // takes rows g, g + 4, g + 8, g + 12); K = 3 reads 8 columns, 6 of them weighted
    static constexpr bool TAIL = K == 5;
    static constexpr int NS = NSF + (TAIL ? 1 : 0);  // B fragments (each hi and lo)
};

struct MmaArgs {
    const void *x;
    void *y;
    const float *w0, *b0, *s0, *wl, *sl;
    int n, C, H, W, L;
    int rotate;
    int vec;         // x rows are read with vector loads (W % 2CW == 0, aligned)
    int store_mode;  // 2: four pixels per store (W % 4 == 0), 1: pixel pairs (W even), 0: single pixels
    int PB, Pw1;     // planes per pass (side by side), level-1 column pitch between them
    int NG, U;       // image groups of PB per channel, units (C NG; a unit is one pass)
    int H1, W1;      // level-1 grid of one plane
    int Gw;          // commit column groups of CW cells per level-1 row
    int commit_items;
    int H2, pair_items;  // level-2 rows ceil(H1 / 2); commit items of two stacked patches (PB H2 Gw)
    int S;           // canvas row stride (dwords)
    int TX, tiles;   // product tiles per tile row, in all
    int aligned;     // 0: a tile takes 16 consecutive strip columns; 1: 16 / MW whole planes
    int MW;          // ... of at most MW = 4, 8 or 16 cells, MW M rows each
    int sy1;         // (unused: level 2 is analysed from the canvas)
    // deep levels l = 2..L at index l - 2 (as in PlaneArgs)
    int hl[kMaxLevels], wls[kMaxLevels];
    int sd[kMaxLevels];
    int syd[kMaxLevels], offd[kMaxLevels];
    int sq[kMaxLevels], offq[kMaxLevels];
    int dend[kMaxLevels];
    int wt;           // weight table (floats)
    int btab;         // B table (MmaBTab words), 16-byte aligned
    int btab_alias;   // 1: the B table lies in the level-2 pattern region
    int zero_floats;  // floats cleared at the start (canvas, bands, patterns, weights)
    int tab;          // deep-level geometry table
    int lds_floats;
    uint32_t m_gw, m_h1, m_tx, m_pw1, m_h2;  // udiv16 reciprocals of Gw, H1, TX, Pw1, H2
    uint32_t m_wls[kMaxLevels];
};

// B fragments (hi and lo halves) of one channel from the LDS weight table: the
// level-1 band weights as float4 over the bands at wt + 4 (v K + u), the base
// weights at base + v K + u (columns of taps, as the table stores them).  Column n
// = 4 rp + 2 rx + ry of B (held by lane n mod 16) belongs to output pixel (ry, rx)
// of cell row rp; its entry at window pixel (rho, kap) is the level-1 tap of that
// window pixel with the Haar sign product folded in, plus the base tap.
template <int K>
__device__ __forceinline__ void mma_b_fragments(const float *smem, int wt, int base, int lane,
                                                wtc_bf16x8 (&bh)[MmaGeom<K>::NS], wtc_bf16x8 (&bl)[MmaGeom<K>::NS]) {
    using G = MmaGeom<K>;
    constexpr int R = (K - 1) / 2;
    const float4 *s4 = reinterpret_cast<const float4 *>(smem);
    // the lane's coordinates made opaque here, so that nothing of this block is
    // hoisted out of a caller's loop (it would stay in registers throughout)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int g4 = ln >> 4, mm = ln & 15;
    const int rp = mm >> 2, ry = mm & 1, rx = (mm >> 1) & 1;
#pragma unroll
    for (int s = 0; s < G::NS; ++s) {
        union { wtc_bf16x8 v; uint32_t w[4]; } fh, fl;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            uint32_t h2[2], l2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                // window pixel (rho, kap) of K element 8 g4 + j + e of step s
                int rho, kap;
                if (G::TAIL && s == G::NSF) {
                    rho = g4 + 4 * ((j + e) >> 1);
                    kap = 8 + ((j + e) & 1);
                } else {
                    const int q = 4 * s + g4;
                    rho = q;
                    kap = j + e;
                }
                float w;
                {  // level-1 tap (uu, vv) at window pixel (py, px)
                    const int py = rho & 1, px = kap & 1, uu = (rho >> 1) - rp, vv = kap >> 1;
                    const bool ok = rho < G::WR && uu >= 0 && uu < K && vv < K;
                    const float4 wb = s4[(wt >> 2) + (ok ? vv * K + uu : 0)];
                    const int sy = ry ^ py, sx = rx ^ px;
                    const float t = (wb.x + (sy ? -wb.y : wb.y)) + ((sx ? -wb.z : wb.z) + ((sy ^ sx) ? -wb.w : wb.w));
                    w = ok ? t : 0.f;
                }
                if (!G::TAIL || s < G::NSF) {  // base tap of output pixel (2 rp + ry, rx)
                    const int uu = rho - 2 * rp - ry + R - G::ROW0, vv = kap - rx + R - G::COL0;
                    const bool ok = rho < G::WR && uu >= 0 && uu < K && vv >= 0 && vv < K;
                    const float t = smem[base + (ok ? vv * K + uu : 0)];
                    w += ok ? t : 0.f;
                }
                const uint16_t h = Act<uint16_t>::one(w);
                h2[e] = h;
                l2[e] = Act<uint16_t>::one(w - __uint_as_float((uint32_t)h << 16));
            }
            fh.w[j >> 1] = h2[0] | (h2[1] << 16);
            fl.w[j >> 1] = l2[0] | (l2[1] << 16);
        }
        bh[s] = fh.v;
        bl[s] = fl.v;
        // one step at a time: the table reads of all steps at once would take more
        // registers than the rest of the kernel
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The B entries of a channel as a table shared by the workgroup.  The entry of B
// column n = (rp, ry, rx) at window pixel (rho, kap) depends on rp and rho only
// through dy = rho - 2 rp: the level-1 tap is (dy >> 1, kap >> 1) with window-pixel
// parities (dy & 1, kap & 1), the base tap (dy - ry - R, kap - rx - R).  Entry
// (2 ry + rx, dy, kap), dy < 2K, holds that value split as hi | lo << 16 (bfloat16
// halves); window pixels with dy outside [0, 2K) carry no weight.  Rows are FC words
// (a multiple of 4: the lanes read window columns 0..7 as two 16-byte words, and
// columns 8, 9 for K = 5).
template <int K>
struct MmaBTab {
    static constexpr int FR = 2 * K;
    static constexpr int FC = K == 5 ? 12 : 8;
    static constexpr int kWords = 4 * FR * FC;
};

template <int K>
__device__ __forceinline__ void mma_btab_build(const float *smem, int wt, int base, uint32_t *ft, int tid, int NT) {
    using BT = MmaBTab<K>;
    constexpr int R = (K - 1) / 2;
    const float4 *s4 = reinterpret_cast<const float4 *>(smem);
    for (int e = tid; e < BT::kWords; e += NT) {
        const int q = e / (BT::FR * BT::FC), r = e - q * (BT::FR * BT::FC);
        const int dy = r / BT::FC, kap = r - dy * BT::FC;
        const int ry = q >> 1, rx = q & 1;
        float w = 0.f;
        {  // level-1 tap (dy >> 1, kap >> 1), the Haar sign product folded in
            const int uu = dy >> 1, vv = kap >> 1;
            const bool ok = vv < K;
            const float4 wb = s4[(wt >> 2) + (ok ? vv * K + uu : 0)];
            const int sy = ry ^ (dy & 1), sx = rx ^ (kap & 1);
            const float t = (wb.x + (sy ? -wb.y : wb.y)) + ((sx ? -wb.z : wb.z) + ((sy ^ sx) ? -wb.w : wb.w));
            w = ok ? t : 0.f;
        }
        {  // base tap of output pixel (ry, rx)
            const int uu = dy - ry - R, vv = kap - rx - R;
            const bool ok = uu >= 0 && uu < K && vv >= 0 && vv < K;
            const float t = smem[base + (ok ? vv * K + uu : 0)];
            w += ok ? t : 0.f;
        }
        const uint32_t h = Act<uint16_t>::one(w);
        const uint32_t l = Act<uint16_t>::one(w - __uint_as_float(h << 16));
        ft[e] = h | (l << 16);
    }
}

// A lane's B fragments (hi and lo halves) from the B table: lane (g4, mm) holds
// column mm = 4 rp + 2 rx + ry and, in step s, window row 4 s + g4, columns 0..7;
// in the tail step (K = 5), columns 8, 9 of window rows g4, g4 + 4, g4 + 8, g4 + 12.
template <int K>
__device__ __forceinline__ void mma_b_from_table(const uint32_t *ft, int lane, wtc_bf16x8 (&bh)[MmaGeom<K>::NS],
                                                 wtc_bf16x8 (&bl)[MmaGeom<K>::NS]) {
    using G = MmaGeom<K>;
    using BT = MmaBTab<K>;
    const int g4 = lane >> 4, mm = lane & 15;
    const int rp = mm >> 2, ry = mm & 1, rx = (mm >> 1) & 1;
    const uint32_t *fq = ft + (2 * ry + rx) * (BT::FR * BT::FC);
    // hi halves of two entries as one bfloat16 pair, and the lo halves
    auto split = [](uint32_t p0, uint32_t p1, uint32_t &h, uint32_t &l) {
        h = __builtin_amdgcn_perm(p1, p0, 0x05040100u);
        l = __builtin_amdgcn_perm(p1, p0, 0x07060302u);
    };
#pragma unroll
    for (int s = 0; s < G::NSF; ++s) {
        const int dy = 4 * s + g4 - 2 * rp;
        const bool ok = dy >= 0 && dy < BT::FR;
        const uint4 *src = reinterpret_cast<const uint4 *>(fq + (ok ? dy : 0) * BT::FC);
        const uint4 v0 = src[0], v1 = src[1];
        const uint32_t p[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        union { wtc_bf16x8 v; uint32_t w[4]; } fh, fl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            split(ok ? p[2 * i] : 0u, ok ? p[2 * i + 1] : 0u, fh.w[i], fl.w[i]);
        }
        bh[s] = fh.v;
        bl[s] = fl.v;
    }
    if constexpr (G::TAIL) {
        union { wtc_bf16x8 v; uint32_t w[4]; } fh, fl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dy = g4 + 4 * i - 2 * rp;
            const bool ok = dy >= 0 && dy < BT::FR;
            const uint2 v = *reinterpret_cast<const uint2 *>(fq + (ok ? dy : 0) * BT::FC + 8);
            split(ok ? v.x : 0u, ok ? v.y : 0u, fh.w[i], fl.w[i]);
        }
        bh[G::NSF] = fh.v;
        bl[G::NSF] = fl.v;
    }
}

// The transposed products of two tiles (their MFMA chains and LDS reads are
// independent, which hides the latency of each): wp[h] points at the canvas dword
// of window row g4, cell column mm of tile h (S: canvas row stride in dwords).
// acc[h] receives the four pixels of cell (g4, mm) of tile h, i = 2 rx + ry, added
// to v[h] (the value every pixel of the cell starts from).
template <int K>
__device__ __forceinline__ void mma_products2(const uint32_t *wp0, const uint32_t *wp1, int S,
                                              const wtc_bf16x8 (&bh)[MmaGeom<K>::NS],
                                              const wtc_bf16x8 (&bl)[MmaGeom<K>::NS], const float (&v)[2],
                                              wtc_f32x4 (&acc)[2]) {
    using G = MmaGeom<K>;
    const uint32_t *wp[2] = {wp0, wp1};
    acc[0] = wtc_f32x4{v[0], v[0], v[0], v[0]};
    acc[1] = wtc_f32x4{v[1], v[1], v[1], v[1]};
#pragma unroll
    for (int s = 0; s < G::NSF; ++s) {
        union { wtc_bf16x8 v; uint32_t w[4]; } A[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t *q = wp[h] + 4 * s * S;
            A[h].w[0] = q[0];
            A[h].w[1] = q[1];
            A[h].w[2] = q[2];
            A[h].w[3] = q[3];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[s], A[h].v, acc[h], 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl[s], A[h].v, acc[h], 0, 0, 0);
    }
    if constexpr (G::TAIL) {  // window columns 8, 9 of rows g4 + 4 e
        union { wtc_bf16x8 v; uint32_t w[4]; } A[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) A[h].w[e] = wp[h][4 * e * S + 4];
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[G::NSF], A[h].v, acc[h], 0, 0, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl[G::NSF], A[h].v, acc[h], 0, 0, 0);
    }
}

template <int K, int CW>
__device__ __forceinline__ void mma_fwd_body(const MmaArgs &args) {
    using G = MmaGeom<K>;
    using T = uint16_t;
    using IO = PatchIO<T, CW>;
    constexpr int R = (K - 1) / 2, KK = K * K;
    constexpr int NT = kMmaThreads;
    constexpr int SLOTS = kPlaneMaxWords / (2 * IO::kWords) > 0 ? kPlaneMaxWords / (2 * IO::kWords) : 1;
    constexpr int WSLOTS = 3;  // weight-table entries per thread carried in registers
    extern __shared__ float smem[];
    float4 *s4 = reinterpret_cast<float4 *>(smem);
    uint32_t *cv = reinterpret_cast<uint32_t *>(smem);  // the canvas: bfloat16 pixel pairs
    const MmaArgs &a0 = args;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int HW = a0.H * a0.W, CHW = a0.C * HW;

    for (int i = tid * 4; i < a0.zero_floats; i += NT * 4)
        *reinterpret_cast<float4 *>(smem + i) = make_float4(0.f, 0.f, 0.f, 0.f);
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

    // A unit is PB images of one channel, in channel-major order: unit u = (channel
    // u / NG, images [(u % NG) PB, ...)).  This workgroup's units are [ubeg, uend).
    const long long G0 = gridDim.x;
    const long long wb = xcd_block(blockIdx.x, gridDim.x);
    const int ubeg = (int)(wb * a0.U / G0), uend = (int)((wb + 1) * a0.U / G0);
    auto unit_of = [&](const auto &A, int u, int &c, int &n0) {
        c = u / A.NG;
        n0 = (u - c * A.NG) * A.PB;
    };
    auto patch_of = [&](const auto &A, int g, int &p, int &i, int &m) {
        const int q = udiv16(g, A.m_gw);
        m = g - q * A.Gw;
        p = udiv16(q, A.m_h1);
        i = q - p * A.H1;
    };
    auto load_patch = [&](const auto &A, uint32_t (&r)[2][IO::kWords], const T *xb, int live, int g) {
        int p, i, m;
        patch_of(A, min(g, A.commit_items - 1), p, i, m);
        load_patch_clamped<T, CW>(r, xb, p, i, m, live, CHW, A.H, A.W, A.vec);
    };
    // Weight-table entry e of channel c (raw factors; folded by fold_weight).  Level
    // l, band b: s(l,b) 4^-l W(l,b) as [l][v][u] float4 over b; base: s0 W0 as [v][u]
    // (the products read x itself); entry (4L + 1) K^2 is the folded bias s0 b.
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
        return lb < nl ? ldexpf(f0, -2 * ((lb >> 2) + 1)) * f1 : (lb == nl ? f0 * f1 : (A.b0 ? f0 * f1 : 0.f));
    };
    auto weight_slot = [&](const auto &A, int e) {
        const int lb = e / KK, tap = e - lb * KK;
        return lb < 4 * A.L ? A.wt + ((lb >> 2) * KK + tap) * 4 + (lb & 3) : A.wt + 4 * A.L * KK + (lb - 4 * A.L) * KK + tap;
    };

    // With CW >= 2 and levels >= 2, a commit item is two patches stacked, pixel rows
    // 4a .. 4a + 3 of 2CW columns: the lane that commits them also forms the level-2
    // bands of their CW / 2 level-2 cells (no separate analysis pass).
    constexpr bool kPair = CW >= 2;
    static_assert(!kPair || SLOTS % 2 == 0, "pairs of patches in the prefetch registers");
    const bool fold = kPair && a0.L >= 2;
    auto pair_of = [&](const auto &A, int d, int &p, int &a, int &m) {
        const int q = udiv16(d, A.m_gw);
        m = d - q * A.Gw;
        p = udiv16(q, A.m_h2);
        a = q - p * A.H2;
    };
    // the two patches of pair item d (the second past the plane when H1 is odd: its
    // loads repeat the first's rows, and it is cleared at the commit)
    auto load_pair = [&](const auto &A, uint32_t (&r0)[2][IO::kWords], uint32_t (&r1)[2][IO::kWords], const T *xb,
                         int live, int d) {
        int p, a, m;
        pair_of(A, min(d, A.pair_items - 1), p, a, m);
        load_patch_clamped<T, CW>(r0, xb, p, 2 * a, m, live, CHW, A.H, A.W, A.vec);
        load_patch_clamped<T, CW>(r1, xb, p, min(2 * a + 1, A.H1 - 1), m, live, CHW, A.H, A.W, A.vec);
    };
    uint32_t raw[SLOTS][2][IO::kWords];
    float wf0[WSLOTS], wf1[WSLOTS];
    // The weight table stays in LDS while consecutive units share a channel: its
    // factors are fetched (and the table rewritten) only for a unit that starts a
    // channel in this workgroup.
    auto prefetch = [&](const auto &A, int u) {
        int c, n0;
        unit_of(A, u, c, n0);
        const bool new_c = u == ubeg || c != (u - 1) / A.NG;
        const int live = min(A.PB, A.n - n0);
        const T *xb = static_cast<const T *>(A.x) + ((size_t)n0 * A.C + c) * HW;
        if (kPair && A.L >= 2) {
#pragma unroll
            for (int k = 0; k < SLOTS / 2; ++k) load_pair(A, raw[2 * k], raw[2 * k + 1], xb, live, tid + k * NT);
        } else {
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) load_patch(A, raw[k], xb, live, tid + k * NT);
        }
        if (new_c) {
#pragma unroll
            for (int k = 0; k < WSLOTS; ++k)
                weight_factors(A, c, min(tid + k * NT, (4 * A.L + 1) * KK), wf0[k], wf1[k]);
        }
    };
    if (ubeg < uend) prefetch(args, ubeg);

    // B fragments of the current channel (hi and lo halves); the channel whose weight
    // table is in LDS
    wtc_bf16x8 bh[G::NS], bl[G::NS];
    int cur_c = -1, tbl_c = -1;
    const int g4 = lane >> 4, mm = lane & 15;  // lane group (K octet) and A row / D column

    for (int u = ubeg; u < uend; ++u) {
        balance_priority(uend - u, uend - ubeg);
        const __attribute__((address_space(4))) MmaArgs *ap =
            (const __attribute__((address_space(4))) MmaArgs *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const auto &a = *ap;
        int c, n0;
        unit_of(a, u, c, n0);
        const int live = min(a.PB, a.n - n0);
        const int H = a.H, W = a.W, L = a.L, S = opaque(a.S);
        const bool full = live == a.PB && !(H & 1);
        __syncthreads();  // the previous pass is done with every array
        // 1. commit: the weight table (for a new channel) and the raw pixels (canvas
        //    rows ROW0 + y)
        {
            if (c != tbl_c) {
                tbl_c = c;
                const int nw = (4 * L + 1) * KK + 1;
#pragma unroll
                for (int k = 0; k < WSLOTS; ++k) {
                    const int e = tid + k * NT;
                    if (e < nw) smem[weight_slot(a, e)] = fold_weight(a, e, wf0[k], wf1[k]);
                }
                for (int e = tid + WSLOTS * NT; e < nw; e += NT) {
                    float f0, f1;
                    weight_factors(a, c, e, f0, f1);
                    smem[weight_slot(a, e)] = fold_weight(a, e, f0, f1);
                }
            }
            const int pw1 = opaque(a.Pw1);
            auto put = [&](const uint32_t (&r)[2][IO::kWords], int p, int i, int m) {
                uint32_t *d = cv + (G::ROW0 + 2 * i) * S + kMmaCL / 2 + p * pw1 + CW * m;
#pragma unroll
                for (int row = 0; row < 2; ++row, d += S) {
                    if constexpr (CW == 4) {
                        *reinterpret_cast<uint4 *>(d) = make_uint4(r[row][0], r[row][1], r[row][2], r[row][3]);
                    } else if constexpr (CW == 2) {
                        *reinterpret_cast<uint2 *>(d) = make_uint2(r[row][0], r[row][1]);
                    } else {
                        d[0] = r[row][0];
                    }
                }
            };
            const T *xb = static_cast<const T *>(a.x) + ((size_t)n0 * a.C + c) * HW;
            if (fold) {
                // level-2 cell e of a pair: the butterflies of the low-pass sums of its
                // four level-1 cells (pixel rows 4a .. 4a + 3, columns 4e .. 4e + 3)
                const int ds = opaque(a.syd[0]);
                float4 *l2 = s4 + opaque(a.offd[0]);
                auto put_pair = [&](uint32_t (&r0)[2][IO::kWords], uint32_t (&r1)[2][IO::kWords], int d) {
                    int p, aa, m;
                    pair_of(a, d, p, aa, m);
                    mask_patch<T, CW>(r0, p, 2 * aa, live, H, full);
                    mask_patch<T, CW>(r1, p, 2 * aa + 1, live, H, full);
                    if (2 * aa + 1 >= a.H1) {
#pragma unroll
                        for (int w = 0; w < IO::kWords; ++w) r1[0][w] = r1[1][w] = 0u;
                    }
                    put(r0, p, 2 * aa, m);
                    if (2 * aa + 1 < a.H1) put(r1, p, 2 * aa + 1, m);
                    float4 *dst = l2 + (aa + R) * ds + kPlaneCO + ((p * pw1 + CW * m) >> 1);
#pragma unroll
                    for (int e = 0; e < CW / 2; ++e) {
                        float cs[2][2];
#pragma unroll
                        for (int cc = 0; cc < 2; ++cc) {
                            const uint32_t t0 = r0[0][2 * e + cc], t1 = r0[1][2 * e + cc];
                            const uint32_t t2 = r1[0][2 * e + cc], t3 = r1[1][2 * e + cc];
                            cs[0][cc] = (Act<T>::lo(t0) + Act<T>::hi(t0)) + (Act<T>::lo(t1) + Act<T>::hi(t1));
                            cs[1][cc] = (Act<T>::lo(t2) + Act<T>::hi(t2)) + (Act<T>::lo(t3) + Act<T>::hi(t3));
                        }
                        const float s0 = cs[0][0] + cs[0][1], s1 = cs[1][0] + cs[1][1];
                        const float d0 = cs[0][0] - cs[0][1], d1 = cs[1][0] - cs[1][1];
                        dst[e] = make_float4(s0 + s1, s0 - s1, d0 + d1, d0 - d1);
                    }
                };
#pragma unroll
                for (int k = 0; k < SLOTS / 2; ++k) {
                    const int d = tid + k * NT;
                    if (d < a.pair_items) put_pair(raw[2 * k], raw[2 * k + 1], d);
                }
                for (int d = tid + (SLOTS / 2) * NT; d < a.pair_items; d += NT) {  // beyond the registers
                    uint32_t r0[2][IO::kWords], r1[2][IO::kWords];
                    load_pair(a, r0, r1, xb, live, d);
                    put_pair(r0, r1, d);
                }
            } else {
#pragma unroll
                for (int k = 0; k < SLOTS; ++k) {
                    const int g = tid + k * NT;
                    if (g >= a.commit_items) continue;
                    int p, i, m;
                    patch_of(a, g, p, i, m);
                    mask_patch<T, CW>(raw[k], p, i, live, H, full);
                    put(raw[k], p, i, m);
                }
                for (int g = tid + SLOTS * NT; g < a.commit_items; g += NT) {
                    uint32_t r[2][IO::kWords];
                    load_patch(a, r, xb, live, g);
                    int p, i, m;
                    patch_of(a, g, p, i, m);
                    mask_patch<T, CW>(r, p, i, live, H, full);
                    put(r, p, i, m);
                }
            }
        }
        __syncthreads();
        // The next unit's loads are issued as soon as the registers are free: the
        // rest of the pass (LDS work and products) is short next to their latency,
        // and nothing in it waits for vector-memory loads.
        if (u + 1 < uend) prefetch(a, u + 1);

        // B fragments of a new channel (the condition is uniform over the workgroup):
        // the workgroup builds the B table, each lane reads its fragments.  Where the
        // table lies in the level-2 pattern region, the reads finish before the deep
        // phase writes the patterns.
        if (c != cur_c) {
            cur_c = c;
            uint32_t *ft = reinterpret_cast<uint32_t *>(smem + opaque(a.btab));
            const int wt = opaque(a.wt);
            mma_btab_build<K>(smem, wt, wt + 4 * L * KK, ft, tid, NT);
            __syncthreads();
            mma_b_from_table<K>(ft, lane, bh, bl);
            if (a.btab_alias) __syncthreads();
        }

        {
            // 2. level 2 from the pixels (a level-2 cell is a 4 x 4 pixel block: the
            //    butterflies of the low-pass sums of its four level-1 cells; formed at
            //    the commit for CW >= 2), then levels 3..L from the low-pass band
            //    above; 3. the deep patterns
            if (L >= 2) {
                if (!fold) {
                    const int Wls = a.wls[0], ds = a.syd[0];
                    float4 *dst = s4 + a.offd[0];
                    for (int q = tid; q < a.hl[0] * Wls; q += NT) {
                        const int i = udiv16(q, a.m_wls[0]), j = q - i * Wls;
                        const uint32_t *sp = cv + (G::ROW0 + 4 * i) * S + kMmaCL / 2 + 2 * j;
                        float cs[2][2];  // low-pass sums of the 2 x 2 level-1 cells, by (row, column)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const uint2 t0 = *reinterpret_cast<const uint2 *>(sp + (2 * h) * S);
                            const uint2 t1 = *reinterpret_cast<const uint2 *>(sp + (2 * h + 1) * S);
                            cs[h][0] = (Act<T>::lo(t0.x) + Act<T>::hi(t0.x)) + (Act<T>::lo(t1.x) + Act<T>::hi(t1.x));
                            cs[h][1] = (Act<T>::lo(t0.y) + Act<T>::hi(t0.y)) + (Act<T>::lo(t1.y) + Act<T>::hi(t1.y));
                        }
                        const float x00 = cs[0][0], x01 = cs[0][1], x10 = cs[1][0], x11 = cs[1][1];
                        const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
                        dst[(i + R) * ds + j + kPlaneCO] = make_float4(s0 + s1, s0 - s1, d0 + d1, d0 - d1);
                    }
                    __syncthreads();
                }
                haar_levels<K>(a, s4, 3, tid, NT);
                deep_patterns<K>(a, s4, smem, tab, tid, NT);
            }
        }

        // 4. products and stores, one tile of 16 x 4 cells at a time.  The product is
        //    formed transposed (the B fragments as the left operand, the pixel
        //    fragments as the right one), so that lane (g4, mm) receives the four
        //    pixels of cell (4 ty + g4, tile column lcol): element i = 2 rx + ry.
        T *yb = static_cast<T *>(a.y) + ((size_t)n0 * a.C + c) * HW;
        const float bias = smem[a.wt + (4 * L + 1) * KK];
        const int smode = opaque(a.store_mode), pw1 = opaque(a.Pw1), W1 = opaque(a.W1);
        // the lane's strip column within a tile, and the tile's first strip column
        const int MW = opaque(a.MW), aligned = opaque(a.aligned);
        const int lcol = aligned ? (mm / MW) * pw1 + (mm & (MW - 1)) : mm;
        const int tstep = aligned ? (16 / MW) * pw1 : 16;
        // deep patterns: Q_l of cell (row, col) at (row >> j, col >> j), j = l - 2,
        // split into a wave-uniform part (tile origin, a multiple of 4 columns) and the
        // lane's part; a level past L reads canvas row 0, which is zero padding throughout
        int qo[kMaxLevels - 1], qs[kMaxLevels - 1], ql[3];
#pragma unroll
        for (int k = 0; k < kMaxLevels - 1; ++k) {
            const bool on = k + 2 <= L;
            qo[k] = on ? opaque(a.offq[k]) : 0;
            qs[k] = on ? opaque(a.sq[k]) : 0;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) ql[j] = (g4 >> j) * qs[j] + (lcol >> j);
        // the lane's A reads: row g4 of the window's step, strip column lcol
        const int la = (kMmaCL - G::COL0) / 2 + g4 * S + lcol;
        constexpr int NW = NT / kWave;
        // two tiles per iteration (t and t + NW; the second may repeat the first, then
        // it stores nothing): their MFMA chains and LDS reads are independent
        for (int t = wave; t < a.tiles; t += 2 * NW) {
            const int t2 = t + NW < a.tiles ? t + NW : t;
            int ty[2], tx[2];
            ty[0] = udiv16(t, a.m_tx);
            tx[0] = t - ty[0] * a.TX;
            ty[1] = udiv16(t2, a.m_tx);
            tx[1] = t2 - ty[1] * a.TX;
            // bias and the deep patterns (they enter all four pixels of the cell): the
            // products accumulate onto them
            float v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int crow = 4 * ty[h] + g4, ccol = tstep * tx[h] + lcol;
                v[h] = bias;
                if (L >= 2) {
                    float q[3];
#pragma unroll
                    for (int j = 0; j < 3; ++j)
                        q[j] = smem[qo[j] + ((4 * ty[h]) >> j) * qs[j] + ((tstep * tx[h]) >> j) + ql[j]];
                    v[h] += q[0] + (q[1] + q[2]);
                    for (int k = 3; k < L - 1; ++k)  // levels 5..L
                        v[h] += smem[qo[k] + (crow >> k) * qs[k] + (ccol >> k)];
                }
            }
            wtc_f32x4 acc[2];
            mma_products2<K>(cv + la + (8 * ty[0]) * S + tstep * tx[0], cv + la + (8 * ty[1]) * S + tstep * tx[1], S, bh,
                             bl, v, acc);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1 && t2 == t) break;
                const int crow = 4 * ty[h] + g4, ccol = tstep * tx[h] + lcol;
                const int p = udiv16(ccol, a.m_pw1);
                const int jc = ccol - p * pw1;
                const int pr = 2 * crow;
                if (p < live && jc < W1 && pr < H) {
                    const float o0 = acc[h][0], o1 = acc[h][1], o2 = acc[h][2], o3 = acc[h][3];
                    T *dst = yb + (p * CHW + pr * W + 2 * jc);
                    const bool row1 = pr + 1 < H;
                    if (smode != 0) {  // pixel pairs (W even)
                        *reinterpret_cast<uint32_t *>(dst) = Act<T>::pack(o0, o2);
                        if (row1) *reinterpret_cast<uint32_t *>(dst + W) = Act<T>::pack(o1, o3);
                    } else {
                        const bool col1 = 2 * jc + 1 < W;
                        act_store(dst, 0, o0);
                        if (col1) act_store(dst, 1, o2);
                        if (row1) {
                            act_store(dst, W, o1);
                            if (col1) act_store(dst, W + 1, o3);
                        }
                    }
                }
            }
        }
    }
}

template <int K, int CW>
__global__ __launch_bounds__(kMmaThreads, 3) void mma_fwd_kernel(MmaArgs a) {
    mma_fwd_body<K, CW>(a);
}

}  // namespace wtc
