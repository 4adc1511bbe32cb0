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
// After the products, a lane holds pixel (ry, rx) of four consecutive cells of one
// cell row; the deeper levels' patterns and the bias enter every pixel of a block
// with a plus sign (they come in through the LL band).  One DPP exchange pairs the
// two pixel columns, and y is stored four pixels per lane.
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
    int sy1;         // (unused: level 2 is analysed from the canvas)
    // deep levels l = 2..L at index l - 2 (as in PlaneArgs)
    int hl[kMaxLevels], wls[kMaxLevels];
    int sd[kMaxLevels];
    int syd[kMaxLevels], offd[kMaxLevels];
    int sq[kMaxLevels], offq[kMaxLevels];
    int dend[kMaxLevels];
    int wt;           // weight table (floats)
    int zero_floats;  // floats cleared at the start (canvas, bands, patterns, weights)
    int tab;          // deep-level geometry table
    int lds_floats;
    uint32_t m_gw, m_h1, m_tx, m_pw1, m_h2;  // udiv16 reciprocals of Gw, H1, TX, Pw1, H2
    uint32_t m_wls[kMaxLevels];
};

template <int CTRL>
__device__ __forceinline__ float dpp_quad(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
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
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
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
    const int ubeg = (int)((long long)blockIdx.x * a0.U / G0), uend = (int)(((long long)blockIdx.x + 1) * a0.U / G0);
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
    auto prefetch = [&](const auto &A, int u) {
        int c, n0;
        unit_of(A, u, c, n0);
        const int live = min(A.PB, A.n - n0);
        const T *xb = static_cast<const T *>(A.x) + ((size_t)n0 * A.C + c) * HW;
        if (kPair && A.L >= 2) {
#pragma unroll
            for (int k = 0; k < SLOTS / 2; ++k) load_pair(A, raw[2 * k], raw[2 * k + 1], xb, live, tid + k * NT);
        } else {
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) load_patch(A, raw[k], xb, live, tid + k * NT);
        }
#pragma unroll
        for (int k = 0; k < WSLOTS; ++k) weight_factors(A, c, min(tid + k * NT, (4 * A.L + 1) * KK), wf0[k], wf1[k]);
    };
    if (ubeg < uend) prefetch(args, ubeg);

    // B fragments of the current channel (hi and lo halves)
    wtc_bf16x8 bh[G::NS], bl[G::NS];
    int cur_c = -1;
    const int g4 = lane >> 4, mm = lane & 15;  // lane group (K octet) and A row / D column

    for (int u = ubeg; u < uend; ++u) {
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
        // 1. commit: the weight table and the raw pixels (canvas rows ROW0 + y)
        {
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

        // B fragments, when the channel changes (wave-uniform)
        if (c != cur_c) {
            cur_c = c;
            const int wt = opaque(a.wt);
            // the lane's coordinates made opaque here, so that nothing of this block
            // is hoisted out of the unit loop (it would stay in registers throughout)
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
                            const float t = smem[wt + 4 * L * KK + (ok ? vv * K + uu : 0)];
                            w += ok ? t : 0.f;
                        }
                        const uint16_t h = Act<T>::one(w);
                        h2[e] = h;
                        l2[e] = Act<T>::one(w - __uint_as_float((uint32_t)h << 16));
                    }
                    fh.w[j >> 1] = h2[0] | (h2[1] << 16);
                    fl.w[j >> 1] = l2[0] | (l2[1] << 16);
                }
                bh[s] = fh.v;
                bl[s] = fl.v;
                // one step at a time: the table reads of all steps at once would take
                // more registers than the rest of the kernel
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // 4. products and stores, one tile of 16 x 4 cells at a time
        T *yb = static_cast<T *>(a.y) + ((size_t)n0 * a.C + c) * HW;
        const float bias = smem[a.wt + (4 * L + 1) * KK];
        const int rp = mm >> 2, ry = mm & 1, rx = (mm >> 1) & 1;
        const int smode = opaque(a.store_mode), pw1 = opaque(a.Pw1), W1 = opaque(a.W1);
        // deep patterns of levels 2..L at level-1 resolution: Q_l of cell (row, col)
        // at (row >> (l - 2), col >> (l - 2)); the offsets and strides held uniform
        int qo[kMaxLevels - 1], qs[kMaxLevels - 1];
#pragma unroll
        for (int k = 0; k < kMaxLevels - 1; ++k) {
            qo[k] = opaque(a.offq[k]);
            qs[k] = opaque(a.sq[k]);
        }
        // Two tiles per iteration (t and t + NT / kWave; the second may repeat the
        // first, then it stores nothing): their products and LDS reads are
        // independent, which hides the latency of each.
        auto products = [&](int t, wtc_f32x4 &dh, wtc_f32x4 &dl) {
            const int ty = udiv16(t, a.m_tx), tx = t - ty * a.TX;
            // canvas row 2 ci0 is window row 0; this lane's A row is cell column cj0 + mm
            const uint32_t *wp = cv + (8 * ty) * S + (kMmaCL - G::COL0) / 2 + 16 * tx + mm;
#pragma unroll
            for (int s = 0; s < G::NSF; ++s) {
                const int q = 4 * s + g4;
                const uint32_t *p = wp + q * S;
                union { wtc_bf16x8 v; uint32_t w[4]; } A;
                A.w[0] = p[0];
                A.w[1] = p[1];
                A.w[2] = p[2];
                A.w[3] = p[3];
                dh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.v, bh[s], dh, 0, 0, 0);
                dl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.v, bl[s], dl, 0, 0, 0);
            }
            if constexpr (G::TAIL) {
                union { wtc_bf16x8 v; uint32_t w[4]; } A;
#pragma unroll
                for (int e = 0; e < 4; ++e) A.w[e] = wp[(g4 + 4 * e) * S + 4];
                dh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.v, bh[G::NSF], dh, 0, 0, 0);
                dl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.v, bl[G::NSF], dl, 0, 0, 0);
            }
        };
        // lane: D column = pixel (ry, rx) of cell row rp, D rows r = cell columns cs0 + r
        auto finish = [&](int t, const wtc_f32x4 &dh, const wtc_f32x4 &dl, bool store) {
            const int ty = udiv16(t, a.m_tx), tx = t - ty * a.TX;
            const int crow = 4 * ty + rp, cs0 = 16 * tx + 4 * g4;
            float4 dz = make_float4(bias, bias, bias, bias);
            if (L >= 2) {
                // levels 2 and 3 (and 4) read unconditionally, a level past L from the
                // level-2 array with its value discarded, so that the reads overlap
                const float4 q2 = *reinterpret_cast<const float4 *>(smem + qo[0] + __umul24(crow, qs[0]) + cs0);
                const bool l3 = L >= 3, l4 = L >= 4;
                const float2 q3 = *reinterpret_cast<const float2 *>(
                    smem + (l3 ? qo[1] + __umul24(crow >> 1, qs[1]) + (cs0 >> 1) : qo[0]));
                const float q4 = smem[l4 ? qo[2] + __umul24(crow >> 2, qs[2]) + (cs0 >> 2) : qo[0]];
                const float v3x = l3 ? q3.x : 0.f, v3y = l3 ? q3.y : 0.f, v4 = l4 ? q4 : 0.f;
                dz.x += q2.x + (v3x + v4);
                dz.y += q2.y + (v3x + v4);
                dz.z += q2.z + (v3y + v4);
                dz.w += q2.w + (v3y + v4);
                for (int k = 3; k < L - 1; ++k) {  // levels 5..L: one value for the four cells
                    const float v = smem[qo[k] + __umul24(crow >> k, qs[k]) + (cs0 >> k)];
                    dz.x += v;
                    dz.y += v;
                    dz.z += v;
                    dz.w += v;
                }
            }
            float y[4] = {(dh[0] + dl[0]) + dz.x, (dh[1] + dl[1]) + dz.y, (dh[2] + dl[2]) + dz.z, (dh[3] + dl[3]) + dz.w};
            // pair the two pixel columns (lane ^ 2 holds the other rx): rx = 0 keeps
            // cells cs0, cs0 + 1, rx = 1 cells cs0 + 2, cs0 + 3, four pixels in a row
            const float snd0 = rx ? y[0] : y[2], snd1 = rx ? y[1] : y[3];
            const float rcv0 = dpp_quad<0x4E>(snd0), rcv1 = dpp_quad<0x4E>(snd1);
            const float o0 = rx ? rcv0 : y[0], o1 = rx ? y[2] : rcv0;
            const float o2 = rx ? rcv1 : y[1], o3 = rx ? y[3] : rcv1;
            const int p = udiv16(cs0, a.m_pw1);
            const int jc = cs0 - p * pw1 + 2 * rx;  // first cell of the four pixels
            const int pr = 2 * crow + ry;
            if (store && p < live && pr < H && jc < W1) {
                T *dst = yb + (p * CHW + pr * W + 2 * jc);
                if (smode == 2) {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(Act<T>::pack(o0, o1), Act<T>::pack(o2, o3));
                } else {
                    const float oo[4] = {o0, o1, o2, o3};
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int col = 2 * (jc + h);
                        if (jc + h >= W1) break;
                        if (smode == 1) {
                            *reinterpret_cast<uint32_t *>(dst + 2 * h) = Act<T>::pack(oo[2 * h], oo[2 * h + 1]);
                        } else {
                            act_store(dst, 2 * h, oo[2 * h]);
                            if (col + 1 < W) act_store(dst, 2 * h + 1, oo[2 * h + 1]);
                        }
                    }
                }
            }
        };
        constexpr int NW = NT / kWave;
        for (int t = wave; t < a.tiles; t += 2 * NW) {
            const int t2 = t + NW < a.tiles ? t + NW : t;
            wtc_f32x4 h1 = {0.f, 0.f, 0.f, 0.f}, l1 = h1, h2 = h1, l2 = h1;
            products(t, h1, l1);
            products(t2, h2, l2);
            finish(t, h1, l1, true);
            finish(t2, h2, l2, t2 != t);
        }
    }
}

template <int K, int CW>
__global__ __launch_bounds__(kMmaThreads, 2) void mma_fwd_kernel(MmaArgs a) {
    mma_fwd_body<K, CW>(a);
}

}  // namespace wtc
