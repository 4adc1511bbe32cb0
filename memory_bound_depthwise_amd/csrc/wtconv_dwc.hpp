// Weight gradients of the base conv and of level 1 on the matrix cores (bfloat16
// activations, planes up to 64 x 64).
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §3 (the layer), §4.3 Eq. 9 (gradients of the folded parameters).
// The raw sums the finalize kernel expects are
//   base:    B[u][v] = sum_P dy[P] x[P + (u - R, v - R)],  and sum_P dy[P];
//   level 1: L_b[u][v] = 1/4 sum_c G_b[c] S_b[c + (u - R, v - R)],
// with S_b, G_b the unscaled level-1 Haar bands of x and dy (Eq. 5 without its
// 1/2: S_b[c] = sum_p h_b(p) x_p[c] over the four polyphase components x_p[c] =
// x[2c + p], h_b the Haar signs).  Both are sign-combinations of the
// cross-correlations of the polyphase components on the level-1 grid,
//   C[q][p][t] = sum_c dy_q[c] x_p[c + t]:
//   L_b[t + R] = 1/4 sum_{q,p} h_b(q) h_b(p) C[q][p][t],
//   B[d + R]  = sum_q C[q][(q + d) mod 2][floor((q + d) / 2)]   (per axis),
// and C takes only products of bfloat16 values, exact in the float32 accumulation
// of a bfloat16 MFMA.
//
// Products.  One 16x16x32 MFMA gives C for four row offsets and four column offsets
// at once: row m = 4 q + i of A is dy_q shifted by ty = ty0 + i rows, column
// n = 4 p + j of B is x_p shifted by tx = tx0 + j columns, and K runs over 32
// consecutive cells of one cell row:
//   D[4q + i][4p + j] = sum_cells dy_q[ci - ty][cj] x_p[ci][cj + tx] = C[q][p][(ty, tx)].
// The offsets needed (-R..R for level 1, floor(-R/2)..floor((R+1)/2) for the base
// alone) take one or two families of four per axis.  LDS holds the components as
// bfloat16 planes (dy with zero rows above and below, x with zero columns to the
// left and right); a lane reads its A row 16 bytes at a time, and its B column as
// five dwords funnel-shifted by one cell when the column offset is odd.
//
// Workgroup r C + c, the r-th of the k workgroups of channel c, walks the image
// groups [r NG / k, (r + 1) NG / k) of that channel, PB images per pass side by
// side (at least R zero cells apart, so no valid offset reaches a neighbour).  At
// the end the wavefronts' products are summed in a fixed order through LDS, the
// sign-combinations above are formed in a fixed order, and the workgroup writes
// its partial rows of the base and level-1 regions (bitwise repeatable).

#pragma once

#include "wtconv_mma.hpp"

namespace wtc {

constexpr int kDwcThreads = 128;  // two wavefronts

// Offsets of the cross-correlations: T0..T1 per axis, in NF families of four.
template <int K, bool kLev>
struct DwcGeom {
    static constexpr int R = (K - 1) / 2;
    static constexpr int T0 = kLev ? -R : -((R + 1) / 2);  // floor(-R / 2)
    static constexpr int T1 = kLev ? R : (R + 1) / 2;
    static constexpr int NF = (T1 - T0 + 4) / 4;
    static constexpr int TYMAX = T0 + 4 * NF - 1;  // largest row offset of a family
};

struct PlaneDwcArgs {
    const void *x, *dy;
    float *pbase;    // base region: [C][k][K*K + 1] (correlations, then sum dy)
    float *plev;     // level-1 region: [C][k][4 K*K], or null without levels
    int n, C, H, W;
    int vec;         // x and dy rows are read with vector loads (W % 2CW == 0, aligned)
    int PB, Pw1;     // planes per pass (side by side), cell pitch between them
    int NG, k;       // image groups of PB per channel, workgroups per channel
    int H1, W1, Gw, commit_items;
    int nch;         // chunks of 32 cells per strip row
    int DT;          // zero rows of the dy planes above row 0
    int Sd, pd;      // dy planes: row stride, plane size (dwords)
    int XL, Sx, px;  // x planes: zero cells left of column 0, row stride, plane size (dwords)
    int xo;          // dword offset of the x planes (the dy planes start at 0)
    int items;       // H1 * nch
    int lds_floats;
    uint32_t m_gw, m_h1, m_nch;  // udiv16 reciprocals of Gw, H1, nch
};

// Products of one item: x canvas row ci of every component, the lane's 8 cells
// from cj on.  A row m = 4 q + i of the lane is dy component q at canvas row
// ci + DT - ty (ty = T0 + 4 fy + i), 16 bytes at a time; B column n = 4 p + j is x
// component p at row ci, cells cj + tx .. (tx = T0 + 4 fx + j, canvas cell XL + ..),
// five dwords funnel-shifted by one cell when the first cell is odd.
template <int K, bool kLev>
__device__ __forceinline__ void dwc_item(const uint32_t *lw, int ci, int cj, int aq, int ai, int DT, int Sd, int pd,
                                         int xo, int XL, int Sx, int pxs,
                                         wtc_f32x4 (&acc)[DwcGeom<K, kLev>::NF][DwcGeom<K, kLev>::NF]) {
    using Gm = DwcGeom<K, kLev>;
    constexpr int NF = Gm::NF, T0 = Gm::T0;
    union { wtc_bf16x8 v; uint32_t w[4]; } A[NF], Bf[NF];
#pragma unroll
    for (int fy = 0; fy < NF; ++fy) {
        const uint32_t *p = lw + aq * pd + (ci + DT - (T0 + 4 * fy + ai)) * Sd + (cj >> 1);
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        A[fy].w[0] = v.x;
        A[fy].w[1] = v.y;
        A[fy].w[2] = v.z;
        A[fy].w[3] = v.w;
    }
#pragma unroll
    for (int fx = 0; fx < NF; ++fx) {
        const int col = XL + cj + T0 + 4 * fx + ai;  // first x cell of this lane's column
        const uint32_t *p = lw + xo + aq * pxs + ci * Sx + (col >> 1);
        uint32_t d5[5];
#pragma unroll
        for (int e = 0; e < 5; ++e) d5[e] = p[e];
        const uint32_t sh = (col & 1) * 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) Bf[fx].w[e] = __builtin_amdgcn_alignbit(d5[e + 1], d5[e], sh);
    }
#pragma unroll
    for (int fy = 0; fy < NF; ++fy)
#pragma unroll
        for (int fx = 0; fx < NF; ++fx)
            acc[fy][fx] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[fy].v, Bf[fx].v, acc[fy][fx], 0, 0, 0);
}

// Fixed-order reduction of a 128-thread workgroup's products (the wavefronts' D
// tiles through LDS) and of its dy sums, then the sign-combinations: the raw base
// sums and sum dy go to partial row `row` of pbase ([rows][K*K + 1]), the level-1
// sums (with kLev) to row `row` of plev ([rows][4 K*K]).  Bitwise repeatable.
template <int K, bool kLev>
__device__ __forceinline__ void dwc_reduce_write(float *smem,
                                                 const wtc_f32x4 (&acc)[DwcGeom<K, kLev>::NF][DwcGeom<K, kLev>::NF],
                                                 float bsum, int tid, size_t row, float *pbase, float *plev) {
    using Gm = DwcGeom<K, kLev>;
    constexpr int R = (K - 1) / 2, KK = K * K, NF = Gm::NF, T0 = Gm::T0;
    constexpr int NT = kDwcThreads;
    const int lane = tid & (kWave - 1), wave = tid / kWave, g4 = lane >> 4, mm = lane & 15;
    // fixed-order reduction: the wavefronts' D tiles through LDS, then the sums
    constexpr int NC = NF * NF * 256;  // C[fy][fx][m][n]
    __syncthreads();                   // the planes are no longer read
#pragma unroll
    for (int fy = 0; fy < NF; ++fy)
#pragma unroll
        for (int fx = 0; fx < NF; ++fx)
#pragma unroll
            for (int i = 0; i < 4; ++i) smem[wave * NC + ((fy * NF + fx) * 16 + 4 * g4 + i) * 16 + mm] = acc[fy][fx][i];
    {
        const float v = wave_sum(bsum);
        if (lane == 0) smem[(NT / kWave) * NC + wave] = v;
    }
    __syncthreads();
    float *Cs = smem + (NT / kWave) * NC + NT / kWave;
    for (int i = tid; i < NC; i += NT) {
        float s = smem[i];
#pragma unroll
        for (int w = 1; w < NT / kWave; ++w) s += smem[w * NC + i];
        Cs[i] = s;
    }
    __syncthreads();
    // C[q][p][(ty, tx)], q = 2 qy + qx and p = 2 py + px
    auto Cv = [&](int q, int p, int ty, int tx) {
        const int fy = (ty - T0) >> 2, iy = (ty - T0) & 3, fx = (tx - T0) >> 2, ix = (tx - T0) & 3;
        return Cs[((fy * NF + fx) * 16 + 4 * q + iy) * 16 + 4 * p + ix];
    };
    for (int o = tid; o < KK + 1; o += NT) {
        float s = 0.f;
        if (o < KK) {
            const int dy_ = o / K - R, dx_ = o % K - R;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int sy = (q >> 1) + dy_, sx = (q & 1) + dx_;
                s += Cv(q, 2 * (sy & 1) + (sx & 1), sy >> 1, sx >> 1);
            }
        } else {
            for (int w = 0; w < NT / kWave; ++w) s += smem[(NT / kWave) * NC + w];
        }
        pbase[row * (KK + 1) + o] = s;
    }
    if constexpr (kLev) {
        for (int o = tid; o < 4 * KK; o += NT) {
            const int b = o / KK, tap = o - b * KK, ty = tap / K - R, tx = tap % K - R;
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    // h_b(q) h_b(p): band 1 flips on odd rows, band 2 on odd columns
                    const int fl = ((b & 1) & ((q >> 1) ^ (p >> 1))) ^ (((b >> 1) & 1) & ((q & 1) ^ (p & 1)));
                    const float v = Cv(q, p, ty, tx);
                    s += fl ? -v : v;
                }
            plev[row * 4 * KK + o] = 0.25f * s;
        }
    }
}

template <int K, int CW, bool kLev>
__global__ __launch_bounds__(kDwcThreads, 2) void plane_dwc_kernel(PlaneDwcArgs a) {
    using Gm = DwcGeom<K, kLev>;
    using T = uint16_t;
    using IO = PatchIO<T, CW>;
    constexpr int R = (K - 1) / 2, KK = K * K, NF = Gm::NF, T0 = Gm::T0;
    constexpr int NT = kDwcThreads;
    constexpr int SLOTS = kPlaneMaxWords / (2 * IO::kWords) > 0 ? kPlaneMaxWords / (2 * IO::kWords) : 1;
    static_assert(CW == 1 || CW == 2 || CW == 4, "commit width");
    extern __shared__ float smem[];
    uint32_t *lw = reinterpret_cast<uint32_t *>(smem);
    // neighbouring workgroups (numbered per XCD) take neighbouring channels of the
    // same images
    const int wb = xcd_block(blockIdx.x, gridDim.x);
    const int r = wb / a.C, c = wb - r * a.C;
    const int g_begin = (int)((long long)r * a.NG / a.k), g_end = (int)((long long)(r + 1) * a.NG / a.k);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, PB = a.PB;
    const int HW = a.H * a.W, CHW = a.C * HW;
    const T *xc = static_cast<const T *>(a.x) + (size_t)c * HW;
    const T *dc = static_cast<const T *>(a.dy) + (size_t)c * HW;

    for (int i = tid * 4; i < a.lds_floats; i += NT * 4)
        *reinterpret_cast<float4 *>(smem + i) = make_float4(0.f, 0.f, 0.f, 0.f);

    auto patch_of = [&](int g, int &p, int &i, int &m) {
        const int q = udiv16(g, a.m_gw);
        m = g - q * a.Gw;
        p = udiv16(q, a.m_h1);
        i = q - p * a.H1;
    };
    auto load_patch = [&](uint32_t (&rw)[2][IO::kWords], const T *base, int live, int g) {
        if (g >= a.commit_items) return;
        int p, i, m;
        patch_of(g, p, i, m);
        load_patch_clamped<T, CW>(rw, base, p, i, m, live, CHW, a.H, a.W, a.vec);
    };
    // the four components of a patch's CW cells (row i, cells CW m .. of plane p) as
    // bfloat16 pairs: component (py, px) takes the px halves of pixel row py
    auto store_patch = [&](int base, int stride, int psize, int row, int col, const uint32_t (&rw)[2][IO::kWords]) {
#pragma unroll
        for (int py = 0; py < 2; ++py)
#pragma unroll
            for (int px = 0; px < 2; ++px) {
                uint32_t *d = lw + base + (2 * py + px) * psize + row * stride + (col >> 1);
                if constexpr (CW == 1) {
                    // one cell: a half of a dword shared with the neighbouring patch
                    uint16_t *h = reinterpret_cast<uint16_t *>(lw + base + (2 * py + px) * psize + row * stride) + col;
                    *h = (uint16_t)(px ? rw[py][0] >> 16 : rw[py][0] & 0xffffu);
                } else {
#pragma unroll
                    for (int e = 0; e < CW / 2; ++e) {
                        const uint32_t w0 = rw[py][2 * e], w1 = rw[py][2 * e + 1];
                        d[e] = px ? (w0 >> 16) | (w1 & 0xffff0000u) : (w0 & 0xffffu) | (w1 << 16);
                    }
                }
            }
    };

    uint32_t xr[SLOTS][2][IO::kWords], dr[SLOTS][2][IO::kWords];
    auto prefetch = [&](int g) {
        const int n0 = g * PB, live = min(PB, a.n - n0);
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
            load_patch(xr[k], xc + (size_t)n0 * CHW, live, tid + k * NT);
            load_patch(dr[k], dc + (size_t)n0 * CHW, live, tid + k * NT);
        }
    };

    wtc_f32x4 acc[NF][NF];
#pragma unroll
    for (int fy = 0; fy < NF; ++fy)
#pragma unroll
        for (int fx = 0; fx < NF; ++fx) acc[fy][fx] = wtc_f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;
    if (g_begin < g_end) prefetch(g_begin);

    const int g4 = lane >> 4, mm = lane & 15;
    // A row of this lane: component q = mm >> 2 of dy, row shift ty0 + (mm & 3);
    // B column: component p = mm >> 2 of x, column shift tx0 + (mm & 3)
    const int aq = mm >> 2, ai = mm & 3;

    for (int g = g_begin; g < g_end; ++g) {
        balance_priority(g_end - g, g_end - g_begin);
        const int n0 = g * PB, live = min(PB, a.n - n0);
        const bool full = live == PB && !(a.H & 1);
        __syncthreads();  // the previous pass is done with the planes
        {
            const int pw1 = opaque(a.Pw1);
            auto commit = [&](uint32_t (&xw)[2][IO::kWords], uint32_t (&dw)[2][IO::kWords], int e) {
                int p, i, m;
                patch_of(e, p, i, m);
                mask_patch<T, CW>(xw, p, i, live, a.H, full);
                mask_patch<T, CW>(dw, p, i, live, a.H, full);
                const int col = p * pw1 + m * CW;
                store_patch(0, a.Sd, a.pd, i + a.DT, col, dw);
                store_patch(a.xo, a.Sx, a.px, i, col + a.XL, xw);
#pragma unroll
                for (int w = 0; w < IO::kWords; ++w)
                    bsum += (Act<T>::lo(dw[0][w]) + Act<T>::hi(dw[0][w])) + (Act<T>::lo(dw[1][w]) + Act<T>::hi(dw[1][w]));
            };
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int e = tid + k * NT;
                if (e < a.commit_items) commit(xr[k], dr[k], e);
            }
            for (int e = tid + SLOTS * NT; e < a.commit_items; e += NT) {  // beyond the registers
                uint32_t xw[2][IO::kWords], dw[2][IO::kWords];
                load_patch(xw, xc + (size_t)n0 * CHW, live, e);
                load_patch(dw, dc + (size_t)n0 * CHW, live, e);
                commit(xw, dw, e);
            }
        }
        __syncthreads();
        if (g + 1 < g_end) prefetch(g + 1);

        // products: item = (cell row ci, chunk of 32 cells)
        const int Sd = opaque(a.Sd), pd = opaque(a.pd), Sx = opaque(a.Sx), pxs = opaque(a.px);
        const int xo = opaque(a.xo), XL = opaque(a.XL), DT = opaque(a.DT);
        for (int it = wave; it < a.items; it += NT / kWave) {
            const int ci = udiv16(it, a.m_nch), cj = 32 * (it - ci * a.nch) + 8 * g4;
            dwc_item<K, kLev>(lw, ci, cj, aq, ai, DT, Sd, pd, xo, XL, Sx, pxs, acc);
        }
    }

    dwc_reduce_write<K, kLev>(smem, acc, bsum, tid, (size_t)c * a.k + r, a.pbase, a.plev);
}

}  // namespace wtc
