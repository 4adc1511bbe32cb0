// Plane-resident weight gradient of the base conv (small planes).
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §3 (the layer) and §4.3 Eq. 9 (gradients of the folded
// parameters).  The base branch is y0 = s0 (W0 * x + b0) with * the k x k
// cross-correlation with zero "same" padding, so dL/dW0[u][v] = s0 sum over pixels
// p of dy[p] x[p + (u - R, v - R)] and dL/db0 = s0 sum dy.  This kernel forms the
// raw sums (the correlation and sum dy) per channel; the finalize kernel applies
// s0 and the Eq. 9 scale gradient.
//
// Layout: LDS holds x and dy of a plane as their polyphase components on the
// level-1 grid, one float4 per cell: X[i][j] = (x[2i][2j], x[2i][2j+1],
// x[2i+1][2j], x[2i+1][2j+1]) with a zero halo of ceil(R/2) cells, and D[i][j] the
// same for dy (no halo).  Small planes sit side by side, PB per pass, with zero
// cells between them.
//
// Workgroup (c, r) of the k workgroups of channel c walks the image groups
// [r NG / k, (r + 1) NG / k) of that channel, PB images per pass:
//   1. commit the prefetched 2 x 2CW pixel patches of x and dy as cells; issue the
//      loads of the next pass;
//   2. one item is one cell column x RH cell rows (2 x 2RH pixels of dy): the lane
//      reads the item's RH dy cells and the (RH + 2 ceil(R/2)) x (2 ceil(R/2) + 1)
//      x cells around them and adds every (pixel, tap) product to its 25 (k^2)
//      tap accumulators, and sum dy to a bias accumulator.
// At the end the lanes' accumulators are summed in a fixed order (bitwise
// repeatable) into the workgroup's partial row [c][r][k^2 + 1].

#pragma once

#include "wtconv_plane.hpp"

namespace wtc {

struct PlaneDwbArgs {
    const void *x, *dy;
    float *partial;        // [C][k][K*K + 1]
    int n, C, H, W;
    int vec;               // x and dy rows are read with vector loads (W % 2CW == 0, aligned)
    int PB, Pw1;           // planes per pass (side by side), cell pitch between them
    int NG, k;             // image groups of PB per channel, workgroups per channel
    int H1, W1;            // level-1 grid of one plane
    int S1;                // strips of RH cell rows
    int sx, ax;            // X cells: row stride; D starts at cell ax
    int sd;                // D cells: row stride
    int Gw;                // commit column groups of CW cells per row
    int commit_items;      // PB * H1 * Gw
    int final_items;       // S1 * PB * W1
    int lds_floats;
    uint32_t m_gw, m_h1, m_strip, m_w1;  // udiv16 reciprocals of Gw, H1, PB*W1, W1
};

__device__ __forceinline__ float cell_comp(const float4 &q, int comp) {
    return comp == 0 ? q.x : comp == 1 ? q.y : comp == 2 ? q.z : q.w;
}

template <int K, typename T, int CW, int RH>
__global__ __launch_bounds__(kPlaneThreads, 2) void plane_dwb_kernel(PlaneDwbArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    constexpr int RC = (R + 1) / 2;
    constexpr int NT = kPlaneThreads;
    using IO = PatchIO<T, CW>;
    constexpr int SLOTS = kPlaneMaxWords / (2 * IO::kWords) > 0 ? kPlaneMaxWords / (2 * IO::kWords) : 1;
    extern __shared__ float smem[];
    float4 *s4 = reinterpret_cast<float4 *>(smem);
    const int c = blockIdx.x / a.k, r = blockIdx.x - c * a.k;
    const int g_begin = (int)((long long)r * a.NG / a.k), g_end = (int)((long long)(r + 1) * a.NG / a.k);
    const int tid = threadIdx.x, PB = a.PB;
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
#pragma unroll
        for (int w = 0; w < IO::kWords; ++w) rw[0][w] = rw[1][w] = 0;
        int p, i, m;
        patch_of(g, p, i, m);
        if (p >= live) return;
        const int col0 = 2 * CW * m;
        const T *src = base + (p * CHW + (2 * i) * a.W + col0);
        IO::load_row(rw[0], src, a.vec, col0, a.W);
        if (2 * i + 1 < a.H) IO::load_row(rw[1], src + a.W, a.vec, col0, a.W);
    };
    // polyphase cells of a patch: CW cells from (row i, cell m CW) of plane p
    auto store_patch = [&](float4 *arr, int stride, int row_off, int col_off, const uint32_t (&rw)[2][IO::kWords],
                           int p, int i, int m) {
        float4 *dst = arr + (i + row_off) * stride + col_off + p * a.Pw1 + m * CW;
#pragma unroll
        for (int q = 0; q < CW; ++q)
            dst[q] = make_float4(IO::elem(rw[0], 2 * q), IO::elem(rw[0], 2 * q + 1), IO::elem(rw[1], 2 * q),
                                 IO::elem(rw[1], 2 * q + 1));
    };

    uint32_t xr[SLOTS][2][IO::kWords], dr[SLOTS][2][IO::kWords];
    auto prefetch = [&](int g) {
        const int n0 = g * PB, live = min(PB, a.n - n0);
#pragma unroll
        for (int k = 0; k < SLOTS; ++k) {
            const int e = tid + k * NT;
            if (e >= a.commit_items) continue;
            load_patch(xr[k], xc + (size_t)n0 * CHW, live, e);
            load_patch(dr[k], dc + (size_t)n0 * CHW, live, e);
        }
    };

    float acc[KK], bsum = 0.f;
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[t] = 0.f;
    if (g_begin < g_end) prefetch(g_begin);

    for (int g = g_begin; g < g_end; ++g) {
        const int n0 = g * PB, live = min(PB, a.n - n0);
        __syncthreads();  // the previous pass is done with the cells
        {
            const int sx = opaque(a.sx), sd = opaque(a.sd), ax = opaque(a.ax);
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int e = tid + k * NT;
                if (e >= a.commit_items) continue;
                int p, i, m;
                patch_of(e, p, i, m);
                store_patch(s4, sx, RC, kPlaneCO, xr[k], p, i, m);
                store_patch(s4 + ax, sd, 0, 0, dr[k], p, i, m);
            }
            for (int e = tid + SLOTS * NT; e < a.commit_items; e += NT) {  // beyond the registers
                uint32_t rw[2][IO::kWords];
                int p, i, m;
                patch_of(e, p, i, m);
                load_patch(rw, xc + (size_t)n0 * CHW, live, e);
                store_patch(s4, sx, RC, kPlaneCO, rw, p, i, m);
                load_patch(rw, dc + (size_t)n0 * CHW, live, e);
                store_patch(s4 + ax, sd, 0, 0, rw, p, i, m);
            }
        }
        __syncthreads();
        if (g + 1 < g_end) prefetch(g + 1);

        for (int t = tid; t < a.final_items; t += NT) {
            const int sx = opaque(a.sx), sd = opaque(a.sd), ax = opaque(a.ax);
            const int s = udiv16(t, a.m_strip), rr = t - s * (PB * a.W1);
            const int p = udiv16(rr, a.m_w1), j = rr - p * a.W1;
            const int col = p * a.Pw1 + j, row0 = s * RH;
            // dy of the item's 2 x 2RH pixels: component 2 ry + rx of cell i
            float4 d[RH];
            const float4 *dcol = s4 + ax + row0 * sd + col;
#pragma unroll
            for (int i = 0; i < RH; ++i) {
                d[i] = dcol[i * sd];
                bsum += (d[i].x + d[i].y) + (d[i].z + d[i].w);
            }
            // pixel (2i+ry, 2j+rx) meets tap (u, w) at x pixel (2i+ry+u-R, 2j+rx+w-R):
            // component (py, px) of cell (i + di, j + dj)
            const float4 *xw = s4 + row0 * sx + col + kPlaneCO;
#pragma unroll
            for (int dj = -RC; dj <= RC; ++dj) {
                float4 xcl[RH + 2 * RC];
#pragma unroll
                for (int tt = 0; tt < RH + 2 * RC; ++tt) xcl[tt] = xw[tt * sx + dj];
#pragma unroll
                for (int px = 0; px < 2; ++px)
#pragma unroll
                    for (int rx = 0; rx < 2; ++rx) {
                        const int w = 2 * dj + px - rx + R;
                        if (w < 0 || w >= K) continue;
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
                                    for (int i = 0; i < RH; ++i)
                                        acc[u * K + w] = fmaf(cell_comp(d[i], 2 * ry + rx),
                                                              cell_comp(xcl[i + di + RC], 2 * py + px), acc[u * K + w]);
                                }
                    }
            }
        }
    }

    // fixed-order reduction of the lanes' accumulators through LDS
    __syncthreads();
    constexpr int SL = KK + 1;
#pragma unroll
    for (int t = 0; t < KK; ++t) smem[tid * (SL + 1) + t] = acc[t];
    smem[tid * (SL + 1) + KK] = bsum;
    __syncthreads();
    if (tid < SL) {
        float sum = 0.f;
        for (int l = 0; l < NT; ++l) sum += smem[l * (SL + 1) + tid];
        a.partial[((size_t)c * a.k + r) * SL + tid] = sum;
    }
}

}  // namespace wtc
