// Weight gradients of the base conv and of level 1 on the matrix cores for planes
// past the plane-resident range (bfloat16 activations), one spatial tile per pass.
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §4.3 Eq. 9.  The same cross-correlations of the polyphase
// components as the plane-resident correlation kernel (wtconv_dwc.hpp: dwc_item,
// dwc_reduce_write), summed over the tiles of the planes.  A pass stages the dy
// cells of one tile of UR x 32 level-1 cells and the x cells its offsets reach:
// x canvas row r is cell row r0 + T0 + r of the plane (r < XR = UR + 4 NF - 1),
// x canvas cell q is cell column c0 - 4 + q, zero outside the plane; the dy canvas
// holds the tile's rows between 4 NF - 1 zero rows above and below, so that an
// item (one x canvas row, the tile's 32 columns) pairs every x cell with the dy
// cells of this tile only.  Each (dy cell, offset) pair of a plane is then counted
// once, in the pass of its dy cell.  With levels >= 2 the pass also writes the
// level-1 carriers (1/2 the sum of each 2 x 2 block, Eq. 5) of x and dy for the
// tile's cells: the input of the level-2 gradient kernel, which otherwise reads
// x and dy once more.
//
// Workgroup r C + c (numbered per XCD) takes passes [r P / k, (r + 1) P / k) of
// channel c, in the order (image, tile row, tile column), and writes partial row
// c k + r of the base and level-1 regions.  The next pass's staging loads are in
// flight while the current one multiplies.

#pragma once

#include "wtconv_dwc.hpp"

namespace wtc {

constexpr int kDwcTileCols = 32;  // tile width in cells (one item covers it)
// tile rows at most: 32-row tiles (less x halo per dy cell) measured slower, their
// registers and LDS leave fewer workgroups resident
constexpr int kDwcTileRows = 16;
constexpr int kDwcTileDySlots = kDwcTileRows * kDwcTileCols / 4 / 128;  // dy staging items per thread
constexpr int kDwcTileXSlots = 2;                                       // x staging items per thread

struct DwcTileArgs {
    const void *x, *dy;
    float *pbase;      // base region: [C][k][K*K + 1]
    float *plev;       // level-1 region: [C][k][4 K*K], or null without levels
    void *xc, *gc;     // level-1 carriers of x and dy, [n][C][Ho][Wo], or null
    int n, C, H, W;
    int Ho, Wo;        // level-1 grid
    int vec;           // W % 8 == 0, x and dy 16-byte aligned: 8-pixel loads
    int UR;            // tile rows (cells), at most kDwcTileRows
    int TYu, TXu;      // tiles per plane
    int P;             // passes per channel: n TYu TXu
    int k;             // workgroups per channel
    int XR, XC;        // x canvas rows, 4-cell chunks per x canvas row
    int Sd, pd;        // dy canvas: row stride, component plane size (dwords)
    int Sx, px, xo;    // x canvas: row stride, component plane size, offset (dwords)
    int lds_floats;
    uint32_t m_xc;     // udiv16 reciprocal of XC
};

// The four polyphase components of 4 cells (8 pixels of two pixel rows, as
// bfloat16 words w[row][0..3]) as bfloat16 pairs: comp[2 py + px][0..1].
__device__ __forceinline__ void dwc_split(const uint4 (&w)[2], uint2 (&comp)[4]) {
#pragma unroll
    for (int py = 0; py < 2; ++py) {
        const uint32_t w0 = w[py].x, w1 = w[py].y, w2 = w[py].z, w3 = w[py].w;
        comp[2 * py] = make_uint2((w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16));
        comp[2 * py + 1] = make_uint2((w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u));
    }
}

template <int K, bool kLev>
__global__ __launch_bounds__(kDwcThreads, 2) void dwc_tile_kernel(DwcTileArgs a) {
    using Gm = DwcGeom<K, kLev>;
    using T = uint16_t;
    constexpr int NF = Gm::NF, T0 = Gm::T0, TYMAX = Gm::TYMAX;
    constexpr int NT = kDwcThreads;
    constexpr int DZ = 4 * NF - 1;  // zero rows of the dy canvas above (and below) the tile
    extern __shared__ float smem[];
    uint32_t *lw = reinterpret_cast<uint32_t *>(smem);
    const int wb = xcd_block(blockIdx.x, gridDim.x);
    const int r = wb / a.C, c = wb - r * a.C;
    const int p_begin = (int)((long long)r * a.P / a.k), p_end = (int)((long long)(r + 1) * a.P / a.k);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int HW = a.H * a.W;
    const int per_img = a.TYu * a.TXu, dy_items = a.UR * (kDwcTileCols / 4), x_items = a.XR * a.XC;

    for (int i = tid * 4; i < a.lds_floats; i += NT * 4)
        *reinterpret_cast<float4 *>(smem + i) = make_float4(0.f, 0.f, 0.f, 0.f);

    auto pass_of = [&](int p, int &nn, int &r0, int &c0) {
        nn = p / per_img;
        const int t = p - nn * per_img, ty = t / a.TXu;
        r0 = a.UR * ty;
        c0 = kDwcTileCols * (t - ty * a.TXu);
    };
    // 8 pixels of pixel rows 2 row, 2 row + 1 from pixel column px0 (zero outside
    // the plane; with vec the chunk lies wholly inside or outside)
    auto load8 = [&](const T *plane, int row, int px0, uint4 (&w)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int y = 2 * row + h;
            w[h] = make_uint4(0u, 0u, 0u, 0u);
            if (y < 0 || y >= a.H) continue;
            const T *src = plane + (size_t)y * a.W;
            if (a.vec) {
                if (px0 >= 0 && px0 < a.W) w[h] = *reinterpret_cast<const uint4 *>(src + px0);
            } else {
                uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int x = px0 + i;
                    const uint32_t e = x >= 0 && x < a.W ? reinterpret_cast<const uint16_t *>(src)[x] : 0u;
                    v[i >> 1] |= e << (16 * (i & 1));
                }
                w[h] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    uint4 dr[kDwcTileDySlots][2], xr[kDwcTileXSlots][2];
    auto prefetch = [&](int p) {
        int nn, r0, c0;
        pass_of(p, nn, r0, c0);
        const size_t pl = ((size_t)nn * a.C + c) * HW;
        const T *xp = static_cast<const T *>(a.x) + pl, *dp = static_cast<const T *>(a.dy) + pl;
#pragma unroll
        for (int s = 0; s < kDwcTileDySlots; ++s) {
            const int e = min(tid + s * NT, dy_items - 1), ar = e >> 3, j = e & 7;
            load8(dp, r0 + ar, 2 * c0 + 8 * j, dr[s]);
        }
#pragma unroll
        for (int s = 0; s < kDwcTileXSlots; ++s) {
            const int e = min(tid + s * NT, x_items - 1), row = udiv16(e, a.m_xc), j = e - row * a.XC;
            load8(xp, r0 + T0 + row, 2 * (c0 - 4) + 8 * j, xr[s]);
        }
    };
    // level-1 carrier of 4 cells from their components: 1/2 ((x00 + x01) + (x10 + x11))
    auto carry = [&](T *dst, int row, int col0, const uint2 (&comp)[4]) {
        if (row >= a.Ho) return;
        float v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int hf = b & 1;
            const uint32_t c00 = b < 2 ? comp[0].x : comp[0].y, c01 = b < 2 ? comp[1].x : comp[1].y;
            const uint32_t c10 = b < 2 ? comp[2].x : comp[2].y, c11 = b < 2 ? comp[3].x : comp[3].y;
            const float x00 = hf ? Act<T>::hi(c00) : Act<T>::lo(c00), x01 = hf ? Act<T>::hi(c01) : Act<T>::lo(c01);
            const float x10 = hf ? Act<T>::hi(c10) : Act<T>::lo(c10), x11 = hf ? Act<T>::hi(c11) : Act<T>::lo(c11);
            v[b] = 0.5f * ((x00 + x01) + (x10 + x11));
        }
        T *o = dst + (size_t)row * a.Wo + col0;
        if (a.vec) {  // Wo % 4 == 0: the four cells are inside or outside together
            if (col0 < a.Wo) *reinterpret_cast<uint2 *>(o) = make_uint2(Act<T>::pack(v[0], v[1]), Act<T>::pack(v[2], v[3]));
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (col0 + b < a.Wo) act_store(o, b, v[b]);
        }
    };

    wtc_f32x4 acc[NF][NF];
#pragma unroll
    for (int fy = 0; fy < NF; ++fy)
#pragma unroll
        for (int fx = 0; fx < NF; ++fx) acc[fy][fx] = wtc_f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;
    if (p_begin < p_end) prefetch(p_begin);
    const int g4 = lane >> 4, mm = lane & 15, aq = mm >> 2, ai = mm & 3;

    for (int p = p_begin; p < p_end; ++p) {
        balance_priority(p_end - p, p_end - p_begin);
        int nn, r0, c0;
        pass_of(p, nn, r0, c0);
        const size_t cpl = ((size_t)nn * a.C + c) * a.Ho * a.Wo;
        __syncthreads();  // the previous pass is done with the canvases
        // dy cells of the tile: components into canvas rows DZ .. DZ + UR - 1, sum dy,
        // and the dy carrier
#pragma unroll
        for (int s = 0; s < kDwcTileDySlots; ++s) {
            const int e = tid + s * NT;
            if (e >= dy_items) continue;
            const int ar = e >> 3, j = e & 7;
            uint2 comp[4];
            dwc_split(dr[s], comp);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2 *>(lw + q * a.pd + (ar + DZ) * a.Sd + 2 * j) = comp[q];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                bsum += ((Act<T>::lo(dr[s][h].x) + Act<T>::hi(dr[s][h].x)) +
                         (Act<T>::lo(dr[s][h].y) + Act<T>::hi(dr[s][h].y))) +
                        ((Act<T>::lo(dr[s][h].z) + Act<T>::hi(dr[s][h].z)) +
                         (Act<T>::lo(dr[s][h].w) + Act<T>::hi(dr[s][h].w)));
            if (a.gc) carry(static_cast<T *>(a.gc) + cpl, r0 + ar, c0 + 4 * j, comp);
        }
        // x cells: canvas rows 0 .. XR - 1, and the x carrier of the tile's own cells
#pragma unroll
        for (int s = 0; s < kDwcTileXSlots; ++s) {
            const int e = tid + s * NT;
            if (e >= x_items) continue;
            const int row = udiv16(e, a.m_xc), j = e - row * a.XC;
            uint2 comp[4];
            dwc_split(xr[s], comp);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2 *>(lw + a.xo + q * a.px + row * a.Sx + 2 * j) = comp[q];
            const int ar = T0 + row;
            if (a.xc && ar >= 0 && ar < a.UR && j >= 1 && j <= kDwcTileCols / 4)
                carry(static_cast<T *>(a.xc) + cpl, r0 + ar, c0 + 4 * (j - 1), comp);
        }
        __syncthreads();
        if (p + 1 < p_end) prefetch(p + 1);

        // products: one item per x canvas row, the tile's 32 columns
        for (int it = wave; it < a.XR; it += NT / kWave)
            dwc_item<K, kLev>(lw, it, 8 * g4, aq, ai, TYMAX, a.Sd, a.pd, a.xo, 4, a.Sx, a.px, acc);
    }

    dwc_reduce_write<K, kLev>(smem, acc, bsum, tid, (size_t)c * a.k + r, a.pbase, a.plev);
}

}  // namespace wtc
