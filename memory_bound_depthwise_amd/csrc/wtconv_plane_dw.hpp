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
// Workgroup r C + c, the r-th of the k workgroups of channel c, walks the image
// groups [r NG / k, (r + 1) NG / k) of that channel, PB images per pass (workgroups
// running side by side take neighbouring channels of the same images, whose planes
// are adjacent in memory):
//   1. commit the prefetched 2 x 2CW pixel patches of x and dy as cells; issue the
//      loads of the next pass;
//   2. one item is one cell column x RH cell rows (2 x 2RH pixels of dy): the lane
//      reads the item's RH dy cells and the (RH + 2 ceil(R/2)) x (2 ceil(R/2) + 1)
//      x cells around them and adds every (pixel, tap) product to its 25 (k^2)
//      tap accumulators, and sum dy to a bias accumulator.
// At the end the lanes' accumulators are summed in a fixed order (bitwise
// repeatable): over each wavefront with DPP, then over the wavefronts, into the
// workgroup's partial row [c][r][k^2 + 1].

#pragma once

#include "wtconv_plane.hpp"

namespace wtc {

constexpr int kDwbThreads = 128;  // threads of a base weight-gradient workgroup

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
__global__ __launch_bounds__(kDwbThreads, 2) void plane_dwb_kernel(PlaneDwbArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    constexpr int RC = (R + 1) / 2;
    constexpr int NT = kDwbThreads;
    using IO = PatchIO<T, CW>;
    constexpr int SLOTS = kPlaneMaxWords / (2 * IO::kWords) > 0 ? kPlaneMaxWords / (2 * IO::kWords) : 1;
    extern __shared__ float smem[];
    float4 *s4 = reinterpret_cast<float4 *>(smem);
    // neighbouring workgroups (numbered per XCD) take neighbouring channels of the
    // same images
    const int wb = xcd_block(blockIdx.x, gridDim.x);
    const int r = wb / a.C, c = wb - r * a.C;
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
    // loads from clamped addresses (see load_patch_clamped); lanes past the last
    // item load nothing (their registers are not used)
    auto load_patch = [&](uint32_t (&rw)[2][IO::kWords], const T *base, int live, int g) {
        if (g >= a.commit_items) return;
        int p, i, m;
        patch_of(g, p, i, m);
        load_patch_clamped<T, CW>(rw, base, p, i, m, live, CHW, a.H, a.W, a.vec);
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
            load_patch(xr[k], xc + (size_t)n0 * CHW, live, tid + k * NT);
            load_patch(dr[k], dc + (size_t)n0 * CHW, live, tid + k * NT);
        }
    };

    float acc[KK], bsum = 0.f;
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[t] = 0.f;
    if (g_begin < g_end) prefetch(g_begin);

    for (int g = g_begin; g < g_end; ++g) {
        balance_priority(g_end - g, g_end - g_begin);
        const int n0 = g * PB, live = min(PB, a.n - n0);
        const bool full = live == PB && !(a.H & 1);  // nothing of the pass's patches needs masking
        __syncthreads();  // the previous pass is done with the cells
        {
            const int sx = opaque(a.sx), sd = opaque(a.sd), ax = opaque(a.ax);
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int e = tid + k * NT;
                if (e >= a.commit_items) continue;
                int p, i, m;
                patch_of(e, p, i, m);
                mask_patch<T, CW>(xr[k], p, i, live, a.H, full);
                mask_patch<T, CW>(dr[k], p, i, live, a.H, full);
                store_patch(s4, sx, RC, kPlaneCO, xr[k], p, i, m);
                store_patch(s4 + ax, sd, 0, 0, dr[k], p, i, m);
            }
            for (int e = tid + SLOTS * NT; e < a.commit_items; e += NT) {  // beyond the registers
                uint32_t rw[2][IO::kWords];
                int p, i, m;
                patch_of(e, p, i, m);
                load_patch(rw, xc + (size_t)n0 * CHW, live, e);
                mask_patch<T, CW>(rw, p, i, live, a.H, full);
                store_patch(s4, sx, RC, kPlaneCO, rw, p, i, m);
                load_patch(rw, dc + (size_t)n0 * CHW, live, e);
                mask_patch<T, CW>(rw, p, i, live, a.H, full);
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

    // fixed-order reduction: every accumulator over its wavefront with DPP
    // (wave_sum), then the wavefronts' sums in order through LDS
    constexpr int SL = KK + 1, NW = NT / kWave;
    const int wave = tid / kWave, lane = tid % kWave;
    __syncthreads();  // the cells are no longer read: LDS holds the wave sums
#pragma unroll
    for (int t = 0; t < SL; ++t) {
        const float v = wave_sum(t < KK ? acc[t] : bsum);
        if (lane == 0) smem[wave * SL + t] = v;
    }
    __syncthreads();
    if (tid < SL) {
        float sum = smem[tid];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += smem[w * SL + tid];
        a.partial[((size_t)c * a.k + r) * SL + tid] = sum;
    }
}

// ---------------------------------------------------------------------------
// Plane-resident weight gradient of the levels.
//
// Level l, band b: the branch is z = s(l,b) (W(l,b) * Y_l,b) on the orthonormal
// Haar coefficients Y_l of x (§3.1), and the synthesis back to pixels is the
// adjoint of the analysis (Prop. 1), so dL/dz = G_l,b, the analysis of dy, and
// dL/dW(l,b)[u][v] = s(l,b) sum_ij G_l,b[i][j] Y_l,b[i+u-R][j+v-R].  With the
// unscaled pyramids of both (S_l = 2^l Y_l, the same for dy) the raw sum is 4^-l
// sum G S; the finalize kernel applies s(l,b) and the Eq. 9 scale gradient.
//
// LDS holds the unscaled bands of x (zero halo of R cells) and of dy, every level,
// band by band and column-major, so that a column of an item's window is
// contiguous and is read 16 bytes at a time.  Each lane is tied to one (level,
// band) for the whole kernel and owns its k^2 tap accumulators; an item is one
// column x RHD rows of that level's grid, and the items of a (level, band) are
// dealt round-robin to its lanes (the lane table comes from the host).  Per pass:
//   1. commit x and dy patches as level-1 bands (butterflies in registers);
//   2. Haar analysis of levels 2..L for x and dy;
//   3. every lane runs its items.
// At the end the lanes of each (level, band) are summed in a fixed order into the
// workgroup's partial row of that level.
// ---------------------------------------------------------------------------

// Workgroup size of the level kernel: its LDS allows three workgroups per compute
// unit, so four wavefronts each keep twelve wavefronts per compute unit.
constexpr int kDwlThreads = 256;

struct PlaneDwlArgs {
    const void *x, *dy;
    float *partial;                 // level l region at off[l-1]: [C][k][4 K^2]
    long long off[kMaxLevels];
    int n, C, H, W, L;
    int vec;                        // x and dy rows are read with vector loads
    int PB, Pw1, NG, k;             // as for the base kernel
    int H1, W1, Gw, commit_items;
    // level l = 1..L at index l-1 (its grid, side-by-side planes included).  Band b
    // of x: element (row r, column j) at xo + b xb + (j + R) xs + (r + R); of dy:
    // go + b gb + j gs + r.  Strides and offsets are multiples of 4 floats.
    int hl[kMaxLevels], wl[kMaxLevels];    // rows, width
    int wr[kMaxLevels], pw[kMaxLevels];    // width of one plane, column pitch between planes
    int ns[kMaxLevels];                    // strips of RHD rows
    int xs[kMaxLevels], xb[kMaxLevels], xo[kMaxLevels];  // x: column stride, band size, offset (floats)
    int gs[kMaxLevels], gb[kMaxLevels], go[kMaxLevels];  // dy: the same
    uint32_t m_wl[kMaxLevels], m_hl[kMaxLevels];          // udiv16 reciprocals of wl, hl
    uint32_t m_row[kMaxLevels], m_wr[kMaxLevels];         // ... of PB wr (items per strip), wr
    uint32_t lane[kDwlThreads];            // level (bits 0-3) | band (4-5) | index in group (8-15) | lanes in group (16-23)
    int groups;                            // (level, band) groups in use: 4 (L - lfirst)
    int lfirst;                            // first level with items, 0-based (1: level 1 runs elsewhere)
    int lane0[kMaxLevels], lanes[kMaxLevels];  // level l: first lane of band 0, lanes per band
    int lds_floats;
    uint32_t m_gw, m_h1;                   // udiv16 reciprocals of Gw, H1
};

template <int K, typename T, int CW, int RHD>
__device__ __forceinline__ void plane_dwl_body(const PlaneDwlArgs &a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    constexpr int NT = kDwlThreads;
    constexpr int WQ = (RHD + 2 * R + 3) / 4;  // 16-byte reads per window column
    static_assert(RHD % 4 == 0, "item rows are read 16 bytes at a time");
    using IO = PatchIO<T, CW>;
    constexpr int SLOTS = kPlaneMaxWords / (2 * IO::kWords) > 0 ? kPlaneMaxWords / (2 * IO::kWords) : 1;
    extern __shared__ float smem[];
    // neighbouring workgroups (numbered per XCD) take neighbouring channels of the
    // same images
    const int wb = xcd_block(blockIdx.x, gridDim.x);
    const int r = wb / a.C, c = wb - r * a.C;
    const int g_begin = (int)((long long)r * a.NG / a.k), g_end = (int)((long long)(r + 1) * a.NG / a.k);
    const int tid = threadIdx.x, PB = a.PB, L = a.L;
    const int HW = a.H * a.W, CHW = a.C * HW;
    const T *xc = static_cast<const T *>(a.x) + (size_t)c * HW;
    const T *dc = static_cast<const T *>(a.dy) + (size_t)c * HW;

    for (int i = tid * 4; i < a.lds_floats; i += NT * 4)
        *reinterpret_cast<float4 *>(smem + i) = make_float4(0.f, 0.f, 0.f, 0.f);

    // commit item g = (p Gw + m) H1 + i: consecutive lanes take consecutive rows of
    // a column group, so that their column-major stores hit distinct banks
    auto patch_of = [&](int g, int &p, int &i, int &m) {
        const int q = udiv16(g, a.m_h1);
        i = g - q * a.H1;
        p = udiv16(q, a.m_gw);
        m = q - p * a.Gw;
    };
    // loads from clamped addresses (see load_patch_clamped); lanes past the last
    // item load nothing (their registers are not used)
    auto load_patch = [&](uint32_t (&rw)[2][IO::kWords], const T *base, int live, int g) {
        if (g >= a.commit_items) return;
        int p, i, m;
        patch_of(g, p, i, m);
        load_patch_clamped<T, CW>(rw, base, p, i, m, live, CHW, a.H, a.W, a.vec);
    };
    // level-1 bands of a patch's CW cells: element (row, col + q) of each band
    // (column stride cs, band size bs); without level-1 items only the low-pass band,
    // which the level-2 analysis reads
    const bool lp_only = a.lfirst > 0;
    auto store_bands = [&](float *base, int cs, int bs, const uint32_t (&rw)[2][IO::kWords], int row, int col) {
#pragma unroll
        for (int q = 0; q < CW; ++q) {
            const float x00 = IO::elem(rw[0], 2 * q), x01 = IO::elem(rw[0], 2 * q + 1);
            const float x10 = IO::elem(rw[1], 2 * q), x11 = IO::elem(rw[1], 2 * q + 1);
            const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
            float *d = base + (col + q) * cs + row;
            d[0] = s0 + s1;
            if (lp_only) continue;
            d[bs] = s0 - s1;
            d[2 * bs] = d0 + d1;
            d[3 * bs] = d0 - d1;
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

    // the lane table, rotated by whole wavefronts per workgroup (so that the
    // wavefronts with the most items fall on different SIMDs); entry pos is this lane's
    const int pos = (tid + kWave * (int)(blockIdx.x & (NT / kWave - 1))) & (NT - 1);
    const uint32_t info = a.lane[pos];
    const int lv = info & 15, band = (info >> 4) & 3, gm = (info >> 8) & 255, gM = (info >> 16) & 255;
    // the lane's item geometry, fixed for the kernel (the level differs between
    // lanes of a wavefront, so it is looked up once, not per item)
    const int li0 = gM > 0 ? lv - 1 : 0;
    // items cover the planes' own columns (not the zero columns between planes)
    const int it_wr = a.wr[li0], it_row = PB * it_wr, it_pw = a.pw[li0];
    const int it_end = gM > 0 ? a.ns[li0] * it_row : 0;
    const uint32_t it_mrow = a.m_row[li0], it_mwr = a.m_wr[li0];
    const int it_xs = a.xs[li0], it_gs = a.gs[li0];
    const int it_x = a.xo[li0] + band * a.xb[li0], it_g = a.go[li0] + band * a.gb[li0];
    float acc[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[t] = 0.f;
    if (g_begin < g_end) prefetch(g_begin);

    for (int g = g_begin; g < g_end; ++g) {
        balance_priority(g_end - g, g_end - g_begin);
        const int n0 = g * PB, live = min(PB, a.n - n0);
        const bool full = live == PB && !(a.H & 1);  // nothing of the pass's patches needs masking
        __syncthreads();  // the previous pass is done with the bands
        {
            const int xs = opaque(a.xs[0]), xb = opaque(a.xb[0]), gs = opaque(a.gs[0]), gb = opaque(a.gb[0]);
            const int pw1 = opaque(a.Pw1);
            float *xbase = smem + a.xo[0] + R * xs + R;
            float *gbase = smem + a.go[0];
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) {
                const int e = tid + k * NT;
                if (e >= a.commit_items) continue;
                int p, i, m;
                patch_of(e, p, i, m);
                mask_patch<T, CW>(xr[k], p, i, live, a.H, full);
                mask_patch<T, CW>(dr[k], p, i, live, a.H, full);
                store_bands(xbase, xs, xb, xr[k], i, p * pw1 + m * CW);
                store_bands(gbase, gs, gb, dr[k], i, p * pw1 + m * CW);
            }
            for (int e = tid + SLOTS * NT; e < a.commit_items; e += NT) {  // beyond the registers
                uint32_t rw[2][IO::kWords];
                int p, i, m;
                patch_of(e, p, i, m);
                load_patch(rw, xc + (size_t)n0 * CHW, live, e);
                mask_patch<T, CW>(rw, p, i, live, a.H, full);
                store_bands(xbase, xs, xb, rw, i, p * pw1 + m * CW);
                load_patch(rw, dc + (size_t)n0 * CHW, live, e);
                mask_patch<T, CW>(rw, p, i, live, a.H, full);
                store_bands(gbase, gs, gb, rw, i, p * pw1 + m * CW);
            }
        }
        __syncthreads();
        if (g + 1 < g_end) prefetch(g + 1);

        // Haar analysis of levels 2..L (unscaled butterflies of the low-pass bands);
        // consecutive lanes take consecutive rows of a column
        for (int l = 1; l < L; ++l) {
            const int Hn = a.hl[l], Wn = a.wl[l];
            const int xs0 = a.xs[l - 1], gs0 = a.gs[l - 1], xs1 = a.xs[l], gs1 = a.gs[l];
            const int xb1 = a.xb[l], gb1 = a.gb[l];
            const float *xsrc = smem + a.xo[l - 1] + R * xs0 + R;  // LL band of the level above
            const float *gsrc = smem + a.go[l - 1];
            float *xdst = smem + a.xo[l] + R * xs1 + R;
            float *gdst = smem + a.go[l];
            for (int q = tid; q < 2 * Hn * Wn; q += NT) {
                const bool isg = q >= Hn * Wn;
                const int qq = isg ? q - Hn * Wn : q;
                const int j = udiv16(qq, a.m_hl[l]), i = qq - j * Hn;
                const int ss = isg ? gs0 : xs0, ds = isg ? gs1 : xs1, db = isg ? gb1 : xb1;
                const float *sp = (isg ? gsrc : xsrc) + (2 * j) * ss + 2 * i;
                const float x00 = sp[0], x10 = sp[1], x01 = sp[ss], x11 = sp[ss + 1];
                const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
                float *dp = (isg ? gdst : xdst) + j * ds + i;
                dp[0] = s0 + s1;
                dp[db] = s0 - s1;
                dp[2 * db] = d0 + d1;
                dp[3 * db] = d0 - d1;
            }
            __syncthreads();
        }

        // this lane's items: column j x RHD rows of (level lv, band)
        if (gM > 0) {
            for (int it = gm; it < it_end; it += gM) {
                const int s = udiv16(it, it_mrow), rem = it - s * it_row;
                const int p = udiv16(rem, it_mwr), j = p * it_pw + (rem - p * it_wr);
                // dy rows s RHD .. + RHD of column j; x window rows s RHD - R ..,
                // columns j - R .. j + R (storage column j + v, row s RHD + t)
                const float4 *gcol = reinterpret_cast<const float4 *>(smem + it_g + j * it_gs + s * RHD);
                const float *xwin = smem + it_x + j * it_xs + s * RHD;
                const int xs = it_xs;
                float gv[RHD];
#pragma unroll
                for (int q = 0; q < RHD / 4; ++q) {
                    const float4 g4 = gcol[q];
                    gv[4 * q] = g4.x;
                    gv[4 * q + 1] = g4.y;
                    gv[4 * q + 2] = g4.z;
                    gv[4 * q + 3] = g4.w;
                }
#pragma unroll
                for (int v = 0; v < K; ++v) {
                    const float4 *cp = reinterpret_cast<const float4 *>(xwin + v * xs);
                    float col[4 * WQ];
#pragma unroll
                    for (int q = 0; q < WQ; ++q) {
                        const float4 c4 = cp[q];
                        col[4 * q] = c4.x;
                        col[4 * q + 1] = c4.y;
                        col[4 * q + 2] = c4.z;
                        col[4 * q + 3] = c4.w;
                    }
#pragma unroll
                    for (int u = 0; u < K; ++u)
#pragma unroll
                        for (int i = 0; i < RHD; ++i) acc[u * K + v] = fmaf(gv[i], col[i + u], acc[u * K + v]);
                }
            }
        }
    }

    // fixed-order reduction: lanes of a group are consecutive in the lane table; the
    // taps go through LDS TC at a time (TC + 1 floats per lane fit the allocation)
    constexpr int TC = KK <= 24 ? KK : (KK + 1) / 2;
#pragma unroll
    for (int t0 = 0; t0 < KK; t0 += TC) {
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TC; ++t)
            if (t0 + t < KK) smem[pos * (TC + 1) + t] = acc[t0 + t];
        __syncthreads();
        const int nt = min(TC, KK - t0);
        for (int q = tid; q < a.groups * nt; q += NT) {
            const int grp = q / nt, tap = q - grp * nt;
            const int l = (grp >> 2) + a.lfirst, b = grp & 3;  // 0-based level
            const int l0 = a.lane0[l] + b * a.lanes[l];
            float sum = 0.f;
            for (int t = l0; t < l0 + a.lanes[l]; ++t) sum += smem[t * (TC + 1) + tap];
            a.partial[a.off[l] + ((size_t)c * a.k + r) * 4 * KK + b * KK + t0 + tap] = ldexpf(sum, -2 * (l + 1));
        }
    }
}

template <int K, typename T, int CW, int RHD>
__global__ __launch_bounds__(kDwlThreads, 3) void plane_dwl_kernel(PlaneDwlArgs a) {
    plane_dwl_body<K, T, CW, RHD>(a);
}
// The same kernel when the correlation kernel takes level 1 (a.lfirst = 1): only
// levels 2..L have items; a symbol of its own, so that traces tell the two apart.
template <int K, typename T, int CW, int RHD>
__global__ __launch_bounds__(kDwlThreads, 3) void plane_dwd_kernel(PlaneDwlArgs a) {
    plane_dwl_body<K, T, CW, RHD>(a);
}

}  // namespace wtc
