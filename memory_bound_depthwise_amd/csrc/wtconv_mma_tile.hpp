// Forward kernel on the matrix cores for planes past the plane-resident range
// (bfloat16 activations, k = 3 or 5, levels >= 1), one spatial tile per pass.
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §4.1-4.2.  On the per-level path the deep levels l = 2..L are
// filtered by the level kernels from the low-pass carriers, deepest first, each
// adding the levels below it, so that level 2 leaves D = sum_{l >= 2} Q_l on the
// level-1 grid in the workspace (the sign patterns Q_l enter every pixel of a
// level-1 cell alike).  This kernel does the rest of the forward pass in one read of
// x and one write of y: the level-1 analysis, filter and synthesis and the base
// conv, as the single banded product of the pixels that the plane-resident
// matrix-core kernel forms (wtconv_mma.hpp: mma_b_fragments, mma_products2), then
// y = product + bias + D per cell.  Level 1 never passes through the workspace.
//
// A pass is a tile of UR x UC level-1 cells (2 UR x 2 UC pixels) of one plane; the
// canvas in LDS holds its pixels and the 2R-pixel halo that the windows of its
// outermost cells reach (zero outside the plane), as bfloat16 pairs: canvas row r is
// pixel row Y0 - 2R + r, canvas column q pixel column X0 - 8 + q.  It is staged in
// chunks of 8 pixels; with rows of a multiple of 8 pixels (vec) the next pass's
// chunks are loaded into registers while the current pass multiplies.  The tile's
// block of D is staged the same way, one pass ahead, as bfloat16 pairs.
//
// Workgroup w (numbered per XCD) takes a contiguous range of passes in the order
// (channel, image, tile row, tile column): neighbouring tiles, whose halos overlap,
// run one after another behind the same L2, and the channel (with it the weight
// table and the B fragments) changes at most a few times per workgroup.  With
// rotate = 1 (and no bias) the kernel computes the input gradient (Prop. 1 / Eq. 1).

#pragma once

#include "wtconv_mma.hpp"

namespace wtc {

constexpr int kTileThreads = 128;  // two wavefronts
constexpr int kTileSlots = 6;      // staged chunks per thread held in registers
constexpr int kTileQSlots = 4;     // staged pattern pairs per thread held in registers

struct MmaTileArgs {
    const void *x;
    void *y;
    const float *w0, *b0, *s0, *wl, *sl;
    const void *q;    // D (activation dtype), [n][C][hq][wq] with hq >= ceil(H / 2) and
                      // wq >= ceil(W / 2) even, or NULL for L = 1
    int hq, wq;
    int n, C, H, W, L;
    int rotate;
    int vec;          // rows of a multiple of 8 pixels, 16-byte aligned: chunk loads
    int pairs;        // y rows take pixel-pair stores (W even, aligned)
    int UR, UC;       // cells per tile (UR a multiple of 4, UC of 16)
    int TYu, TXu;     // tiles per plane
    int rows, chunks; // canvas rows, 8-pixel chunks per canvas row
    int items;        // rows * chunks <= kTileSlots * kTileThreads
    int S;            // canvas row stride (dwords)
    int U;            // passes: C * n * TYu * TXu
    int qitems;       // pairs of D per pass: UR rows of UC / 2 (0 for L = 1)
    int qbase;        // LDS dword offset of the staged block of D
    int wt;           // weight table (floats)
    int lds_floats;
    uint32_t m_chunks, m_tx, m_qp;  // udiv16 reciprocals of chunks, UC / 16 and UC / 2
};

template <int K>
__global__ __launch_bounds__(kTileThreads, 3) void mma_tile_kernel(MmaTileArgs args) {
    using G = MmaGeom<K>;
    using T = uint16_t;
    constexpr int R = (K - 1) / 2, KK = K * K;
    constexpr int NT = kTileThreads;
    extern __shared__ float smem[];
    uint32_t *cv = reinterpret_cast<uint32_t *>(smem);
    const MmaTileArgs &a0 = args;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g4 = lane >> 4, mm = lane & 15;
    const long long G0 = gridDim.x;
    const long long wb = xcd_block(blockIdx.x, gridDim.x);
    const int ubeg = (int)(wb * a0.U / G0), uend = (int)((wb + 1) * a0.U / G0);
    const int HW = a0.H * a0.W;

    // pass u: channel c, image nn, pixel origin (Y0, X0) of its tile
    auto pass_of = [&](const auto &A, int u, int &c, int &nn, int &Y0, int &X0) {
        const int per_plane = A.TYu * A.TXu;
        const int pl = u / per_plane, t = u - pl * per_plane;
        c = pl / A.n;
        nn = pl - c * A.n;
        const int ty = t / A.TXu;
        Y0 = 2 * A.UR * ty;
        X0 = 2 * A.UC * (t - ty * A.TXu);
    };
    // chunk e of the canvas: 8 pixels of pixel row Y, columns X .. X + 7
    auto chunk_of = [&](const auto &A, int e, int Y0, int X0, int &Y, int &X) {
        const int r = udiv16(e, A.m_chunks), k = e - r * A.chunks;
        Y = Y0 - 2 * R + r;
        X = X0 - 8 + 8 * k;
    };
    auto load_chunk = [&](const auto &A, const T *xp, int Y, int X) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (Y >= 0 && Y < A.H && X >= 0 && X < A.W) v = *reinterpret_cast<const uint4 *>(xp + (size_t)Y * A.W + X);
        return v;
    };
    // unaligned rows: the chunk's pixels one at a time
    auto load_chunk_scalar = [&](const auto &A, const T *xp, int Y, int X) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (Y >= 0 && Y < A.H) {
            const uint16_t *row = reinterpret_cast<const uint16_t *>(xp) + (size_t)Y * A.W;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int xi = X + i;
                const uint32_t h = xi >= 0 && xi < A.W ? row[xi] : 0u;
                w[i >> 1] |= h << (16 * (i & 1));
            }
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    };

    // pair e of the pass's block of D: row r, pair j (clamped into D: rows and pairs
    // past the plane repeat its last ones; their cells store nothing)
    auto load_qpair = [&](const auto &A, int e, int c, int nn, int Y0, int X0) {
        const int half = A.UC >> 1, r = udiv16(e, A.m_qp), j = e - r * half;
        const int row = min((Y0 >> 1) + r, A.hq - 1), pair = min((X0 >> 2) + j, (A.wq >> 1) - 1);
        const uint32_t *qp = static_cast<const uint32_t *>(A.q);
        return qp[(((size_t)nn * A.C + c) * A.hq * A.wq) / 2 + (size_t)row * (A.wq >> 1) + pair];
    };

    uint4 raw[kTileSlots];
    uint32_t qraw[kTileQSlots];
    auto prefetch = [&](const auto &A, int u) {
        int c, nn, Y0, X0;
        pass_of(A, u, c, nn, Y0, X0);
        const T *xp = static_cast<const T *>(A.x) + ((size_t)nn * A.C + c) * HW;
        if (A.vec) {
#pragma unroll
            for (int k = 0; k < kTileSlots; ++k) {
                int Y, X;
                chunk_of(A, min(tid + k * NT, A.items - 1), Y0, X0, Y, X);
                raw[k] = load_chunk(A, xp, Y, X);
            }
        }
#pragma unroll
        for (int k = 0; k < kTileQSlots; ++k) {
            const int e = tid + k * NT;
            if (e < A.qitems) qraw[k] = load_qpair(A, e, c, nn, Y0, X0);
        }
    };
    if (ubeg < uend) prefetch(args, ubeg);

    wtc_bf16x8 bh[G::NS], bl[G::NS];
    float bias = 0.f;
    int cur_c = -1;

    for (int u = ubeg; u < uend; ++u) {
        balance_priority(uend - u, uend - ubeg);
        const __attribute__((address_space(4))) MmaTileArgs *ap =
            (const __attribute__((address_space(4))) MmaTileArgs *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const auto &a = *ap;
        int c, nn, Y0, X0;
        pass_of(a, u, c, nn, Y0, X0);
        const int S = opaque(a.S), wt = opaque(a.wt);
        const bool new_c = c != cur_c;
        __syncthreads();  // the previous pass is done with the canvas and the table
        // 1. the weight table of a new channel: level-1 band weights s(1,b) W(1,b) / 4
        //    as float4 over the bands at wt + 4 (v K + u), the base weights s0 W0 at
        //    wt + 4 K^2 + v K + u, the folded bias s0 b0 at wt + 5 K^2
        if (new_c && tid < 5 * KK + 1) {
            const int e = tid;
            float val;
            if (e < 5 * KK) {
                const int tap = e < 4 * KK ? e % KK : e - 4 * KK;  // v K + u (column-major)
                const int v = tap / K, uu = tap - v * K;
                const int src = a.rotate ? (K - 1 - uu) * K + (K - 1 - v) : uu * K + v;
                if (e < 4 * KK) {
                    const int b = e / KK;
                    val = ldexpf(a.sl[c * 4 + b], -2) * a.wl[((size_t)c * 4 + b) * KK + src];
                    smem[wt + 4 * tap + b] = val;
                } else {
                    val = a.s0[c] * a.w0[(size_t)c * KK + src];
                    smem[wt + 4 * KK + tap] = val;
                }
            } else {
                smem[wt + 5 * KK] = a.b0 ? a.s0[c] * a.b0[c] : 0.f;
            }
        }
        // 2. the canvas
        {
            const T *xp = static_cast<const T *>(a.x) + ((size_t)nn * a.C + c) * HW;
            if (a.vec) {
#pragma unroll
                for (int k = 0; k < kTileSlots; ++k) {
                    const int e = tid + k * NT;
                    if (e < a.items) {
                        const int r = udiv16(e, a.m_chunks), kk = e - r * a.chunks;
                        *reinterpret_cast<uint4 *>(cv + r * S + 4 * kk) = raw[k];
                    }
                }
            } else {
                for (int e = tid; e < a.items; e += NT) {
                    int Y, X;
                    chunk_of(a, e, Y0, X0, Y, X);
                    const int r = udiv16(e, a.m_chunks), kk = e - r * a.chunks;
                    *reinterpret_cast<uint4 *>(cv + r * S + 4 * kk) = load_chunk_scalar(a, xp, Y, X);
                }
            }
#pragma unroll
            for (int k = 0; k < kTileQSlots; ++k) {
                const int e = tid + k * NT;
                if (e < a.qitems) cv[a.qbase + e] = qraw[k];
            }
        }
        __syncthreads();
        // 3. the B fragments of a new channel; the next pass's chunks go out
        if (new_c) {
            cur_c = c;
            mma_b_fragments<K>(smem, wt, wt + 4 * KK, lane, bh, bl);
            bias = smem[wt + 5 * KK];
        }
        if (u + 1 < uend) prefetch(a, u + 1);

        // 4. products and stores: tile t = (ty, tx) of 4 x 16 cells; lane (g4, mm)
        //    receives the four pixels of cell (4 ty + g4, 16 tx + mm) of the pass
        T *yp = static_cast<T *>(a.y) + ((size_t)nn * a.C + c) * HW;
        const int la = (kMmaCL - G::COL0) / 2 + g4 * S + mm;
        const int tiles = (a.UR >> 2) * (a.UC >> 4), ntx = a.UC >> 4;
        const int cr0 = Y0 >> 1, cc0 = X0 >> 1;  // level-1 cell of the pass origin
        const int H = a.H, W = a.W, pairs = opaque(a.pairs);
        const bool deep = a.L >= 2;
        const uint16_t *qs16 = reinterpret_cast<const uint16_t *>(cv);
        constexpr int NW = NT / kWave;
        for (int t = wave; t < tiles; t += 2 * NW) {
            const int t2 = t + NW < tiles ? t + NW : t;
            int ty[2], tx[2];
            ty[0] = udiv16(t, a.m_tx);
            tx[0] = t - ty[0] * ntx;
            ty[1] = udiv16(t2, a.m_tx);
            tx[1] = t2 - ty[1] * ntx;
            // bias and the deep patterns of the cell, from the staged block of D: the
            // products accumulate onto them
            float v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int lr = 4 * ty[h] + g4, lc = 16 * tx[h] + mm;
                v[h] = bias + (deep ? Act<T>::lo(qs16[2 * a.qbase + lr * a.UC + lc]) : 0.f);
            }
            wtc_f32x4 acc[2];
            mma_products2<K>(cv + la + (8 * ty[0]) * S + 16 * tx[0], cv + la + (8 * ty[1]) * S + 16 * tx[1], S, bh, bl,
                             v, acc);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1 && t2 == t) break;
                const int lr = 4 * ty[h] + g4, lc = 16 * tx[h] + mm;
                const int pr = 2 * (cr0 + lr), pc = 2 * (cc0 + lc);
                if (pr < H && pc < W) {
                    const float o0 = acc[h][0], o1 = acc[h][1], o2 = acc[h][2], o3 = acc[h][3];
                    T *dst = yp + ((size_t)pr * W + pc);
                    const bool row1 = pr + 1 < H;
                    if (pairs) {
                        *reinterpret_cast<uint32_t *>(dst) = Act<T>::pack(o0, o2);
                        if (row1) *reinterpret_cast<uint32_t *>(dst + W) = Act<T>::pack(o1, o3);
                    } else {
                        const bool col1 = pc + 1 < W;
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

}  // namespace wtc
