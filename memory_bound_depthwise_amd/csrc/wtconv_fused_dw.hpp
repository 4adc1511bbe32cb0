// Plane-resident weight-gradient kernel of the WTConv levels for small planes
// (H, W <= 64).
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §2.2 Eq. 1 and §4.3 Eq. 9.  The folded-weight gradient of band b
// of level l is the correlation
//     dW~(l)[b][u][v] = sum_{n,i,j} G(l)[b][i][j] Y(l)[b][i+u-R][j+v-R],
// with Y(l) the level-l Haar analysis of x and G(l) that of dy: the gradient at the
// level-l coefficients is the analysis of dy (backward through synthesis is
// analysis, Eq. 1).  Eq. 9 then gives dW = s dW~ and ds = <dW~, W> (finalize
// kernel).
//
// One workgroup (256 threads) owns one channel and walks a range of its planes,
// PB per pass.  Per pass, in LDS: the unscaled pyramids S_l(x) = 2^l Y(l) (with a
// zero halo of R for the correlation windows) and S_l(dy) = 2^l G(l) (centre only).
// Level 1 comes straight from the prefetched 2 x 2 pixel blocks of x and dy; deeper
// levels from the low-pass band of the level above.  Each lane owns one
// (level, band) pair for the whole kernel - lanes are allocated to pairs in
// proportion to their work so that all pairs finish in the same number of rounds -
// and accumulates its k x k tap sums over 8-row column strips.  At the end the
// lanes of each pair are summed in a fixed order (LDS) into one partial row per
// workgroup, scaled by 4^-l (exact).

#pragma once

#include "wtconv_fused.hpp"

namespace wtc {

constexpr int kDwMaxRounds = 4;    // items per lane per pass
constexpr int kDwRawWords = 16;    // prefetch words per thread and tensor

struct FusedDwArgs {
    const void *x, *dy;
    float *partial;   // level l region: [C][nblk][4 K K] at partial + off[l]
    long long off[kMaxLevels];
    int n, C, H, W, L;
    int PB, NB, nblk;
    int VE;           // elements per prefetch row segment (W % VE == 0, even, aligned); 1 = scalar blocks
    // LDS layout (floats, first plane block; PB blocks plane_floats apart)
    int plane_floats, lds_floats;
    int yb[kMaxLevels], ybs[kMaxLevels], ys[kMaxLevels];  // x pyramid: base, band stride, row stride (halo R)
    int gb[kMaxLevels], gbs[kMaxLevels];                  // dy pyramid: base, band stride (row stride = W_l)
    int hl[kMaxLevels + 1], wl_[kMaxLevels + 1], sp[kMaxLevels + 1];
    // lane allocation: pair t = 4 l + b owns lanes [lane0[t], lane0[t] + lanes[t])
    int lane0[4 * kMaxLevels], lanes[4 * kMaxLevels];
    int rounds;
    int blocks;        // level-1 blocks per plane (H1 W1)
    int bpv;           // blocks per prefetch slot (VE / 2, or 1)
    uint32_t m_w1, m_blocks;                      // fdiv: W1, blocks-per-plane
    uint32_t m_per[kMaxLevels], m_wl[kMaxLevels];  // fdiv: Hl Wl, Wl
};

// Prefetched 2 x 2 pixel blocks of one tensor: slot k covers coarse row i and the
// BPV blocks starting at coarse column j0 of plane p.
template <typename T, int VE>
struct BlockPrefetch {
    static constexpr int BPV = VE >= 2 ? VE / 2 : 1;
    static constexpr int kRowWords = VE >= 2 ? (VE * (int)sizeof(T) + 3) / 4 : (2 * (int)sizeof(T) + 3) / 4;
    static constexpr int kSlots = kDwRawWords / (2 * kRowWords);

    // slot geometry shared by x and dy: returns false when the slot is past the pass
    __device__ __forceinline__ static bool where(const FusedDwArgs &a, int v, int &p, int &i, int &j0) {
        const int spp = a.blocks / BPV;  // slots per plane
        if (v >= a.PB * spp) return false;
        const int e = v * BPV;
        p = fdiv(e, a.m_blocks);
        const int off = e - p * a.blocks;
        i = fdiv(off, a.m_w1);
        j0 = off - i * a.wl_[1];
        return true;
    }

    __device__ __forceinline__ static void load(const FusedDwArgs &a, uint32_t *raw, const T *base, int live,
                                                int CHW, int tid) {
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            int p, i, j0;
            uint32_t *r = raw + k * 2 * kRowWords;
#pragma unroll
            for (int q = 0; q < 2 * kRowWords; ++q) r[q] = 0u;
            if (!where(a, tid + k * 256, p, i, j0) || p >= live) continue;
            const T *src = base + (p * CHW + (2 * i) * a.W + 2 * j0);
            const bool row1 = 2 * i + 1 < a.H;
            if constexpr (VE >= 2) {
                if constexpr (sizeof(T) == 2) {
                    if constexpr (VE == 8) {
                        const uint4 q0 = *reinterpret_cast<const uint4 *>(src);
                        r[0] = q0.x; r[1] = q0.y; r[2] = q0.z; r[3] = q0.w;
                        if (row1) {
                            const uint4 q1 = *reinterpret_cast<const uint4 *>(src + a.W);
                            r[4] = q1.x; r[5] = q1.y; r[6] = q1.z; r[7] = q1.w;
                        }
                    } else if constexpr (VE == 4) {
                        const uint2 q0 = *reinterpret_cast<const uint2 *>(src);
                        r[0] = q0.x; r[1] = q0.y;
                        if (row1) {
                            const uint2 q1 = *reinterpret_cast<const uint2 *>(src + a.W);
                            r[2] = q1.x; r[3] = q1.y;
                        }
                    } else {
                        r[0] = *reinterpret_cast<const uint32_t *>(src);
                        if (row1) r[1] = *reinterpret_cast<const uint32_t *>(src + a.W);
                    }
                } else {
                    if constexpr (VE == 4) {
                        const uint4 q0 = *reinterpret_cast<const uint4 *>(src);
                        r[0] = q0.x; r[1] = q0.y; r[2] = q0.z; r[3] = q0.w;
                        if (row1) {
                            const uint4 q1 = *reinterpret_cast<const uint4 *>(src + a.W);
                            r[4] = q1.x; r[5] = q1.y; r[6] = q1.z; r[7] = q1.w;
                        }
                    } else {
                        const uint2 q0 = *reinterpret_cast<const uint2 *>(src);
                        r[0] = q0.x; r[1] = q0.y;
                        if (row1) {
                            const uint2 q1 = *reinterpret_cast<const uint2 *>(src + a.W);
                            r[2] = q1.x; r[3] = q1.y;
                        }
                    }
                }
            } else {
                // one block from scalars; odd sizes pad with zeros
                const bool col1 = 2 * j0 + 1 < a.W;
                if constexpr (sizeof(T) == 2) {
                    const uint16_t *s16 = reinterpret_cast<const uint16_t *>(src);
                    r[0] = (uint32_t)s16[0] | (col1 ? (uint32_t)s16[1] << 16 : 0u);
                    if (row1) r[1] = (uint32_t)s16[a.W] | (col1 ? (uint32_t)s16[a.W + 1] << 16 : 0u);
                } else {
                    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
                    r[0] = s32[0];
                    if (col1) r[1] = s32[1];
                    if (row1) {
                        r[2] = s32[a.W];
                        if (col1) r[3] = s32[a.W + 1];
                    }
                }
            }
        }
    }

    // pixel t of row rr (0 or 1) of slot k as float32
    __device__ __forceinline__ static float px(const uint32_t *raw, int k, int rr, int t) {
        const uint32_t *r = raw + k * 2 * kRowWords + rr * kRowWords;
        if constexpr (kHalf<T>) {
            const uint32_t wv = r[t >> 1];
            return (t & 1) ? Act<T>::hi(wv) : Act<T>::lo(wv);
        } else {
            return __uint_as_float(r[t]);
        }
    }

    // butterflies of the slot's blocks into the level-1 region of a pyramid:
    // band b of block (i, j) at dst + b * band_stride + (i + halo) * row_stride + j + halo
    __device__ __forceinline__ static void commit(const FusedDwArgs &a, const uint32_t *raw, float *smem,
                                                  int region, int band_stride, int row_stride, int halo,
                                                  int tid) {
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            int p, i, j0;
            if (!where(a, tid + k * 256, p, i, j0)) continue;
            float *d = smem + p * a.plane_floats + region + (i + halo) * row_stride + j0 + halo;
#pragma unroll
            for (int q = 0; q < BPV; ++q) {
                const float x00 = px(raw, k, 0, 2 * q), x01 = px(raw, k, 0, 2 * q + 1);
                const float x10 = px(raw, k, 1, 2 * q), x11 = px(raw, k, 1, 2 * q + 1);
                const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
                d[q] = s0 + s1;
                d[q + band_stride] = s0 - s1;
                d[q + 2 * band_stride] = d0 + d1;
                d[q + 3 * band_stride] = d0 - d1;
            }
        }
    }
};

template <int K, typename T, int VE>
__device__ __forceinline__ void fused_dw_body(const FusedDwArgs &a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    using BP = BlockPrefetch<T, VE>;
    extern __shared__ float smem[];
    const int c = blockIdx.x % a.C, nb = blockIdx.x / a.C;
    const int n_begin = nb * a.NB, n_end = min(a.n, n_begin + a.NB);
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int L = a.L, PB = a.PB, PF = a.plane_floats;

    for (int i = tid; i < a.lds_floats; i += nthr) smem[i] = 0.f;

    // this lane's (level, band) pair and its items, packed per round:
    //   d0 = x-window offset (0-15) | dy offset (16-31);  d1 = rows (0-7) | x stride (8-15) | dy stride (16-23)
    int pair = -1;
    for (int t = 0; t < 4 * L; ++t)
        if (tid >= a.lane0[t] && tid < a.lane0[t] + a.lanes[t]) pair = t;
    uint32_t d0[kDwMaxRounds], d1[kDwMaxRounds];
#pragma unroll
    for (int r = 0; r < kDwMaxRounds; ++r) {
        d0[r] = d1[r] = 0;
        if (pair < 0 || r >= a.rounds) continue;
        const int l = pair >> 2, b = pair & 3;
        const int Wl = a.wl_[l + 1], per = a.sp[l + 1] * Wl;
        const int m = (tid - a.lane0[pair]) + r * a.lanes[pair];
        if (m >= PB * per) continue;
        const int p = m / per, rem = m - p * per, s = rem / Wl, j = rem - s * Wl;
        const int xo = p * PF + a.yb[l] + b * a.ybs[l] + (s * kRH) * a.ys[l] + j;
        const int go = p * PF + a.gb[l] + b * a.gbs[l] + (s * kRH) * Wl + j;
        const int rows = min(kRH, a.hl[l + 1] - s * kRH);
        d0[r] = (uint32_t)xo | ((uint32_t)go << 16);
        d1[r] = (uint32_t)rows | ((uint32_t)a.ys[l] << 8) | ((uint32_t)Wl << 16);
    }

    float acc[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) acc[i] = 0.f;

    const int CHW = a.C * a.H * a.W, HW = a.H * a.W;
    const T *x = static_cast<const T *>(a.x);
    const T *dy = static_cast<const T *>(a.dy);
    uint32_t rx[kDwRawWords], rg[kDwRawWords];
    {
        const int live = min(PB, n_end - n_begin);
        const size_t base = ((size_t)n_begin * a.C + c) * HW;
        BP::load(a, rx, x + base, live, CHW, tid);
        BP::load(a, rg, dy + base, live, CHW, tid);
    }

    for (int n0 = n_begin; n0 < n_end; n0 += PB) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kDwMaxRounds; ++r) asm volatile("" : "+v"(d0[r]), "+v"(d1[r]));
        int t = tid;
        asm volatile("" : "+v"(t));
        // level 1 of both pyramids from the prefetched blocks (planes past n_end are 0)
        BP::commit(a, rx, smem, a.yb[0], a.ybs[0], a.ys[0], R, t);
        BP::commit(a, rg, smem, a.gb[0], a.gbs[0], a.wl_[1], 0, t);
        __syncthreads();
        if (n0 + PB < n_end) {
            const int live = min(PB, n_end - n0 - PB);
            const size_t base = ((size_t)(n0 + PB) * a.C + c) * HW;
            BP::load(a, rx, x + base, live, CHW, t);
            BP::load(a, rg, dy + base, live, CHW, t);
        }
        // deeper levels: butterflies of the low-pass band of the level above
        for (int l = 1; l < L; ++l) {
            const int Hp = a.hl[l], Wp = a.wl_[l];  // grid of the level above
            const int Wl = a.wl_[l + 1], per = a.hl[l + 1] * Wl;
            const uint32_t m_per = a.m_per[l], m_wl = a.m_wl[l];
            for (int q = t; q < PB * per; q += nthr) {
                const int p = fdiv(q, m_per), rem = q - p * per, i = fdiv(rem, m_wl), j = rem - i * Wl;
                // x side: the halo of the level above pads odd sizes
                const float *sx = smem + p * PF + a.yb[l - 1] + (2 * i + R) * a.ys[l - 1] + 2 * j + R;
                float x00 = sx[0], x01 = sx[1], x10 = sx[a.ys[l - 1]], x11 = sx[a.ys[l - 1] + 1];
                float s0 = x00 + x01, s1 = x10 + x11, e0 = x00 - x01, e1 = x10 - x11;
                float *dxp = smem + p * PF + a.yb[l] + (i + R) * a.ys[l] + j + R;
                const int bx = a.ybs[l];
                dxp[0] = s0 + s1;
                dxp[bx] = s0 - s1;
                dxp[2 * bx] = e0 + e1;
                dxp[3 * bx] = e0 - e1;
                // dy side: centre-only layout, pad odd sizes explicitly
                const float *sg = smem + p * PF + a.gb[l - 1] + (2 * i) * Wp + 2 * j;
                const bool c1 = 2 * j + 1 < Wp, r1 = 2 * i + 1 < Hp;
                const float g00 = sg[0], g01 = c1 ? sg[1] : 0.f;
                const float g10 = r1 ? sg[Wp] : 0.f, g11 = (r1 && c1) ? sg[Wp + 1] : 0.f;
                s0 = g00 + g01;
                s1 = g10 + g11;
                e0 = g00 - g01;
                e1 = g10 - g11;
                float *dgp = smem + p * PF + a.gb[l] + i * Wl + j;
                const int bg = a.gbs[l];
                dgp[0] = s0 + s1;
                dgp[bg] = s0 - s1;
                dgp[2 * bg] = e0 + e1;
                dgp[3 * bg] = e0 - e1;
            }
            __syncthreads();
        }
        // correlations of this lane's (level, band) pair (planes past n_end are all
        // zero and add nothing)
#pragma unroll
        for (int r = 0; r < kDwMaxRounds; ++r) {
            const int rows = d1[r] & 0xffu;
            if (rows == 0) continue;
            const int xs = (d1[r] >> 8) & 0xffu, gs = (d1[r] >> 16) & 0xffu;
            const float *gp = smem + (d0[r] >> 16);
            float g[kRH];
#pragma unroll
            for (int i = 0; i < kRH; ++i) g[i] = i < rows ? gp[i * gs] : 0.f;
            corr_strip<K>(smem + (d0[r] & 0xffffu), xs, g, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // fixed-order reduction of each pair's lanes, 8 taps at a time through LDS
    constexpr int CH = 8;
    float *red = smem;  // [256][CH + 1]
#pragma unroll
    for (int t0 = 0; t0 < KK; t0 += CH) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (t0 + i < KK) red[tid * (CH + 1) + i] = acc[t0 + i];
        __syncthreads();
        for (int q = tid; q < 4 * L * CH; q += nthr) {
            const int pr = q / CH, i = q - pr * CH, tap = t0 + i, l = pr >> 2, b = pr & 3;
            if (tap >= KK) continue;
            float sum = 0.f;
            for (int ln = 0; ln < a.lanes[pr]; ++ln) sum += red[(a.lane0[pr] + ln) * (CH + 1) + i];
            // S_l(x) S_l(dy) = 4^l Y G: scale back (exact)
            a.partial[a.off[l] + ((size_t)c * a.nblk + nb) * 4 * KK + b * KK + tap] = ldexpf(sum, -2 * (l + 1));
        }
    }
}

template <int K, typename T, int VE>
__global__ __launch_bounds__(256, (K <= 5 ? 4 : 2)) void fused_dw_kernel(FusedDwArgs a) {
    fused_dw_body<K, T, VE>(a);
}

}  // namespace wtc
