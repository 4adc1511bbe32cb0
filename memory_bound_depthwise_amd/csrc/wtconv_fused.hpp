// Plane-resident forward kernel of the WTConv layer for small planes (H, W <= 64).
//
// Paper: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation", §4.  The paper fuses the analysis and the filtering of each level
// (§4.1) and collapses the synthesis into one closed-form pass (§4.2, Prop. 2);
// its level kernels still hand the filtered coefficients of every level to the
// synthesis pass through HBM.  On gfx950 a whole plane of the WTConvNeXt stages
// (56 x 56 and smaller) and all of its levels fit in the 160 KB LDS of a compute
// unit, so this kernel keeps the complete pyramid on chip and moves only x in and y
// out: 2N elements per pass instead of the paper's 4N + (13/3)N(1 - 4^-L) - N 4^-L.
//
// One workgroup (256 threads) owns one channel and walks a range of planes of it,
// PB planes per pass.  Per pass, all in LDS:
//   1. commit the prefetched x planes (float32, zero halo of R = (K-1)/2);
//      issue the loads of the next pass's planes (they land during steps 2-6);
//   2. Haar analysis level by level (Eq. 5, unscaled: S_l = 2^l Y_l); level l reads
//      the low-pass band of level l-1 (the carrier), whose zero halo doubles as the
//      pad-to-even of odd sizes;
//   3. the k x k depthwise conv of every (level, band) pair: one item is one column
//      x 8 rows of one band of one level, all items of the pass share the 256 lanes
//      and each lane reads its item's folded weights from an LDS table:
//      s(l) W(l) 4^-l, i.e. the scale (Eq. 8), the analysis factor 2^-l of S_l and
//      the synthesis weight 2^-l of Eq. 7 (powers of two: exact);
//   4. the filtered coefficients overwrite their band (centre only; halos stay 0);
//   5. each coefficient block is replaced by its four sign patterns (Eq. 12/13),
//      slot 2 ry + rx holding LL + (-1)^ry LH + (-1)^rx HL + (-1)^(ry+rx) HH;
//   6. final pass: base conv with s0 W0 (scalar registers), bias s0 b, plus for each
//      level the slot selected by bit l-1 of the output coordinate at (y >> l,
//      x >> l) (Prop. 2, Eq. 7); one store of y.
// With rotate = 1 (and no bias) the same kernel computes the input gradient.

#pragma once

#include "wtconv_kernels.hpp"

namespace wtc {

constexpr int kFusedMaxItems = 3;  // conv items per thread per pass
constexpr int kFusedMaxFinal = 2;  // final-pass items per thread per pass
// prefetch buffer per thread (32-bit words)
template <typename T>
constexpr int fused_raw_words() { return sizeof(T) == 2 ? 8 : 16; }

// Balanced item-to-thread map: item round k covers items [256 k, 256 k + r_k) and
// gives each of the four wavefronts a contiguous chunk of ceil(r_k / 4) items, so no
// wavefront (and no SIMD) carries a whole extra round.  Returns -1 when the thread
// has no item in round k.
__device__ __forceinline__ int balanced_item(int total, int k, int tid) {
    const int first = k * 256, r = min(256, total - first);
    if (r <= 0) return -1;
    const int chunk = (r + 3) >> 2, w = tid >> 6, lane = tid & 63;
    if (lane >= chunk) return -1;
    const int li = w * chunk + lane;
    return li < r ? first + li : -1;
}

struct FusedArgs {
    const void *x;
    void *y;
    const float *w0, *b0, *s0, *wl, *sl;
    int n, C, H, W, L;
    int rotate;
    int PB;            // planes per pass
    int NB, nblk;      // planes per workgroup, workgroups per channel
    int VE;            // elements per prefetch vector (W % VE == 0, pointer aligned)
    // LDS layout, in floats; a plane's block is repeated PB times, plane_floats apart
    int plane_floats;
    int wtab;          // weight table [L][4][KKP] (shared by the planes)
    int xoff, xs;      // x region offset (first plane block) and row stride
    int yb[kMaxLevels], bs[kMaxLevels], sy[kMaxLevels];  // level l+1: base (first plane block), band stride, row stride
    int hl[kMaxLevels + 1], wl_[kMaxLevels + 1];         // grid of level l (l = 0: pixels)
    int sp[kMaxLevels + 1];                              // 8-row strips of level l's grid
    int items_end[kMaxLevels];  // cumulative conv items per plane, by level (4 bands each)
    int conv_items;             // per plane
    int lds_floats;             // total
    // multiply-high reciprocals (see fdiv) of the divisors used per element
    uint32_t m_hw, m_w, m_conv, m_fin;
    uint32_t m_per[kMaxLevels], m_wl[kMaxLevels];  // level l+1: Hl*Wl and Wl
};

template <int K>
__device__ __forceinline__ void conv_strip_dyn(const float *src, int stride, const float *w, float *acc) {
#pragma unroll
    for (int v = 0; v < K; ++v) {
        float col[kRH + K - 1];
#pragma unroll
        for (int i = 0; i < kRH + K - 1; ++i) col[i] = src[i * stride + v];
#pragma unroll
        for (int u = 0; u < K; ++u)
#pragma unroll
            for (int i = 0; i < kRH; ++i) acc[i] = fmaf(w[u * K + v], col[i + u], acc[i]);
    }
}

// Prefetch of PB planes of x into registers: vector v of the pass covers elements
// [v VE, v VE + VE) of the concatenated planes; slots are v = tid + k 256.  Global
// offsets are 32-bit from the uniform base of plane (n0, c); PB C H W < 2^30.
template <typename T, int VE>
struct XPrefetch {
    static constexpr int kRawWords = fused_raw_words<T>();
    static constexpr int kWordsPerVec = (VE * (int)sizeof(T) + 3) / 4;
    static constexpr int kSlots = kRawWords / kWordsPerVec;

    __device__ __forceinline__ static void load(uint32_t *raw, const T *xbase, int live_planes, int CHW, int HW,
                                                uint32_t m_hw, int PB, int tid) {
        const int total = PB * HW / VE;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int v = tid + k * 256;
            if (v >= total) continue;
            const int e = v * VE, p = fdiv(e, m_hw), off = e - p * HW;
            if (p >= live_planes) continue;
            const T *src = xbase + (p * CHW + off);
            uint32_t *r = raw + k * kWordsPerVec;
            if constexpr (sizeof(T) == 2) {
                if constexpr (VE == 8) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(src);
                    r[0] = q.x; r[1] = q.y; r[2] = q.z; r[3] = q.w;
                } else if constexpr (VE == 4) {
                    const uint2 q = *reinterpret_cast<const uint2 *>(src);
                    r[0] = q.x; r[1] = q.y;
                } else if constexpr (VE == 2) {
                    r[0] = *reinterpret_cast<const uint32_t *>(src);
                } else {
                    r[0] = *reinterpret_cast<const uint16_t *>(src);
                }
            } else {
                if constexpr (VE == 4) {
                    const uint4 q = *reinterpret_cast<const uint4 *>(src);
                    r[0] = q.x; r[1] = q.y; r[2] = q.z; r[3] = q.w;
                } else if constexpr (VE == 2) {
                    const uint2 q = *reinterpret_cast<const uint2 *>(src);
                    r[0] = q.x; r[1] = q.y;
                } else {
                    r[0] = *reinterpret_cast<const uint32_t *>(src);
                }
            }
        }
    }

    // Element t of slot k as float32.
    __device__ __forceinline__ static float elem(const uint32_t *raw, int k, int t) {
        const uint32_t *r = raw + k * kWordsPerVec;
        if constexpr (kHalf<T>) {
            if constexpr (VE == 1) return Act<T>::lo(r[0]);
            const uint32_t wv = r[t >> 1];
            return (t & 1) ? Act<T>::hi(wv) : Act<T>::lo(wv);
        } else {
            return __uint_as_float(r[t]);
        }
    }

    // Write the slots into the x regions of LDS (centre of each plane's region).
    __device__ __forceinline__ static void commit(const uint32_t *raw, float *smem, int live_planes, int HW,
                                                  uint32_t m_hw, int W, uint32_t m_w, int PB, int plane_floats,
                                                  int xoff, int xs, int R, int tid) {
        const int total = PB * HW / VE;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int v = tid + k * 256;
            if (v >= total) continue;
            const int e = v * VE, p = fdiv(e, m_hw), off = e - p * HW;
            const int row = fdiv(off, m_w), col = off - row * W;
            float *d = smem + p * plane_floats + xoff + (row + R) * xs + col + R;
            const bool live = p < live_planes;
#pragma unroll
            for (int t = 0; t < VE; ++t) d[t] = live ? elem(raw, k, t) : 0.f;
        }
    }
};

template <int K, typename T, int VE>
__device__ __forceinline__ void fused_fwd_body(const FusedArgs &a) {
    constexpr int R = (K - 1) / 2, KK = K * K, KKP = (KK + 3) & ~3;
    using XP = XPrefetch<T, VE>;
    extern __shared__ float smem[];
    const int c = blockIdx.x % a.C, nb = blockIdx.x / a.C;
    const int n_begin = nb * a.NB, n_end = min(a.n, n_begin + a.NB);
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int H = a.H, W = a.W, HW = H * W, L = a.L, PB = a.PB, PF = a.plane_floats;

    for (int i = tid; i < a.lds_floats; i += nthr) smem[i] = 0.f;
    // folded level weights: s(l) W(l) 4^-l (rotated for the input gradient)
    for (int i = tid; i < L * 4 * KK; i += nthr) {
        const int lb = i / KK, tap = i - lb * KK, l = lb >> 2, b = lb & 3;
        const int u = tap / K, v = tap - u * K;
        const int src = a.rotate ? (K - 1 - u) * K + (K - 1 - v) : tap;
        const size_t pc = ((size_t)l * a.C + c) * 4 + b;
        smem[a.wtab + lb * KKP + tap] = a.sl[pc] * a.wl[pc * KK + src] * ldexpf(1.0f, -2 * (l + 1));
    }
    // conv items of this thread: (plane, level, band, strip, column), packed as
    //   cd0 = window offset (bits 0-15) | row stride (16-23) | valid rows (24-31)
    //   cd1 = weight-table offset
    uint32_t cd0[kFusedMaxItems], cd1[kFusedMaxItems];
#pragma unroll
    for (int k = 0; k < kFusedMaxItems; ++k) {
        cd0[k] = cd1[k] = 0;
        const int it = balanced_item(PB * a.conv_items, k, tid);
        if (it < 0) continue;
        const int p = fdiv(it, a.m_conv);
        int loc = it - p * a.conv_items, l = 0;
        while (loc >= a.items_end[l]) ++l;
        loc -= l ? a.items_end[l - 1] : 0;
        const int Wl = a.wl_[l + 1], per_band = a.sp[l + 1] * Wl;
        const int b = loc / per_band, r = loc - b * per_band, s = r / Wl, j = r - s * Wl;
        const int win = p * PF + a.yb[l] + b * a.bs[l] + (s * kRH) * a.sy[l] + j;
        const int rows = min(kRH, a.hl[l + 1] - s * kRH);
        cd0[k] = (uint32_t)win | ((uint32_t)a.sy[l] << 16) | ((uint32_t)rows << 24);
        cd1[k] = (uint32_t)(a.wtab + (l * 4 + b) * KKP);
    }
    // final-pass items: (plane, strip, column) of the pixel grid, packed as
    //   fd = column (0-7) | strip (8-15) | plane (16-23) | valid rows (24-31)
    uint32_t fd[kFusedMaxFinal];
    const int fin_per_plane = a.sp[0] * W;
#pragma unroll
    for (int k = 0; k < kFusedMaxFinal; ++k) {
        const int it = balanced_item(PB * fin_per_plane, k, tid);
        fd[k] = 0;
        if (it < 0) continue;
        const int p = fdiv(it, a.m_fin), r = it - p * fin_per_plane, s = fdiv(r, a.m_w), j = r - s * W;
        fd[k] = (uint32_t)j | ((uint32_t)s << 8) | ((uint32_t)p << 16) | ((uint32_t)min(kRH, H - s * kRH) << 24);
    }

    const int CHW = a.C * HW;
    const T *x = static_cast<const T *>(a.x);
    T *y = static_cast<T *>(a.y);
    uint32_t raw[XP::kRawWords];
    XP::load(raw, x + ((size_t)n_begin * a.C + c) * HW, min(PB, n_end - n_begin), CHW, HW, a.m_hw, PB, tid);

    for (int n0 = n_begin; n0 < n_end; n0 += PB) {
        __syncthreads();  // previous pass done with every region
        // Keep the item descriptors opaque to loop-invariant code motion: addresses
        // derived from them are recomputed each pass instead of being held in
        // registers across all phases.
#pragma unroll
        for (int k = 0; k < kFusedMaxItems; ++k) asm volatile("" : "+v"(cd0[k]), "+v"(cd1[k]));
#pragma unroll
        for (int k = 0; k < kFusedMaxFinal; ++k) asm volatile("" : "+v"(fd[k]));
        int t = tid;
        asm volatile("" : "+v"(t));
        const int live = min(PB, n_end - n0);
        XP::commit(raw, smem, live, HW, a.m_hw, W, a.m_w, PB, PF, a.xoff, a.xs, R, t);
        __syncthreads();
        if (n0 + PB < n_end)
            XP::load(raw, x + ((size_t)(n0 + PB) * a.C + c) * HW, min(PB, n_end - n0 - PB), CHW, HW, a.m_hw, PB,
                     t);

        // 2. Haar analysis, unscaled: S_l = butterfly of S_{l-1}'s low-pass band
        for (int l = 0; l < L; ++l) {
            const int Hl = a.hl[l + 1], Wl = a.wl_[l + 1], per = Hl * Wl;
            const uint32_t m_per = a.m_per[l], m_wl = a.m_wl[l];
            const int s_off = l == 0 ? a.xoff : a.yb[l - 1];
            const int s_str = l == 0 ? a.xs : a.sy[l - 1];
            const int d_off = a.yb[l], d_str = a.sy[l], bsl = a.bs[l];
            for (int q = t; q < PB * per; q += nthr) {
                const int p = fdiv(q, m_per), rem = q - p * per, i = fdiv(rem, m_wl), j = rem - i * Wl;
                const float *sp = smem + p * PF + s_off + (2 * i + R) * s_str + 2 * j + R;
                const float x00 = sp[0], x01 = sp[1], x10 = sp[s_str], x11 = sp[s_str + 1];
                const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
                float *dp = smem + p * PF + d_off + (i + R) * d_str + j + R;
                dp[0] = s0 + s1;
                dp[bsl] = s0 - s1;
                dp[2 * bsl] = d0 + d1;
                dp[3 * bsl] = d0 - d1;
            }
            __syncthreads();
        }

        // 3. k x k conv of every (level, band) item; one item at a time so that only
        //    one item's weights are live
        float z[kFusedMaxItems][kRH];
#pragma unroll
        for (int k = 0; k < kFusedMaxItems; ++k) {
#pragma unroll
            for (int i = 0; i < kRH; ++i) z[k][i] = 0.f;
            if ((cd0[k] >> 24) == 0) continue;
            float w[KK];
            const float *wp = smem + cd1[k];
#pragma unroll
            for (int tp = 0; tp < KK; ++tp) w[tp] = wp[tp];
            conv_strip_dyn<K>(smem + (cd0[k] & 0xffffu), (cd0[k] >> 16) & 0xffu, w, z[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // 4. filtered coefficients replace their band (centre rows only)
#pragma unroll
        for (int k = 0; k < kFusedMaxItems; ++k) {
            const int str = (cd0[k] >> 16) & 0xffu, rows = cd0[k] >> 24;
            float *dst = smem + (cd0[k] & 0xffffu) + R * str + R;
#pragma unroll
            for (int i = 0; i < kRH; ++i)
                if (i < rows) dst[i * str] = z[k][i];
        }
        __syncthreads();
        // 5. sign patterns of every block, in place: slot 2 ry + rx
        for (int l = 0; l < L; ++l) {
            const int Hl = a.hl[l + 1], Wl = a.wl_[l + 1], per = Hl * Wl, bsl = a.bs[l];
            const uint32_t m_per = a.m_per[l], m_wl = a.m_wl[l];
            const int d_off = a.yb[l], d_str = a.sy[l];
            for (int q = t; q < PB * per; q += nthr) {
                const int p = fdiv(q, m_per), rem = q - p * per, i = fdiv(rem, m_wl), j = rem - i * Wl;
                float *zp = smem + p * PF + d_off + (i + R) * d_str + j + R;
                const float LL = zp[0], LH = zp[bsl], HL = zp[2 * bsl], HH = zp[3 * bsl];
                zp[0] = (LL + LH) + (HL + HH);
                zp[bsl] = (LL + LH) - (HL + HH);
                zp[2 * bsl] = (LL - LH) + (HL - HH);
                zp[3 * bsl] = (LL - LH) - (HL - HH);
            }
        }
        __syncthreads();
        // 6. base conv + bias + closed-form synthesis, one store
        float w0[KK];
        const float sc0 = a.s0[c];
#pragma unroll
        for (int i = 0; i < KK; ++i) {
            const int u = i / K, v = i - u * K;
            w0[i] = uniform(sc0 * a.w0[(size_t)c * KK + (a.rotate ? (K - 1 - u) * K + (K - 1 - v) : i)]);
        }
        const float bias = a.b0 ? uniform(sc0 * a.b0[c]) : 0.f;
        T *ybase = y + ((size_t)n0 * a.C + c) * HW;
#pragma unroll
        for (int k = 0; k < kFusedMaxFinal; ++k) {
            const int rows = fd[k] >> 24, p = (fd[k] >> 16) & 0xffu;
            if (rows == 0 || p >= live) continue;
            const int s = (fd[k] >> 8) & 0xffu, j = fd[k] & 0xffu;
            float acc[kRH];
#pragma unroll
            for (int i = 0; i < kRH; ++i) acc[i] = bias;
            conv_strip<K>(smem + p * PF + a.xoff + (s * kRH) * a.xs + j, a.xs, w0, acc);
            // Level l+1 adds slot 2 ry + rx of the block at (y >> (l+1), x >> (l+1)),
            // ry = bit l of y = 8s + i, rx = bit l of x = j.  For l <= 2, ry and the
            // block row offset from 8s depend on i only; for l >= 3 they depend on s.
#pragma unroll
            for (int l = 0; l < kMaxLevels; ++l) {
                if (l >= L) break;
                const int sy = a.sy[l], bs2 = 2 * a.bs[l];
                const float *zb = smem + p * PF + a.yb[l] + ((j >> l) & 1) * a.bs[l] + (j >> (l + 1)) + R;
                if (l <= 2) {
                    const float *zr = zb + ((s << (2 - l)) + R) * sy;
#pragma unroll
                    for (int i = 0; i < kRH; ++i) acc[i] += zr[((i >> l) & 1) * bs2 + (i >> (l + 1)) * sy];
                } else {
                    const float v = zb[((s >> (l - 3)) & 1) * bs2 + ((s >> (l - 2)) + R) * sy];
#pragma unroll
                    for (int i = 0; i < kRH; ++i) acc[i] += v;
                }
            }
            const int yoff = p * CHW + (s * kRH) * W + j;
            if constexpr (kHalf<T>) {
#pragma unroll
                for (int i = 0; i < kRH; i += 2) {
                    const uint32_t pk = Act<T>::pack(acc[i], acc[i + 1]);
                    if (i < rows) reinterpret_cast<uint16_t *>(ybase)[yoff + i * W] = (uint16_t)pk;
                    if (i + 1 < rows) reinterpret_cast<uint16_t *>(ybase)[yoff + (i + 1) * W] = (uint16_t)(pk >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kRH; ++i)
                    if (i < rows) ybase[yoff + i * W] = acc[i];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int K, typename T, int VE>
__global__ __launch_bounds__(256, (K <= 5 ? 4 : 2)) void fused_fwd_kernel(FusedArgs a) {
    fused_fwd_body<K, T, VE>(a);
}

}  // namespace wtc
