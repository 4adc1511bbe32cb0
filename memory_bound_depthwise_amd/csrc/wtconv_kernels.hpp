// Device code of the WTConv layer for gfx950 (CDNA4, wave64).
//
// The layer is the wavelet convolution of "Fast and Memory-Efficient Wavelet
// Convolutions via I/O-Aware Reformulation" (§2.1 Algorithm 1), evaluated in the
// I/O-aware form of its §4:
//   * the Haar butterfly (Eq. 5) is recomputed on chip from an LDS-staged tile of
//     the level's carrier; the subbands never reach HBM (§4.1);
//   * the learned scales, the analysis 1/2 and the synthesis weight 2^-l are folded
//     into the k x k weights when a workgroup loads them (Eq. 8; powers of two are
//     exact, so this changes no rounding);
//   * synthesis of all levels is one closed-form pass indexed by the bits of the
//     output coordinate (Proposition 2, Eq. 7).
//
// Storage of the level coefficients.  Eq. 7 adds, for level l, the sign-selected
// combination c_LL + s_y c_LH + s_x c_HL + s_y s_x c_HH of the coefficients at
// (y >> l, x >> l), where s_y is set by bit l-1 of y.  The level kernel evaluates
// the four sign patterns of each coefficient block once (the one-step synthesis of
// Appendix A, Eq. 12/13) and stores them as a 2 x 2 block of a plane twice the
// coefficient grid, Q(l)[2i + ry][2j + rx].  The closed-form pass then reads level
// l at (y >> (l-1), x >> (l-1)): bit l-1 of the coordinate, which Eq. 7 turns into a
// sign, becomes the low address bit.  Q(l) holds as many values as Z(l) (four per
// block), and level 1 is read with unit stride, aligned with the output row.
//
// Compute layout (all convolution-shaped kernels).  A lane owns one column of the
// output tile and a strip of RH = 8 consecutive rows; consecutive lanes own
// consecutive columns.  For each horizontal tap v the lane reads its 8 + K - 1
// column values from LDS (consecutive lanes read consecutive words: no bank
// conflicts) and applies the K vertical taps from registers, so one LDS read feeds
// 8K/(8+K-1) FMAs.  The folded k x k weights of a channel (and band) are the same
// for a whole wavefront and are moved to scalar registers with readfirstlane: each
// multiply-accumulate is one v_fmac_f32 with a scalar operand.
//
// All arithmetic is float32; activations are float32 or bfloat16 in memory.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wtconv.h"

namespace wtc {

constexpr int kMaxLevels = WTCONV_MAX_LEVELS;
constexpr int kWave = 64;
constexpr int kRH = 8;  // rows per lane strip

// ---------------------------------------------------------------------------
// Activation storage
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float act_load(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float act_load(const uint16_t *p, size_t i) { return bf16_bits_to_f32(p[i]); }

// float32 -> bfloat16, round to nearest, ties to even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}
typedef float wtc_float2 __attribute__((ext_vector_type(2)));
typedef __bf16 wtc_bf16x2 __attribute__((ext_vector_type(2)));
// Two values packed low, high in one conversion.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    const wtc_float2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, wtc_bf16x2));
}

// Exact quotient n / d for n, d < 2^16, with m = ceil(2^32 / d) computed on the host
// (m = 0 encodes d = 1): the error term n (m d - 2^32) / (d 2^32) stays below 1/d.
__device__ __forceinline__ int fdiv(int n, uint32_t m) { return m ? (int)__umulhi((uint32_t)n, m) : n; }

__device__ __forceinline__ void act_store(float *p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void act_store(uint16_t *p, size_t i, float v) { p[i] = (uint16_t)f32_to_bf16(v); }

// Two adjacent elements (element index i even, so the pair is aligned).
__device__ __forceinline__ void act_store2(float *p, size_t i, float a, float b) {
    *reinterpret_cast<float2 *>(p + i) = make_float2(a, b);
}
__device__ __forceinline__ void act_store2(uint16_t *p, size_t i, float a, float b) {
    *reinterpret_cast<uint32_t *>(p + i) = f32x2_to_bf16x2(a, b);
}
__device__ __forceinline__ void act_load2(const float *p, size_t i, float &a, float &b) {
    const float2 v = *reinterpret_cast<const float2 *>(p + i);
    a = v.x;
    b = v.y;
}
__device__ __forceinline__ void act_load2(const uint16_t *p, size_t i, float &a, float &b) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(p + i);
    a = bf16_bits_to_f32(v & 0xffffu);
    b = bf16_bits_to_f32(v >> 16);
}

// VW consecutive elements starting at element i (i a multiple of VW, base aligned).
template <int VW>
__device__ __forceinline__ void act_loadv(const float *p, size_t i, float *out) {
    if constexpr (VW == 1) {
        out[0] = p[i];
    } else if constexpr (VW == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(p + i);
        out[0] = v.x;
        out[1] = v.y;
    } else {
        static_assert(VW == 4, "float vectors are at most 16 bytes");
        const float4 v = *reinterpret_cast<const float4 *>(p + i);
        out[0] = v.x;
        out[1] = v.y;
        out[2] = v.z;
        out[3] = v.w;
    }
}
template <int VW>
__device__ __forceinline__ void act_loadv(const uint16_t *p, size_t i, float *out) {
    if constexpr (VW == 1) {
        out[0] = bf16_bits_to_f32(p[i]);
    } else if constexpr (VW == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(p + i);
        out[0] = bf16_bits_to_f32(v & 0xffffu);
        out[1] = bf16_bits_to_f32(v >> 16);
    } else if constexpr (VW == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p + i);
        out[0] = bf16_bits_to_f32(v.x & 0xffffu);
        out[1] = bf16_bits_to_f32(v.x >> 16);
        out[2] = bf16_bits_to_f32(v.y & 0xffffu);
        out[3] = bf16_bits_to_f32(v.y >> 16);
    } else {
        static_assert(VW == 8, "bf16 vectors are at most 16 bytes");
        const uint4 v = *reinterpret_cast<const uint4 *>(p + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = bf16_bits_to_f32(w[k] & 0xffffu);
            out[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
        }
    }
}

__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ---------------------------------------------------------------------------
// Wavefront reduction with DPP: quad butterflies, half-row and row mirrors leave
// every lane with the sum of its 16-lane row; the four row sums are then read
// and added in a fixed order, so the result is the same on every run.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);  // row_half_mirror
    v += dpp_move<0x140>(v);  // row_mirror
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// ---------------------------------------------------------------------------
// Launch arguments
// ---------------------------------------------------------------------------

// Tiling of the output grid of a kernel.  A tile is TY rows x TX columns, computed
// as SP strips of kRH rows; a workgroup pass stacks PB planes of one channel in LDS
// and a workgroup walks NB planes in all.  VW is the element count of the vector
// loads that stage pixel rows (rows and tile origins are multiples of it).
struct Tiling {
    int TY, TX, SP;
    int tiles_x, tiles;
    int PB, NB, nblk;
    int VW;
};

struct LevelArgs {
    const void *in;   // carrier of the level above, [n][C][Hi][Wi]
    void *qout;       // [n][C][2 Ho][2 Wo]: four synthesised values per coefficient block
    void *cout;       // carrier of this level, [n][C][Ho][Wo] (NULL at the deepest level)
    const float *wl;  // this level's kernels, [C][4][K][K]
    const float *sl;  // this level's scales, [C][4]
    int n, C, Hi, Wi, Ho, Wo;
    float wscale;     // 2^-(l+1): synthesis weight 2^-l times the analysis 1/2
    int rotate;       // 1: kernels turned by 180 degrees (input gradient)
    int pairs;        // 1: Wi even and the input aligned for two-element loads
    Tiling t;
};

struct SynthArgs {
    const void *x;    // [n][C][H][W]
    void *y;          // [n][C][H][W]
    const float *w0, *b0, *s0;
    const void *q[kMaxLevels];  // Q of level l+1, [n][C][Hq][Wq]
    int wq[kMaxLevels];         // row length of Q
    long long qplane[kMaxLevels];
    int n, C, H, W, L;
    int rotate;
    Tiling t;
};

struct DwLevelArgs {
    const void *xin, *gin;  // carriers of x and dy at the level above
    void *xc, *gc;          // carriers of this level (NULL at the deepest level)
    float *partial;         // [C][G][4 K K], G = nblk * tiles
    int n, C, Hi, Wi, Ho, Wo;
    int pairs;
    Tiling t;
};

struct DwBaseArgs {
    const void *x, *dy;
    float *partial;  // [C][G][K K + 1]
    int n, C, H, W;
    Tiling t;
};

struct FinalizeArgs {
    const float *partial;
    long long off[kMaxLevels + 1];  // region offsets: 0 = base, l = level l
    int G[kMaxLevels + 1];          // partial rows per channel in each region
    int C, L;
    const float *w0, *b0, *s0, *wl, *sl;
    float *dw0, *db0, *ds0, *dwl, *dsl;
};

// Decompose the flat workgroup index as (tile, channel, plane block).
struct BlockPos {
    int tile, c, nb, ty0, tx0;
};

__device__ __forceinline__ BlockPos block_pos(const Tiling &t, int C) {
    int bid = blockIdx.x;
    BlockPos b;
    b.tile = bid % t.tiles;
    bid /= t.tiles;
    b.c = bid % C;
    b.nb = bid / C;
    b.ty0 = (b.tile / t.tiles_x) * t.TY;
    b.tx0 = (b.tile % t.tiles_x) * t.TX;
    return b;
}

// Staged width of a pixel tile with an R-column halo, starting at the multiple of
// VW at or left of tx0 - R.
__host__ __device__ __forceinline__ int stage_col0(int tx0, int R, int VW) {
    const int c = tx0 - R;
    return c >= 0 ? c / VW * VW : -((-c + VW - 1) / VW) * VW;
}
__host__ __device__ __forceinline__ int stage_width(int TX, int R, int VW) {
    // worst case over tile origins: VW - 1 extra on the left, rounded up on the right
    return ((TX + 2 * R + VW - 1 + VW - 1) / VW) * VW;
}

// ---------------------------------------------------------------------------
// Haar staging shared by the level kernels: every coefficient block in rows
// [r0, r0 + rows) x cols [c0, c0 + cols) of the coefficient grid is loaded once
// and transformed once (Eq. 5 without its 1/2, which lives in the weights).
// Blocks outside the grid, at or below row vr1 (<= Ho), or outside the plane range
// are zero: the conv's zero padding.  The raw low-pass value of blocks inside [cr0, cr1) x [cc0, cc1) is
// written to the next carrier.
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ void haar_stage(const T *__restrict__ in, T *__restrict__ carrier, float *bands,
                                           int bandsz, int stride, int PB, int rows, int cols, int r0, int c0,
                                           int n0, int n_end, int c, int C, int Hi, int Wi, int Ho, int Wo,
                                           int vr1, int cr0, int cr1, int cc0, int cc1, int pairs) {
    const int per_plane = rows * cols;
    const size_t in_plane = (size_t)Hi * Wi, out_plane = (size_t)Ho * Wo;
    for (int idx = threadIdx.x; idx < PB * per_plane; idx += blockDim.x) {
        const int p = idx / per_plane, rem = idx - p * per_plane;
        const int ci = rem / cols, cj = rem - ci * cols;
        const int nn = n0 + p, gi = r0 + ci, gj = c0 + cj;
        float x00 = 0.f, x01 = 0.f, x10 = 0.f, x11 = 0.f;
        const bool inside = nn < n_end && gi >= 0 && gi < vr1 && gj >= 0 && gj < Wo;
        if (inside) {
            const T *src = in + ((size_t)nn * C + c) * in_plane;
            const size_t o0 = (size_t)(2 * gi) * Wi + 2 * gj;
            const bool r1 = 2 * gi + 1 < Hi;
            if (pairs) {
                act_load2(src, o0, x00, x01);
                if (r1) act_load2(src, o0 + Wi, x10, x11);
            } else {
                const bool c1 = 2 * gj + 1 < Wi;
                x00 = act_load(src, o0);
                if (c1) x01 = act_load(src, o0 + 1);
                if (r1) {
                    x10 = act_load(src, o0 + Wi);
                    if (c1) x11 = act_load(src, o0 + Wi + 1);
                }
            }
        }
        const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
        float *dst = bands + (size_t)p * 4 * bandsz + ci * stride + cj;
        dst[0] = s0 + s1;           // 2 LL
        dst[bandsz] = s0 - s1;      // 2 LH
        dst[2 * bandsz] = d0 + d1;  // 2 HL
        dst[3 * bandsz] = d0 - d1;  // 2 HH
        if (carrier && inside && gi >= cr0 && gi < cr1 && gj >= cc0 && gj < cc1)
            act_store(carrier, ((size_t)nn * C + c) * out_plane + (size_t)gi * Wo + gj, 0.5f * (s0 + s1));
    }
}

// Stage a pixel tile: rows [r0, r0 + rows) x cols [c0, c0 + width) of PB planes,
// zero outside the plane, at or below row row_hi (<= H), and, when mask_lo <
// mask_hi, outside those columns;
// converted to float32 in LDS with row stride `width`.  c0 and width are multiples
// of VW and W is a multiple of VW, so each vector is wholly inside or outside.
template <int VW, typename T>
__device__ __forceinline__ void pixel_stage_v(const T *__restrict__ src, float *dst, int PB, int rows, int width,
                                              int r0, int c0, int n0, int n_end, int c, int C, int H, int W,
                                              int row_hi, int mask_lo, int mask_hi) {
    const int vpr = width / VW, per_plane = rows * vpr;
    const size_t plane = (size_t)H * W;
    for (int idx = threadIdx.x; idx < PB * per_plane; idx += blockDim.x) {
        const int p = idx / per_plane, rem = idx - p * per_plane;
        const int ri = rem / vpr, vc = rem - ri * vpr;
        const int nn = n0 + p, gi = r0 + ri, gc = c0 + vc * VW;
        float v[VW];
#pragma unroll
        for (int e = 0; e < VW; ++e) v[e] = 0.f;
        if (nn < n_end && gi >= 0 && gi < row_hi && gc >= 0 && gc < W)
            act_loadv<VW>(src + ((size_t)nn * C + c) * plane, (size_t)gi * W + gc, v);
        float *d = dst + (size_t)p * rows * width + ri * width + vc * VW;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            const int col = gc + e;
            d[e] = (mask_lo < mask_hi && (col < mask_lo || col >= mask_hi)) ? 0.f : v[e];
        }
    }
}

template <typename T>
__device__ __forceinline__ void pixel_stage(const T *__restrict__ src, float *dst, int VW, int PB, int rows,
                                            int width, int r0, int c0, int n0, int n_end, int c, int C, int H,
                                            int W, int row_hi, int mask_lo, int mask_hi) {
#define WTC_STAGE(V) pixel_stage_v<V>(src, dst, PB, rows, width, r0, c0, n0, n_end, c, C, H, W, row_hi, mask_lo, mask_hi)
    switch (VW) {
        case 8:
            if constexpr (sizeof(T) == 2) {
                WTC_STAGE(8);
                return;
            }
            [[fallthrough]];
        case 4: WTC_STAGE(4); return;
        case 2: WTC_STAGE(2); return;
        default: WTC_STAGE(1); return;
    }
#undef WTC_STAGE
}

// One lane's strip of an K x K cross-correlation: out[i] += sum_{u,v} w[u][v] *
// src[(i + u) * stride + v] for i < kRH, w in scalar registers.
template <int K>
__device__ __forceinline__ void conv_strip(const float *src, int stride, const float *w, float *acc) {
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

// One lane's strip of a K x K weight gradient: acc[u][v] += sum_i g[i] *
// src[(i + u) * stride + v].
template <int K>
__device__ __forceinline__ void corr_strip(const float *src, int stride, const float *g, float *acc) {
#pragma unroll
    for (int v = 0; v < K; ++v) {
        float col[kRH + K - 1];
#pragma unroll
        for (int i = 0; i < kRH + K - 1; ++i) col[i] = src[i * stride + v];
#pragma unroll
        for (int u = 0; u < K; ++u)
#pragma unroll
            for (int i = 0; i < kRH; ++i) acc[u * K + v] = fmaf(g[i], col[i + u], acc[u * K + v]);
    }
}

// ---------------------------------------------------------------------------
// Level kernel: Haar analysis + 4-band depthwise conv (+ carrier), §4.1 / Fig. 1b.
// Output grid: the level's coefficient grid (Ho x Wo).  Wavefront b filters band b;
// a combine pass writes the four sign patterns of each block.  256 threads.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void level_fwd_kernel(LevelArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C);
    const int c = bp.c;
    const int HY = t.SP * kRH + K - 1, HXP = t.TX + K - 1, bandsz = HY * HXP;
    float *band = smem;                              // [PB][4][HY][HXP]
    float *zbuf = smem + (size_t)t.PB * 4 * bandsz;  // [4][PB][TY][TX]
    const int n0 = bp.nb * t.PB;

    haar_stage<T>(static_cast<const T *>(a.in), static_cast<T *>(a.cout), band, bandsz, HXP, t.PB, HY, HXP,
                  bp.ty0 - R, bp.tx0 - R, n0, a.n, c, a.C, a.Hi, a.Wi, a.Ho, a.Wo, a.Ho, bp.ty0, bp.ty0 + t.TY,
                  bp.tx0, bp.tx0 + t.TX, a.pairs);

    const int b = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // this wavefront's band
    const int lane = threadIdx.x & (kWave - 1);
    float w[KK];
    {
        const float sc = a.sl[c * 4 + b] * a.wscale;
        const float *wb = a.wl + (size_t)(c * 4 + b) * KK;
#pragma unroll
        for (int i = 0; i < KK; ++i) {
            const int u = i / K, v = i - u * K;
            w[i] = uniform(sc * wb[a.rotate ? (K - 1 - u) * K + (K - 1 - v) : i]);
        }
    }
    __syncthreads();

    const int per_plane = t.SP * t.TX;
    for (int it = lane; it < t.PB * per_plane; it += kWave) {
        const int p = it / per_plane, rem = it - p * per_plane;
        const int s = rem / t.TX, j = rem - s * t.TX;
        float acc[kRH];
#pragma unroll
        for (int i = 0; i < kRH; ++i) acc[i] = 0.f;
        conv_strip<K>(band + (size_t)(p * 4 + b) * bandsz + (s * kRH) * HXP + j, HXP, w, acc);
        float *z = zbuf + ((size_t)(b * t.PB + p) * t.TY + s * kRH) * t.TX + j;
#pragma unroll
        for (int i = 0; i < kRH; ++i)
            if (s * kRH + i < t.TY) z[i * t.TX] = acc[i];
    }
    __syncthreads();

    // Combine: q[ry][rx] = LL + (-1)^ry LH + (-1)^rx HL + (-1)^(ry+rx) HH (Eq. 12/13).
    T *q = static_cast<T *>(a.qout);
    const int Wq = 2 * a.Wo;
    const size_t q_plane = (size_t)4 * a.Ho * a.Wo, zb = (size_t)t.PB * t.TY * t.TX;
    const int per_tile = t.TY * t.TX;
    for (int idx = threadIdx.x; idx < t.PB * per_tile; idx += blockDim.x) {
        const int p = idx / per_tile, rem = idx - p * per_tile;
        const int r = rem / t.TX, j = rem - r * t.TX;
        const int nn = n0 + p, gi = bp.ty0 + r, gj = bp.tx0 + j;
        if (nn >= a.n || gi >= a.Ho || gj >= a.Wo) continue;
        const float *z = zbuf + (size_t)p * per_tile + rem;
        const float LL = z[0], LH = z[zb], HL = z[2 * zb], HH = z[3 * zb];
        T *qp = q + ((size_t)nn * a.C + c) * q_plane + (size_t)(2 * gi) * Wq + 2 * gj;
        act_store2(qp, 0, (LL + LH) + (HL + HH), (LL + LH) - (HL + HH));
        act_store2(qp, Wq, (LL - LH) + (HL - HH), (LL - LH) - (HL - HH));
    }
}

// ---------------------------------------------------------------------------
// Closed-form synthesis + base conv + bias, one store (§4.2 Prop. 2, §4.3, §4.4).
// Output grid: pixels.  256 threads.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void synth_kernel(SynthArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C);
    const int c = bp.c;
    const int HY = t.SP * kRH + K - 1, HXW = stage_width(t.TX, R, t.VW), plsz = HY * HXW;
    const int ca = stage_col0(bp.tx0, R, t.VW), off = bp.tx0 - R - ca;
    const int n0 = bp.nb * t.PB;

    pixel_stage<T>(static_cast<const T *>(a.x), smem, t.VW, t.PB, HY, HXW, bp.ty0 - R, ca, n0, a.n, c, a.C, a.H,
                   a.W, a.H, 0, 0);

    float w[KK];
    const float sc = a.s0[c];
#pragma unroll
    for (int i = 0; i < KK; ++i) {
        const int u = i / K, v = i - u * K;
        w[i] = uniform(sc * a.w0[(size_t)c * KK + (a.rotate ? (K - 1 - u) * K + (K - 1 - v) : i)]);
    }
    const float bias = a.b0 ? uniform(sc * a.b0[c]) : 0.f;
    __syncthreads();

    T *y = static_cast<T *>(a.y);
    const size_t plane = (size_t)a.H * a.W;
    const int per_plane = t.SP * t.TX;
    for (int it = threadIdx.x; it < t.PB * per_plane; it += blockDim.x) {
        const int p = it / per_plane, rem = it - p * per_plane;
        const int s = rem / t.TX, j = rem - s * t.TX;
        const int nn = n0 + p, gx = bp.tx0 + j, gy0 = bp.ty0 + s * kRH;
        if (nn >= a.n || gx >= a.W) continue;
        const int rows = min(kRH, min(a.H, bp.ty0 + t.TY) - gy0);  // rows of this strip in the tile
        const size_t pidx = (size_t)nn * a.C + c;
        // Eq. 7: level l contributes Q(l)[y >> (l-1)][x >> (l-1)]
        float acc[kRH];
#pragma unroll
        for (int i = 0; i < kRH; ++i) acc[i] = bias;
        for (int l = 0; l < a.L; ++l) {
            const T *ql = static_cast<const T *>(a.q[l]) + pidx * (size_t)a.qplane[l] + (gx >> l);
#pragma unroll
            for (int i = 0; i < kRH; ++i)
                if (i < rows) acc[i] += act_load(ql, (size_t)((gy0 + i) >> l) * a.wq[l]);
        }
        conv_strip<K>(smem + (size_t)p * plsz + (s * kRH) * HXW + j + off, HXW, w, acc);
        T *yp = y + pidx * plane + (size_t)gy0 * a.W + gx;
#pragma unroll
        for (int i = 0; i < kRH; ++i)
            if (i < rows) act_store(yp, (size_t)i * a.W, acc[i]);
    }
}

// ---------------------------------------------------------------------------
// Weight gradient, level l: the folded-weight gradient of band b is
//   dW~[b][u][v] = sum_{n,i,j} G[b][i][j] * Y[b][i+u-R][j+v-R]
// with Y the level-l analysis of x and G the level-l analysis of dy (the gradient
// at Z(l), Eq. 1: backward through synthesis is analysis).  Both analyses are
// recomputed from the carriers in LDS; the carriers of the next level are written
// on the way.  Wavefront b owns band b; per-lane tap accumulators are reduced with
// DPP into one partial row per workgroup.  256 threads.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void dw_level_kernel(DwLevelArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C);
    const int c = bp.c;
    const int lane = threadIdx.x & (kWave - 1);
    const int b = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int HY = t.SP * kRH + K - 1, HXP = t.TX + K - 1, ysz = HY * HXP;
    const int GY = t.SP * kRH, gsz = GY * t.TX;
    float *ys = smem;                          // [PB][4][HY][HXP]
    float *gs = ys + (size_t)t.PB * 4 * ysz;   // [PB][4][GY][TX]
    float *red = gs + (size_t)t.PB * 4 * gsz;  // [4][KK]

    const T *xin = static_cast<const T *>(a.xin);
    const T *gin = static_cast<const T *>(a.gin);
    const int n_begin = bp.nb * t.NB;
    const int n_end = min(a.n, n_begin + t.NB);

    float acc[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) acc[i] = 0.f;

    const int per_plane = t.SP * t.TX;
    for (int n0 = n_begin; n0 < n_end; n0 += t.PB) {
        __syncthreads();
        haar_stage<T>(xin, static_cast<T *>(a.xc), ys, ysz, HXP, t.PB, HY, HXP, bp.ty0 - R, bp.tx0 - R, n0, n_end,
                      c, a.C, a.Hi, a.Wi, a.Ho, a.Wo, a.Ho, bp.ty0, bp.ty0 + t.TY, bp.tx0, bp.tx0 + t.TX, a.pairs);
        // G only on the tile itself; rows past the tile are zero (no double count)
        haar_stage<T>(gin, static_cast<T *>(a.gc), gs, gsz, t.TX, t.PB, GY, t.TX, bp.ty0, bp.tx0, n0, n_end, c,
                      a.C, a.Hi, a.Wi, a.Ho, a.Wo, min(a.Ho, bp.ty0 + t.TY), bp.ty0, bp.ty0 + t.TY, bp.tx0,
                      bp.tx0 + t.TX, a.pairs);
        __syncthreads();
        for (int it = lane; it < t.PB * per_plane; it += kWave) {
            const int p = it / per_plane, rem = it - p * per_plane;
            const int s = rem / t.TX, j = rem - s * t.TX;
            const float *gp = gs + (size_t)(p * 4 + b) * gsz + (s * kRH) * t.TX + j;
            float g[kRH];
#pragma unroll
            for (int i = 0; i < kRH; ++i) g[i] = gp[i * t.TX];
            corr_strip<K>(ys + (size_t)(p * 4 + b) * ysz + (s * kRH) * HXP + j, HXP, g, acc);
        }
    }

#pragma unroll
    for (int i = 0; i < KK; ++i) {
        const float v = wave_sum(acc[i]);
        if (lane == 0) red[b * KK + i] = v;
    }
    __syncthreads();
    const int G = t.nblk * t.tiles, g = bp.nb * t.tiles + bp.tile;
    float *out = a.partial + ((size_t)c * G + g) * 4 * KK;
    for (int i = threadIdx.x; i < 4 * KK; i += blockDim.x) out[i] = 0.25f * red[i];  // the two analysis halves
}

// ---------------------------------------------------------------------------
// Weight gradient, base path: dW~0[u][v] = sum dy[y][x] * x[y+u-R][x+v-R] and
// db~ = sum dy; the same two-stage reduction.  256 threads.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void dw_base_kernel(DwBaseArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C);
    const int c = bp.c;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
    const int HY = t.SP * kRH + K - 1, HXW = stage_width(t.TX, R, t.VW), xsz = HY * HXW;
    const int ca = stage_col0(bp.tx0, R, t.VW), off = bp.tx0 - R - ca;
    const int GY = t.SP * kRH, GW = stage_width(t.TX, 0, t.VW), gsz = GY * GW;
    const int ga = stage_col0(bp.tx0, 0, t.VW), goff = bp.tx0 - ga;
    float *xs = smem;                       // [PB][HY][HXW]
    float *gs = xs + (size_t)t.PB * xsz;    // [PB][GY][GW]
    float *red = gs + (size_t)t.PB * gsz;   // [nwaves][KK + 1]

    const T *x = static_cast<const T *>(a.x);
    const T *dy = static_cast<const T *>(a.dy);
    const int n_begin = bp.nb * t.NB;
    const int n_end = min(a.n, n_begin + t.NB);
    const int row_end = min(a.H, bp.ty0 + t.TY);

    float acc[KK + 1];
#pragma unroll
    for (int i = 0; i <= KK; ++i) acc[i] = 0.f;

    const int per_plane = t.SP * t.TX;
    for (int n0 = n_begin; n0 < n_end; n0 += t.PB) {
        __syncthreads();
        pixel_stage<T>(x, xs, t.VW, t.PB, HY, HXW, bp.ty0 - R, ca, n0, n_end, c, a.C, a.H, a.W, a.H, 0, 0);
        // dy only on the tile: rows and columns past the tile are zero
        pixel_stage<T>(dy, gs, t.VW, t.PB, GY, GW, bp.ty0, ga, n0, n_end, c, a.C, a.H, a.W, row_end, bp.tx0,
                       bp.tx0 + t.TX);
        __syncthreads();
        for (int it = threadIdx.x; it < t.PB * per_plane; it += blockDim.x) {
            const int p = it / per_plane, rem = it - p * per_plane;
            const int s = rem / t.TX, j = rem - s * t.TX;
            const float *gp = gs + (size_t)p * gsz + (s * kRH) * GW + j + goff;
            float g[kRH];
#pragma unroll
            for (int i = 0; i < kRH; ++i) {
                g[i] = gp[i * GW];
                acc[KK] += g[i];
            }
            corr_strip<K>(xs + (size_t)p * xsz + (s * kRH) * HXW + j + off, HXW, g, acc);
        }
    }

#pragma unroll
    for (int i = 0; i <= KK; ++i) {
        const float v = wave_sum(acc[i]);
        if (lane == 0) red[wave * (KK + 1) + i] = v;
    }
    __syncthreads();
    const int G = t.nblk * t.tiles, g = bp.nb * t.tiles + bp.tile;
    float *out = a.partial + ((size_t)c * G + g) * (KK + 1);
    for (int i = threadIdx.x; i <= KK; i += blockDim.x) {
        float s = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) s += red[wv * (KK + 1) + i];
        out[i] = s;
    }
}

// ---------------------------------------------------------------------------
// Finalize: fixed-order sum of the workgroup partials, then Eq. 9.
// Grid: (C, L + 1); blockIdx.y = 0 is the base path, l >= 1 is level l.
// ---------------------------------------------------------------------------

template <int K>
__global__ __launch_bounds__(128) void dw_finalize_kernel(FinalizeArgs a) {
    constexpr int KK = K * K;
    __shared__ float sum[4 * KK];
    const int c = blockIdx.x, region = blockIdx.y, tid = threadIdx.x;
    const int slots = region == 0 ? KK + 1 : 4 * KK;
    const int G = a.G[region];
    const float *part = a.partial + a.off[region] + (size_t)c * G * slots;
    for (int i = tid; i < slots; i += blockDim.x) {
        float s = 0.f;
        for (int g = 0; g < G; ++g) s += part[(size_t)g * slots + i];
        sum[i] = s;
    }
    __syncthreads();
    if (region == 0) {
        const float sc = a.s0[c];
        for (int i = tid; i < KK; i += blockDim.x) a.dw0[(size_t)c * KK + i] = sc * sum[i];
        if (tid == 0) {
            if (a.db0) a.db0[c] = sc * sum[KK];
            float ds = 0.f;
            for (int i = 0; i < KK; ++i) ds = fmaf(sum[i], a.w0[(size_t)c * KK + i], ds);
            if (a.b0) ds = fmaf(sum[KK], a.b0[c], ds);
            a.ds0[c] = ds;
        }
    } else {
        const size_t pc = (size_t)(region - 1) * a.C + c;
        for (int i = tid; i < 4 * KK; i += blockDim.x)
            a.dwl[pc * 4 * KK + i] = a.sl[pc * 4 + i / KK] * sum[i];
        if (tid < 4) {
            float ds = 0.f;
            for (int i = 0; i < KK; ++i) ds = fmaf(sum[tid * KK + i], a.wl[(pc * 4 + tid) * KK + i], ds);
            a.dsl[pc * 4 + tid] = ds;
        }
    }
}

}  // namespace wtc
