// Device code of the WTConv layer for gfx950 (CDNA4, wave64).
//
// The layer is the wavelet convolution of "Fast and Memory-Efficient Wavelet
// Convolutions via I/O-Aware Reformulation" (§2.1 Algorithm 1), evaluated in the
// I/O-aware form of its §4:
//   * the Haar butterfly (Eq. 5) is recomputed on chip from an LDS-staged tile of
//     the level's carrier; the subbands never reach HBM (§4.1);
//   * the learned scales, the analysis 1/2 and the synthesis weight 2^-l are folded
//     into the k x k weights when a workgroup loads them (Eq. 8; powers of two are
//     exact, so the folding changes no rounding);
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
// All arithmetic is float32; activations are float32 or bfloat16 in memory.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wtconv.h"

namespace wtc {

constexpr int kMaxLevels = WTCONV_MAX_LEVELS;
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Activation storage
// ---------------------------------------------------------------------------

__device__ __forceinline__ float act_load(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float act_load(const uint16_t *p, size_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

__device__ __forceinline__ void act_store(float *p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void act_store(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }

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

// Tiling of one plane and grouping of planes into a workgroup.  Tiles are TY rows
// by TX columns of the kernel's output grid; a workgroup takes one tile of PB
// planes of one channel at a time (stacked in LDS) and walks NB planes in all.
struct Tiling {
    int TY, TX;     // tile rows / columns
    int SP;         // strips per tile row (strip width is the kernel's S)
    int tiles_x;    // tiles per plane row
    int tiles;      // tiles per plane
    int PB;         // planes stacked per pass
    int NB;         // planes per workgroup (multiple of PB)
    int nblk;       // ceil(n / NB)
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
    Tiling t;
};

struct SynthArgs {
    const void *x;    // [n][C][H][W]
    void *y;          // [n][C][H][W]
    const float *w0, *b0, *s0;
    const void *q[kMaxLevels];  // Q(l) of level l+1, [n][C][Hq][Wq]
    int wq[kMaxLevels];         // row length of Q(l)
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

__device__ __forceinline__ BlockPos block_pos(const Tiling &t, int C, int TYstep, int TXstep) {
    int bid = blockIdx.x;
    BlockPos b;
    b.tile = bid % t.tiles;
    bid /= t.tiles;
    b.c = bid % C;
    b.nb = bid / C;
    b.ty0 = (b.tile / t.tiles_x) * TYstep;
    b.tx0 = (b.tile % t.tiles_x) * TXstep;
    return b;
}

// ---------------------------------------------------------------------------
// Level kernel: Haar analysis + 4-band depthwise conv (+ carrier), §4.1 / Fig. 1b.
// Output grid: the level's coefficient grid (Ho x Wo); strip of S coefficients.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void level_fwd_kernel(LevelArgs a) {
    constexpr int R = (K - 1) / 2, S = 4, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C, t.TY, t.TX);
    const int c = bp.c, tid = threadIdx.x;
    const int HY = t.TY + K - 1, HXP = t.SP * S + K - 1, bandsz = HY * HXP;
    float *wsh = smem;             // [4][K][K] folded weights
    float *band = smem + 4 * KK;   // [PB][4][HY][HXP]

    for (int i = tid; i < 4 * KK; i += blockDim.x) {
        const int b = i / KK, tap = i - b * KK, u = tap / K, v = tap - u * K;
        const int src = a.rotate ? (K - 1 - u) * K + (K - 1 - v) : tap;
        wsh[i] = a.sl[c * 4 + b] * a.wl[(size_t)(c * 4 + b) * KK + src] * a.wscale;
    }

    // Stage: every coefficient block of the tile plus an R-block halo is loaded
    // once and transformed once (Eq. 5, without its 1/2, which lives in the
    // weights).  Blocks outside the coefficient grid are the conv's zero padding.
    const T *in = static_cast<const T *>(a.in);
    const size_t in_plane = (size_t)a.Hi * a.Wi;
    const int per_plane = bandsz;
    for (int idx = tid; idx < t.PB * per_plane; idx += blockDim.x) {
        const int p = idx / per_plane, rem = idx - p * per_plane;
        const int ci = rem / HXP, cj = rem - ci * HXP;
        const int nn = bp.nb * t.PB + p;
        const int gi = bp.ty0 + ci - R, gj = bp.tx0 + cj - R;
        float x00 = 0.f, x01 = 0.f, x10 = 0.f, x11 = 0.f;
        const bool inside = nn < a.n && gi >= 0 && gi < a.Ho && gj >= 0 && gj < a.Wo;
        if (inside) {
            const T *src = in + ((size_t)nn * a.C + c) * in_plane;
            const int r0 = 2 * gi, c0 = 2 * gj;
            const bool c1 = c0 + 1 < a.Wi, r1 = r0 + 1 < a.Hi;
            x00 = act_load(src, (size_t)r0 * a.Wi + c0);
            if (c1) x01 = act_load(src, (size_t)r0 * a.Wi + c0 + 1);
            if (r1) {
                x10 = act_load(src, (size_t)(r0 + 1) * a.Wi + c0);
                if (c1) x11 = act_load(src, (size_t)(r0 + 1) * a.Wi + c0 + 1);
            }
        }
        const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
        float *dst = band + (size_t)p * 4 * bandsz + ci * HXP + cj;
        dst[0] = s0 + s1;           // 2 LL
        dst[bandsz] = s0 - s1;      // 2 LH
        dst[2 * bandsz] = d0 + d1;  // 2 HL
        dst[3 * bandsz] = d0 - d1;  // 2 HH
        if (a.cout && inside && ci >= R && ci < R + t.TY && cj >= R && cj < R + t.TX)
            act_store(static_cast<T *>(a.cout), ((size_t)nn * a.C + c) * a.Ho * a.Wo + (size_t)gi * a.Wo + gj,
                      0.5f * (s0 + s1));
    }
    __syncthreads();

    T *q = static_cast<T *>(a.qout);
    const int Wq = 2 * a.Wo;
    const size_t q_plane = (size_t)4 * a.Ho * a.Wo;
    const int per_tile = t.TY * t.SP;
    for (int it = tid; it < t.PB * per_tile; it += blockDim.x) {
        const int p = it / per_tile, rem = it - p * per_tile;
        const int r = rem / t.SP, j0 = (rem - r * t.SP) * S;
        const int nn = bp.nb * t.PB + p, gi = bp.ty0 + r, gj0 = bp.tx0 + j0;
        if (nn >= a.n || gi >= a.Ho || j0 >= t.TX || gj0 >= a.Wo) continue;
        // q[ry][rx] collects the synthesis of the block at in-block position
        // (ry, rx): band b enters with sign (-1)^(ry*[b is LH or HH] + rx*[b is HL
        // or HH]) (Eq. 12/13).  The band loop stays rolled so that only one band's
        // k x k weights are live at a time.
        float q00[S], q01[S], q10[S], q11[S];
#pragma unroll
        for (int s = 0; s < S; ++s) q00[s] = q01[s] = q10[s] = q11[s] = 0.f;
#pragma unroll 1
        for (int b = 0; b < 4; ++b) {
            float acc[S];
#pragma unroll
            for (int s = 0; s < S; ++s) acc[s] = 0.f;
            const float *src = band + (size_t)p * 4 * bandsz + b * bandsz + r * HXP + j0;
            const float *wb = wsh + b * KK;
#pragma unroll
            for (int u = 0; u < K; ++u) {
                float win[S + K - 1];
#pragma unroll
                for (int e = 0; e < S + K - 1; ++e) win[e] = src[u * HXP + e];
#pragma unroll
                for (int v = 0; v < K; ++v) {
                    const float w = wb[u * K + v];
#pragma unroll
                    for (int s = 0; s < S; ++s) acc[s] = fmaf(w, win[s + v], acc[s]);
                }
            }
            const float sy = (b & 1) ? -1.f : 1.f;  // LH, HH flip the lower row
            const float sx = (b & 2) ? -1.f : 1.f;  // HL, HH flip the right column
#pragma unroll
            for (int s = 0; s < S; ++s) {
                q00[s] += acc[s];
                q01[s] = fmaf(sx, acc[s], q01[s]);
                q10[s] = fmaf(sy, acc[s], q10[s]);
                q11[s] = fmaf(sx * sy, acc[s], q11[s]);
            }
        }
        T *qp = q + ((size_t)nn * a.C + c) * q_plane;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int gj = gj0 + s;
            if (gj >= a.Wo || j0 + s >= t.TX) continue;
            const size_t o = (size_t)(2 * gi) * Wq + 2 * gj;
            act_store(qp, o, q00[s]);
            act_store(qp, o + 1, q01[s]);
            act_store(qp, o + Wq, q10[s]);
            act_store(qp, o + Wq + 1, q11[s]);
        }
    }
}

// ---------------------------------------------------------------------------
// Closed-form synthesis + base conv + bias, one store (§4.2 Prop. 2, §4.3, §4.4).
// Output grid: pixels; strip of S pixels.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void synth_kernel(SynthArgs a) {
    constexpr int R = (K - 1) / 2, S = 8, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C, t.TY, t.TX);
    const int c = bp.c, tid = threadIdx.x;
    const int HY = t.TY + K - 1, HXP = t.SP * S + K - 1, plsz = HY * HXP;
    float *wsh = smem;      // [K][K] folded base weights
    float *xs = smem + KK;  // [PB][HY][HXP]

    const float sc = a.s0[c];
    for (int i = tid; i < KK; i += blockDim.x) {
        const int u = i / K, v = i - u * K;
        const int src = a.rotate ? (K - 1 - u) * K + (K - 1 - v) : i;
        wsh[i] = sc * a.w0[(size_t)c * KK + src];
    }
    const float bias = a.b0 ? sc * a.b0[c] : 0.f;

    const T *x = static_cast<const T *>(a.x);
    const size_t plane = (size_t)a.H * a.W;
    for (int idx = tid; idx < t.PB * plsz; idx += blockDim.x) {
        const int p = idx / plsz, rem = idx - p * plsz;
        const int ci = rem / HXP, cj = rem - ci * HXP;
        const int nn = bp.nb * t.PB + p;
        const int gi = bp.ty0 + ci - R, gj = bp.tx0 + cj - R;
        float v = 0.f;
        if (nn < a.n && gi >= 0 && gi < a.H && gj >= 0 && gj < a.W)
            v = act_load(x + ((size_t)nn * a.C + c) * plane, (size_t)gi * a.W + gj);
        xs[idx] = v;
    }
    __syncthreads();

    T *y = static_cast<T *>(a.y);
    const int per_tile = t.TY * t.SP;
    for (int it = tid; it < t.PB * per_tile; it += blockDim.x) {
        const int p = it / per_tile, rem = it - p * per_tile;
        const int r = rem / t.SP, j0 = (rem - r * t.SP) * S;
        const int nn = bp.nb * t.PB + p, gy = bp.ty0 + r, gx0 = bp.tx0 + j0;
        if (nn >= a.n || gy >= a.H || j0 >= t.TX || gx0 >= a.W) continue;
        float acc[S];
#pragma unroll
        for (int s = 0; s < S; ++s) acc[s] = bias;
        const float *src = xs + (size_t)p * plsz + r * HXP + j0;
#pragma unroll
        for (int u = 0; u < K; ++u) {
            float win[S + K - 1];
#pragma unroll
            for (int e = 0; e < S + K - 1; ++e) win[e] = src[u * HXP + e];
#pragma unroll
            for (int v = 0; v < K; ++v) {
                const float w = wsh[u * K + v];
#pragma unroll
                for (int s = 0; s < S; ++s) acc[s] = fmaf(w, win[s + v], acc[s]);
            }
        }
        const size_t pidx = (size_t)nn * a.C + c;
        bool valid[S];
#pragma unroll
        for (int s = 0; s < S; ++s) valid[s] = (gx0 + s < a.W) && (j0 + s < t.TX);
        // Eq. 7: level l contributes at (y >> (l-1), x >> (l-1)) of Q(l).
        for (int l = 0; l < a.L; ++l) {
            const T *ql = static_cast<const T *>(a.q[l]) + pidx * (size_t)a.qplane[l] + (size_t)(gy >> l) * a.wq[l];
#pragma unroll
            for (int s = 0; s < S; ++s)
                if (valid[s]) acc[s] += act_load(ql, (size_t)((gx0 + s) >> l));
        }
        T *yp = y + pidx * plane + (size_t)gy * a.W + gx0;
#pragma unroll
        for (int s = 0; s < S; ++s)
            if (valid[s]) act_store(yp, s, acc[s]);
    }
}

// ---------------------------------------------------------------------------
// Weight gradient, level l: the folded-weight gradient of band b is
//   dW~[b][u][v] = sum_{n,i,j} G[b][i][j] * Y[b][i+u-R][j+v-R]
// with Y the level-l analysis of x and G the level-l analysis of dy (the gradient
// at Z(l), Eq. 1: backward through synthesis is analysis).  Both analyses are
// recomputed from the carriers in LDS; the carriers of the next level are written
// on the way.  Each wavefront owns one band; per-lane tap accumulators are reduced
// with DPP, then across wavefronts in LDS, into one partial row per workgroup.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void dw_level_kernel(DwLevelArgs a) {
    constexpr int R = (K - 1) / 2, S = 8, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C, t.TY, t.TX);
    const int c = bp.c, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = blockDim.x / kWave;
    const int band = wave & 3, wib = wave >> 2, nwb = nwaves >> 2;
    const int HY = t.TY + K - 1, HXP = t.SP * S + K - 1, ysz = HY * HXP;
    const int GW = t.SP * S, gsz = t.TY * GW;
    float *ys = smem;                        // [PB][4][HY][HXP]
    float *gs = ys + (size_t)t.PB * 4 * ysz;  // [PB][4][TY][GW]
    float *red = gs + (size_t)t.PB * 4 * gsz; // [nwb][4][KK]

    const T *xin = static_cast<const T *>(a.xin);
    const T *gin = static_cast<const T *>(a.gin);
    const size_t in_plane = (size_t)a.Hi * a.Wi, out_plane = (size_t)a.Ho * a.Wo;
    const int n_begin = bp.nb * t.NB;
    const int n_end = min(a.n, n_begin + t.NB);

    float acc[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) acc[i] = 0.f;

    for (int n0 = n_begin; n0 < n_end; n0 += t.PB) {
        __syncthreads();
        for (int idx = tid; idx < t.PB * ysz; idx += blockDim.x) {
            const int p = idx / ysz, rem = idx - p * ysz;
            const int ci = rem / HXP, cj = rem - ci * HXP;
            const int nn = n0 + p;
            const int gi = bp.ty0 + ci - R, gj = bp.tx0 + cj - R;
            float x00 = 0.f, x01 = 0.f, x10 = 0.f, x11 = 0.f;
            const bool inside = nn < n_end && gi >= 0 && gi < a.Ho && gj >= 0 && gj < a.Wo;
            if (inside) {
                const T *src = xin + ((size_t)nn * a.C + c) * in_plane;
                const int r0 = 2 * gi, c0 = 2 * gj;
                const bool c1 = c0 + 1 < a.Wi, r1 = r0 + 1 < a.Hi;
                x00 = act_load(src, (size_t)r0 * a.Wi + c0);
                if (c1) x01 = act_load(src, (size_t)r0 * a.Wi + c0 + 1);
                if (r1) {
                    x10 = act_load(src, (size_t)(r0 + 1) * a.Wi + c0);
                    if (c1) x11 = act_load(src, (size_t)(r0 + 1) * a.Wi + c0 + 1);
                }
            }
            const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
            float *dst = ys + (size_t)p * 4 * ysz + ci * HXP + cj;
            dst[0] = s0 + s1;
            dst[ysz] = s0 - s1;
            dst[2 * ysz] = d0 + d1;
            dst[3 * ysz] = d0 - d1;
            if (a.xc && inside && ci >= R && ci < R + t.TY && cj >= R && cj < R + t.TX)
                act_store(static_cast<T *>(a.xc), ((size_t)nn * a.C + c) * out_plane + (size_t)gi * a.Wo + gj,
                          0.5f * (s0 + s1));
        }
        for (int idx = tid; idx < t.PB * gsz; idx += blockDim.x) {
            const int p = idx / gsz, rem = idx - p * gsz;
            const int ci = rem / GW, cj = rem - ci * GW;
            const int nn = n0 + p;
            const int gi = bp.ty0 + ci, gj = bp.tx0 + cj;
            float x00 = 0.f, x01 = 0.f, x10 = 0.f, x11 = 0.f;
            const bool inside = nn < n_end && ci < t.TY && gi < a.Ho && cj < t.TX && gj < a.Wo;
            if (inside) {
                const T *src = gin + ((size_t)nn * a.C + c) * in_plane;
                const int r0 = 2 * gi, c0 = 2 * gj;
                const bool c1 = c0 + 1 < a.Wi, r1 = r0 + 1 < a.Hi;
                x00 = act_load(src, (size_t)r0 * a.Wi + c0);
                if (c1) x01 = act_load(src, (size_t)r0 * a.Wi + c0 + 1);
                if (r1) {
                    x10 = act_load(src, (size_t)(r0 + 1) * a.Wi + c0);
                    if (c1) x11 = act_load(src, (size_t)(r0 + 1) * a.Wi + c0 + 1);
                }
            }
            const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
            float *dst = gs + (size_t)p * 4 * gsz + ci * GW + cj;
            dst[0] = s0 + s1;
            dst[gsz] = s0 - s1;
            dst[2 * gsz] = d0 + d1;
            dst[3 * gsz] = d0 - d1;
            if (a.gc && inside)
                act_store(static_cast<T *>(a.gc), ((size_t)nn * a.C + c) * out_plane + (size_t)gi * a.Wo + gj,
                          0.5f * (s0 + s1));
        }
        __syncthreads();

        const int per_tile = t.TY * t.SP;
        for (int it = wib * kWave + lane; it < t.PB * per_tile; it += nwb * kWave) {
            const int p = it / per_tile, rem = it - p * per_tile;
            const int r = rem / t.SP, j0 = (rem - r * t.SP) * S;
            const float *g = gs + (size_t)p * 4 * gsz + band * gsz + r * GW + j0;
            float gv[S];
#pragma unroll
            for (int s = 0; s < S; ++s) gv[s] = g[s];
            const float *src = ys + (size_t)p * 4 * ysz + band * ysz + r * HXP + j0;
#pragma unroll
            for (int u = 0; u < K; ++u) {
                float win[S + K - 1];
#pragma unroll
                for (int e = 0; e < S + K - 1; ++e) win[e] = src[u * HXP + e];
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int s = 0; s < S; ++s) acc[u * K + v] = fmaf(gv[s], win[s + v], acc[u * K + v]);
            }
        }
    }

#pragma unroll
    for (int i = 0; i < KK; ++i) {
        const float v = wave_sum(acc[i]);
        if (lane == 0) red[(wib * 4 + band) * KK + i] = v;
    }
    __syncthreads();
    const int G = t.nblk * t.tiles, g = bp.nb * t.tiles + bp.tile;
    float *out = a.partial + ((size_t)c * G + g) * 4 * KK;
    for (int i = tid; i < 4 * KK; i += blockDim.x) {
        float s = 0.f;
        for (int w = 0; w < nwb; ++w) s += red[w * 4 * KK + i];
        out[i] = 0.25f * s;  // the two analysis halves
    }
}

// ---------------------------------------------------------------------------
// Weight gradient, base path: dW~0[u][v] = sum dy[y][x] * x[y+u-R][x+v-R] and
// db~ = sum dy; same two-stage reduction.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void dw_base_kernel(DwBaseArgs a) {
    constexpr int R = (K - 1) / 2, S = 8, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C, t.TY, t.TX);
    const int c = bp.c, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = blockDim.x / kWave;
    const int HY = t.TY + K - 1, HXP = t.SP * S + K - 1, xsz = HY * HXP;
    const int GW = t.SP * S, gsz = t.TY * GW;
    float *xs = smem;                         // [PB][HY][HXP]
    float *gs = xs + (size_t)t.PB * xsz;      // [PB][TY][GW]
    float *red = gs + (size_t)t.PB * gsz;     // [nwaves][KK + 1]

    const T *x = static_cast<const T *>(a.x);
    const T *dy = static_cast<const T *>(a.dy);
    const size_t plane = (size_t)a.H * a.W;
    const int n_begin = bp.nb * t.NB;
    const int n_end = min(a.n, n_begin + t.NB);

    float acc[KK + 1];
#pragma unroll
    for (int i = 0; i <= KK; ++i) acc[i] = 0.f;

    for (int n0 = n_begin; n0 < n_end; n0 += t.PB) {
        __syncthreads();
        for (int idx = tid; idx < t.PB * xsz; idx += blockDim.x) {
            const int p = idx / xsz, rem = idx - p * xsz;
            const int ci = rem / HXP, cj = rem - ci * HXP;
            const int nn = n0 + p, gi = bp.ty0 + ci - R, gj = bp.tx0 + cj - R;
            float v = 0.f;
            if (nn < n_end && gi >= 0 && gi < a.H && gj >= 0 && gj < a.W)
                v = act_load(x + ((size_t)nn * a.C + c) * plane, (size_t)gi * a.W + gj);
            xs[idx] = v;
        }
        for (int idx = tid; idx < t.PB * gsz; idx += blockDim.x) {
            const int p = idx / gsz, rem = idx - p * gsz;
            const int ci = rem / GW, cj = rem - ci * GW;
            const int nn = n0 + p, gi = bp.ty0 + ci, gj = bp.tx0 + cj;
            float v = 0.f;
            if (nn < n_end && ci < t.TY && gi < a.H && cj < t.TX && gj < a.W)
                v = act_load(dy + ((size_t)nn * a.C + c) * plane, (size_t)gi * a.W + gj);
            gs[idx] = v;
        }
        __syncthreads();

        const int per_tile = t.TY * t.SP;
        for (int it = tid; it < t.PB * per_tile; it += blockDim.x) {
            const int p = it / per_tile, rem = it - p * per_tile;
            const int r = rem / t.SP, j0 = (rem - r * t.SP) * S;
            const float *g = gs + (size_t)p * gsz + r * GW + j0;
            float gv[S];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                gv[s] = g[s];
                acc[KK] += gv[s];
            }
            const float *src = xs + (size_t)p * xsz + r * HXP + j0;
#pragma unroll
            for (int u = 0; u < K; ++u) {
                float win[S + K - 1];
#pragma unroll
                for (int e = 0; e < S + K - 1; ++e) win[e] = src[u * HXP + e];
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int s = 0; s < S; ++s) acc[u * K + v] = fmaf(gv[s], win[s + v], acc[u * K + v]);
            }
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
    for (int i = tid; i <= KK; i += blockDim.x) {
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += red[w * (KK + 1) + i];
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
