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
// column values from LDS (consecutive lanes read consecutive words or cells: no
// bank conflicts) and applies the K vertical taps from registers, so one LDS read
// feeds 8K/(8+K-1) FMAs.  In the synthesis and base-gradient kernels the folded
// k x k weights of a channel are the same for the whole workgroup and sit in scalar
// registers (readfirstlane): each multiply-accumulate is one v_fmac_f32 with a
// scalar operand.  The level kernel stages one float4 cell of the four bands per
// coefficient block and reads the four bands' weights as float4 from LDS.
//
// All arithmetic is float32; activations are float32, bfloat16 or IEEE half in
// memory.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wtconv.h"

namespace wtc {

constexpr int kMaxLevels = WTCONV_MAX_LEVELS;
constexpr int kWave = 64;
constexpr int kRH = 8;  // rows per lane strip

// ---------------------------------------------------------------------------
// Activation storage
// ---------------------------------------------------------------------------

// Three storage types: float (float32), uint16_t (bfloat16 bits) and wtc_f16
// (IEEE half bits).  Every kernel loads the raw words of its activations and
// converts them with Act<T>; the 16-bit types share all load and store code, and
// differ only in the conversions below.  All arithmetic is float32.
struct wtc_f16 {
    uint16_t bits;
};
typedef float wtc_float2 __attribute__((ext_vector_type(2)));
typedef __bf16 wtc_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 wtc_halfx2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Act;
template <>
struct Act<float> {
    static constexpr bool half = false;
};
template <>
struct Act<uint16_t> {  // bfloat16: the high half of a float32
    static constexpr bool half = true;
    __device__ __forceinline__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ __forceinline__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    // round to nearest, ties to even (gfx950 v_cvt_pk_bf16_f32), low half = a
    __device__ __forceinline__ static uint32_t pack(float a, float b) {
        const wtc_float2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, wtc_bf16x2));
    }
    __device__ __forceinline__ static uint16_t one(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
};
template <>
struct Act<wtc_f16> {  // IEEE binary16
    static constexpr bool half = true;
    __device__ __forceinline__ static float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    __device__ __forceinline__ static float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    // round to nearest, ties to even, low half = a
    __device__ __forceinline__ static uint32_t pack(float a, float b) {
        const wtc_float2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, wtc_halfx2));
    }
    __device__ __forceinline__ static uint16_t one(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
};
template <typename T>
constexpr bool kHalf = Act<T>::half;
template <typename T>
using if_half = typename std::enable_if<Act<T>::half, int>::type;

__device__ __forceinline__ float act_load(const float *p, size_t i) { return p[i]; }
template <typename T, if_half<T> = 0>
__device__ __forceinline__ float act_load(const T *p, size_t i) {
    return Act<T>::lo(reinterpret_cast<const uint16_t *>(p)[i]);
}

// Exact quotient n / d for n, d < 2^16, with m = ceil(2^32 / d) computed on the host
// (m = 0 encodes d = 1): the error term n (m d - 2^32) / (d 2^32) stays below 1/d.
__device__ __forceinline__ int fdiv(int n, uint32_t m) { return m ? (int)__umulhi((uint32_t)n, m) : n; }

__device__ __forceinline__ void act_store(float *p, size_t i, float v) { p[i] = v; }
template <typename T, if_half<T> = 0>
__device__ __forceinline__ void act_store(T *p, size_t i, float v) {
    reinterpret_cast<uint16_t *>(p)[i] = Act<T>::one(v);
}

// Two adjacent elements (element index i even, so the pair is aligned).
__device__ __forceinline__ void act_store2(float *p, size_t i, float a, float b) {
    *reinterpret_cast<float2 *>(p + i) = make_float2(a, b);
}
template <typename T, if_half<T> = 0>
__device__ __forceinline__ void act_store2(T *p, size_t i, float a, float b) {
    *reinterpret_cast<uint32_t *>(p + i) = Act<T>::pack(a, b);
}
__device__ __forceinline__ void act_load2(const float *p, size_t i, float &a, float &b) {
    const float2 v = *reinterpret_cast<const float2 *>(p + i);
    a = v.x;
    b = v.y;
}
template <typename T, if_half<T> = 0>
__device__ __forceinline__ void act_load2(const T *p, size_t i, float &a, float &b) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(p + i);
    a = Act<T>::lo(v);
    b = Act<T>::hi(v);
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
template <int VW, typename T, if_half<T> = 0>
__device__ __forceinline__ void act_loadv(const T *p, size_t i, float *out) {
    const uint16_t *q = reinterpret_cast<const uint16_t *>(p);
    if constexpr (VW == 1) {
        out[0] = Act<T>::lo(q[i]);
    } else if constexpr (VW == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(q + i);
        out[0] = Act<T>::lo(v);
        out[1] = Act<T>::hi(v);
    } else if constexpr (VW == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(q + i);
        out[0] = Act<T>::lo(v.x);
        out[1] = Act<T>::hi(v.x);
        out[2] = Act<T>::lo(v.y);
        out[3] = Act<T>::hi(v.y);
    } else {
        static_assert(VW == 8, "16-bit vectors are at most 16 bytes");
        const uint4 v = *reinterpret_cast<const uint4 *>(q + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = Act<T>::lo(w[k]);
            out[2 * k + 1] = Act<T>::hi(w[k]);
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
    // the deeper levels' patterns summed on this level's grid, [n][C][2 Ho'][2 Wo']
    // for the next level's Ho' x Wo' (its value at cell (i, j) enters all four
    // patterns of block (i, j)), or NULL
    const void *deeper;
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

// Staging loops take their indices in batches of kStageBatch per thread: every load
// of a batch is issued, from an address clamped into the tensor, before any of them
// is used (out-of-range values are masked afterwards).  A load that is converted or
// tested right after it is issued makes the wavefront wait for it alone, and a
// loop of such loads pays one memory latency per iteration.
constexpr int kStageBatch = 4;

// The four raw elements of one 2 x 2 pixel block: with `pairs`, one two-element
// load per row (bfloat16: one word per row in w[0], w[1]; float32: w[0..3]);
// otherwise one element per word, (x00, x01, x10, x11).
template <typename T>
__device__ __forceinline__ void block_load_raw(const T *src, size_t o0, size_t o1, int dc, bool pairs,
                                               uint32_t (&w)[4]) {
    if (pairs) {
        if constexpr (sizeof(T) == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(src + o0);
            w[1] = *reinterpret_cast<const uint32_t *>(src + o1);
        } else {
            const uint2 a = *reinterpret_cast<const uint2 *>(src + o0), b = *reinterpret_cast<const uint2 *>(src + o1);
            w[0] = a.x;
            w[1] = a.y;
            w[2] = b.x;
            w[3] = b.y;
        }
    } else {
        if constexpr (sizeof(T) == 2) {
            const uint16_t *s16 = reinterpret_cast<const uint16_t *>(src);
            w[0] = s16[o0];
            w[1] = s16[o0 + dc];
            w[2] = s16[o1];
            w[3] = s16[o1 + dc];
        } else {
            const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
            w[0] = s32[o0];
            w[1] = s32[o0 + dc];
            w[2] = s32[o1];
            w[3] = s32[o1 + dc];
        }
    }
}
template <typename T>
__device__ __forceinline__ void block_unpack(const uint32_t (&w)[4], bool pairs, float &x00, float &x01, float &x10,
                                             float &x11) {
    if constexpr (kHalf<T>) {
        if (pairs) {
            x00 = Act<T>::lo(w[0]);
            x01 = Act<T>::hi(w[0]);
            x10 = Act<T>::lo(w[1]);
            x11 = Act<T>::hi(w[1]);
        } else {
            x00 = Act<T>::lo(w[0]);
            x01 = Act<T>::lo(w[1]);
            x10 = Act<T>::lo(w[2]);
            x11 = Act<T>::lo(w[3]);
        }
    } else {
        x00 = __uint_as_float(w[0]);
        x01 = __uint_as_float(w[1]);
        x10 = __uint_as_float(w[2]);
        x11 = __uint_as_float(w[3]);
    }
}

// q / d and q % d for 0 <= q < 2^23, d >= 1, given rd = 1 / d in float: the float
// quotient of q + 1/2 is within one of the true one, and the remainder fixes it.
__device__ __forceinline__ void small_divmod(int q, int d, float rd, int &quo, int &rem) {
    int v = (int)(((float)q + 0.5f) * rd);
    int r = q - v * d;
    if (r < 0) {
        --v;
        r += d;
    } else if (r >= d) {
        ++v;
        r -= d;
    }
    quo = v;
    rem = r;
}

// Threads walk a staged grid with a fixed column each: thread t takes column
// t % cols and rows t / cols, t / cols + step, ... (step = threads / cols; cols is
// at most the thread count), so nothing is divided per element.
// kCells: the four bands of a block go to one float4 cell, bands + 4 (p bandsz +
// ci stride + cj); otherwise to four arrays of bandsz floats each.
template <typename T, bool kCells = false>
__device__ __forceinline__ void haar_stage(const T *__restrict__ in, T *__restrict__ carrier, float *bands,
                                           int bandsz, int stride, int PB, int rows, int cols, int r0, int c0,
                                           int n0, int n_end, int c, int C, int Hi, int Wi, int Ho, int Wo,
                                           int vr1, int cr0, int cr1, int cc0, int cc1, int pairs) {
    const size_t in_plane = (size_t)Hi * Wi, out_plane = (size_t)Ho * Wo;
    const int step = blockDim.x / cols, cj = threadIdx.x % cols, rs = threadIdx.x / cols;
    if (rs >= step) return;
    const int gj = c0 + cj, gjc = min(max(gj, 0), Wo - 1);
    const bool col_in = gj >= 0 && gj < Wo, c1 = 2 * gjc + 1 < Wi;
    const bool carry_col = carrier && col_in && gj >= cc0 && gj < cc1;
    for (int p = 0; p < PB; ++p) {
        const int nn = n0 + p;
        const bool plane_in = nn < n_end && col_in;
        const T *src = in + ((size_t)min(nn, n_end - 1) * C + c) * in_plane + 2 * gjc;
        float *dst0 = bands + (size_t)p * 4 * bandsz + (kCells ? 4 * cj : cj);
        for (int base = rs; base < rows; base += kStageBatch * step) {
            uint32_t raw[kStageBatch][4];
#pragma unroll
            for (int k = 0; k < kStageBatch; ++k) {
                // clamped into the image: the block itself when it is inside
                const int gi = min(max(r0 + min(base + k * step, rows - 1), 0), Ho - 1);
                const size_t o0 = (size_t)(2 * gi) * Wi, o1 = 2 * gi + 1 < Hi ? o0 + Wi : o0;
                block_load_raw<T>(src, o0, o1, c1 ? 1 : 0, pairs, raw[k]);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of every use
            // rows past the end repeat the last row (the same values to the same
            // place): no branch, so the loads are not sunk into one
#pragma unroll
            for (int k = 0; k < kStageBatch; ++k) {
                const int ci = min(base + k * step, rows - 1);
                const int gi = r0 + ci;
                const bool inside = plane_in && gi >= 0 && gi < vr1;
                float x00, x01, x10, x11;
                block_unpack<T>(raw[k], pairs, x00, x01, x10, x11);
                const bool r1 = 2 * gi + 1 < Hi;
                x00 = inside ? x00 : 0.f;
                x01 = inside && c1 ? x01 : 0.f;
                x10 = inside && r1 ? x10 : 0.f;
                x11 = inside && r1 && c1 ? x11 : 0.f;
                const float s0 = x00 + x01, s1 = x10 + x11, d0 = x00 - x01, d1 = x10 - x11;
                if constexpr (kCells) {
                    *reinterpret_cast<float4 *>(dst0 + 4 * ci * stride) = make_float4(s0 + s1, s0 - s1, d0 + d1, d0 - d1);
                } else {
                    float *dst = dst0 + ci * stride;
                    dst[0] = s0 + s1;           // 2 LL
                    dst[bandsz] = s0 - s1;      // 2 LH
                    dst[2 * bandsz] = d0 + d1;  // 2 HL
                    dst[3 * bandsz] = d0 - d1;  // 2 HH
                }
                if (carry_col && inside && gi >= cr0 && gi < cr1 && base + k * step < rows)
                    act_store(carrier, ((size_t)nn * C + c) * out_plane + (size_t)gi * Wo + gj, 0.5f * (s0 + s1));
            }
        }
    }
}

// Raw words of VW consecutive elements (converted once the batch is in flight).
template <int VW, typename T>
struct RawVec {
    static constexpr int kWords = (VW * (int)sizeof(T) + 3) / 4;
    uint32_t w[kWords];
};
template <int VW, typename T>
__device__ __forceinline__ void raw_load(const T *p, RawVec<VW, T> &r) {
    constexpr int bytes = VW * (int)sizeof(T);
    if constexpr (bytes == 16) {
        const uint4 q = *reinterpret_cast<const uint4 *>(p);
        r.w[0] = q.x;
        r.w[1] = q.y;
        r.w[2] = q.z;
        r.w[3] = q.w;
    } else if constexpr (bytes == 8) {
        const uint2 q = *reinterpret_cast<const uint2 *>(p);
        r.w[0] = q.x;
        r.w[1] = q.y;
    } else if constexpr (bytes == 4) {
        r.w[0] = *reinterpret_cast<const uint32_t *>(p);
    } else {
        static_assert(bytes == 2, "one bfloat16");
        r.w[0] = *reinterpret_cast<const uint16_t *>(p);
    }
}
template <int VW, typename T>
__device__ __forceinline__ float raw_elem(const RawVec<VW, T> &r, int e) {
    if constexpr (kHalf<T>) {
        const uint32_t wv = r.w[e >> 1];
        return (e & 1) ? Act<T>::hi(wv) : Act<T>::lo(wv);
    } else {
        return __uint_as_float(r.w[e]);
    }
}

// VW floats to LDS in 16-byte (or narrower) writes.
template <int VW>
__device__ __forceinline__ void lds_store(float *d, const float *v) {
    if constexpr (VW == 8) {
        reinterpret_cast<float4 *>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4 *>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else if constexpr (VW == 4) {
        *reinterpret_cast<float4 *>(d) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (VW == 2) {
        *reinterpret_cast<float2 *>(d) = make_float2(v[0], v[1]);
    } else {
        d[0] = v[0];
    }
}

// Stage a pixel tile: rows [r0, r0 + rows) x cols [c0, c0 + width) of PB planes,
// zero outside the plane, at or below row row_hi (<= H), and, when mask_lo <
// mask_hi, outside those columns;
// converted to float32 in LDS with row stride `width`.  c0 and width are multiples
// of VW and W is a multiple of VW, so each vector is wholly inside or outside; dst
// is aligned to VW floats.  Thread t stages vector column t % (width / VW) (of each
// chunk of at most blockDim.x columns).
template <int VW, typename T>
__device__ __forceinline__ void pixel_stage_v(const T *__restrict__ src, float *dst, int PB, int rows, int width,
                                              int r0, int c0, int n0, int n_end, int c, int C, int H, int W,
                                              int row_hi, int mask_lo, int mask_hi) {
    const int vpr = width / VW, nthr = blockDim.x;
    const size_t plane = (size_t)H * W;
    // vector columns in chunks of at most one per thread (one chunk unless a row
    // holds more vectors than the workgroup has threads)
    for (int vc0 = 0; vc0 < vpr; vc0 += nthr) {
        const int ncols = min(vpr - vc0, nthr);
        const int step = nthr / ncols, vc = vc0 + (int)threadIdx.x % ncols, rs = (int)threadIdx.x / ncols;
        if (rs >= step) continue;
        const int gc = c0 + vc * VW, gcc = min(max(gc, 0), W - VW);
        bool keep[VW];
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            const int col = gc + e;
            keep[e] = gc >= 0 && gc < W && !(mask_lo < mask_hi && (col < mask_lo || col >= mask_hi));
        }
        for (int p = 0; p < PB; ++p) {
            const int nn = n0 + p;
            const bool plane_in = nn < n_end;
            const T *sp = src + ((size_t)min(nn, n_end - 1) * C + c) * plane + gcc;
            float *dp = dst + (size_t)p * rows * width + vc * VW;
            for (int base = rs; base < rows; base += kStageBatch * step) {
                RawVec<VW, T> raw[kStageBatch];
#pragma unroll
                for (int k = 0; k < kStageBatch; ++k) {
                    const int gi = min(max(r0 + min(base + k * step, rows - 1), 0), H - 1);
                    raw_load<VW, T>(sp + (size_t)gi * W, raw[k]);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of every use
                // rows past the end repeat the last row (the same values to the same
                // place): no branch, so the loads are not sunk into one
#pragma unroll
                for (int k = 0; k < kStageBatch; ++k) {
                    const int ri = min(base + k * step, rows - 1);
                    const int gi = r0 + ri;
                    const bool rin = plane_in && gi >= 0 && gi < row_hi;
                    float v[VW];
#pragma unroll
                    for (int e = 0; e < VW; ++e) v[e] = rin && keep[e] ? raw_elem<VW, T>(raw[k], e) : 0.f;
                    lds_store<VW>(dp + (size_t)ri * width, v);
                }
            }
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
// Output grid: the level's coefficient grid (Ho x Wo).  The staged tile holds one
// float4 cell of the four unscaled bands per coefficient block; a lane filters all
// four bands of one column x kRH rows (weights of the four bands as float4 from an
// LDS table: s(l,b) 2^-(l+1) W(l,b), Eq. 8 with the analysis 1/2 and the synthesis
// weight 2^-l folded in) and stores the four sign patterns of each block (Eq.
// 12/13) as a 2 x 2 block of Q(l).  256 threads.
// ---------------------------------------------------------------------------

template <int K, typename T>
__global__ __launch_bounds__(256) void level_fwd_kernel(LevelArgs a) {
    constexpr int R = (K - 1) / 2, KK = K * K;
    extern __shared__ float smem[];
    const Tiling &t = a.t;
    const BlockPos bp = block_pos(t, a.C);
    const int c = bp.c;
    const int HY = t.SP * kRH + K - 1, HXP = t.TX + K - 1, cells = HY * HXP;
    float4 *band = reinterpret_cast<float4 *>(smem);  // [PB][HY][HXP] cells
    float4 *wtab = band + (size_t)t.PB * cells;         // [v][u] float4 over the bands
    const int n0 = bp.nb * t.PB;
    const int tid = threadIdx.x;

    // weight table: thread e < 4 KK folds band e / KK, tap e % KK (row u, column v)
    float wraw = 0.f, sraw = 0.f;
    if (tid < 4 * KK) {
        const int b = tid / KK, tap = tid - b * KK, u = tap / K, v = tap - u * K;
        wraw = a.wl[(size_t)(c * 4 + b) * KK + (a.rotate ? (K - 1 - u) * K + (K - 1 - v) : tap)];
        sraw = a.sl[c * 4 + b];
    }
    haar_stage<T, true>(static_cast<const T *>(a.in), static_cast<T *>(a.cout), smem, cells, HXP, t.PB, HY, HXP,
                        bp.ty0 - R, bp.tx0 - R, n0, a.n, c, a.C, a.Hi, a.Wi, a.Ho, a.Wo, a.Ho, bp.ty0, bp.ty0 + t.TY,
                        bp.tx0, bp.tx0 + t.TX, a.pairs);
    if (tid < 4 * KK) {
        const int b = tid / KK, tap = tid - b * KK, u = tap / K, v = tap - u * K;
        reinterpret_cast<float *>(wtab)[(v * K + u) * 4 + b] = sraw * a.wscale * wraw;
    }
    __syncthreads();

    // thread: column threadIdx.x % TX, strips (plane, strip) = threadIdx.x / TX, + step, ...
    T *q = static_cast<T *>(a.qout);
    const int Wq = 2 * a.Wo;
    const size_t q_plane = (size_t)4 * a.Ho * a.Wo;
    const int step = blockDim.x / t.TX, j = tid % t.TX, q0 = tid / t.TX, nq = t.PB * t.SP;
    const float rsp = 1.f / (float)t.SP;
    const int gj = bp.tx0 + j;
    for (int qi = q0 < step ? q0 : nq; qi < nq; qi += step) {
        int p, s;
        small_divmod(qi, t.SP, rsp, p, s);
        float z[4][kRH];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < kRH; ++i) z[b][i] = 0.f;
        const float4 *win = band + (size_t)p * cells + (s * kRH) * HXP + j;
#pragma unroll 1
        for (int v = 0; v < K; ++v) {  // rolled: unrolled, every column's reads go out up front
            float4 wb[K];
#pragma unroll
            for (int u = 0; u < K; ++u) wb[u] = wtab[v * K + u];
            float4 cl[kRH + K - 1];
#pragma unroll
            for (int tt = 0; tt < kRH + K - 1; ++tt) cl[tt] = win[tt * HXP + v];
#pragma unroll
            for (int u = 0; u < K; ++u)
#pragma unroll
                for (int i = 0; i < kRH; ++i) {
                    z[0][i] = fmaf(wb[u].x, cl[i + u].x, z[0][i]);
                    z[1][i] = fmaf(wb[u].y, cl[i + u].y, z[1][i]);
                    z[2][i] = fmaf(wb[u].z, cl[i + u].z, z[2][i]);
                    z[3][i] = fmaf(wb[u].w, cl[i + u].w, z[3][i]);
                }
        }
        // q[ry][rx] = LL + (-1)^ry LH + (-1)^rx HL + (-1)^(ry+rx) HH (Eq. 12/13)
        const int nn = n0 + p, gi0 = bp.ty0 + s * kRH;
        const int rows = min(kRH, min(a.Ho, bp.ty0 + t.TY) - gi0);
        if (nn >= a.n || gj >= a.Wo || rows <= 0) continue;
        T *qp = q + ((size_t)nn * a.C + c) * q_plane + (size_t)(2 * gi0) * Wq + 2 * gj;
        float dz[kRH];
#pragma unroll
        for (int i = 0; i < kRH; ++i) dz[i] = 0.f;
        if (a.deeper) {
            // the deeper grid is 2 Ho' x 2 Wo' with Ho' = ceil(Ho / 2): rows of this
            // level's grid are all inside it
            const int Wd = 2 * ((a.Wo + 1) / 2), Hd = 2 * ((a.Ho + 1) / 2);
            const T *dp = static_cast<const T *>(a.deeper) + ((size_t)nn * a.C + c) * Hd * Wd + (size_t)gi0 * Wd + gj;
#pragma unroll
            for (int i = 0; i < kRH; ++i)
                if (i < rows) dz[i] = act_load(dp, (size_t)i * Wd);
        }
#pragma unroll
        for (int i = 0; i < kRH; ++i) {
            if (i >= rows) break;
            const float a0 = z[0][i] + z[1][i], a1 = z[0][i] - z[1][i];
            const float b0 = z[2][i] + z[3][i], b1 = z[2][i] - z[3][i];
            act_store2(qp + 2 * i * Wq, 0, (a0 + b0) + dz[i], (a0 - b0) + dz[i]);
            act_store2(qp + (2 * i + 1) * Wq, 0, (a1 + b1) + dz[i], (a1 - b1) + dz[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Level-1 carrier alone: the normalised low-pass band 1/2 (x00 + x01 + x10 + x11)
// of every 2 x 2 block (Eq. 5), the input of the level-2 kernel when the level-1
// filter and synthesis run elsewhere (the tiled matrix-core forward).  The same
// sums, in the same order and with the same rounding, as the carrier the level
// kernel writes.  Thread: four consecutive blocks of one block row; grid.y walks
// the planes.
// ---------------------------------------------------------------------------

struct CarrierArgs {
    const void *in;  // [planes][Hi][Wi]
    void *out;       // [planes][Ho][Wo]
    int planes, Hi, Wi, Ho, Wo;
    int groups;      // ceil(Wo / 4) groups of four blocks per row
    int vec;         // Wi % 8 == 0 and the input 16-byte aligned: one 8-pixel load per row
};

template <typename T>
__global__ __launch_bounds__(256) void carrier_kernel(CarrierArgs a) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.Ho * a.groups) return;
    const int i = idx / a.groups, g = idx - i * a.groups;
    const bool r1 = 2 * i + 1 < a.Hi;
    for (int p = blockIdx.y; p < a.planes; p += gridDim.y) {
        const T *src = static_cast<const T *>(a.in) + (size_t)p * a.Hi * a.Wi + (size_t)(2 * i) * a.Wi + 8 * g;
        T *dst = static_cast<T *>(a.out) + (size_t)p * a.Ho * a.Wo + (size_t)i * a.Wo + 4 * g;
        float x[2][8];
        if constexpr (kHalf<T>) {
            if (a.vec) {
                const uint4 v0 = *reinterpret_cast<const uint4 *>(src);
                const uint4 v1 = r1 ? *reinterpret_cast<const uint4 *>(src + a.Wi) : make_uint4(0u, 0u, 0u, 0u);
                const uint32_t w[2][4] = {{v0.x, v0.y, v0.z, v0.w}, {v1.x, v1.y, v1.z, v1.w}};
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[r][2 * e] = Act<T>::lo(w[r][e]);
                        x[r][2 * e + 1] = Act<T>::hi(w[r][e]);
                    }
            } else {
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool in = 8 * g + e < a.Wi && (r == 0 || r1);
                        x[r][e] = in ? act_load(src, (size_t)r * a.Wi + e) : 0.f;
                    }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool in = 8 * g + e < a.Wi && (r == 0 || r1);
                    x[r][e] = in ? act_load(src, (size_t)r * a.Wi + e) : 0.f;
                }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (4 * g + b >= a.Wo) break;
            const float s0 = x[0][2 * b] + x[0][2 * b + 1], s1 = x[1][2 * b] + x[1][2 * b + 1];
            act_store(dst, b, 0.5f * (s0 + s1));
        }
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

    // every load first, then one wait: not one memory latency per weight
    float w[KK], raw[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) {
        const int u = i / K, v = i - u * K;
        raw[i] = a.w0[(size_t)c * KK + (a.rotate ? (K - 1 - u) * K + (K - 1 - v) : i)];
    }
    const float sc = a.s0[c], braw = a.b0 ? a.b0[c] : 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < KK; ++i) w[i] = uniform(sc * raw[i]);
    const float bias = uniform(sc * braw);
    __syncthreads();

    T *y = static_cast<T *>(a.y);
    const size_t plane = (size_t)a.H * a.W;
    // thread: column threadIdx.x % TX, strips (plane, strip) = threadIdx.x / TX, + step, ...
    const int step = blockDim.x / t.TX, j = threadIdx.x % t.TX, q0 = threadIdx.x / t.TX, nq = t.PB * t.SP;
    const float rsp = 1.f / (float)t.SP;
    for (int q = q0 < step ? q0 : nq; q < nq; q += step) {
        int p, s;
        small_divmod(q, t.SP, rsp, p, s);
        const int nn = n0 + p, gx = bp.tx0 + j, gy0 = bp.ty0 + s * kRH;
        if (nn >= a.n || gx >= a.W) continue;
        const int rows = min(kRH, min(a.H, bp.ty0 + t.TY) - gy0);  // rows of this strip in the tile
        const size_t pidx = (size_t)nn * a.C + c;
        // Eq. 7: level l + 1 contributes Q(l+1)[y >> l][x >> l].  gy0 is a multiple of
        // kRH = 8 (the tiling keeps TY one), so row i of the strip reads row
        // (gy0 >> l) + (i >> l) of level l + 1: 8, 4, 2, then 1 distinct values.  They
        // are loaded raw (row clamped into the plane) before the conv and added after
        // it, so that their latency overlaps the conv.
        uint32_t qraw[kMaxLevels][kRH];
        const int ylast = a.H - 1;
#pragma unroll
        for (int l = 0; l < kMaxLevels; ++l) {
            if (l < a.L) {
                const T *ql = static_cast<const T *>(a.q[l]) + pidx * (size_t)a.qplane[l] + (gx >> l);
#pragma unroll
                for (int r = 0; r < (kRH >> l > 0 ? kRH >> l : 1); ++r) {
                    const int row = min((gy0 >> l) + r, ylast >> l);
                    if constexpr (kHalf<T>)  // converted after the conv: no wait here
                        qraw[l][r] = reinterpret_cast<const uint16_t *>(ql)[(size_t)row * a.wq[l]];
                    else
                        qraw[l][r] = reinterpret_cast<const uint32_t *>(ql)[(size_t)row * a.wq[l]];
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of the conv
        float acc[kRH];
#pragma unroll
        for (int i = 0; i < kRH; ++i) acc[i] = 0.f;
        conv_strip<K>(smem + (size_t)p * plsz + (s * kRH) * HXW + j + off, HXW, w, acc);
        __builtin_amdgcn_sched_barrier(0);
        auto qval = [&](uint32_t w) {
            if constexpr (kHalf<T>)
                return Act<T>::lo(w);
            else
                return __uint_as_float(w);
        };
        // levels 4 and deeper read one row for the whole strip: summed once
        float deep = bias;
#pragma unroll
        for (int l = 3; l < kMaxLevels; ++l)
            if (l < a.L) deep += qval(qraw[l][0]);
#pragma unroll
        for (int i = 0; i < kRH; ++i) {
            float qsum = deep;
#pragma unroll
            for (int l = 0; l < 3; ++l)
                if (l < a.L) qsum += qval(qraw[l][i >> l]);
            acc[i] += qsum;
        }
        T *yp = y + pidx * plane + (size_t)gy0 * a.W + gx;
        // a whole strip stores without a branch per row, so that the conv is not sunk
        // into per-row blocks (and the coefficient loads not waited for before it)
        if (rows == kRH) {
#pragma unroll
            for (int i = 0; i < kRH; ++i) act_store(yp, (size_t)i * a.W, acc[i]);
        } else {
#pragma unroll
            for (int i = 0; i < kRH; ++i)
                if (i < rows) act_store(yp, (size_t)i * a.W, acc[i]);
        }
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

    // lane: column lane % TX, strips (plane, strip) = lane / TX, + kWave / TX, ...
    const int wstep = kWave / t.TX, j = lane % t.TX, q0 = lane / t.TX, nq = t.PB * t.SP;
    const float rsp = 1.f / (float)t.SP;
    for (int n0 = n_begin; n0 < n_end; n0 += t.PB) {
        __syncthreads();
        haar_stage<T>(xin, static_cast<T *>(a.xc), ys, ysz, HXP, t.PB, HY, HXP, bp.ty0 - R, bp.tx0 - R, n0, n_end,
                      c, a.C, a.Hi, a.Wi, a.Ho, a.Wo, a.Ho, bp.ty0, bp.ty0 + t.TY, bp.tx0, bp.tx0 + t.TX, a.pairs);
        // G only on the tile itself; rows past the tile are zero (no double count)
        haar_stage<T>(gin, static_cast<T *>(a.gc), gs, gsz, t.TX, t.PB, GY, t.TX, bp.ty0, bp.tx0, n0, n_end, c,
                      a.C, a.Hi, a.Wi, a.Ho, a.Wo, min(a.Ho, bp.ty0 + t.TY), bp.ty0, bp.ty0 + t.TY, bp.tx0,
                      bp.tx0 + t.TX, a.pairs);
        __syncthreads();
        for (int q = q0 < wstep ? q0 : nq; q < nq; q += wstep) {
            int p, s;
            small_divmod(q, t.SP, rsp, p, s);
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

    // thread: column threadIdx.x % TX, strips (plane, strip) = threadIdx.x / TX, + step, ...
    const int step = blockDim.x / t.TX, j = threadIdx.x % t.TX, q0 = threadIdx.x / t.TX, nq = t.PB * t.SP;
    const float rsp = 1.f / (float)t.SP;
    for (int n0 = n_begin; n0 < n_end; n0 += t.PB) {
        __syncthreads();
        pixel_stage<T>(x, xs, t.VW, t.PB, HY, HXW, bp.ty0 - R, ca, n0, n_end, c, a.C, a.H, a.W, a.H, 0, 0);
        // dy only on the tile: rows and columns past the tile are zero
        pixel_stage<T>(dy, gs, t.VW, t.PB, GY, GW, bp.ty0, ga, n0, n_end, c, a.C, a.H, a.W, row_end, bp.tx0,
                       bp.tx0 + t.TX);
        __syncthreads();
        for (int q = q0 < step ? q0 : nq; q < nq; q += step) {
            int p, s;
            small_divmod(q, t.SP, rsp, p, s);
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
        // the same sequential order of additions; loads eight at a time so that
        // they are in flight together
        float s = 0.f;
        int g = 0;
        for (; g + 8 <= G; g += 8) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = part[(size_t)(g + k) * slots + i];
#pragma unroll
            for (int k = 0; k < 8; ++k) s += v[k];
        }
        for (; g < G; ++g) s += part[(size_t)g * slots + i];
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
