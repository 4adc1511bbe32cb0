/*
 * wtconv.h — C ABI of the MI355X (gfx950) WTConv layer library, libwtconv.so.
 *
 * The layer is the wavelet convolution of "Fast and Memory-Efficient Wavelet
 * Convolutions via I/O-Aware Reformulation" (Aflalo, Finder, Amoyal, Treister,
 * Freifeld), §2.1 Algorithm 1:
 *
 *   for l = 1..L: Y(l) = Haar analysis of the carrier X(l-1) (X(0) = x; Eq. 5),
 *                 Z(l) = s(l) * (Y(l) depthwise-conv W(l))  over the 4C bands,
 *                 X(l) = low-pass band of Y(l) (raw, unfiltered)
 *   R(L+1) = 0; for l = L..1: R(l) = synthesis((Z(l)_LL + R(l+1)) || Z(l)_H)
 *   y = s0 * (x depthwise-conv W0 + b) + R(1)
 *
 * Conventions used by every entry point (readings of points the paper leaves open):
 *   - depthwise convolution is cross-correlation with zero padding (k-1)/2, the
 *     output the size of the input, in each level's own coefficient grid;
 *   - an odd plane is zero-padded at the bottom/right to even before each
 *     analysis level, and synthesis crops back, so any H, W >= 1 is accepted;
 *   - the four bands are ordered LL, LH, HL, HH as in Eq. 5, and the 4C
 *     coefficient channels are channel-major, band-minor;
 *   - each level has one scale per (channel, band): s(l) is [C][4];
 *   - only the base path has a bias.
 *
 * Memory: every pointer argument is DEVICE memory owned by the caller (for
 * example torch CUDA tensors).  The library allocates nothing and keeps no state
 * between calls other than the optional profiling records below.  Activations
 * are NCHW contiguous in the dtype of the descriptor; all parameters and all
 * parameter gradients are float32, contiguous:
 *   w0 [C][k][k], b0 [C] (may be NULL = no bias), s0 [C],
 *   wl [levels][C][4][k][k], sl [levels][C][4]  (may be NULL when levels == 0).
 * bf16 values are stored as bfloat16 bit patterns and f16 values as IEEE
 * binary16 bit patterns (16 bits each); arithmetic is float32 throughout; 16-bit
 * results are rounded to nearest, ties to even.
 * Intermediates in the workspace use the activation dtype.
 *
 * Streams: each call enqueues its kernels on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without synchronising.  Argument errors are
 * reported before anything is enqueued; a failed launch returns WTCONV_ERR_HIP.
 * Calls that share a workspace must be ordered on one stream.
 *
 * Thread safety: calls are reentrant; only the profiling switch is global.
 */
#ifndef WTCONV_H
#define WTCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WTCONV_VERSION 1
#define WTCONV_MAX_LEVELS 8

/* Symbols of the library's C interface (everything else in it is hidden). */
#if defined(__GNUC__)
#define WTCONV_API __attribute__((visibility("default")))
#else
#define WTCONV_API
#endif

/* Activation storage type. */
enum wtconv_dtype { WTCONV_F32 = 0, WTCONV_BF16 = 1, WTCONV_F16 = 2 };

/* Operation selector for wtconv_workspace_size. */
enum wtconv_op { WTCONV_OP_FORWARD = 0, WTCONV_OP_BACKWARD_INPUT = 1, WTCONV_OP_BACKWARD_WEIGHT = 2 };

/* Status codes (0 = success, negative = error; nothing was enqueued on error,
 * except for WTCONV_ERR_HIP which may follow earlier successful launches). */
enum wtconv_status {
    WTCONV_OK = 0,
    WTCONV_ERR_SHAPE = -1,     /* n, c, h or w negative, or a tensor too large */
    WTCONV_ERR_KERNEL = -2,    /* k is not one of the compiled sizes 3, 5, 7 */
    WTCONV_ERR_LEVELS = -3,    /* levels < 0 or > WTCONV_MAX_LEVELS */
    WTCONV_ERR_DTYPE = -4,     /* dtype is not a wtconv_dtype */
    WTCONV_ERR_NULL = -5,      /* a required pointer (or the descriptor) is NULL */
    WTCONV_ERR_WORKSPACE = -6, /* workspace NULL or smaller than wtconv_workspace_size */
    WTCONV_ERR_ALIGN = -7,     /* a pointer is not aligned to its element size */
    WTCONV_ERR_OP = -8,        /* unknown wtconv_op */
    WTCONV_ERR_HIP = -9,       /* a kernel launch failed */
    WTCONV_ERR_SCRATCH = -10   /* wtconv_backward_weight_noalloc: the shape needs more workspace
                                  than WTCONV_STATIC_SCRATCH_BYTES */
};

/* Shape of one layer call.  An empty tensor (any of n, c, h, w equal to 0) is
 * valid: forward and backward_input do nothing, backward_weight writes zero
 * gradients. */
typedef struct wtconv_desc {
    int32_t n, c, h, w; /* activation shape, NCHW */
    int32_t k;          /* odd kernel size of the base and every level: 3, 5 or 7 */
    int32_t levels;     /* Haar decomposition levels L, 0..WTCONV_MAX_LEVELS */
    int32_t dtype;      /* enum wtconv_dtype */
    int32_t reserved;   /* must be 0 */
} wtconv_desc;

/* Bytes of device workspace the operation needs for this shape (written to
 * *bytes; 0 is possible).  Returns a status code. */
WTCONV_API int wtconv_workspace_size(const wtconv_desc *desc, int op, size_t *bytes);

/* Forward pass, §2.1 Algorithm 1 evaluated as in §4 of the paper.  Planes up to
 * 64 x 64 with L >= 1: one launch of a kernel that keeps a plane and its whole
 * Haar pyramid in LDS (bands recomputed with the butterfly of Eq. 5, filtered
 * with scale-folded weights, Eq. 8, synthesised in closed form, Proposition 2 /
 * Eq. 7, plus the base convolution and bias); no workspace.  Larger planes: per
 * level, one kernel recomputes the butterfly from an LDS-staged tile of the
 * carrier and filters the four bands; one final kernel adds the base
 * convolution, the bias and the bit-indexed synthesis of all levels and stores
 * y (L + 1 launches, coefficients and carriers in the workspace).
 *   x [n][c][h][w] in, y [n][c][h][w] out (must not alias x). */
WTCONV_API int wtconv_forward(const wtconv_desc *desc, const void *x, const float *w0, const float *b0,
                   const float *s0, const float *wl, const float *sl, void *y, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Input gradient dx = dL/dx for the upstream gradient dy.  The layer is linear
 * in x and the Haar matrix is its own transpose (§2.2 Proposition 1, Eq. 1), so
 * the adjoint is the forward pipeline run on dy with every k x k kernel turned
 * by 180 degrees and no bias (scales unchanged).
 *   dy [n][c][h][w] in, dx [n][c][h][w] out (must not alias dy).
 * The same kernels and workspace as the forward pass. */
WTCONV_API int wtconv_backward_input(const wtconv_desc *desc, const void *dy, const float *w0, const float *s0,
                          const float *wl, const float *sl, void *dx, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Parameter gradients for input x and upstream gradient dy, recovered from the
 * folded-weight gradients with §4.3 Eq. 9:
 *   dW = s * dW~,  db = s0 * db~,  ds = <dW~, W> (+ db~ * b on the base path).
 * Outputs are overwritten (not accumulated), float32:
 *   dw0 [C][k][k], db0 [C] (may be NULL), ds0 [C], dwl [L][C][4][k][k], dsl [L][C][4].
 * Reductions are two-stage with a fixed order (lanes, then a fixed-order sum
 * over workgroup partials kept in the workspace), so results are bitwise
 * repeatable for a given shape.  Planes up to 64 x 64: three launches (levels,
 * base, finalize); larger planes: L + 2 (one per level, base, finalize). */
WTCONV_API int wtconv_backward_weight(const wtconv_desc *desc, const void *x, const void *dy, const float *w0,
                           const float *b0, const float *s0, const float *wl, const float *sl,
                           float *dw0, float *db0, float *ds0, float *dwl, float *dsl,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the library's static device scratch used by
 * wtconv_backward_weight_noalloc (one array per device, held until the process
 * ends). */
#define WTCONV_STATIC_SCRATCH_BYTES (16u << 20)

/* wtconv_backward_weight without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus the workspace), kernels
 * and results as wtconv_backward_weight; its workspace is a static array of
 * WTCONV_STATIC_SCRATCH_BYTES per device inside the library (the device address is
 * looked up once per device, on its first call there).  No allocation happens in
 * the call.  A shape whose weight-gradient workspace (wtconv_workspace_size with
 * WTCONV_OP_BACKWARD_WEIGHT) exceeds WTCONV_STATIC_SCRATCH_BYTES is refused with
 * WTCONV_ERR_SCRATCH before anything is enqueued; every shape that the
 * plane-resident kernels handle at ordinary channel counts fits.  All calls on one
 * device share its array: calls that overlap in time on that device (different
 * streams, or host threads without ordering) race and give wrong results; calls
 * ordered on one stream are safe.  Nothing in the array needs clearing between
 * calls (each call writes every value it reads). */
WTCONV_API int wtconv_backward_weight_noalloc(const wtconv_desc *desc, const void *x, const void *dy,
                                              const float *w0, const float *b0, const float *s0, const float *wl,
                                              const float *sl, float *dw0, float *db0, float *ds0, float *dwl,
                                              float *dsl, void *stream);

/* Launch plan of an operation for this shape, assuming activation pointers aligned
 * to 16 bytes (as device allocations are): one entry per kernel launch the call
 * would enqueue, in order, named as the profiling records name them (see below).
 * Writes up to max_entries entries and the total count to *n_entries.  Host only:
 * nothing is enqueued.  Returns a status code. */
typedef struct wtconv_launch {
    char name[64];       /* kernel family, k, dtype and level, e.g. "level_fwd<5,bf16>#2" */
    int64_t workgroups;  /* grid size in workgroups */
    int32_t threads;     /* workgroup size */
    int32_t lds_bytes;   /* dynamic LDS per workgroup */
    int32_t variant;     /* plane-resident kernels: the compiled variant, 16 CW + RH (cells per
                            staging item, cell rows per item), plus 256 for the base-only
                            forward of levels = 0; 0 for the other kernels */
    int32_t reserved;    /* 0 */
} wtconv_launch;

WTCONV_API int wtconv_plan_launches(const wtconv_desc *desc, int op, wtconv_launch *out, int max_entries,
                         int *n_entries);

/* Human-readable text of a status code (static storage). */
WTCONV_API const char *wtconv_status_string(int status);

/* Library version (WTCONV_VERSION). */
WTCONV_API int wtconv_version(void);

/* ---- Per-kernel timing (tracing) ----------------------------------------
 * While profiling is on, every kernel launch is bracketed by two hipEvents
 * recorded on the launch stream.  wtconv_profile_end waits for those events,
 * aggregates them by kernel name into `out` (up to `max_entries` entries, the
 * count written to *n_entries) and switches profiling off.  Not meant to be
 * used from several threads at once. */
typedef struct wtconv_kernel_time {
    char name[64];   /* kernel family, k, dtype and level, e.g. "level_fwd<5,bf16>#1" */
    int32_t count;   /* launches recorded */
    double total_ms; /* sum of event-to-event durations */
    double min_ms, max_ms;
} wtconv_kernel_time;

WTCONV_API int wtconv_profile_begin(void);
WTCONV_API int wtconv_profile_end(wtconv_kernel_time *out, int max_entries, int *n_entries);

#ifdef __cplusplus
}
#endif

#endif /* WTCONV_H */
