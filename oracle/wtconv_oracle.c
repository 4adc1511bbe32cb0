/*
 * CPU oracle of the WTConv layer, forward and backward, in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link, load
 * or call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the GPU library.
 *
 * Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
 * Reformulation" (Aflalo, Finder, Amoyal, Treister, Freifeld), §2.1 Algorithm 1
 * (the operator as the reference implements it), §2.2 Proposition 1 and Eq. 1
 * (Haar matrix and its differentiation), §4.1 Eq. 5 (analysis of a 2x2 block),
 * Appendix A Eq. 12 (synthesis of one block).
 *
 * This is the plain, unfused definition: every level materialises its Haar
 * coefficients, filters them, scales them, and the reconstruction runs as the
 * level-by-level cascade.  None of the fused identities (scale folding, the
 * bit-indexed closed form, rotated-kernel input gradients) is used here.
 *
 * Readings of points the pages leave open (each is also listed with the design
 * notes of the repository):
 *   - the level scale has one entry per (channel, band), i.e. 4C values per level;
 *   - the 4C coefficient channels are ordered channel-major, band-minor, with the
 *     bands in Eq. 5 order (LL, LH, HL, HH);
 *   - an odd plane is zero-padded at the bottom/right before each analysis and
 *     the synthesis output is cropped back to the size before padding;
 *   - convolution is cross-correlation with zero padding (k-1)/2 on each side, in
 *     the level's own coefficient grid; k is odd;
 *   - only the base path has a bias (absent bias = 0).
 *
 * Layouts (all row-major, float64):
 *   x, y, dy, dx : [n][C][H][W]
 *   W0 [C][k][k], b0 [C] (may be NULL), s0 [C]
 *   Wl [L][C][4][k][k], sl [L][C][4]
 *   z_out (optional): for l = 1..L in turn, [n][C][4][H_l][W_l] of the filtered,
 *   scaled level coefficients Z^(l); H_l = ceil(H_{l-1} / 2), H_0 = H.
 *
 * Work is split over channels with OpenMP: every channel is an independent
 * computation (the convolutions are depthwise), so this changes no arithmetic.
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define WO_OK 0
#define WO_EINVAL (-1)
#define WO_ENOMEM (-2)

int wo_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Size of one side after zero padding to even and one Haar level. */
static int half_up(int v) { return (v + 1) / 2; }

static double at(const double *p, int h, int w, int i, int j) {
    return (i >= 0 && i < h && j >= 0 && j < w) ? p[(size_t)i * w + j] : 0.0;
}

/* Eq. 5: normalized Haar analysis of the block [a b; c d]; out = (LL, LH, HL, HH). */
static void haar_block(double a, double b, double c, double d, double out[4]) {
    out[0] = 0.5 * (a + b + c + d);
    out[1] = 0.5 * (a + b - c - d);
    out[2] = 0.5 * (a - b + c - d);
    out[3] = 0.5 * (a - b - c + d);
}

/* One analysis level of an h x w plane (zero-padded to even at the bottom/right).
 * bands: [4][ceil(h/2)][ceil(w/2)]. */
void wo_haar_analysis(int h, int w, const double *x, double *bands) {
    int ho = half_up(h), wo = half_up(w);
    size_t plane = (size_t)ho * wo;
    for (int i = 0; i < ho; ++i)
        for (int j = 0; j < wo; ++j) {
            double o[4];
            haar_block(at(x, h, w, 2 * i, 2 * j), at(x, h, w, 2 * i, 2 * j + 1),
                       at(x, h, w, 2 * i + 1, 2 * j), at(x, h, w, 2 * i + 1, 2 * j + 1), o);
            for (int b = 0; b < 4; ++b) bands[b * plane + (size_t)i * wo + j] = o[b];
        }
}

/* One synthesis level (Appendix A, Eq. 12): pixel (ry, rx) of a block receives
 * 1/2 (LL + (-1)^ry LH + (-1)^rx HL + (-1)^(ry+rx) HH).  The result is cropped
 * to h x w; bands are [4][ceil(h/2)][ceil(w/2)]. */
void wo_haar_synthesis(int h, int w, const double *bands, double *x) {
    int ho = half_up(h), wo = half_up(w);
    size_t plane = (size_t)ho * wo;
    for (int y = 0; y < h; ++y)
        for (int xx = 0; xx < w; ++xx) {
            size_t q = (size_t)(y / 2) * wo + (xx / 2);
            double sy = (y % 2) ? -1.0 : 1.0;
            double sx = (xx % 2) ? -1.0 : 1.0;
            x[(size_t)y * w + xx] = 0.5 * (bands[q] + sy * bands[plane + q] +
                                           sx * bands[2 * plane + q] + sy * sx * bands[3 * plane + q]);
        }
}

/* Depthwise convolution of one plane: cross-correlation with a k x k kernel,
 * zero padding p = (k-1)/2, output the same size as the input. */
static void xcorr(int h, int w, int k, const double *in, const double *ker, double *out) {
    int p = (k - 1) / 2;
    for (int i = 0; i < h; ++i)
        for (int j = 0; j < w; ++j) {
            double acc = 0.0;
            for (int u = 0; u < k; ++u)
                for (int v = 0; v < k; ++v)
                    acc += ker[u * k + v] * at(in, h, w, i + u - p, j + v - p);
            out[(size_t)i * w + j] = acc;
        }
}

/* Adjoint of xcorr with respect to its input: every output gradient g[i][j]
 * is sent back to the input pixels it read.  out is overwritten. */
static void xcorr_input_adjoint(int h, int w, int k, const double *g, const double *ker, double *out) {
    int p = (k - 1) / 2;
    memset(out, 0, sizeof(double) * (size_t)h * w);
    for (int i = 0; i < h; ++i)
        for (int j = 0; j < w; ++j)
            for (int u = 0; u < k; ++u)
                for (int v = 0; v < k; ++v) {
                    int ii = i + u - p, jj = j + v - p;
                    if (ii >= 0 && ii < h && jj >= 0 && jj < w)
                        out[(size_t)ii * w + jj] += ker[u * k + v] * g[(size_t)i * w + j];
                }
}

/* Gradient of xcorr with respect to its kernel, accumulated into dker. */
static void xcorr_kernel_grad(int h, int w, int k, const double *g, const double *in, double *dker) {
    int p = (k - 1) / 2;
    for (int u = 0; u < k; ++u)
        for (int v = 0; v < k; ++v) {
            double acc = 0.0;
            for (int i = 0; i < h; ++i)
                for (int j = 0; j < w; ++j)
                    acc += g[(size_t)i * w + j] * at(in, h, w, i + u - p, j + v - p);
            dker[u * k + v] += acc;
        }
}

static int check_shape(int n, int C, int H, int W, int k, int L) {
    if (n < 0 || C < 0 || H < 0 || W < 0) return WO_EINVAL;
    if (k < 1 || (k % 2) == 0) return WO_EINVAL;
    if (L < 0 || L > 16) return WO_EINVAL;
    return WO_OK;
}

/* Per-level plane sizes: hs[l], ws[l] for l = 0..L. */
static void level_sizes(int H, int W, int L, int *hs, int *ws) {
    hs[0] = H;
    ws[0] = W;
    for (int l = 1; l <= L; ++l) {
        hs[l] = half_up(hs[l - 1]);
        ws[l] = half_up(ws[l - 1]);
    }
}

/* Scratch for one channel plane at every level. */
typedef struct {
    double *Y[17];  /* Haar coefficients of the carrier, [4][H_l][W_l] */
    double *Zc[17]; /* unscaled convolution output, [4][H_l][W_l] */
    double *Z[17];  /* scaled, filtered coefficients */
    double *g[17];  /* backward: gradient at the level's coefficients */
    double *gy[17]; /* backward: gradient at Y */
    double *r0, *r1, *base, *tmp;
} scratch_t;

static void scratch_free(scratch_t *s, int L) {
    for (int l = 1; l <= L; ++l) {
        free(s->Y[l]);
        free(s->Zc[l]);
        free(s->Z[l]);
        free(s->g[l]);
        free(s->gy[l]);
    }
    free(s->r0);
    free(s->r1);
    free(s->base);
    free(s->tmp);
}

static int scratch_alloc(scratch_t *s, const int *hs, const int *ws, int L) {
    memset(s, 0, sizeof(*s));
    int ok = 1;
    size_t full = (size_t)hs[0] * ws[0] + 1;
    for (int l = 1; l <= L; ++l) {
        size_t e = 4 * (size_t)hs[l] * ws[l] + 1;
        s->Y[l] = malloc(e * sizeof(double));
        s->Zc[l] = malloc(e * sizeof(double));
        s->Z[l] = malloc(e * sizeof(double));
        s->g[l] = malloc(e * sizeof(double));
        s->gy[l] = malloc(e * sizeof(double));
        ok = ok && s->Y[l] && s->Zc[l] && s->Z[l] && s->g[l] && s->gy[l];
    }
    s->r0 = malloc(full * sizeof(double));
    s->r1 = malloc(full * sizeof(double));
    s->base = malloc(full * sizeof(double));
    s->tmp = malloc(full * sizeof(double));
    ok = ok && s->r0 && s->r1 && s->base && s->tmp;
    if (!ok) {
        scratch_free(s, L);
        return WO_ENOMEM;
    }
    return WO_OK;
}

/* Downward half of Algorithm 1 for one plane: for each level, Haar analysis of the
 * carrier (Eq. 5), depthwise filtering of the four bands, per-(channel, band)
 * scaling; the raw low-pass band is carried to the next level. */
static void decompose(const double *xp, int c, int C, int k, int L, const int *hs, const int *ws,
                      const double *Wl, const double *sl, scratch_t *s) {
    const double *carrier = xp;
    for (int l = 1; l <= L; ++l) {
        size_t pl = (size_t)hs[l] * ws[l];
        wo_haar_analysis(hs[l - 1], ws[l - 1], carrier, s->Y[l]);
        for (int b = 0; b < 4; ++b) {
            const double *ker = Wl + ((((size_t)(l - 1) * C + c) * 4 + b) * k * k);
            double sc = sl[((size_t)(l - 1) * C + c) * 4 + b];
            xcorr(hs[l], ws[l], k, s->Y[l] + b * pl, ker, s->Zc[l] + b * pl);
            for (size_t e = 0; e < pl; ++e) s->Z[l][b * pl + e] = sc * s->Zc[l][b * pl + e];
        }
        carrier = s->Y[l]; /* the LL band is the first band */
    }
}

/* Upward half of Algorithm 1: R^(L+1) = 0; R^(l) = synthesis of the level-l
 * coefficients with R^(l+1) added to their low-pass band, cropped to the size of
 * level l-1.  Returns R^(1) (hs[0] x ws[0]) in s->r0 or s->r1. */
static double *reconstruct(int L, const int *hs, const int *ws, scratch_t *s) {
    double *R = NULL;
    double *bufs[2] = {s->r0, s->r1};
    int which = 0;
    for (int l = L; l >= 1; --l) {
        size_t pl = (size_t)hs[l] * ws[l];
        double *T = s->g[l]; /* reuse as scratch for the summed bands */
        memcpy(T, s->Z[l], 4 * pl * sizeof(double));
        if (R)
            for (size_t e = 0; e < pl; ++e) T[e] += R[e];
        double *out = bufs[which];
        which ^= 1;
        wo_haar_synthesis(hs[l - 1], ws[l - 1], T, out);
        R = out;
    }
    return R;
}

int wo_forward(int n, int C, int H, int W, int k, int L, const double *x, const double *W0,
               const double *b0, const double *s0, const double *Wl, const double *sl, double *y,
               double *z_out) {
    if (check_shape(n, C, H, W, k, L)) return WO_EINVAL;
    if ((size_t)n * C * H * W == 0) return WO_OK;
    if (!x || !W0 || !s0 || !y || (L > 0 && (!Wl || !sl))) return WO_EINVAL;
    int hs[17], ws[17];
    level_sizes(H, W, L, hs, ws);
    size_t zoff[17];
    zoff[1] = 0;
    for (int l = 1; l < L; ++l) zoff[l + 1] = zoff[l] + (size_t)n * C * 4 * hs[l] * ws[l];
    int status = WO_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int c = 0; c < C; ++c) {
        scratch_t s;
        if (scratch_alloc(&s, hs, ws, L) != WO_OK) {
#pragma omp atomic write
            status = WO_ENOMEM;
            continue;
        }
        size_t P = (size_t)H * W;
        for (int i = 0; i < n; ++i) {
            const double *xp = x + ((size_t)i * C + c) * P;
            double *yp = y + ((size_t)i * C + c) * P;
            decompose(xp, c, C, k, L, hs, ws, Wl, sl, &s);
            if (z_out)
                for (int l = 1; l <= L; ++l) {
                    size_t e = 4 * (size_t)hs[l] * ws[l];
                    memcpy(z_out + zoff[l] + ((size_t)i * C + c) * e, s.Z[l], e * sizeof(double));
                }
            double *R = L > 0 ? reconstruct(L, hs, ws, &s) : NULL;
            /* base path: s0 * (x conv W0 + b) + R^(1) */
            xcorr(H, W, k, xp, W0 + (size_t)c * k * k, s.base);
            double bias = b0 ? b0[c] : 0.0;
            for (size_t e = 0; e < P; ++e) yp[e] = s0[c] * (s.base[e] + bias) + (R ? R[e] : 0.0);
        }
        scratch_free(&s, L);
    }
    return status;
}

/* Reverse mode of wo_forward, stage by stage.  The adjoint of "zero pad, then
 * analyse" is "synthesise, then crop", and vice versa (Eq. 1: the Haar matrix is
 * symmetric and its own inverse).
 *
 * Outputs (each may be NULL to skip): dx [n][C][H][W]; dW0 [C][k][k]; db0 [C];
 * ds0 [C]; dWl [L][C][4][k][k]; dsl [L][C][4].  Gradients are with respect to the
 * unscaled kernels W, the bias b and the scales s. */
int wo_backward(int n, int C, int H, int W, int k, int L, const double *x, const double *dy,
                const double *W0, const double *b0, const double *s0, const double *Wl,
                const double *sl, double *dx, double *dW0, double *db0, double *ds0, double *dWl,
                double *dsl) {
    if (check_shape(n, C, H, W, k, L)) return WO_EINVAL;
    size_t kk = (size_t)k * k;
    if (dW0) memset(dW0, 0, sizeof(double) * C * kk);
    if (db0) memset(db0, 0, sizeof(double) * C);
    if (ds0) memset(ds0, 0, sizeof(double) * C);
    if (dWl) memset(dWl, 0, sizeof(double) * L * C * 4 * kk);
    if (dsl) memset(dsl, 0, sizeof(double) * L * C * 4);
    if ((size_t)n * C * H * W == 0) return WO_OK;
    if (!x || !dy || !W0 || !s0 || (L > 0 && (!Wl || !sl))) return WO_EINVAL;
    int hs[17], ws[17];
    level_sizes(H, W, L, hs, ws);
    int status = WO_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int c = 0; c < C; ++c) {
        scratch_t s;
        if (scratch_alloc(&s, hs, ws, L) != WO_OK) {
#pragma omp atomic write
            status = WO_ENOMEM;
            continue;
        }
        size_t P = (size_t)H * W;
        double *dker = malloc(kk * sizeof(double));
        if (!dker) {
#pragma omp atomic write
            status = WO_ENOMEM;
            scratch_free(&s, L);
            continue;
        }
        double bias = b0 ? b0[c] : 0.0;
        for (int i = 0; i < n; ++i) {
            const double *xp = x + ((size_t)i * C + c) * P;
            const double *gp = dy + ((size_t)i * C + c) * P;
            /* recompute the forward intermediates of this plane */
            decompose(xp, c, C, k, L, hs, ws, Wl, sl, &s);

            /* reconstruction cascade, reversed: dR^(1) = dy; the gradient at the
             * level-l coefficients is the analysis of dR^(l); its low-pass band is
             * dR^(l+1). */
            const double *dR = gp;
            for (int l = 1; l <= L; ++l) {
                wo_haar_analysis(hs[l - 1], ws[l - 1], dR, s.g[l]);
                dR = s.g[l];
            }

            /* per level: scale, filter and kernel gradients; gradient at Y */
            for (int l = 1; l <= L; ++l) {
                size_t pl = (size_t)hs[l] * ws[l];
                for (int b = 0; b < 4; ++b) {
                    size_t pidx = ((size_t)(l - 1) * C + c) * 4 + b;
                    const double *ker = Wl + pidx * kk;
                    const double *gZ = s.g[l] + b * pl;
                    double sc = sl[pidx];
                    if (dsl) {
                        double acc = 0.0;
                        for (size_t e = 0; e < pl; ++e) acc += gZ[e] * s.Zc[l][b * pl + e];
                        dsl[pidx] += acc;
                    }
                    /* gradient at the unscaled convolution output */
                    for (size_t e = 0; e < pl; ++e) s.tmp[e] = sc * gZ[e];
                    if (dWl) {
                        memset(dker, 0, kk * sizeof(double));
                        xcorr_kernel_grad(hs[l], ws[l], k, s.tmp, s.Y[l] + b * pl, dker);
                        for (size_t t = 0; t < kk; ++t) dWl[pidx * kk + t] += dker[t];
                    }
                    xcorr_input_adjoint(hs[l], ws[l], k, s.tmp, ker, s.gy[l] + b * pl);
                }
            }

            /* analysis cascade, reversed: the carrier of level l is the LL band of
             * Y^(l), so its gradient joins the LL gradient of level l; the gradient
             * at the carrier of level l-1 is the synthesis of the level-l gradient. */
            double *dX = NULL;
            double *bufs[2] = {s.r0, s.r1};
            int which = 0;
            for (int l = L; l >= 1; --l) {
                size_t pl = (size_t)hs[l] * ws[l];
                if (dX)
                    for (size_t e = 0; e < pl; ++e) s.gy[l][e] += dX[e];
                wo_haar_synthesis(hs[l - 1], ws[l - 1], s.gy[l], bufs[which]);
                dX = bufs[which];
                which ^= 1;
            }

            /* base path: y_base = s0 * (x conv W0 + b) */
            for (size_t e = 0; e < P; ++e) s.tmp[e] = s0[c] * gp[e];
            if (dW0) xcorr_kernel_grad(H, W, k, s.tmp, xp, dW0 + (size_t)c * kk);
            if (db0) {
                double acc = 0.0;
                for (size_t e = 0; e < P; ++e) acc += s.tmp[e];
                db0[c] += acc;
            }
            if (ds0) {
                xcorr(H, W, k, xp, W0 + (size_t)c * kk, s.base);
                double acc = 0.0;
                for (size_t e = 0; e < P; ++e) acc += gp[e] * (s.base[e] + bias);
                ds0[c] += acc;
            }
            if (dx) {
                double *dxp = dx + ((size_t)i * C + c) * P;
                xcorr_input_adjoint(H, W, k, s.tmp, W0 + (size_t)c * kk, dxp);
                if (L > 0)
                    for (size_t e = 0; e < P; ++e) dxp[e] += dX[e];
            }
        }
        free(dker);
        scratch_free(&s, L);
    }
    return status;
}
