/*
 * Driver for a sanitizer build of the CPU oracle (oracle/wtconv_oracle.c), built
 * with gcc -fsanitize=address,undefined by tests/test_oracle_sanitized.py.  It runs
 * the oracle's forward and backward on odd sizes, every kernel size, up to five
 * levels, with and without bias and with outputs skipped (NULL), and checks two
 * properties that hold for any input: the dot-product adjoint identity
 * <M v, g> = <v, M^T g> (Eq. 1 of the layer's paper) and the Haar round trip.
 * The sanitizers report any out-of-bounds access, leak or undefined behaviour.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int wo_forward(int n, int C, int H, int W, int k, int L, const double *x, const double *W0, const double *b0,
               const double *s0, const double *Wl, const double *sl, double *y, double *z_out);
int wo_backward(int n, int C, int H, int W, int k, int L, const double *x, const double *dy, const double *W0,
                const double *b0, const double *s0, const double *Wl, const double *sl, double *dx, double *dW0,
                double *db0, double *ds0, double *dWl, double *dsl);
void wo_haar_analysis(int h, int w, const double *x, double *bands);
void wo_haar_synthesis(int h, int w, const double *bands, double *x);

static unsigned long long state = 0x9E3779B97F4A7C15ULL;
static double rnd(void) { /* xorshift64*, uniform in [-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1DULL) >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static double *vec(size_t n) {
    double *p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

static int run(int n, int C, int H, int W, int k, int L, int bias) {
    size_t N = (size_t)n * C * H * W, kk = (size_t)k * k;
    size_t nl = (size_t)(L ? L : 1) * C;
    double *x = vec(N), *g = vec(N), *W0 = vec(C * kk), *b0 = bias ? vec(C) : NULL, *s0 = vec(C);
    double *Wl = vec(nl * 4 * kk), *sl = vec(nl * 4);
    double *y = calloc(N ? N : 1, sizeof(double)), *dx = calloc(N ? N : 1, sizeof(double));
    double *dW0 = calloc(C * kk, sizeof(double)), *db0 = calloc(C, sizeof(double)), *ds0 = calloc(C, sizeof(double));
    double *dWl = calloc(nl * 4 * kk, sizeof(double)), *dsl = calloc(nl * 4, sizeof(double));
    int bad = 0;
    /* the adjoint identity needs the linear map: no bias in this forward */
    if (wo_forward(n, C, H, W, k, L, x, W0, NULL, s0, Wl, sl, y, NULL)) bad = 1;
    if (wo_backward(n, C, H, W, k, L, x, g, W0, b0, s0, Wl, sl, dx, dW0, db0, ds0, dWl, dsl)) bad = 1;
    double lhs = 0, rhs = 0, scale = 0;
    for (size_t i = 0; i < N; ++i) {
        lhs += y[i] * g[i];
        rhs += x[i] * dx[i];
        scale += fabs(y[i] * g[i]) + fabs(x[i] * dx[i]);
    }
    if (fabs(lhs - rhs) > 1e-12 * (scale + 1.0)) {
        fprintf(stderr, "adjoint mismatch %d %d %d %d k=%d L=%d: %g vs %g\n", n, C, H, W, k, L, lhs, rhs);
        bad = 1;
    }
    /* outputs may be skipped one group at a time */
    if (wo_backward(n, C, H, W, k, L, x, g, W0, b0, s0, Wl, sl, dx, NULL, NULL, NULL, NULL, NULL)) bad = 1;
    if (wo_backward(n, C, H, W, k, L, x, g, W0, b0, s0, Wl, sl, NULL, dW0, db0, ds0, dWl, dsl)) bad = 1;
    /* forward with the coefficients returned */
    {
        size_t total = 0;
        int h = H, w = W;
        for (int l = 1; l <= L; ++l) {
            h = (h + 1) / 2;
            w = (w + 1) / 2;
            total += (size_t)n * C * 4 * h * w;
        }
        double *z = calloc(total ? total : 1, sizeof(double));
        if (wo_forward(n, C, H, W, k, L, x, W0, b0, s0, Wl, sl, y, z)) bad = 1;
        free(z);
    }
    free(x); free(g); free(W0); free(b0); free(s0); free(Wl); free(sl);
    free(y); free(dx); free(dW0); free(db0); free(ds0); free(dWl); free(dsl);
    return bad;
}

static int haar_round_trip(int h, int w) {
    double *x = vec((size_t)h * w), *r = calloc((size_t)h * w, sizeof(double));
    double *b = calloc(4 * (size_t)((h + 1) / 2) * ((w + 1) / 2), sizeof(double));
    wo_haar_analysis(h, w, x, b);
    wo_haar_synthesis(h, w, b, r);
    int bad = 0;
    for (int i = 0; i < h * w; ++i)
        if (fabs(r[i] - x[i]) > 1e-14) bad = 1;
    free(x); free(r); free(b);
    return bad;
}

int main(void) {
    static const int shapes[][6] = {
        {1, 2, 16, 16, 5, 2}, {2, 3, 7, 9, 3, 3}, {1, 2, 1, 1, 5, 3}, {2, 1, 13, 11, 7, 5},
        {1, 3, 5, 3, 5, 5}, {3, 2, 9, 14, 5, 0}, {1, 1, 33, 17, 3, 4}, {0, 2, 8, 8, 5, 2},
        {1, 2, 0, 8, 5, 1}, {2, 2, 6, 1, 7, 2},
    };
    int bad = 0;
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        for (int bias = 0; bias < 2; ++bias) {
            const int *s = shapes[i];
            if (run(s[0], s[1], s[2], s[3], s[4], s[5], bias)) {
                fprintf(stderr, "case %zu (bias %d) failed\n", i, bias);
                bad = 1;
            }
        }
    static const int planes[][2] = {{1, 1}, {2, 3}, {7, 7}, {8, 5}, {13, 16}};
    for (size_t i = 0; i < sizeof(planes) / sizeof(planes[0]); ++i)
        if (haar_round_trip(planes[i][0], planes[i][1])) {
            fprintf(stderr, "Haar round trip %d x %d failed\n", planes[i][0], planes[i][1]);
            bad = 1;
        }
    printf(bad ? "FAILED\n" : "ok\n");
    return bad;
}
