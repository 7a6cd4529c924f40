/*
 * oracle_checks.c - host driver that runs every entry point of the fp64
 * oracle (oracle/gdn_oracle.c) on small inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer. Test infrastructure only.
 *
 * Each call covers a layout corner: packed sequences with an empty one and a
 * one-token one, d_k != d_v, grouped channels of the convolution, a NULL
 * initial state and a NULL final state, and the argument checks (a NULL
 * pointer or a decreasing offset must return -1 without touching memory).
 * Any out-of-bounds access or undefined operation aborts the process under
 * the sanitizers; the few invariants checked here (beta = 0 with alpha = 1
 * keeps the state; S_t k_t = v_t for a unit key and beta = 1) make a
 * silently wrong build fail too. Exit status 0 means every check passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gdn_recurrent(const double *, const double *, const double *, const double *,
                         const double *, const double *, double *, double *, const int64_t *,
                         int, int, int, int, double, int);
int oracle_gdn_recurrent_channel(const double *, const double *, const double *, const double *,
                                 const double *, const double *, double *, double *,
                                 const int64_t *, int, int, int, int, double, int);
int oracle_causal_conv_silu(const double *, const double *, double *, const int64_t *, int, int,
                            int, int);
int oracle_l2norm_rows(double *, int64_t, int, double);
int oracle_gates(const double *, const double *, const double *, const double *, double *,
                 double *, int64_t, int);
int oracle_gated_rmsnorm(const double *, const double *, const double *, double *, int64_t, int,
                         double);

static uint64_t lcg = 12345;
static double rnd(void)
{
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(lcg >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *arr(size_t n)
{
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static int fails = 0;
#define CHECK(c, msg) do { if (!(c)) { fprintf(stderr, "FAIL: %s\n", msg); ++fails; } } while (0)

int main(void)
{
    enum { H = 3, DK = 8, DV = 5, N = 4 };
    const int64_t cu[N + 1] = {0, 0, 1, 9, 20};       /* empty, one token, 8, 11 */
    const int64_t T = cu[N];
    double *q = arr(T * H * DK), *k = arr(T * H * DK), *v = arr(T * H * DV);
    double *g = arr(T * H), *beta = arr(T * H), *o = arr(T * H * DV);
    double *s0 = arr((size_t)N * H * DV * DK), *s1 = arr((size_t)N * H * DV * DK);
    for (int64_t i = 0; i < T * H; ++i) { g[i] = -fabs(g[i]); beta[i] = 0.5 * (beta[i] + 1.0); }

    CHECK(oracle_gdn_recurrent(q, k, v, g, beta, s0, s1, o, cu, N, H, DK, DV, 0.5, 2) == 0, "recurrent");
    CHECK(memcmp(s0, s1, sizeof(double) * H * DV * DK) == 0, "empty sequence keeps its state");
    CHECK(oracle_gdn_recurrent(q, k, v, g, beta, NULL, NULL, o, cu, N, H, DK, DV, 1.0, 1) == 0, "no states");

    /* per-channel decay: g is [T][H][DK] */
    double *gc = arr(T * H * DK);
    for (int64_t i = 0; i < T * H * DK; ++i) gc[i] = -fabs(gc[i]);
    CHECK(oracle_gdn_recurrent_channel(q, k, v, gc, beta, s0, s1, o, cu, N, H, DK, DV, 0.5, 2) == 0, "channel");

    /* beta = 0, alpha = 1: the state passes through unchanged */
    double *z = calloc(T * H, sizeof(double));
    CHECK(oracle_gdn_recurrent(q, k, v, z, z, s0, s1, o, cu, N, H, DK, DV, 1.0, 1) == 0, "identity run");
    CHECK(memcmp(s0, s1, sizeof(double) * (size_t)N * H * DV * DK) == 0, "beta = 0, alpha = 1 keeps S");

    /* unit key, beta = 1: S_1 k_1 = v_1 for one token from any S_0 */
    {
        const int64_t cu1[2] = {0, 1};
        double kk[DK], qq[DK], vv[DV], one = 1.0, g0 = -0.3, oo[DV];
        double S0[DV * DK], S1[DV * DK], nk = 0.0;
        for (int j = 0; j < DK; ++j) { kk[j] = rnd(); qq[j] = rnd(); nk += kk[j] * kk[j]; }
        for (int j = 0; j < DK; ++j) kk[j] /= sqrt(nk);
        for (int i = 0; i < DV; ++i) vv[i] = rnd();
        for (int i = 0; i < DV * DK; ++i) S0[i] = rnd();
        CHECK(oracle_gdn_recurrent(qq, kk, vv, &g0, &one, S0, S1, oo, cu1, 1, 1, DK, DV, 1.0, 1) == 0, "one token");
        for (int i = 0; i < DV; ++i) {
            double r = 0.0;
            for (int j = 0; j < DK; ++j) r += S1[i * DK + j] * kk[j];
            CHECK(fabs(r - vv[i]) < 1e-12, "S_t k_t = v_t");
        }
    }

    /* argument checks never touch memory */
    const int64_t bad[3] = {0, 5, 2};
    CHECK(oracle_gdn_recurrent(NULL, k, v, g, beta, NULL, NULL, o, cu, N, H, DK, DV, 1.0, 1) == -1, "NULL q");
    CHECK(oracle_gdn_recurrent(q, k, v, g, beta, NULL, NULL, o, bad, 2, H, DK, DV, 1.0, 1) == -1, "decreasing cu");
    CHECK(oracle_gdn_recurrent_channel(q, k, v, gc, beta, NULL, NULL, o, bad, 2, H, DK, DV, 1.0, 1) == -1, "channel decreasing cu");

    /* prologue / epilogue pieces */
    {
        enum { C = 7 };
        double *x = arr(T * C), *w = arr(C * 4), *y = arr(T * C);
        CHECK(oracle_causal_conv_silu(x, w, y, cu, N, C, 4, 1) == 0, "conv");
        double *rows = arr(T * DK);
        CHECK(oracle_l2norm_rows(rows, T, DK, 1e-6) == 0, "l2norm");
        double *a = arr(T * H), *b = arr(T * H), *A = arr(H), *gg = arr(T * H), *bb = arr(T * H);
        for (int h = 0; h < H; ++h) A[h] = fabs(A[h]) + 0.5;
        CHECK(oracle_gates(a, b, A, NULL, gg, bb, T, H) == 0, "gates");
        CHECK(oracle_gates(a, b, A, A, gg, bb, T, H) == 0, "gates with bias");
        double *yy = arr(T * H * DV), *zz = arr(T * H * DV), *out = arr(T * H * DV), *nw = arr(DV);
        CHECK(oracle_gated_rmsnorm(yy, zz, NULL, out, T * H, DV, 1e-6) == 0, "rmsnorm");
        CHECK(oracle_gated_rmsnorm(yy, zz, nw, out, T * H, DV, 1e-6) == 0, "rmsnorm weighted");
        free(x); free(w); free(y); free(rows); free(a); free(b); free(A); free(gg); free(bb);
        free(yy); free(zz); free(out); free(nw);
    }
    free(q); free(k); free(v); free(g); free(beta); free(o); free(s0); free(s1); free(gc); free(z);
    if (fails) { fprintf(stderr, "%d check(s) failed\n", fails); return 1; }
    printf("oracle sanitizer checks: ok\n");
    return 0;
}
