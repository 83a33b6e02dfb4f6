/*
 * Driver for the C oracle built with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Every tensor is its own heap block of exactly
 * the size its shape implies, so a read or write one element past any of
 * them is reported.  Runs both routines over small shapes (empty sequence,
 * single token, N = 1, ragged sizes, several groups), with each optional
 * input present and absent, each flag on and off, on one and two threads;
 * checks the return codes, that bad arguments are refused, and that every
 * output is finite.  Exit status 0: no finding.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_s6_fwd(const double* u, const double* delta, const double* A, const double* Bm,
                  const double* Cm, const double* Dskip, const double* z,
                  const double* delta_bias, int delta_softplus, int zoh, const double* h0,
                  double* y, double* h_last, int64_t B, int64_t L, int64_t D, int64_t N,
                  int nthreads);
int oracle_ssd_fwd(const double* X, const double* delta, const double* A, const double* Bm,
                   const double* Cm, const double* Dskip, const double* z,
                   const double* delta_bias, int delta_softplus, const double* h0, double* Y,
                   double* h_last, int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                   int64_t N, int nthreads);

static uint64_t g_state = 12345;
static double uniform(void) {   /* xorshift64*, in [-1, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

/* exactly n doubles (one byte for n = 0, so every pointer is a valid block) */
static double* vec(int64_t n, double scale, double shift) {
    double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    for (int64_t i = 0; i < n; ++i) p[i] = shift + scale * uniform();
    return p;
}

static int g_fail = 0;
static void finite(const char* what, const double* p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) { fprintf(stderr, "%s[%lld] not finite\n", what, (long long)i); ++g_fail; return; }
}

static void s6_case(int64_t B, int64_t L, int64_t D, int64_t N, int opt) {
    const int has_D = opt & 1, has_z = opt & 2, has_bias = opt & 4, has_h0 = opt & 8;
    const int softplus = (opt >> 4) & 1, zoh = (opt >> 5) & 1, threads = 1 + ((opt >> 6) & 1);
    double *u = vec(B * L * D, 1, 0), *dl = vec(B * L * D, 0.5, softplus ? -1.0 : 0.6);
    double *A = vec(D * N, 0.5, -1.0), *Bm = vec(B * L * N, 1, 0), *Cm = vec(B * L * N, 1, 0);
    double *Dk = has_D ? vec(D, 1, 0) : NULL, *z = has_z ? vec(B * L * D, 2, 0) : NULL;
    double *bias = has_bias ? vec(D, 0.5, 0) : NULL, *h0 = has_h0 ? vec(B * D * N, 1, 0) : NULL;
    double *y = vec(B * L * D, 0, 0), *hl = vec(B * D * N, 0, 0);
    if (oracle_s6_fwd(u, dl, A, Bm, Cm, Dk, z, bias, softplus, zoh, h0, y, (opt & 128) ? NULL : hl,
                      B, L, D, N, threads) != 0) {
        fprintf(stderr, "s6 (%lld,%lld,%lld,%lld) opt %d failed\n", (long long)B, (long long)L,
                (long long)D, (long long)N, opt);
        ++g_fail;
    }
    finite("s6 y", y, B * L * D);
    if (!(opt & 128)) finite("s6 h_last", hl, B * D * N);
    free(u); free(dl); free(A); free(Bm); free(Cm); free(Dk); free(z); free(bias); free(h0);
    free(y); free(hl);
}

static void ssd_case(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int opt) {
    const int has_D = opt & 1, has_z = opt & 2, has_bias = opt & 4, has_h0 = opt & 8;
    const int softplus = (opt >> 4) & 1, threads = 1 + ((opt >> 5) & 1);
    double *X = vec(B * L * H * P, 1, 0), *dl = vec(B * L * H, 0.5, softplus ? -1.0 : 0.6);
    double *A = vec(H, 0.5, -1.0), *Bm = vec(B * L * G * N, 1, 0), *Cm = vec(B * L * G * N, 1, 0);
    double *Dk = has_D ? vec(H, 1, 0) : NULL, *z = has_z ? vec(B * L * H * P, 2, 0) : NULL;
    double *bias = has_bias ? vec(H, 0.5, 0) : NULL, *h0 = has_h0 ? vec(B * H * P * N, 1, 0) : NULL;
    double *Y = vec(B * L * H * P, 0, 0), *hl = vec(B * H * P * N, 0, 0);
    if (oracle_ssd_fwd(X, dl, A, Bm, Cm, Dk, z, bias, softplus, h0, Y, (opt & 64) ? NULL : hl,
                       B, L, H, P, G, N, threads) != 0) {
        fprintf(stderr, "ssd (%lld,%lld,%lld,%lld,%lld,%lld) opt %d failed\n", (long long)B,
                (long long)L, (long long)H, (long long)P, (long long)G, (long long)N, opt);
        ++g_fail;
    }
    finite("ssd Y", Y, B * L * H * P);
    if (!(opt & 64)) finite("ssd h_last", hl, B * H * P * N);
    free(X); free(dl); free(A); free(Bm); free(Cm); free(Dk); free(z); free(bias); free(h0);
    free(Y); free(hl);
}

int main(void) {
    static const int64_t s6_shapes[][4] = {
        {1, 0, 1, 1}, {1, 1, 1, 1}, {2, 5, 3, 7}, {1, 33, 16, 16}, {3, 17, 5, 64}, {1, 2, 70, 2}};
    for (size_t i = 0; i < sizeof(s6_shapes) / sizeof(s6_shapes[0]); ++i)
        for (int opt = 0; opt < 256; opt += (i < 2 ? 1 : 7))
            s6_case(s6_shapes[i][0], s6_shapes[i][1], s6_shapes[i][2], s6_shapes[i][3], opt);
    static const int64_t ssd_shapes[][6] = {
        {1, 0, 1, 1, 1, 1}, {1, 1, 1, 1, 1, 1}, {2, 9, 4, 3, 2, 5}, {1, 70, 2, 8, 1, 16},
        {2, 13, 6, 4, 3, 2}};
    for (size_t i = 0; i < sizeof(ssd_shapes) / sizeof(ssd_shapes[0]); ++i)
        for (int opt = 0; opt < 128; opt += (i < 2 ? 1 : 5))
            ssd_case(ssd_shapes[i][0], ssd_shapes[i][1], ssd_shapes[i][2], ssd_shapes[i][3],
                     ssd_shapes[i][4], ssd_shapes[i][5], opt);
    /* refused arguments */
    double one = 1.0, out = 0.0;
    if (oracle_s6_fwd(NULL, &one, &one, &one, &one, NULL, NULL, NULL, 1, 0, NULL, &out, NULL,
                      1, 1, 1, 1, 1) != -1 ||
        oracle_s6_fwd(&one, &one, &one, &one, &one, NULL, NULL, NULL, 1, 0, NULL, &out, NULL,
                      1, 1, 1, 0, 1) != -1 ||
        oracle_ssd_fwd(&one, &one, &one, &one, &one, NULL, NULL, NULL, 1, NULL, &out, NULL,
                       1, 1, 3, 1, 2, 1, 1) != -1 ||
        oracle_ssd_fwd(&one, &one, &one, &one, &one, NULL, NULL, NULL, 1, NULL, &out, NULL,
                       -1, 1, 1, 1, 1, 1, 1) != -1) {
        fprintf(stderr, "a bad argument was accepted\n");
        ++g_fail;
    }
    if (g_fail) return 1;
    printf("oracle_asan: no finding\n");
    return 0;
}
