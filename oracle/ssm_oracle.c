/*
 * ssm_oracle.c -- plain fp64 CPU reference for the selective scan (S6) and
 * for the Mamba-2 scalar-decay (SSD) form.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or table with the
 * HIP library; it is compiled with plain `gcc -O2` (no -ffast-math).
 *
 * Every routine below is the plain definition of what the method computes,
 * evaluated token by token in double precision.  The faster GPU formulations
 * (segment carry, chunked block matrices) are exact reorganisations of these
 * sums, so this loop is the yardstick for them.  The expanded per-token state
 * tensor of shape [B, L, D, N] is never formed: one channel's N-wide state is
 * carried through time.
 *
 * Sources (web pages, cited by title and section):
 *  [P5] "Selective state space" article of the Transformer-math series
 *       (aicassindra.com), sections "The mechanism: parameters as functions
 *       of the input" (shapes, A = -exp(A_log), softplus step) and
 *       "Discretization becomes a per-token operation" (elementwise
 *       exp(delta*A), first-order input term delta*B, readout sum over n).
 *  [P4] "12. Selective State Space" (runlocalai.co course), the reference
 *       `selective_scan` routine: sequential loop over t with
 *       h = dA*h + dB*u and y_t = h . C_t.
 *  [P1] "Selective State-Space Models (Mamba) and Hardware-Aware Scans"
 *       (temporalbook, section 13.2), section 2 "Selection" (softplus keeps
 *       the step positive) and section 4 (the gated block: the second branch
 *       multiplies the SSM output).
 *  [P2] "Mamba & Mamba-2 Architecture" (ai360xpert), section 3 "Mamba-2 and
 *       State Space Duality": scalar A per head times identity, the
 *       1-semiseparable matrix, Y = (M o (C B^T)) X.
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *  - input term: first-order delta*B (what the pages say implementations use);
 *    the exact zero-order-hold term is available through `zoh` = 1;
 *  - softplus(x) = log(1 + e^x), evaluated as max(x,0) + log1p(exp(-|x|));
 *    delta_bias is added inside the softplus;
 *  - skip and gate: y = (sum_n C h + Dskip*u) * silu(z), silu(z) = z*sigma(z);
 *  - initial state zero unless h0 is given;
 *  - SSD: head h reads group g = h / (H/G) of B and C; delta scales the
 *    input side (delta_s * X_s), consistent with the first-order input term.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_version(void) { return 1; }

/* log(1 + e^x) without overflow: for x > 0, x + log(1 + e^-x). */
static double sp(double x) {
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* z * sigma(z); exp(-z) may overflow to +inf for very negative z, giving
 * z / inf = -0, which is the correct limit. */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * S6 forward, one (b, d) channel at a time.
 *   u, delta, z, y : [B, L, D]   (z may be NULL)
 *   A              : [D, N]      continuous-time diagonal, already -exp(A_log)
 *   Bm, Cm         : [B, L, N]   shared by all D channels of a batch row
 *   Dskip, delta_bias : [D] or NULL
 *   h0, h_last     : [B, D, N]   (h0 may be NULL = zeros; h_last may be NULL)
 *   zoh            : 0 -> dB = delta*B (first order); 1 -> exact ZOH,
 *                    dB = (exp(delta*A) - 1) / A * B  (delta*B where A == 0)
 * Returns 0, or -1 on a bad argument.
 */
int oracle_s6_fwd(const double* u, const double* delta, const double* A,
                  const double* Bm, const double* Cm, const double* Dskip,
                  const double* z, const double* delta_bias, int delta_softplus,
                  int zoh, const double* h0, double* y, double* h_last,
                  int64_t B, int64_t L, int64_t D, int64_t N, int nthreads) {
    if (!u || !delta || !A || !Bm || !Cm || !y) return -1;
    if (B < 0 || L < 0 || D < 0 || N <= 0) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t channels = B * D;
#pragma omp parallel
    {
        double* h = (double*)malloc((size_t)N * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t c = 0; c < channels; ++c) {
            const int64_t b = c / D, d = c % D;
            for (int64_t n = 0; n < N; ++n)
                h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * D + d;  /* [B,L,D] index */
                const int64_t r = (b * L + t) * N;      /* row of B_t, C_t */
                double x = delta[i] + (delta_bias ? delta_bias[d] : 0.0);
                const double dt = delta_softplus ? sp(x) : x;
                const double ut = u[i];
                for (int64_t n = 0; n < N; ++n) {
                    const double a = A[d * N + n];
                    const double dA = exp(dt * a);
                    double dB;
                    if (zoh && a != 0.0)
                        dB = expm1(dt * a) / a * Bm[r + n];
                    else
                        dB = dt * Bm[r + n];
                    h[n] = dA * h[n] + dB * ut;
                }
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += Cm[r + n] * h[n];
                if (Dskip) acc += Dskip[d] * ut;
                if (z) acc *= silu(z[i]);
                y[i] = acc;
            }
            if (h_last)
                for (int64_t n = 0; n < N; ++n) h_last[(b * D + d) * N + n] = h[n];
        }
        free(h);
    }
    return 0;
}

/*
 * SSD (Mamba-2) forward: scalar decay per head, P-wide head, N-wide state.
 *   X, Y, z : [B, L, H, P]   (z may be NULL)
 *   delta   : [B, L, H]
 *   A       : [H]            scalar, negative
 *   Bm, Cm  : [B, L, G, N]   head h reads group h / (H / G)
 *   Dskip, delta_bias : [H] or NULL
 *   h0, h_last : [B, H, P, N]
 * For each (b, h) the state is a P x N matrix:
 *   S_t = exp(delta_t * A_h) * S_{t-1} + delta_t * X_t (outer) B_t
 *   Y_t = S_t C_t (+ Dskip_h * X_t) (* silu(z_t))
 * which is the recurrence whose unrolled matrix is the 1-semiseparable M of
 * the SSD section; no chunk size enters the definition.
 */
int oracle_ssd_fwd(const double* X, const double* delta, const double* A,
                   const double* Bm, const double* Cm, const double* Dskip,
                   const double* z, const double* delta_bias, int delta_softplus,
                   const double* h0, double* Y, double* h_last, int64_t B,
                   int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                   int nthreads) {
    if (!X || !delta || !A || !Bm || !Cm || !Y) return -1;
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0) return -1;
    if (H % G != 0) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t heads_per_group = H / G;
    const int64_t pairs = B * H;
#pragma omp parallel
    {
        double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t c = 0; c < pairs; ++c) {
            const int64_t b = c / H, hh = c % H, g = hh / heads_per_group;
            for (int64_t k = 0; k < P * N; ++k)
                S[k] = h0 ? h0[(b * H + hh) * P * N + k] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double x = delta[(b * L + t) * H + hh] +
                           (delta_bias ? delta_bias[hh] : 0.0);
                const double dt = delta_softplus ? sp(x) : x;
                const double a = exp(dt * A[hh]);
                const double* xt = X + ((b * L + t) * H + hh) * P;
                const double* bt = Bm + ((b * L + t) * G + g) * N;
                const double* ct = Cm + ((b * L + t) * G + g) * N;
                double* yt = Y + ((b * L + t) * H + hh) * P;
                for (int64_t p = 0; p < P; ++p) {
                    const double w = dt * xt[p];
                    double* row = S + p * N;
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        row[n] = a * row[n] + w * bt[n];
                        acc += ct[n] * row[n];
                    }
                    if (Dskip) acc += Dskip[hh] * xt[p];
                    if (z) acc *= silu(z[((b * L + t) * H + hh) * P + p]);
                    yt[p] = acc;
                }
            }
            if (h_last)
                for (int64_t k = 0; k < P * N; ++k)
                    h_last[(b * H + hh) * P * N + k] = S[k];
        }
        free(S);
    }
    return 0;
}
