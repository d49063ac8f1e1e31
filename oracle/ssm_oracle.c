/*
 * ssm_oracle.c — plain, sequential, fp64 reference of the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY (see ssm_oracle.h). No blocking, no reordering, no parallel scan:
 * every (b, d) row is walked from t = 0 to L − 1 exactly as the recurrence is written.
 */
#include "ssm_oracle.h"

#include <math.h>
#include <stddef.h>

/* Zero-order hold for one diagonal entry.
 * "State Space Models（SSM）とMamba" §2.2 and "Mambaとは？Transformer以外の系列モデル",
 * section 状態空間モデルを一つの式から理解する: Ā = exp(ΔA), B̄ = (ΔA)^{-1}(exp(ΔA) − I)·ΔB.
 * For a scalar (diagonal) entry a this is B̄ = (exp(Δa) − 1)/a · B; expm1 keeps it accurate for
 * small Δa, and at a = 0 the expression's limit Δ·B is used (Ā = 1). */
void oracle_zoh(double delta, double a, double *abar, double *bcoef) {
    double u = delta * a;
    *abar = exp(u);
    *bcoef = (a != 0.0) ? expm1(u) / a : delta;
}

/* silu(v) = v · σ(v) = v / (1 + exp(−v)); the gate branch of the Mamba block
 * ("Mambaとは？…", section Mamba blockのarchitecture). */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* One (b, d) row. h[N] holds the running state on entry and on exit.
 * x, dl, z, y: the row's L values with stride 1; Bt, Ct: [L][N] of this batch row;
 * a: A[d][0..N); dskip: D[d] (0 if absent). */
static void scan_row(const double *x, const double *dl, const double *a, const double *Bt,
                     const double *Ct, double dskip, const double *z, double *h, double *y, long L,
                     long N) {
    for (long t = 0; t < L; ++t) {
        const double xt = x[t];
        const double dt = dl[t];
        double acc = 0.0;
        for (long n = 0; n < N; ++n) {
            double abar, bcoef;
            oracle_zoh(dt, a[n], &abar, &bcoef);
            /* h_t = Ā h_{t−1} + B̄ x_t ("State Space Models（SSM）とMamba" §2.2, discrete update). */
            h[n] = abar * h[n] + bcoef * Bt[t * N + n] * xt;
            /* y_t = C h_t with the just-updated state (both pages update first, then read). */
            acc += Ct[t * N + n] * h[n];
        }
        /* + D x_t: the skip term of the kasblo page's output equation. */
        double yt = acc + dskip * xt;
        if (z) yt *= silu(z[t]);
        y[t] = yt;
    }
}

int oracle_scan_fwd(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *h0,
                    double *y, double *h, long b, long d, long L, long N) {
    if (!x || !delta || !A || !B || !C || !y) return -1;
    if (b < 0 || d < 0 || L < 0 || N < 0) return -1;
    double hrow[4096];
    if (N > 4096) return -1;
    for (long ib = 0; ib < b; ++ib) {
        for (long id = 0; id < d; ++id) {
            const size_t row = (size_t)ib * (size_t)d + (size_t)id;
            for (long n = 0; n < N; ++n) hrow[n] = h0 ? h0[row * (size_t)N + (size_t)n] : 0.0;
            scan_row(x + row * (size_t)L, delta + row * (size_t)L, A + (size_t)id * (size_t)N,
                     B + (size_t)ib * (size_t)L * (size_t)N, C + (size_t)ib * (size_t)L * (size_t)N,
                     D ? D[id] : 0.0, z ? z + row * (size_t)L : NULL, hrow, y + row * (size_t)L, L,
                     N);
            if (h)
                for (long n = 0; n < N; ++n) h[row * (size_t)N + (size_t)n] = hrow[n];
        }
    }
    return 0;
}

int oracle_scan_step(double *state, const double *x, const double *delta, const double *A,
                     const double *B, const double *C, const double *D, const double *z,
                     double *y, long b, long d, long N) {
    if (!state || !x || !delta || !A || !B || !C || !y) return -1;
    if (b < 0 || d < 0 || N < 0) return -1;
    for (long ib = 0; ib < b; ++ib) {
        for (long id = 0; id < d; ++id) {
            const size_t row = (size_t)ib * (size_t)d + (size_t)id;
            /* A single token: the same row update with L = 1, starting from the stored state. */
            scan_row(x + row, delta + row, A + (size_t)id * (size_t)N, B + (size_t)ib * (size_t)N,
                     C + (size_t)ib * (size_t)N, D ? D[id] : 0.0, z ? z + row : NULL,
                     state + row * (size_t)N, y + row, 1, N);
        }
    }
    return 0;
}
