/*
 * ssm_oracle.c — plain, sequential, fp64 reference of the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY (see ssm_oracle.h). No blocking, no reordering, no parallel scan:
 * every (b, d) row is walked from t = 0 to L − 1 exactly as the recurrence is written.
 */
#include "ssm_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

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

/* ---------------------------------------------------------------------------------------------
 * Gradients of the prefill scan.
 *
 * The pages define only the forward computation; its gradients follow from the chain rule applied
 * to that definition, step by step and in reverse time order. The forward states are recomputed
 * from the inputs rather than stored ("Mambaとは？…", section hardware-awareとは memory trafficまで
 * 設計すること: intermediate states are recomputed for the backward pass).
 *
 * With β = (e^{Δa} − 1)/a (Δ at a = 0), h_t = Ā_t h_{t−1} + β_t B_t x_t,
 * ys_t = Σ_n C_tn h_tn + D x_t and y_t = ys_t · silu(z_t) (or ys_t without a gate), and λ_t the
 * total derivative of the loss with respect to h_t:
 *   λ_t = dys_t · C_t + Ā_{t+1} λ_{t+1}        (λ after the last step: the given d_final_state)
 *   dĀ_t = λ_t h_{t−1},  dβ_t = λ_t B_t x_t
 *   ∂Ā/∂Δ = a Ā,  ∂Ā/∂a = Δ Ā,  ∂β/∂Δ = Ā,  ∂β/∂a = (Δ Ā − β)/a  (Δ²/2 at a = 0)
 * and d(initial state) = Ā_0 λ_0.
 * ------------------------------------------------------------------------------------------- */

/* ∂β/∂a for one entry: (Δ·e^{Δa} − β)/a, and its limit Δ²/2 at a = 0. Near 0 the quotient is
 * a difference of nearly equal terms, so its Taylor series Δ²·Σ_{k≥0} (k+1)(Δa)^k/(k+2)! is summed
 * there instead (to well below fp64 rounding for |Δa| < 2^-6). */
static double dbeta_da(double delta, double a, double abar, double beta) {
    const double v = delta * a;
    if (fabs(v) < 0.015625) {
        double term = 0.5, sum = 0.0; /* term_k = (k+1) v^k / (k+2)! */
        double vk = 1.0, fact = 2.0;  /* v^k, (k+2)! */
        for (int k = 0; k < 12; ++k) {
            term = (double)(k + 1) * vk / fact;
            sum += term;
            vk *= v;
            fact *= (double)(k + 3);
        }
        return delta * delta * sum;
    }
    return (delta * abar - beta) / a;
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_scan_bwd(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *h0,
                    const double *dy, const double *dh_final, double *dx, double *ddelta,
                    double *dA, double *dB, double *dC, double *dD, double *dz, double *dh0,
                    long b, long d, long L, long N) {
    if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return -1;
    if (b < 0 || d < 0 || L < 0 || N < 0 || N > 4096) return -1;
    if (z && !dz) return -1;
    memset(dA, 0, sizeof(double) * (size_t)d * (size_t)N);
    memset(dB, 0, sizeof(double) * (size_t)b * (size_t)L * (size_t)N);
    memset(dC, 0, sizeof(double) * (size_t)b * (size_t)L * (size_t)N);
    if (dD) memset(dD, 0, sizeof(double) * (size_t)d);
    double *hs = (double *)malloc(sizeof(double) * ((size_t)L + 1) * (size_t)(N > 0 ? N : 1));
    double *lam = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!hs || !lam) {
        free(hs);
        free(lam);
        return -1;
    }
    for (long ib = 0; ib < b; ++ib) {
        for (long id = 0; id < d; ++id) {
            const size_t row = (size_t)ib * (size_t)d + (size_t)id;
            const double *xr = x + row * (size_t)L, *dr = delta + row * (size_t)L;
            const double *zr = z ? z + row * (size_t)L : NULL, *dyr = dy + row * (size_t)L;
            const double *a = A + (size_t)id * (size_t)N;
            const double *Bt = B + (size_t)ib * (size_t)L * (size_t)N;
            const double *Ct = C + (size_t)ib * (size_t)L * (size_t)N;
            const double dskip = D ? D[id] : 0.0;
            /* forward recomputation: hs[t + 1][n] = h_t, hs[0][n] = initial state */
            for (long n = 0; n < N; ++n) hs[n] = h0 ? h0[row * (size_t)N + (size_t)n] : 0.0;
            for (long t = 0; t < L; ++t) {
                for (long n = 0; n < N; ++n) {
                    double abar, beta;
                    oracle_zoh(dr[t], a[n], &abar, &beta);
                    hs[(size_t)(t + 1) * (size_t)N + (size_t)n] =
                        abar * hs[(size_t)t * (size_t)N + (size_t)n] + beta * Bt[t * N + n] * xr[t];
                }
            }
            /* backward, t = L−1 … 0; lam holds Ā_{t+1} λ_{t+1} on entry to step t */
            for (long n = 0; n < N; ++n) lam[n] = dh_final ? dh_final[row * (size_t)N + (size_t)n] : 0.0;
            for (long t = L - 1; t >= 0; --t) {
                const double xt = xr[t], dt = dr[t];
                const double *h = hs + (size_t)(t + 1) * (size_t)N;
                const double *hp = hs + (size_t)t * (size_t)N;
                double ys = dskip * xt;
                for (long n = 0; n < N; ++n) ys += Ct[t * N + n] * h[n];
                double dys = dyr[t];
                if (zr) {
                    const double sg = sigmoid(zr[t]);
                    dys = dyr[t] * zr[t] * sg;                                   /* ∂y/∂ys = silu(z) */
                    dz[row * (size_t)L + (size_t)t] = dyr[t] * ys * sg * (1.0 + zr[t] * (1.0 - sg));
                }
                if (dD) dD[id] += dys * xt;
                double gx = dys * dskip, gd = 0.0;
                for (long n = 0; n < N; ++n) {
                    double abar, beta;
                    oracle_zoh(dt, a[n], &abar, &beta);
                    const double ln = dys * Ct[t * N + n] + lam[n];             /* λ_t */
                    const double dab = ln * hp[n];                              /* ∂L/∂Ā_t */
                    const double dbe = ln * Bt[t * N + n] * xt;                 /* ∂L/∂β_t */
                    dC[((size_t)ib * (size_t)L + (size_t)t) * (size_t)N + (size_t)n] += dys * h[n];
                    dB[((size_t)ib * (size_t)L + (size_t)t) * (size_t)N + (size_t)n] += ln * beta * xt;
                    gx += ln * beta * Bt[t * N + n];
                    gd += dab * a[n] * abar + dbe * abar;
                    dA[(size_t)id * (size_t)N + (size_t)n] += dab * dt * abar + dbe * dbeta_da(dt, a[n], abar, beta);
                    lam[n] = abar * ln;
                }
                dx[row * (size_t)L + (size_t)t] = gx;
                ddelta[row * (size_t)L + (size_t)t] = gd;
            }
            if (dh0)
                for (long n = 0; n < N; ++n) dh0[row * (size_t)N + (size_t)n] = lam[n];
        }
    }
    free(hs);
    free(lam);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * The short causal depthwise Conv1D that feeds the scan in a Mamba block, and its SiLU
 * ("Mambaとは？…", section Mamba blockのarchitecture: the main branch mixes neighbouring tokens with a
 * short causal Conv1D, then applies SiLU, then the selective SSM; section training、prefill、decode:
 * in decode every layer keeps a Conv1D state next to the SSM state). Per channel d with taps
 * w[d][0..W) and bias c_d:  u_t = c_d + Σ_{k<W} w[d][k] · xin_{t−(W−1)+k},  x_t = silu(u_t) (or u_t),
 * where inputs before t = 0 come from the given state (the W−1 preceding inputs, oldest first) or are
 * zero. The state left behind holds the last W−1 inputs of the extended sequence.
 * ------------------------------------------------------------------------------------------- */
int oracle_conv1d(const double *xin, const double *w, const double *bias, const double *state_in, int apply_silu,
                  double *x_out, double *state_out, long b, long d, long L, long W) {
    if (!xin || !w || !x_out || b < 0 || d < 0 || L < 0 || W < 1) return -1;
    const long H = W - 1;
    double *ext = (double *)malloc(sizeof(double) * (size_t)(L + H > 0 ? L + H : 1));
    if (!ext) return -1;
    for (long ib = 0; ib < b; ++ib) {
        for (long id = 0; id < d; ++id) {
            const size_t row = (size_t)ib * (size_t)d + (size_t)id;
            /* the extended input: H values of history, then the L new ones */
            for (long k = 0; k < H; ++k) ext[k] = state_in ? state_in[row * (size_t)H + (size_t)k] : 0.0;
            for (long t = 0; t < L; ++t) ext[H + t] = xin[row * (size_t)L + (size_t)t];
            for (long t = 0; t < L; ++t) {
                double u = bias ? bias[id] : 0.0;
                for (long k = 0; k < W; ++k) u += w[(size_t)id * (size_t)W + (size_t)k] * ext[t + k];
                x_out[row * (size_t)L + (size_t)t] = apply_silu ? silu(u) : u;
            }
            if (state_out)
                for (long k = 0; k < H; ++k) state_out[row * (size_t)H + (size_t)k] = ext[L + k];
        }
    }
    free(ext);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * The time-invariant case as a convolution ("State Space Models（SSM）とMamba" §2.3; "Mambaとは？…",
 * section 固定SSMには「再帰」と「畳み込み」の二つの顔がある): when Ā, B̄ and C are the same at every step,
 * the zero-state recurrence unrolls into y = x ∗ K̄ with K̄ = (CB̄, CĀB̄, CĀ²B̄, …, CĀ^{L−1}B̄). Here every
 * channel is its own system with a diagonal A, so K̄_k = Σ_n C_n Ā_n^k B̄_n; Ā^k is the running product.
 * ------------------------------------------------------------------------------------------- */
int oracle_lti_kernel(const double *delta, const double *A, const double *B, const double *C, double *K,
                      long d, long L, long N) {
    if (!delta || !A || !B || !C || !K || d < 0 || L < 0 || N < 1) return -1;
    for (long id = 0; id < d; ++id) {
        double *Kd = K + (size_t)id * (size_t)L;
        for (long k = 0; k < L; ++k) Kd[k] = 0.0;
        for (long n = 0; n < N; ++n) {
            const size_t i = (size_t)id * (size_t)N + (size_t)n;
            double abar, bcoef;
            oracle_zoh(delta[id], A[i], &abar, &bcoef);
            const double cb = C[i] * bcoef * B[i];
            double power = 1.0; /* Ā^k */
            for (long k = 0; k < L; ++k) {
                Kd[k] += cb * power;
                power *= abar;
            }
        }
    }
    return 0;
}

/* y = x ∗ K̄ (causal: y_t = Σ_{s≤t} K̄_{t−s} x_s) plus the skip term D·x, then the gate, as in the
 * recurrent form's readout (same sources as scan_row). */
int oracle_lti_conv(const double *x, const double *K, const double *D, const double *z, double *y, long b,
                    long d, long L) {
    if (!x || !K || !y || b < 0 || d < 0 || L < 0) return -1;
    for (long ib = 0; ib < b; ++ib) {
        for (long id = 0; id < d; ++id) {
            const size_t row = ((size_t)ib * (size_t)d + (size_t)id) * (size_t)L;
            const double *Kd = K + (size_t)id * (size_t)L;
            for (long t = 0; t < L; ++t) {
                double acc = 0.0;
                for (long s = 0; s <= t; ++s) acc += Kd[t - s] * x[row + (size_t)s];
                double yt = acc + (D ? D[id] : 0.0) * x[row + (size_t)t];
                if (z) yt *= silu(z[row + (size_t)t]);
                y[row + (size_t)t] = yt;
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * The scalar-decay selective SSM written as one matrix acting on the whole sequence. Unrolling the
 * recurrence ("Mambaとは？…", section Mambaの核心は入力依存のDelta、B、C; "State Space Models（SSM）とMamba"
 * §4.2) gives y_t = Σ_{s<=t} C_t (Π_{r=s+1..t} Ā_r) B̄_s x_s. When A is one scalar a per head, the product
 * of the Ā_r is the scalar exp(a Σ Δ_r), so the sequence map is y = (causal mask ∘ decay ∘ C Bᵀ)(β ∘ x):
 * a masked linear attention with queries C, keys B and values x ("State Space Models（SSM）とMamba" §4.6:
 * Mamba-2's state space duality relates SSMs and linear attention). Evaluated here entry by entry,
 * O(L²) per head, with the decay exponent summed afresh for every (t, s).
 * ------------------------------------------------------------------------------------------- */
int oracle_ssd_quadratic(const double *x, const double *delta, const double *A, const double *B, const double *C,
                         const double *D, const double *z, double *y, long b, long H, long P, long L, long N) {
    if (!x || !delta || !A || !B || !C || !y || b < 0 || H < 0 || P < 1 || L < 0 || N < 1) return -1;
    const long d = H * P;
    for (long ib = 0; ib < b; ++ib) {
        const double *Bb = B + (size_t)ib * (size_t)L * (size_t)N;
        const double *Cb = C + (size_t)ib * (size_t)L * (size_t)N;
        for (long h = 0; h < H; ++h) {
            const double a = A[h];
            const double *dl = delta + ((size_t)ib * (size_t)H + (size_t)h) * (size_t)L;
            for (long t = 0; t < L; ++t) {
                for (long p = 0; p < P; ++p) {
                    const long ch = h * P + p;
                    const double *xr = x + ((size_t)ib * (size_t)d + (size_t)ch) * (size_t)L;
                    double acc = 0.0;
                    for (long s = 0; s <= t; ++s) {
                        double cb = 0.0; /* C_t · B_s */
                        for (long n = 0; n < N; ++n) cb += Cb[(size_t)t * (size_t)N + (size_t)n] * Bb[(size_t)s * (size_t)N + (size_t)n];
                        double sum = 0.0; /* Σ_{r=s+1..t} Δ_r */
                        for (long r = s + 1; r <= t; ++r) sum += dl[r];
                        double abar_s, beta_s;
                        oracle_zoh(dl[s], a, &abar_s, &beta_s);
                        acc += cb * exp(a * sum) * beta_s * xr[s];
                    }
                    double yt = acc + (D ? D[ch] : 0.0) * xr[t];
                    if (z) yt *= silu(z[((size_t)ib * (size_t)d + (size_t)ch) * (size_t)L + (size_t)t]);
                    y[((size_t)ib * (size_t)d + (size_t)ch) * (size_t)L + (size_t)t] = yt;
                }
            }
        }
    }
    return 0;
}
