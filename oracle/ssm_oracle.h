/*
 * ssm_oracle.h — fp64 sequential reference of the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link, load or call this
 * library: only the test suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or constant with the GPU library.
 *
 * Sources (page title, then section / equation):
 *   [SSM-intro]  "State Space Models（SSM）とMamba" (hatohato.jp ai_intro):
 *                §2.1 continuous-time SSM, §2.2 ZOH discretisation and the discrete update,
 *                §2.3 an LTI system as a convolution y = x ∗ K̄, K̄ = (CB̄, CĀB̄, CĀ²B̄, …),
 *                §4.2 selective SSM (per-token Δ, B, C).
 *   [kasblo]     "Mambaとは？Transformer以外の系列モデル" (kasblo.com):
 *                section "状態空間モデルを一つの式から理解する" (ẋ = Ah + Bx, y = Ch + Dx; ZOH for
 *                Ā and B̄; the recurrent form h_t = Ā h_{t−1} + B̄ x_t, y_t = C h_t + D x_t),
 *                section "Mambaの核心は入力依存のDelta、B、C" (Δ_t, B_t, C_t per token; A not),
 *                section "Mamba blockのarchitecture" (main-branch output times SiLU of the gate).
 *   [sharin]     "Mamba / SSMと拡散LM" (sharin-2a1.pages.dev), section ① (the scan updates the state
 *                first and then reads it out at the same step).
 *
 * Readings where the pages leave a step open (each one is listed in the design notes):
 *   - A is diagonal, stored per channel as A[d][n]; B_t and C_t are shared by all channels of a batch
 *     row, stored as B[b][t][n], C[b][t][n].
 *   - ZOH for a diagonal entry a: Ā = exp(Δ·a), B̄ = (exp(Δ·a) − 1)/a · B; at a = 0 the continuous
 *     limit Ā = 1, B̄ = Δ·B is used.
 *   - The readout uses the updated state h_t, plus the skip term D·x_t (D may be absent = 0).
 *   - The optional gate multiplies the SSM output by silu(z) = z / (1 + exp(−z)).
 *   - Prefill starts from the zero state unless an initial state is given.
 *
 * Layout (all row-major, all values fp64):
 *   x, delta, z, y : [b][d][L]
 *   A              : [d][N]
 *   B, C           : [b][L][N]
 *   D              : [d]
 *   h0, h          : [b][d][N]
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Sequential prefill scan over every (b, d) row. D, z, h0 and h may be NULL.
 * Returns 0 on success, -1 on a NULL required pointer or a negative size. */
int oracle_scan_fwd(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *h0,
                    double *y, double *h, long b, long d, long L, long N);

/* One recurrent step per (b, d): state[b][d][N] is read as h_{t−1} and overwritten with h_t.
 * x, delta, z, y are [b][d]; B, C are [b][N]. D and z may be NULL. Returns 0 or -1. */
int oracle_scan_step(double *state, const double *x, const double *delta, const double *A,
                     const double *B, const double *C, const double *D, const double *z,
                     double *y, long b, long d, long N);

/* Gradients of oracle_scan_fwd for an upstream gradient dy [b][d][L] (and, optionally, a
 * gradient dh_final [b][d][N] on the final state). Outputs: dx, ddelta, dz [b][d][L]; dA [d][N];
 * dB, dC [b][L][N]; dD [d]; dh0 [b][d][N] (gradient on the initial state). D, z, h0, dh_final, dD,
 * dh0 may be NULL (dz is required when z is given). Forward states are recomputed.
 * Returns 0 or -1. */
int oracle_scan_bwd(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *h0,
                    const double *dy, const double *dh_final, double *dx, double *ddelta,
                    double *dA, double *dB, double *dC, double *dD, double *dz, double *dh0,
                    long b, long d, long L, long N);

/* Causal depthwise Conv1D (+ SiLU when apply_silu) per (b, d) row: xin, x_out [b][d][L]; w [d][W];
 * bias [d] or NULL; state_in / state_out [b][d][W−1] (the W−1 inputs before the sequence, oldest
 * first / the last W−1 inputs after it) or NULL (zeros / not written). Returns 0 or -1. */
int oracle_conv1d(const double *xin, const double *w, const double *bias, const double *state_in, int apply_silu,
                  double *x_out, double *state_out, long b, long d, long L, long W);

/* Time-invariant (LTI) convolution kernel per channel: with Ā = exp(Δ_d·A[d][n]) and B̄ the ZOH of
 * B[d][n] (as in oracle_zoh), K[d][k] = Σ_n C[d][n] · Ā^k · B̄ for k = 0 … L−1. delta [d]; A, B, C
 * [d][N] (every channel its own single-input single-output system); K [d][L]. Returns 0 or -1. */
int oracle_lti_kernel(const double *delta, const double *A, const double *B, const double *C, double *K,
                      long d, long L, long N);

/* LTI output by direct causal convolution: y[b][d][t] = Σ_{s≤t} K[d][t−s]·x[b][d][s] + D[d]·x[b][d][t],
 * then times silu(z[b][d][t]) when z is given. x, z, y [b][d][L]; K [d][L]; D [d]. D and z may be
 * NULL. Returns 0 or -1. */
int oracle_lti_conv(const double *x, const double *K, const double *D, const double *z, double *y, long b,
                    long d, long L);

/* The scalar-decay case in its quadratic ("dual", masked-attention) form. Channels come in H heads of P
 * (d = H·P, channel h·P + p); every head has one scalar a_h (A = a_h·I for all N states) and one step
 * delta[b][h][t] shared by its P channels; B, C [b][L][N] as for oracle_scan_fwd. Then
 *   y[b][hP+p][t] = Σ_{s<=t} (C_t·B_s) · exp(a_h Σ_{r=s+1..t} Δ_r) · β_s · x[b][hP+p][s] + D·x, (· silu(z)),
 * with β_s = (exp(Δ_s a_h) − 1)/a_h (Δ_s at a_h = 0), the recurrence of oracle_scan_fwd unrolled.
 * x, z, y [b][H·P][L]; delta [b][H][L]; A [H]; D [H·P] or NULL; z may be NULL. Returns 0 or -1. */
int oracle_ssd_quadratic(const double *x, const double *delta, const double *A, const double *B, const double *C,
                         const double *D, const double *z, double *y, long b, long H, long P, long L, long N);

/* ZOH coefficients of one diagonal entry: *abar = exp(delta·a), *bcoef = (exp(delta·a) − 1)/a
 * (delta at a = 0), so that B̄ = bcoef · B. */
void oracle_zoh(double delta, double a, double *abar, double *bcoef);

#ifdef __cplusplus
}
#endif
#endif
