/* oracle_driver.c — runs every oracle entry point under the address and undefined-behaviour sanitizers on
 * small inputs and edge cases (N = 1, L = 0 and 1, W = 1, A = 0, NULL optionals). It checks nothing
 * numerically (the pins do that); a sanitizer report or a nonzero status fails it. */
#include <stdio.h>
#include <stdlib.h>

#include "ssm_oracle.h"

static unsigned long long rs = 88172645463325252ull;
static double rnd(void) { /* xorshift64 in [-1, 1) */
    rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
    return (double)(rs >> 11) / (double)(1ull << 52) - 1.0;
}
static double *arr(long n) {
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

int main(void) {
    int bad = 0;
    const long shapes[][4] = {{1, 1, 1, 1}, {2, 3, 17, 4}, {1, 2, 0, 3}, {3, 5, 40, 16}};
    for (int s = 0; s < 4; ++s) {
        const long b = shapes[s][0], d = shapes[s][1], L = shapes[s][2], N = shapes[s][3];
        double *x = arr(b * d * L), *dl = arr(b * d * L), *z = arr(b * d * L), *A = arr(d * N), *B = arr(b * L * N);
        double *C = arr(b * L * N), *D = arr(d), *h0 = arr(b * d * N), *dy = arr(b * d * L), *dh = arr(b * d * N);
        for (long i = 0; i < b * d * L; ++i) dl[i] = 0.01 + 0.5 * (dl[i] + 1.0);
        for (long i = 0; i < d * N; ++i) A[i] = (i % 3 == 0) ? 0.0 : -(1.0 + A[i]);
        double *y = arr(b * d * L), *h = arr(b * d * N);
        bad |= oracle_scan_fwd(x, dl, A, B, C, D, z, h0, y, h, b, d, L, N);
        bad |= oracle_scan_fwd(x, dl, A, B, C, NULL, NULL, NULL, y, h, b, d, L, N);
        double *st = arr(b * d * N), *ys = arr(b * d), *xs = arr(b * d), *dls = arr(b * d), *zs = arr(b * d);
        double *Bs = arr(b * N), *Cs = arr(b * N);
        for (long i = 0; i < b * d; ++i) dls[i] = 0.01 + 0.5 * (dls[i] + 1.0);
        bad |= oracle_scan_step(st, xs, dls, A, Bs, Cs, D, zs, ys, b, d, N);
        bad |= oracle_scan_step(st, xs, dls, A, Bs, Cs, NULL, NULL, ys, b, d, N);
        free(xs); free(dls); free(zs); free(Bs); free(Cs);
        double *dx = arr(b * d * L), *ddl = arr(b * d * L), *dA = arr(d * N), *dB = arr(b * L * N), *dC = arr(b * L * N);
        double *dD = arr(d), *dz = arr(b * d * L), *dh0 = arr(b * d * N);
        if (L > 0) bad |= oracle_scan_bwd(x, dl, A, B, C, D, z, h0, dy, dh, dx, ddl, dA, dB, dC, dD, dz, dh0, b, d, L, N);
        for (long W = 1; W <= 4; W += 3) {
            double *w = arr(d * W), *cs = arr(b * d * (W - 1)), *xo = arr(b * d * L), *so = arr(b * d * (W - 1));
            bad |= oracle_conv1d(x, w, D, W > 1 ? cs : NULL, 1, xo, W > 1 ? so : NULL, b, d, L, W);
            bad |= oracle_conv1d(x, w, NULL, NULL, 0, xo, NULL, b, d, L, W);
            free(w); free(cs); free(xo); free(so);
        }
        double *dd = arr(d), *K = arr(d * L), *Bd = arr(d * N), *Cd = arr(d * N);
        for (long i = 0; i < d; ++i) dd[i] = 0.1 + 0.5 * (dd[i] + 1.0);
        bad |= oracle_lti_kernel(dd, A, Bd, Cd, K, d, L, N);
        if (L > 0) bad |= oracle_lti_conv(x, K, D, z, y, b, d, L);
        double abar, bc;
        oracle_zoh(0.5, 0.0, &abar, &bc);
        oracle_zoh(0.5, -1.0, &abar, &bc);
        free(x); free(dl); free(z); free(A); free(B); free(C); free(D); free(h0); free(dy); free(dh); free(y); free(h);
        free(st); free(ys); free(dx); free(ddl); free(dA); free(dB); free(dC); free(dD); free(dz); free(dh0);
        free(dd); free(K); free(Bd); free(Cd);
    }
    {   /* the scalar-decay form: H = 2 heads of P = 3 channels */
        const long b = 1, H = 2, P = 3, L = 9, N = 2, d = H * P;
        double *x = arr(b * d * L), *dl = arr(b * H * L), *A = arr(H), *B = arr(b * L * N), *C = arr(b * L * N);
        double *D = arr(d), *z = arr(b * d * L), *y = arr(b * d * L);
        for (long i = 0; i < b * H * L; ++i) dl[i] = 0.05 + 0.2 * (dl[i] + 1.0);
        A[0] = 0.0; A[1] = -1.5;
        bad |= oracle_ssd_quadratic(x, dl, A, B, C, D, z, y, b, H, P, L, N);
        free(x); free(dl); free(A); free(B); free(C); free(D); free(z); free(y);
    }
    if (bad) { printf("oracle driver: an entry point rejected valid arguments\n"); return 1; }
    printf("oracle driver: every entry point ran clean\n");
    return 0;
}
