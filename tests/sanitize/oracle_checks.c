/*
 * Sanitized run of the fp64 oracle (oracle/fhd_oracle.c), built with
 * -fsanitize=address,undefined by tests/test_sanitize_cpu.py. Every input
 * and output is a malloc'd buffer of exactly the size the call may touch,
 * so an out-of-bounds read or write, a leak or undefined behaviour in the
 * oracle fails the run. The checks are closed forms of the F^H D equation
 * (page "Case study -- iterative MRI reconstruction", section 17.3) and its
 * forward operator (section 17.2): a single sample's pure phase ramp, the
 * k = 0 sum, adjointness, and results independent of the thread count.
 * Exit status 0 when every check holds.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

int oracle_fhd(const double *kx, const double *ky, const double *kz, const double *Dr,
               const double *Di, const double *x, const double *y, const double *z,
               double *rho_r, double *rho_i, long M, long N, int threads);
int oracle_forward(const double *kx, const double *ky, const double *kz, const double *rho_r,
                   const double *rho_i, const double *x, const double *y, const double *z,
                   double *Dr, double *Di, long M, long N, int threads);

static unsigned long long g_state = 0x9e3779b97f4a7c15ull;
static double uniform(double lo, double hi)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (double)(g_state >> 11) / 9007199254740992.0;
}

static double *vec(long n, double lo, double hi)
{
    double *v = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (long i = 0; i < n; ++i) v[i] = uniform(lo, hi);
    return v;
}

static int failures = 0;
static void expect(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

int main(void)
{
    const double two_pi = 2.0 * M_PI;
    /* one sample: |rho_n| = |D| and arg rho_n = 2 pi k.x_n + arg D */
    {
        const long M = 1, N = 37;
        double *kx = vec(M, -9, 9), *ky = vec(M, -9, 9), *kz = vec(M, -9, 9);
        double *Dr = vec(M, -2, 2), *Di = vec(M, -2, 2);
        double *x = vec(N, -0.5, 0.5), *y = vec(N, -0.5, 0.5), *z = vec(N, -0.5, 0.5);
        double *rr = vec(N, 0, 0), *ri = vec(N, 0, 0);
        expect(oracle_fhd(kx, ky, kz, Dr, Di, x, y, z, rr, ri, M, N, 4) == 0, "single sample call");
        for (long n = 0; n < N; ++n) {
            const double ph = two_pi * (kx[0] * x[n] + ky[0] * y[n] + kz[0] * z[n]);
            const double er = Dr[0] * cos(ph) - Di[0] * sin(ph), ei = Dr[0] * sin(ph) + Di[0] * cos(ph);
            expect(fabs(rr[n] - er) < 1e-12 && fabs(ri[n] - ei) < 1e-12, "single sample ramp");
        }
        free(kx); free(ky); free(kz); free(Dr); free(Di); free(x); free(y); free(z); free(rr); free(ri);
    }
    /* k = 0: every voxel gets sum D */
    {
        const long M = 50, N = 9;
        double *k = vec(M, 0, 0), *Dr = vec(M, -1, 1), *Di = vec(M, -1, 1);
        double *x = vec(N, -0.5, 0.5), *rr = vec(N, 0, 0), *ri = vec(N, 0, 0);
        double sr = 0, si = 0;
        for (long m = 0; m < M; ++m) { sr += Dr[m]; si += Di[m]; }
        expect(oracle_fhd(k, k, k, Dr, Di, x, x, x, rr, ri, M, N, 3) == 0, "dc call");
        for (long n = 0; n < N; ++n) expect(fabs(rr[n] - sr) < 1e-12 && fabs(ri[n] - si) < 1e-12, "dc sum");
        free(k); free(Dr); free(Di); free(x); free(rr); free(ri);
    }
    /* adjointness <F^H D, rho> = <D, F rho>, and thread counts 1, 3, 64 agree bitwise */
    {
        const long M = 23, N = 31;
        double *kx = vec(M, -6, 6), *ky = vec(M, -6, 6), *kz = vec(M, -6, 6);
        double *Dr = vec(M, -1, 1), *Di = vec(M, -1, 1);
        double *x = vec(N, -0.5, 0.5), *y = vec(N, -0.5, 0.5), *z = vec(N, -0.5, 0.5);
        double *pr = vec(N, -1, 1), *pi = vec(N, -1, 1);
        double *ar = vec(N, 0, 0), *ai = vec(N, 0, 0), *fr = vec(M, 0, 0), *fi = vec(M, 0, 0);
        double *br = vec(N, 0, 0), *bi = vec(N, 0, 0);
        expect(oracle_fhd(kx, ky, kz, Dr, Di, x, y, z, ar, ai, M, N, 1) == 0, "adjoint call");
        expect(oracle_forward(kx, ky, kz, pr, pi, x, y, z, fr, fi, M, N, 5) == 0, "forward call");
        double lr = 0, li = 0, rr_ = 0, ri_ = 0, scale = 0;
        for (long n = 0; n < N; ++n) {   /* sum (F^H D)_n conj(rho_n) */
            lr += ar[n] * pr[n] + ai[n] * pi[n];
            li += ai[n] * pr[n] - ar[n] * pi[n];
            scale += fabs(ar[n]) + fabs(ai[n]);
        }
        for (long m = 0; m < M; ++m) {   /* sum D_m conj((F rho)_m) */
            rr_ += Dr[m] * fr[m] + Di[m] * fi[m];
            ri_ += Di[m] * fr[m] - Dr[m] * fi[m];
        }
        expect(fabs(lr - rr_) < 1e-11 * scale && fabs(li - ri_) < 1e-11 * scale, "adjointness");
        expect(oracle_fhd(kx, ky, kz, Dr, Di, x, y, z, br, bi, M, N, 64) == 0, "threads > outputs");
        expect(memcmp(ar, br, (size_t)N * sizeof(double)) == 0 && memcmp(ai, bi, (size_t)N * sizeof(double)) == 0,
               "thread count independence");
        free(kx); free(ky); free(kz); free(Dr); free(Di); free(x); free(y); free(z);
        free(pr); free(pi); free(ar); free(ai); free(fr); free(fi); free(br); free(bi);
    }
    /* empty and bad sizes */
    expect(oracle_fhd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 2) == 0, "empty adjoint");
    expect(oracle_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 2) == 0, "empty forward");
    expect(oracle_fhd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, -1, 3, 2) == -1, "negative M");
    if (failures) return 1;
    printf("oracle checks passed under the sanitizers\n");
    return 0;
}
