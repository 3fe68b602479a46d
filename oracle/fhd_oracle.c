/*
 * fp64 CPU oracle for the F^H D step of iterative non-Cartesian MRI
 * reconstruction, and for the forward operator F it is the adjoint of.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the independent truth that the GPU
 * path is checked against. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the GPU library never does, and
 * the two share no code, headers, tables or helpers.
 *
 * Definitions (page "Case study -- iterative MRI reconstruction"):
 *   section 17.3, the F^H D equation: for every voxel n,
 *       rho_n = sum_{m<M} D_m * exp(+i * 2*pi * (k_m . x_n))
 *   section 17.2: F maps an image to k-space; it is the adjoint of F^H,
 *       D_m = sum_{n<N} rho_n * exp(-i * 2*pi * (k_m . x_n))
 * k is in cycles per field of view and x in field-of-view units, so the
 * phase in radians is 2*pi times the dot product. There is no weighting and
 * no normalisation: the sum is taken as written.
 *
 * Both functions are the plain double sums, in order m = 0..M-1 (adjoint) or
 * n = 0..N-1 (forward), with libm sin/cos in double and M_PI. They are
 * parallelised only across outputs (each thread owns a contiguous range of
 * outputs), so every output's summation order is fixed and the result does
 * not depend on the thread count. Build without -ffast-math and with
 * -ffp-contract=off.
 *
 * Parity pins (all in the CPU test suite): single-sample phase ramp, k = 0
 * sum, Cartesian-grid identity against numpy's inverse FFT, F^H F = N I on a
 * Cartesian grid, adjointness <F^H D, rho> = <D, F rho>, conjugation
 * symmetry, hand-worked fixtures, and textual mutants of this file that the
 * pins must reject.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdlib.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

typedef struct {
    /* sample side (length M) */
    const double *kx, *ky, *kz;
    /* voxel side (length N) */
    const double *x, *y, *z;
    /* values summed over: D (length M) for the adjoint, rho (length N) for F */
    const double *in_re, *in_im;
    /* results: rho (length N) for the adjoint, D (length M) for F */
    double *out_re, *out_im;
    long M, N;
    long first, last; /* output range [first, last) owned by this worker */
} oracle_job;

/* F^H D for voxels [first, last): rho_n = sum_m D_m exp(+i 2 pi k_m . x_n). */
static void *adjoint_worker(void *arg)
{
    const oracle_job *j = (const oracle_job *)arg;
    for (long n = j->first; n < j->last; ++n) {
        const double xn = j->x[n], yn = j->y[n], zn = j->z[n];
        double sum_re = 0.0, sum_im = 0.0;
        for (long m = 0; m < j->M; ++m) {
            const double theta = 2.0 * M_PI * (j->kx[m] * xn + j->ky[m] * yn + j->kz[m] * zn);
            const double c = cos(theta), s = sin(theta);
            /* (D_re + i D_im) * (c + i s) */
            sum_re += j->in_re[m] * c - j->in_im[m] * s;
            sum_im += j->in_re[m] * s + j->in_im[m] * c;
        }
        j->out_re[n] = sum_re;
        j->out_im[n] = sum_im;
    }
    return NULL;
}

/* F rho for samples [first, last): D_m = sum_n rho_n exp(-i 2 pi k_m . x_n). */
static void *forward_worker(void *arg)
{
    const oracle_job *j = (const oracle_job *)arg;
    for (long m = j->first; m < j->last; ++m) {
        const double kxm = j->kx[m], kym = j->ky[m], kzm = j->kz[m];
        double sum_re = 0.0, sum_im = 0.0;
        for (long n = 0; n < j->N; ++n) {
            const double theta = 2.0 * M_PI * (kxm * j->x[n] + kym * j->y[n] + kzm * j->z[n]);
            const double c = cos(theta), s = sin(theta);
            /* (rho_re + i rho_im) * (c - i s) */
            sum_re += j->in_re[n] * c + j->in_im[n] * s;
            sum_im += j->in_im[n] * c - j->in_re[n] * s;
        }
        j->out_re[m] = sum_re;
        j->out_im[m] = sum_im;
    }
    return NULL;
}

/* Split [0, count) into `threads` contiguous ranges and run `fn` on each. */
static int run_split(oracle_job base, long count, int threads, void *(*fn)(void *))
{
    if (threads < 1) threads = 1;
    if (threads > count) threads = (int)(count > 0 ? count : 1);
    oracle_job *jobs = (oracle_job *)calloc((size_t)threads, sizeof(oracle_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    char *spawned = (char *)calloc((size_t)threads, 1);
    if (!jobs || !tid || !spawned) {
        free(jobs);
        free(tid);
        free(spawned);
        return -1;
    }
    for (int t = 0; t < threads; ++t) {
        jobs[t] = base;
        jobs[t].first = count * t / threads;
        jobs[t].last = count * (t + 1) / threads;
    }
    /* threads 1.. run on new threads; range 0 (and any that fail to spawn)
     * runs on the calling thread */
    for (int t = 1; t < threads; ++t)
        spawned[t] = pthread_create(&tid[t], NULL, fn, &jobs[t]) == 0;
    fn(&jobs[0]);
    for (int t = 1; t < threads; ++t) {
        if (spawned[t])
            pthread_join(tid[t], NULL);
        else
            fn(&jobs[t]);
    }
    free(jobs);
    free(tid);
    free(spawned);
    return 0;
}

/*
 * rho = F^H D over N voxels and M samples, all arrays fp64.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_fhd(const double *kx, const double *ky, const double *kz,
               const double *Dr, const double *Di,
               const double *x, const double *y, const double *z,
               double *rho_r, double *rho_i, long M, long N, int threads)
{
    if (M < 0 || N < 0) return -1;
    if (N == 0) return 0;
    oracle_job b = {kx, ky, kz, x, y, z, Dr, Di, rho_r, rho_i, M, N, 0, 0};
    return run_split(b, N, threads, adjoint_worker);
}

/*
 * D = F rho over M samples and N voxels, all arrays fp64.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_forward(const double *kx, const double *ky, const double *kz,
                   const double *rho_r, const double *rho_i,
                   const double *x, const double *y, const double *z,
                   double *Dr, double *Di, long M, long N, int threads)
{
    if (M < 0 || N < 0) return -1;
    if (M == 0) return 0;
    oracle_job b = {kx, ky, kz, x, y, z, rho_r, rho_i, Dr, Di, M, N, 0, 0};
    return run_split(b, M, threads, forward_worker);
}
