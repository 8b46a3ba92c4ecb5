/*
 * pcs_cpu.c -- plain C, fp64 recurrence of the per-coordinate selective scan
 * (the Mamba 1 preset).
 *
 * TEST INFRASTRUCTURE ONLY: the CPU oracle at full size and the timed CPU
 * baseline.  Loaded only by the test suite, the smoke check and the benchmark's
 * CPU baseline; the GPU library never links it and shares no code with it.
 *
 * For every batch b, channel d (group g = d G / D) and state coordinate n,
 * token by token ("Diagonal Equivalence in State Space Models ...",
 * section 5.1 "Per-coordinate scan" and the Mamba 1 row of its table of
 * copied-weight presets; "Mamba-3: Improved Sequence Modeling using State Space
 * Principles", section "How Mamba gets its recurrence from a differential
 * equation": decay exp(dt A), gain dt):
 *     h[n] <- exp(dt a[d][n]) h[n] + dt B[g][n] x,   a = -exp(A_log)
 *     y     = sum_n C[g][n] h[n]
 * Inputs are float32 arrays of storage-exact values, upcast to double.
 * Channels are independent; OpenMP runs them in parallel.
 *
 * Layouts (row-major): x, dt, y [b][L][D]; A_log [D][N]; B, C [b][L][G][N];
 * h0, h1 [b][D][N] (h0 may be NULL: zero).  Only channels d in [d0, d1) of every
 * batch are computed; y and h1 hold those channels only: y [b][L][d1 - d0],
 * h1 [b][d1 - d0][N].
 */
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int m3ref_pcs(int b, int L, int D, int G, int N, int d0, int d1, const float* x, const float* dt,
              const float* A_log, const float* B, const float* C, const float* h0, double* y, double* h1,
              int nthreads) {
    if (b < 0 || L < 0 || D < 1 || G < 1 || D % G || N < 1 || d0 < 0 || d1 > D || d0 > d1) return 1;
    const int W = d1 - d0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 4)
    for (long s = 0; s < (long)b * W; ++s) {
        const int bi = (int)(s / W), d = d0 + (int)(s % W), g = d * G / D;
        double* h = (double*)malloc(sizeof(double) * N);
        double* a = (double*)malloc(sizeof(double) * N);
        for (int n = 0; n < N; ++n) {
            a[n] = -exp((double)A_log[(size_t)d * N + n]);
            h[n] = h0 ? (double)h0[((size_t)bi * D + d) * N + n] : 0.0;
        }
        for (int t = 0; t < L; ++t) {
            const size_t tk = ((size_t)bi * L + t);
            const double st = dt[tk * D + d], xv = x[tk * D + d];
            const float* Bt = B + (tk * G + g) * N;
            const float* Ct = C + (tk * G + g) * N;
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                h[n] = exp(st * a[n]) * h[n] + st * (double)Bt[n] * xv;
                acc += (double)Ct[n] * h[n];
            }
            y[tk * W + (d - d0)] = acc;
        }
        for (int n = 0; n < N; ++n) h1[((size_t)bi * W + (d - d0)) * N + n] = h[n];
        free(h);
        free(a);
    }
    return 0;
}
