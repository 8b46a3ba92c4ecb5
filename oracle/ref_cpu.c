/*
 * ref_cpu.c -- plain C, fp64 sequential recurrence of the Mamba-3 scan.
 *
 * TEST INFRASTRUCTURE ONLY: the CPU oracle and the timed CPU baseline.  It is
 * loaded only by the test suite, the smoke check and the benchmark's CPU
 * baseline; the GPU library never links it and shares no code with it.
 *
 * What it computes, token by token for every selected (batch, head) stream,
 * is the recurrence of "Mamba-3: Improved Sequence Modeling using State Space
 * Principles" (intuitivepapers.ai):
 *   - "How the exponential-trapezoidal update works":
 *       h_t = a_t h_{t-1} + b_t X_{t-1}^T B_{t-1} + g_t X_t^T B_t,
 *       a_t = exp(dt_t A_t),  b_t = a_t dt_t (1 - lam_t),  g_t = lam_t dt_t,
 *     with the rate A_t = -exp(A_log) per head, or per token the negated
 *     heavy-tail activation of a rate input u (1 + u for u >= 0, 1 / (1 - u)
 *     for u < 0), clamped at -1e-4 (remarks after the decode listing)
 *   - "Computing the rotation as a data-dependent RoPE": phi_t = phi_{t-1} +
 *     dt_t theta_t per pair; B and C (bias added first) turned by phi_t on
 *     adjacent pairs (2i, 2i+1), counter-clockwise; the lagged term uses the
 *     previous token's turned B; the carry is (h, phi, B_prev, x_prev).
 *   - "MIMO: a rank-4 state update": X_t is R x P, B_t, C_t are R x N; the R
 *     writes are summed into one P x N state which is read R times,
 *     y_{t,r} = h_t C_{t,r}.
 * Inputs are float32 arrays holding storage-exact values (bf16 values are
 * exact in float32) and are upcast to double; all arithmetic is double.
 * Streams are independent, so OpenMP runs them in parallel.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TWO_PI 6.283185307179586476925286766559

/* Layouts (row-major, contiguous):
 *   x      [b][L][H][R][P]      B, C  [b][L][G][R][N]
 *   dt,lam [b][L][H]            theta [b][L][H][npairs]  (NULL if npairs == 0)
 *   A_log  [H]                  A_raw [b][L][H] per-token rate inputs (NULL = static rates)
 *   B_bias, C_bias [H][R][N] (NULL = no bias)
 *   h0 [b][H][P][N], phi0 [b][H][npairs], Bp0 [b][H][R][N], xp0 [b][H][R][P] (each may be NULL = 0)
 * Outputs, for selected stream k (k < nsel, stream (sel_b[k], sel_h[k])):
 *   y [k][L][R][P], h_out [k][P][N], phi_out [k][npairs] (in [0, 2pi)),
 *   Bp_out [k][R][N], xp_out [k][R][P]   (each output may be NULL)
 * Returns 0, or -1 on a bad argument, -2 if memory runs out.
 */
int m3ref_scan(int batch, int L, int H, int G, int P, int N, int R, int npairs,
               const float* x, const float* B, const float* C,
               const float* dt, const float* lam, const float* theta,
               const float* A_log, const float* A_raw, const float* B_bias, const float* C_bias,
               const float* h0, const float* phi0, const float* Bp0, const float* xp0,
               int nsel, const int* sel_b, const int* sel_h,
               double* y, double* h_out, double* phi_out, double* Bp_out, double* xp_out,
               int nthreads)
{
    if (batch < 1 || L < 0 || H < 1 || G < 1 || H % G || P < 1 || N < 1 || R < 1 ||
        npairs < 0 || 2 * npairs > N || nsel < 0 || (npairs > 0 && !theta))
        return -1;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int k = 0; k < nsel; ++k) {
        const int bi = sel_b[k], h = sel_h[k], g = h * G / H;
        if (bi < 0 || bi >= batch || h < 0 || h >= H) { status = -1; continue; }
        double* hs  = (double*)calloc((size_t)P * N, sizeof(double));
        double* phi = (double*)calloc((size_t)npairs + 1, sizeof(double));
        double* Bp  = (double*)calloc((size_t)R * N, sizeof(double));
        double* Xp  = (double*)calloc((size_t)R * P, sizeof(double));
        double* Bt  = (double*)calloc((size_t)R * N, sizeof(double));
        double* Ct  = (double*)calloc((size_t)R * N, sizeof(double));
        if (!hs || !phi || !Bp || !Xp || !Bt || !Ct) {
            status = -2;
            free(hs); free(phi); free(Bp); free(Xp); free(Bt); free(Ct);
            continue;
        }
        const size_t sh = (size_t)bi * H + h;
        if (h0)   for (int i = 0; i < P * N; ++i) hs[i] = h0[sh * P * N + i];
        if (phi0) for (int i = 0; i < npairs; ++i) phi[i] = phi0[sh * npairs + i];
        if (Bp0)  for (int i = 0; i < R * N; ++i) Bp[i] = Bp0[sh * R * N + i];
        if (xp0)  for (int i = 0; i < R * P; ++i) Xp[i] = xp0[sh * R * P + i];
        const double a_static = A_raw ? 0.0 : exp((double)A_log[h]);

        for (int t = 0; t < L; ++t) {
            const size_t tok = ((size_t)bi * L + t) * H + h;      /* index into [b][L][H] */
            const double d = dt[tok], lm = lam[tok];
            double rate = -a_static;
            if (A_raw) {
                const double u = A_raw[tok];
                const double ht = u >= 0.0 ? 1.0 + u : 1.0 / (1.0 - u);
                rate = -ht < -1e-4 ? -ht : -1e-4;
            }
            const double alpha = exp(d * rate);
            const double beta = alpha * d * (1.0 - lm);
            const double gamma = lm * d;
            for (int i = 0; i < npairs; ++i) phi[i] += d * (double)theta[tok * npairs + i];

            /* biased, then rotated B and C for every rank */
            const size_t bc = (((size_t)bi * L + t) * G + g) * (size_t)R * N;
            for (int r = 0; r < R; ++r) {
                for (int n = 0; n < N; ++n) {
                    double bv = B[bc + (size_t)r * N + n], cv = C[bc + (size_t)r * N + n];
                    if (B_bias) bv += B_bias[((size_t)h * R + r) * N + n];
                    if (C_bias) cv += C_bias[((size_t)h * R + r) * N + n];
                    Bt[r * N + n] = bv;
                    Ct[r * N + n] = cv;
                }
                for (int i = 0; i < npairs; ++i) {
                    const double c = cos(phi[i]), s = sin(phi[i]);
                    double* vb = &Bt[r * N + 2 * i];
                    double* vc = &Ct[r * N + 2 * i];
                    double e = vb[0], o = vb[1];
                    vb[0] = e * c - o * s; vb[1] = e * s + o * c;
                    e = vc[0]; o = vc[1];
                    vc[0] = e * c - o * s; vc[1] = e * s + o * c;
                }
            }
            const float* X = x + tok * (size_t)R * P;

            /* h <- alpha h + beta Xp^T Bp + gamma X^T Bt */
            for (int p = 0; p < P; ++p)
                for (int n = 0; n < N; ++n) {
                    double acc = alpha * hs[p * N + n];
                    for (int r = 0; r < R; ++r)
                        acc += beta * Xp[r * P + p] * Bp[r * N + n]
                             + gamma * (double)X[r * P + p] * Bt[r * N + n];
                    hs[p * N + n] = acc;
                }
            /* y_r = h C_r */
            if (y) {
                double* yo = y + ((size_t)k * L + t) * (size_t)R * P;
                for (int r = 0; r < R; ++r)
                    for (int p = 0; p < P; ++p) {
                        double acc = 0.0;
                        for (int n = 0; n < N; ++n) acc += hs[p * N + n] * Ct[r * N + n];
                        yo[r * P + p] = acc;
                    }
            }
            memcpy(Bp, Bt, sizeof(double) * (size_t)R * N);
            for (int i = 0; i < R * P; ++i) Xp[i] = X[i];
        }
        if (h_out) memcpy(h_out + (size_t)k * P * N, hs, sizeof(double) * (size_t)P * N);
        if (phi_out)
            for (int i = 0; i < npairs; ++i) {
                double w = fmod(phi[i], TWO_PI);
                if (w < 0) w += TWO_PI;
                phi_out[(size_t)k * npairs + i] = w;
            }
        if (Bp_out) memcpy(Bp_out + (size_t)k * R * N, Bp, sizeof(double) * (size_t)R * N);
        if (xp_out) memcpy(xp_out + (size_t)k * R * P, Xp, sizeof(double) * (size_t)R * P);
        free(hs); free(phi); free(Bp); free(Xp); free(Bt); free(Ct);
    }
    return status;
}

int m3ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
