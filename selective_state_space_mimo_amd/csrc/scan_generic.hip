// Chunked scan on the vector ALU, any supported shape, f32 or bf16 I/O.
//
// This is the full-fp32-product route (the f32 workloads need products
// rounded no further than fp32) and the route for shapes that have no MFMA
// specialisation.  One workgroup of 256 threads per (batch, head) stream walks
// the sequence chunk by chunk; everything of a chunk lives in LDS as fp32.
//
// The chunked form (quadratic inside a chunk, state carried between chunks)
// follows "The trapezoid term as a two-tap filter" of "Mamba-3: Improved
// Sequence Modeling using State Space Principles" and section 2.4 of
// "Diagonal Equivalence in State Space Models ..." (chunk-local cumulative
// log-decays, so every decay factor is exp of a difference l_t - l_s <= 0).
//
// The carried state is kept "folded": Hf = H + d_next * X_e^T Bt_e, i.e. the
// state after the chunk's last token e plus the lagged share of token e's
// write that the next token's beta = alpha * d will deliver (d_u =
// dt_u (1 - lam_u)).  With that fold every chunk reads
//   y_t  = exp(l_t) Hf_in C_t + sum_{s<=t} exp(l_t - l_s)(g_s + [s<t] d_{s+1}) (C_t.B_s) x_s
//   Hf_out = exp(l_e) Hf_in + sum_s exp(l_e - l_s)(g_s + d_{s+1}) X_s^T B_s
// where d_{e+1} is the next chunk's first token (0 after the last token, so
// the final Hf is the true state).
#include "m3_internal.h"

namespace m3 {

namespace {

constexpr int kThreads = 256;

struct GenLds {
    float *Hs, *Bt, *Ct, *X, *S, *ell, *gam, *del, *phis, *phic;
};

__device__ GenLds carve(float* sm, int P, int N, int R, int np, int qg) {
    GenLds l;
    l.Hs = sm;
    l.Bt = l.Hs + P * N;
    l.Ct = l.Bt + qg * R * N;
    l.X = l.Ct + qg * R * N;
    l.S = l.X + qg * R * P;
    l.ell = l.S + (qg * R) * (qg * R);
    l.gam = l.ell + qg;
    l.del = l.gam + qg;
    l.phis = l.del + qg + 1;
    l.phic = l.phis + qg * (np > 0 ? np : 1);
    return l;
}

__global__ __launch_bounds__(kThreads) void scan_generic_kernel(ScanArgs a, int qg) {
    extern __shared__ float sm[];
    const int P = a.P, N = a.N, R = a.R, np = a.np, L = a.L, H = a.H;
    const int bi = blockIdx.x / H, h = blockIdx.x % H, g = h * a.G / H;
    const int tid = threadIdx.x;
    GenLds s = carve(sm, P, N, R, np, qg);
    const bool dyn = a.rate_law != 0;                // per-token rate input, [b][L][H]
    const float ah = dyn ? 0.f : expf(a.A_log[h]);
    const size_t sh = (size_t)bi * H + h;           // stream index into [b][H]
    const size_t tok0 = (size_t)bi * L;              // token base into [b][L]

    // ---- prologue: running angle and the folded incoming state -------------
    for (int i = tid; i < np; i += kThreads) s.phic[i] = a.phi0 ? a.phi0[sh * np + i] : 0.f;
    {
        const size_t t0 = tok0 * H + h;
        const float d0 = a.dt[t0] * (1.f - a.lam[t0]);
        for (int e = tid; e < P * N; e += kThreads) {
            const int p = e / N, n = e % N;
            float v = a.h0 ? ld_io(a.h0, sh * P * N + e, a.st_bf16) : 0.f;
            if (a.Bp0 && a.xp0) {
                float u = 0.f;
                for (int r = 0; r < R; ++r)
                    u += ld_io(a.xp0, (sh * R + r) * P + p, a.io_bf16) *
                         ld_io(a.Bp0, (sh * R + r) * N + n, a.io_bf16);
                v += d0 * u;
            }
            s.Hs[e] = v;
        }
    }
    __syncthreads();

    int nlast = 0;
    for (int c0 = 0; c0 < L; c0 += qg) {
        const int n = min(qg, L - c0), M = n * R;
        nlast = n;
        // ---- per-token scalars ------------------------------------------------
        for (int t = tid; t <= n; t += kThreads) {
            if (t < n) {
                const size_t ti = (tok0 + c0 + t) * H + h;
                const float dt = a.dt[ti], lm = a.lam[ti];
                s.ell[t] = dyn ? dt * heavy_tail_rate(a.A_log[ti]) : -dt * ah;
                s.gam[t] = lm * dt;
                s.del[t] = dt * (1.f - lm);
            } else {
                const size_t ti = (tok0 + c0 + n) * H + h;
                s.del[n] = (c0 + n < L) ? a.dt[ti] * (1.f - a.lam[ti]) : 0.f;
            }
        }
        for (int i = tid; i < np; i += kThreads) {
            float ph = s.phic[i];
            for (int t = 0; t < n; ++t) {
                const size_t ti = (tok0 + c0 + t) * H + h;
                ph += a.dt[ti] * a.theta[ti * np + i];
                s.phis[t * np + i] = ph;
            }
        }
        __syncthreads();
        if (tid == 0)
            for (int t = 1; t < n; ++t) s.ell[t] += s.ell[t - 1];   // chunk-local cumsum of log alpha
        // ---- biased, turned B and C; x -----------------------------------------
        for (int e = tid; e < M * N; e += kThreads) {
            const int row = e / N, k = e % N, t = row / R, r = row % R;
            const size_t src = (((tok0 + c0 + t) * a.G + g) * R + r) * N;
            float bv, cv;
            if (k < 2 * np) {
                const int k0 = k & ~1;
                float b0 = ld_io(a.B, src + k0, a.io_bf16), b1 = ld_io(a.B, src + k0 + 1, a.io_bf16);
                float c0v = ld_io(a.C, src + k0, a.io_bf16), c1v = ld_io(a.C, src + k0 + 1, a.io_bf16);
                if (a.Bb) { b0 += a.Bb[(h * R + r) * N + k0]; b1 += a.Bb[(h * R + r) * N + k0 + 1]; }
                if (a.Cb) { c0v += a.Cb[(h * R + r) * N + k0]; c1v += a.Cb[(h * R + r) * N + k0 + 1]; }
                float sn, cs;
                sincosf(s.phis[t * np + (k >> 1)], &sn, &cs);
                if ((k & 1) == 0) { bv = b0 * cs - b1 * sn; cv = c0v * cs - c1v * sn; }
                else              { bv = b0 * sn + b1 * cs; cv = c0v * sn + c1v * cs; }
            } else {
                bv = ld_io(a.B, src + k, a.io_bf16);
                cv = ld_io(a.C, src + k, a.io_bf16);
                if (a.Bb) bv += a.Bb[(h * R + r) * N + k];
                if (a.Cb) cv += a.Cb[(h * R + r) * N + k];
            }
            s.Bt[e] = bv;
            s.Ct[e] = cv;
        }
        for (int e = tid; e < M * P; e += kThreads) {
            const int row = e / P, p = e % P, t = row / R, r = row % R;
            s.X[e] = ld_io(a.x, (((tok0 + c0 + t) * H + h) * R + r) * P + p, a.io_bf16);
        }
        __syncthreads();
        // ---- masked scores S[i][j] = w(t_i, s_j) (C_i . B_j) -----------------
        for (int e = tid; e < M * M; e += kThreads) {
            const int i = e / M, j = e % M, ti = i / R, sj = j / R;
            float v = 0.f;
            if (sj <= ti) {
                float dot = 0.f;
                for (int k = 0; k < N; ++k) dot += s.Ct[i * N + k] * s.Bt[j * N + k];
                const float w = expf(s.ell[ti] - s.ell[sj]) * (s.gam[sj] + (sj < ti ? s.del[sj + 1] : 0.f));
                v = w * dot;
            }
            s.S[e] = v;
        }
        __syncthreads();
        // ---- outputs ------------------------------------------------------------
        for (int e = tid; e < M * P; e += kThreads) {
            const int i = e / P, p = e % P, t = i / R, r = i % R;
            float off = 0.f;
            for (int k = 0; k < N; ++k) off += s.Ct[i * N + k] * s.Hs[p * N + k];
            float acc = expf(s.ell[t]) * off;
            for (int j = 0; j < (t + 1) * R; ++j) acc += s.S[i * M + j] * s.X[j * P + p];
            st_io(a.y, (((tok0 + c0 + t) * H + h) * R + r) * P + p, acc, a.io_bf16);
        }
        __syncthreads();
        // ---- folded state update -----------------------------------------------
        const float le = s.ell[n - 1];
        for (int e = tid; e < P * N; e += kThreads) {
            const int p = e / N, k = e % N;
            float acc = expf(le) * s.Hs[e];
            for (int j = 0; j < M; ++j) {
                const int sj = j / R;
                const float v = expf(le - s.ell[sj]) * (s.gam[sj] + s.del[sj + 1]);
                acc += v * s.X[j * P + p] * s.Bt[j * N + k];
            }
            s.Hs[e] = acc;
        }
        for (int i = tid; i < np; i += kThreads) s.phic[i] = wrap_2pi(s.phis[(n - 1) * np + i]);
        __syncthreads();
    }

    // ---- final carry --------------------------------------------------------------
    if (a.h1)
        for (int e = tid; e < P * N; e += kThreads) st_io(a.h1, sh * P * N + e, s.Hs[e], a.st_bf16);
    if (a.phi1)
        for (int i = tid; i < np; i += kThreads) a.phi1[sh * np + i] = s.phic[i];
    const int last = (nlast - 1) * R;
    if (a.Bp1)
        for (int e = tid; e < R * N; e += kThreads) st_io(a.Bp1, sh * R * N + e, s.Bt[last * N + e], a.io_bf16);
    if (a.xp1)
        for (int e = tid; e < R * P; e += kThreads) st_io(a.xp1, sh * R * P + e, s.X[last * P + e], a.io_bf16);
}

}  // namespace

size_t scan_generic_lds_bytes(int P, int N, int R, int np, int qg) {
    size_t f = (size_t)P * N + 2 * (size_t)qg * R * N + (size_t)qg * R * P + (size_t)(qg * R) * (qg * R) +
               3 * (size_t)qg + 1 + (size_t)qg * (np > 0 ? np : 1) + (np > 0 ? np : 1);
    return f * sizeof(float);
}

// Largest chunk <= Q whose working set fits 64 KiB of LDS (0 if none does).
int scan_generic_chunk(int P, int N, int R, int np, int Q) {
    for (int q = Q; q >= 1; --q)
        if (scan_generic_lds_bytes(P, N, R, np, q) <= 65536) return q;
    return 0;
}

hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t st) {
    const int qg = scan_generic_chunk(a.P, a.N, a.R, a.np, a.Q);
    if (qg < 1) return hipErrorInvalidValue;
    const size_t lds = scan_generic_lds_bytes(a.P, a.N, a.R, a.np, qg);
    hipLaunchKernelGGL(scan_generic_kernel, dim3(a.b * a.H), dim3(kThreads), lds, st, a, qg);
    return hipGetLastError();
}

hipError_t launch_decode_generic(const DecodeArgs& d, hipStream_t st) {
    // One decode step is the scan over one token with the carry read and
    // written in place (each workgroup reads its stream's carry before it
    // writes it back).
    ScanArgs a{};
    a.b = d.b; a.L = 1; a.H = d.H; a.G = d.G; a.P = d.P; a.N = d.N; a.R = d.R; a.np = d.np; a.Q = 1;
    a.io_bf16 = d.io_bf16; a.st_bf16 = d.st_bf16;
    a.x = d.x; a.B = d.B; a.C = d.C; a.dt = d.dt; a.lam = d.lam; a.theta = d.theta; a.A_log = d.A_log;
    a.rate_law = d.rate_law;
    a.Bb = d.Bb; a.Cb = d.Cb;
    a.h0 = d.h; a.phi0 = d.phi; a.Bp0 = d.Bp; a.xp0 = d.xp;
    a.y = d.y;
    a.h1 = d.h; a.phi1 = d.phi; a.Bp1 = d.Bp; a.xp1 = d.xp;
    a.nseg = 1; a.seglen = 1;
    return launch_scan_generic(a, st);
}

}  // namespace m3
