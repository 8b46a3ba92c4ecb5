// Backward pass of the scan: the gradients of a loss with respect to every input of
// the scan (x, B, C, dt, lambda, theta, the rate input, the biases and the initial
// carry), given the loss's gradients with respect to its outputs (dy and, optionally,
// the final carry).
//
// "Diagonal Equivalence in State Space Models: Characterization, Retrieval Rank, and
// Selective Extensions" (paperpeel.com), section 2.5 "Parallel scan and gradients":
// the state sensitivity G_t = d loss / d H_t runs backward through the transposed
// transition (a scalar decay here), G_t = alpha_{t+1} G_{t+1} + sum_r dy_t[r] (x) Ct_t[r];
// the initial carry's gradient is what is left at the start; a sensitivity for the
// final state enters as the terminal condition (section 5.5 and appendix C.2: every
// carry is differentiable).  The recurrence differentiated is the three-term update
// of "Mamba-3: Improved Sequence Modeling using State Space Principles"
// (intuitivepapers.ai), sections "How the exponential-trapezoidal update works",
// "Computing the rotation as a data-dependent RoPE" and "MIMO: a rank-4 state update".
//
// Two sweeps per (batch, head) stream, one workgroup (4 waves) each; the P x N fp32
// state (P <= 64, N <= 128) lives in registers, 32 values per lane (lg = lane / 16,
// l16 = lane % 16).  The replay gives wave w the columns 32 w .. 32 w + 31 of every row
// (its readout, a sum over rows, then finishes inside the wave); the sensitivity sweep gives
// wave w the rows 16 w .. 16 w + 15 (its v, a sum over columns, finishes inside the wave,
// and w = G^T X is kept as one partial row per wave, summed when a group's outputs are
// formed).  Tokens are staged a group at a time in LDS; the per-token work is wave-local
// (no barrier, no LDS atomics), the per-token outputs are formed after each group.
//
//   replay (forward): H_t again, token by token (never stored), read against dy:
//     dCt_t[r] = H_t^T dy_t[r], <dy_t, y_t> = sum_r Ct_t[r] . dCt_t[r]; the running
//     angles phi_t (kept for the reverse sweep) and the C side of the angle gradient.
//   adjoint (reverse): G from the last token back, with per token
//     v[r] = G_{t+1} Bt_t[r] (P values) and w[r] = G_{t+1}^T X_t[r] (N values);
//     with K_t = sum_r dy_t[r] (x) Ct_t[r] and G_t = alpha_{t+1} G_{t+1} + K_t:
//       dX_t  = (gamma_t alpha_{t+1} + beta_{t+1}) v + gamma_t K_t Bt_t   (+ d x_prev at the end)
//       dBt_t = (gamma_t alpha_{t+1} + beta_{t+1}) w + gamma_t K_t^T X_t  (+ d B_prev at the end)
//       d gamma_t = alpha_{t+1} X_t . v + sum_{r,r'} (dy_t[r'] . X_t[r]) (Ct_t[r'] . Bt_t[r])
//       d beta_{t+1} = X_t . v
//     (the K_t terms are R x R dot products: no second pass over the state).
// The decay's gradient uses the cumulative log-decay l_t = sum_{k <= t} log alpha_k:
// l_k multiplies every term read at k and divides every term written at k, so
//   d loss / d l_k = <dy_k, y_k> (+ <dH_L, H_L> at the last token) - <dX_k, X_k>_writes
// with <dX_k, X_k>_writes = gamma_k d gamma_k + beta_{k+1} d beta_{k+1}, and
// d loss / d log alpha_t = sum_{k >= t} d loss / d l_k: the reverse sweep never needs H_t.
// Shared B and C (G < H): the per-head gradients are summed into fp32 buffers by
// atomic adds and converted to the I/O dtype at the end.
#include <algorithm>

#include "m3_internal.h"

namespace m3 {

namespace {

constexpr int kT = 8;                 // tokens per staged group (replay)
constexpr int kTA = 4;                // tokens per staged group (adjoint: per-wave partial rows fit two groups per CU)
constexpr int kR4 = 4, kPP = 64, kNN = 128, kThreads = 256;

// Turned B and C rows keep column n = 16 nt + l16 at 64 (nt / 4) + 4 l16 + nt % 4: a lane's
// eight columns are two 16-byte runs, and the 16 lanes of a row group read 64 consecutive
// words per access (no bank conflict; the four row groups read the same words).
__device__ __forceinline__ int bpos(int n) { return ((n >> 6) << 6) + ((n & 15) << 2) + ((n >> 4) & 3); }


template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
// involutions inside a row of 16 lanes pairing the two halves of each level
template <int LEVEL>
__device__ __forceinline__ float row_partner(float v) {
    if constexpr (LEVEL == 8) return dpp_mov<0x140>(v);        // row mirror
    else if constexpr (LEVEL == 4) return dpp_mov<0x141>(v);   // row half mirror
    else if constexpr (LEVEL == 2) return dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    else return dpp_mov<0xB1>(v);                              // quad_perm [1,0,3,2]
}
template <int LEVEL, int CNT>
__device__ __forceinline__ void rs_row_level(float* v, bool up) {
    constexpr int HALF = CNT / 2;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const float keep = up ? v[i + HALF] : v[i];
        const float send = up ? v[i] : v[i + HALF];
        v[i] = keep + row_partner<LEVEL>(send);
    }
}
// Sum of v[16] over the 16 lanes of a row, scattered: lane l16 returns entry l16.
__device__ __forceinline__ float rs_row16(float (&v)[16], int l16) {
    rs_row_level<8, 16>(v, l16 & 8);
    rs_row_level<4, 8>(v, l16 & 4);
    rs_row_level<2, 4>(v, l16 & 2);
    rs_row_level<1, 2>(v, l16 & 1);
    return v[0];
}
// Lane swaps across wave halves and across 16-lane rows (VALU, no LDS round trip):
// swap32(a, b) returns (a with its upper 32 lanes replaced by b's lower 32, b with its lower
// 32 lanes replaced by a's upper 32); swap16 does the same between the odd rows of a and
// the even rows of b.
__device__ __forceinline__ float2 swap32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 swap16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// One reduce-scatter level across halves: the lower half keeps lo, the upper half keeps hi,
// each adding its partner's copy.
__device__ __forceinline__ float rs32(float lo, float hi, bool upper) {
    const float2 w = swap32(lo, hi);
    return upper ? hi + w.x : lo + w.y;
}
__device__ __forceinline__ float rs16(float lo, float hi, bool odd) {
    const float2 w = swap16(lo, hi);
    return odd ? hi + w.x : lo + w.y;
}
// Sum of part[r][nt] over the four 16-lane groups, scattered: group lg keeps tiles
// nt = 2 lg + i (i < 2) in out[r][i].
template <int R>
__device__ __forceinline__ void rs_groups(const float (&part)[R][8], float (&out)[R][2], int lg) {
    const bool h2 = lg & 2, h1 = lg & 1;
    float k4[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) k4[r][i] = rs32(part[r][i], part[r][4 + i], h2);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 2; ++i) out[r][i] = rs16(k4[r][i], k4[r][2 + i], h1);
}
// all-reduce inside each 8-lane half-row (involutions generating the group of 8)
__device__ __forceinline__ float sum8(float c) {
    c += row_partner<4>(c);
    c += row_partner<2>(c);
    c += row_partner<1>(c);
    return c;
}
__device__ __forceinline__ float wave_sum(float v) {
    float2 w = swap32(v, v);
    v = w.x + w.y;
    w = swap16(v, v);
    v = w.x + w.y;
    v += row_partner<8>(v);
    return sum8(v);
}
// Sum of v[8] over the wave, scattered: lanes with lane % 8 == 0 return entry
// 4 (lane >> 5 & 1) + 2 (lane >> 4 & 1) + (lane >> 3 & 1).
__device__ __forceinline__ float rs_wave8(float (&v)[8], int lane) {
    float a[4], b[2];
    const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = rs32(v[i], v[4 + i], h5);
#pragma unroll
    for (int i = 0; i < 2; ++i) b[i] = rs16(a[i], a[2 + i], h4);
    float c = (h3 ? b[1] : b[0]) + row_partner<8>(h3 ? b[0] : b[1]);
    return sum8(c);
}
// Sum of v[4] over the wave, scattered: lanes with lane % 16 == 0 return entry lane / 16.
__device__ __forceinline__ float rs_wave4(float (&v)[4], int lane) {
    const bool h5 = lane & 32, h4 = lane & 16;
    float a[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = rs32(v[i], v[2 + i], h5);
    float c = rs16(a[0], a[1], h4);
    c += row_partner<8>(c);
    return sum8(c);
}
__device__ __forceinline__ void lds_add(float* p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float rate_of(const BwdArgs& a, int h, size_t tok_h) {
    return a.rate_law ? heavy_tail_rate(a.A[tok_h]) : -expf(a.A[h]);
}
// d rate / d u of the heavy-tail law (0 where the clamp at -1e-4 holds)
__device__ __forceinline__ float heavy_tail_rate_grad(float u) {
    const float ht = u >= 0.f ? 1.f + u : 1.f / (1.f - u);
    const float d = u >= 0.f ? 1.f : 1.f / ((1.f - u) * (1.f - u));
    return -ht < -1e-4f ? -d : 0.f;
}

template <bool BF>
__device__ __forceinline__ float ldt(const void* p, size_t i) {
    if constexpr (BF) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}
// The raw inputs one thread stages for a group of KT tokens (rank r, pair j, row j), all
// loaded before any of them is used; indices are clamped into the tensors, and the values of
// slots that are not staged (past the group's tokens, ranks or pairs) are ignored.
template <int KT>
struct RawGroup {
    float b0[KT], b1[KT], c0[KT], c1[KT], x[KT], dy[KT], dt[KT], ang[KT];
};
template <int KT, bool BF>
__device__ __forceinline__ void load_group(RawGroup<KT>& g, const BwdArgs& a, int bi, int h, int gr, int r, int j,
                                           int t0, int nv, const float* ang, bool with_dt) {
    const int R = a.R, N = a.N, P = a.P, H = a.H, np = a.np;
    const int rr = min(r, R - 1), jb = min(j, N / 2 - 1), jx = min(j, P - 1), ja = np > 0 ? min(j, np - 1) : 0;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const size_t tok = (size_t)bi * a.L + t0 + min(k, nv - 1);
        const size_t bc = ((tok * a.G + gr) * R + rr) * N + 2 * jb;
        const size_t xi = ((tok * H + h) * R + rr) * P + jx;
        g.b0[k] = ldt<BF>(a.B, bc);
        g.b1[k] = ldt<BF>(a.B, bc + 1);
        g.c0[k] = ldt<BF>(a.C, bc);
        g.c1[k] = ldt<BF>(a.C, bc + 1);
        g.x[k] = ldt<BF>(a.x, xi);
        g.dy[k] = ldt<BF>(a.dy, xi);
        g.dt[k] = with_dt ? a.dt[tok * H + h] : 0.f;
        g.ang[k] = np > 0 ? ang[(tok * H + h) * np + ja] : 0.f;
    }
}
template <int KT>
__device__ __forceinline__ void load_group_io(RawGroup<KT>& g, const BwdArgs& a, int bi, int h, int gr, int r, int j,
                                              int t0, int nv, const float* ang, bool with_dt) {
    if (a.io_bf16) load_group<KT, true>(g, a, bi, h, gr, r, j, t0, nv, ang, with_dt);
    else load_group<KT, false>(g, a, bi, h, gr, r, j, t0, nv, ang, with_dt);
}
// sin and cos of a phase in [0, 2 pi), as the forward pass turns B and C: the hardware form for
// bf16 I/O (the matrix-core forward's), the full-precision one for f32 I/O (the f32 forward's)
__device__ __forceinline__ void phase_sincos(float phi, bool fast, float* s, float* c) {
    if (fast) __sincosf(phi, s, c);
    else sincosf(phi, s, c);
}
__device__ __forceinline__ float2 turn(float m0, float m1, bool turns, float c, float s) {
    if (!turns) return make_float2(m0, m1);
    return make_float2(m0 * c - m1 * s, m0 * s + m1 * c);
}


// ============================== forward replay ==============================
// The replay carries the folded state U_t = H_t + delta_{t+1} X_t^T Bt_t (delta = dt (1 - lam),
// beta = alpha delta), whose recurrence has one rank-R write per token:
//   U_t = alpha_t U_{t-1} + (gamma_t + delta_{t+1}) X_t^T Bt_t,   U_{-1} = H_0 + delta_0 X_prev^T B_prev,
// so dCt_t[r] = H_t^T dy_t[r] = U_t^T dy_t[r] - delta_{t+1} sum_r' (X_t[r'] . dy_t[r]) Bt_t[r']
// (an R x R correction formed after each group; delta_L = 0 at the last token).
template <int R>
__global__ __launch_bounds__(kThreads, 2) void bwd_replay_kernel(BwdArgs a) {
    __shared__ __align__(16) float sX[kT + 1][kR4][kPP];     // slot 0: x_prev (initial fold only)
    __shared__ __align__(16) float sBt[kT + 1][kR4][kNN];    // turned B; slot 0: B_prev
    __shared__ __align__(16) float sDY[kT][kR4][kPP];
    __shared__ __align__(16) float sCt[kT][kR4][kNN];        // turned C
    __shared__ float sDC[kT][kR4][kNN];                     // U^T dy
    __shared__ float sDot[kT][kR4][4];                      // [r][r'] = X[r'] . dy[r]
    __shared__ float sDPH[kT][kR4][64];                     // C side of the angle gradient, per rank
    __shared__ float sDL[kT];
    __shared__ float sAl[kT], sCo[kT], sDn[kT];             // alpha_t, gamma_t + delta_{t+1}, delta_{t+1}
    __shared__ float sRed[4];

    const int bh = blockIdx.x, H = a.H, bi = bh / H, h = bh % H, g = h * a.G / H;
    const int L = a.L, P = a.P, N = a.N, np = a.np;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, l16 = lane & 15;
    // staging / output role: rank r = w, pair j (columns 2 j, 2 j + 1) and row j
    const int r = w, j = lane;
    const bool pok = r < R && 2 * j < N, xok = r < R && j < P, turns = pok && j < np;
    // The replay's state layout: wave w owns columns 32 w .. 32 w + 31 of every row, lane
    // (lg, l16) rows 16 pt + 4 lg + v of columns 32 w + 16 c + l16, so the readout U^T dy
    // (a sum over rows) finishes inside the wave.
    const int ncol = 32 * w + l16;

    float S[4][4][2];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int p = 16 * pt + 4 * lg + v, n = ncol + 16 * c;
                S[pt][v][c] = (a.h0 && p < P && n < N) ? ld_io(a.h0, ((size_t)bh * P + p) * N + n, a.st_bf16) : 0.f;
            }
    float bb0 = 0.f, bb1 = 0.f, cb0 = 0.f, cb1 = 0.f;
    if (pok && a.Bb) { bb0 = a.Bb[((size_t)h * R + r) * N + 2 * j]; bb1 = a.Bb[((size_t)h * R + r) * N + 2 * j + 1]; }
    if (pok && a.Cb) { cb0 = a.Cb[((size_t)h * R + r) * N + 2 * j]; cb1 = a.Cb[((size_t)h * R + r) * N + 2 * j + 1]; }
    float phi = (turns && a.phi0) ? a.phi0[(size_t)bh * np + j] : 0.f;
    float gC0 = 0.f, gC1 = 0.f;                 // C bias gradient partials

    // rank-R write S += sum_q (f x_q[rows]) (x) b_q[cols] from staged rows
    auto write = [&](const float (*sx)[kPP], const float (*sb)[kNN], float f) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const float b0 = sb[q][ncol], b1 = sb[q][ncol + 16];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const float4 xv = ld4(&sx[q][16 * pt + 4 * lg]);
                const float xq[4] = {f * xv.x, f * xv.y, f * xv.z, f * xv.w};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    S[pt][v][0] = fmaf(xq[v], b0, S[pt][v][0]);
                    S[pt][v][1] = fmaf(xq[v], b1, S[pt][v][1]);
                }
            }
        }
    };
    // the initial fold U_{-1} = H_0 + delta_0 X_prev^T B_prev
    sX[0][r][j] = (xok && a.xp0) ? ld_io(a.xp0, ((size_t)bh * R + r) * P + j, a.io_bf16) : 0.f;
    {
        const bool ok = pok && a.Bp0;
        sBt[0][r][2 * j] = ok ? ld_io(a.Bp0, ((size_t)bh * R + r) * N + 2 * j, a.io_bf16) : 0.f;
        sBt[0][r][2 * j + 1] = ok ? ld_io(a.Bp0, ((size_t)bh * R + r) * N + 2 * j + 1, a.io_bf16) : 0.f;
    }
    if (tid == 0 && L > 0) {
        const size_t th = (size_t)bi * L * H + h;
        sDn[0] = a.dt[th] * (1.f - a.lam[th]);
    }
    __syncthreads();
    if (L > 0) write(sX[0], sBt[0], sDn[0]);
    __syncthreads();

    for (int t0 = 0; t0 < L; t0 += kT) {
        const int nv = min(kT, L - t0);
        // ---- stage kT tokens: angles, turned B and C, x, dy, per-token scalars ----
        float cs[kT], sn[kT];
        {
            RawGroup<kT> rg;
            load_group_io<kT>(rg, a, bi, h, g, r, j, t0, nv, a.theta, true);
#pragma unroll
            for (int k = 0; k < kT; ++k) {
                const bool valid = k < nv;
                const size_t tok = (size_t)bi * L + t0 + k;
                cs[k] = 1.f; sn[k] = 0.f;
                if (valid && turns) {
                    phi = wrap_2pi(phi + rg.dt[k] * rg.ang[k]);
                    phase_sincos(phi, a.io_bf16, &sn[k], &cs[k]);
                    if (r == 0) a.wphi[(tok * H + h) * np + j] = phi;
                }
                const bool ok = valid && pok;
                const float2 bt = turn(rg.b0[k] + bb0, rg.b1[k] + bb1, turns, cs[k], sn[k]);
                const float2 ct = turn(rg.c0[k] + cb0, rg.c1[k] + cb1, turns, cs[k], sn[k]);
                sBt[k + 1][r][2 * j] = ok ? bt.x : 0.f;
                sBt[k + 1][r][2 * j + 1] = ok ? bt.y : 0.f;
                sCt[k][r][2 * j] = ok ? ct.x : 0.f;
                sCt[k][r][2 * j + 1] = ok ? ct.y : 0.f;
                sX[k + 1][r][j] = (valid && xok) ? rg.x[k] : 0.f;
                sDY[k][r][j] = (valid && xok) ? rg.dy[k] : 0.f;
            }
        }
        if (tid < kT) {
            // alpha_t and gamma_t + delta_{t+1} of token t = t0 + tid (delta_L = 0)
            float al = 1.f, ga = 0.f, dn = 0.f;
            if (tid < nv) {
                const size_t th = ((size_t)bi * L + t0 + tid) * H + h;
                const float dtv = a.dt[th], lm = a.lam[th];
                al = expf(dtv * rate_of(a, h, th));
                ga = lm * dtv;
                if (t0 + tid + 1 < L) dn = a.dt[th + H] * (1.f - a.lam[th + H]);
            }
            sAl[tid] = al; sCo[tid] = ga + dn; sDn[tid] = dn;
            sDL[tid] = 0.f;
        }
        __syncthreads();
        // ---- per token (wave-local): U_t, then U_t^T dy_t (complete per wave: plain stores) ----
        for (int k = 0; k < nv; ++k) {
            const float al = sAl[k];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    S[pt][v][0] *= al;
                    S[pt][v][1] *= al;
                }
            write(sX[k + 1], sBt[k + 1], sCo[k]);
            float part[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                part[q][0] = part[q][1] = 0.f;
                if (q < R) {
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const float4 d = ld4(&sDY[k][q][16 * pt + 4 * lg]);
                        const float dq[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            part[q][0] = fmaf(S[pt][v][0], dq[v], part[q][0]);
                            part[q][1] = fmaf(S[pt][v][1], dq[v], part[q][1]);
                        }
                    }
                }
            }
            // sum over the four 16-lane groups, scattered: group lg keeps rank lg's two columns
            float k4[4];
            const bool h2 = lg & 2, h1 = lg & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) k4[i] = rs32(part[i >> 1][i & 1], part[2 + (i >> 1)][i & 1], h2);
            const float o0 = rs16(k4[0], k4[2], h1), o1 = rs16(k4[1], k4[3], h1);
            if (lg < R) {
                sDC[k][lg][ncol] = o0;
                sDC[k][lg][ncol + 16] = o1;
            }
        }
        __syncthreads();
        // ---- per token R x R dots X[r'] . dy[r] (wave r) ----
        // (the per-token loops of the dots and outputs run over the group's fixed size, tokens
        // past the valid ones skipped, so that the wave reductions of different tokens interleave)
        if (r < R) {
#pragma unroll
            for (int k = 0; k < kT; ++k) {
                if (k >= nv) break;
                float d4[4];
                const float dyr = xok ? sDY[k][r][j] : 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) d4[q] = (q < R && xok) ? sX[k + 1][q][j] * dyr : 0.f;
                const float d = rs_wave4(d4, lane);
                if ((lane & 15) == 0) sDot[k][r][lane >> 4] = d;
            }
        }
        __syncthreads();
        // ---- per token outputs: dC (corrected, turned back), bias partials, angle and <dy, y> terms ----
#pragma unroll
        for (int k = 0; k < kT; ++k) {
            if (k >= nv) break;
            const size_t tok = (size_t)bi * L + t0 + k;
            float dl = 0.f, dph = 0.f;
            if (pok) {
                float d0 = sDC[k][r][2 * j], d1 = sDC[k][r][2 * j + 1];
                const float dn = sDn[k];
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    const float m = -dn * sDot[k][r][q];
                    d0 = fmaf(m, sBt[k + 1][q][2 * j], d0);
                    d1 = fmaf(m, sBt[k + 1][q][2 * j + 1], d1);
                }
                const float c0 = sCt[k][r][2 * j], c1 = sCt[k][r][2 * j + 1];
                dl = c0 * d0 + c1 * d1;
                float e0 = d0, e1 = d1;
                if (turns) {
                    dph = -d0 * c1 + d1 * c0;
                    e0 = d0 * cs[k] + d1 * sn[k];
                    e1 = -d0 * sn[k] + d1 * cs[k];
                }
                float* acc = a.accC + ((tok * a.G + g) * R + r) * N + 2 * j;
                unsafeAtomicAdd(acc, e0);
                unsafeAtomicAdd(acc + 1, e1);
                gC0 += e0;
                gC1 += e1;
            }
            sDPH[k][r][j] = dph;
            dl = wave_sum(dl);
            if (lane == 0 && r < R) lds_add(&sDL[k], dl);
        }
        __syncthreads();
        if (w == 0 && j < np)
            for (int k = 0; k < nv; ++k)
                a.wdphi[(((size_t)bi * L + t0 + k) * H + h) * np + j] =
                    sDPH[k][0][j] + sDPH[k][1][j] + sDPH[k][2][j] + sDPH[k][3][j];
        if (tid < nv) a.wdl[((size_t)bi * L + t0 + tid) * H + h] = sDL[tid];
    }
    // <dH_L, H_L>, the final state's reader term of the last token (U_{L-1} = H_{L-1})
    float fin = 0.f;
    if (a.dh1) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int p = 16 * pt + 4 * lg + v, n = ncol + 16 * c;
                    if (p < P && n < N) fin += S[pt][v][c] * a.dh1[((size_t)bh * P + p) * N + n];
                }
    }
    fin = wave_sum(fin);
    if (lane == 0) sRed[w] = fin;
    __syncthreads();
    if (tid == 0) a.wdlf[bh] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
    if (pok && a.dCb) {
        unsafeAtomicAdd(a.dCb + ((size_t)h * R + r) * N + 2 * j, gC0);
        unsafeAtomicAdd(a.dCb + ((size_t)h * R + r) * N + 2 * j + 1, gC1);
    }
}

// ============================== reverse adjoint ==============================
// v and w of one token against the state S (G_{t+1}): v[r][row] stored to sv, w summed
// into sw (both [R4][..] rows of that token)
template <int R>
__device__ __forceinline__ void contract(const float (&S)[4][8], const float (*sx)[kPP], const float (*sb)[kNN],
                                         float (*sv)[kPP], float (*sw)[kNN], int prow, int lg, int l16) {
    float vp[16];
    float wp[R][8];
#pragma unroll
    for (int i = 0; i < 16; ++i) vp[i] = 0.f;
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const float4 b0 = ld4(&sb[q][l16 * 4]), b1 = ld4(&sb[q][64 + l16 * 4]);
        const float bq[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float4 xv = ld4(&sx[q][prow]);
        const float xq[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float s = 0.f;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) s = fmaf(S[v][nt], bq[nt], s);
            vp[4 * q + v] = s;
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            wp[q][nt] = S[0][nt] * xq[0] + S[1][nt] * xq[1] + S[2][nt] * xq[2] + S[3][nt] * xq[3];
    }
    const float vr = rs_row16(vp, l16);
    const int q = l16 >> 2;
    if (q < R) sv[q][prow + (l16 & 3)] = vr;
    float red[R][2];
    rs_groups<R>(wp, red, lg);
#pragma unroll
    for (int qq = 0; qq < R; ++qq)
#pragma unroll
        for (int i = 0; i < 2; ++i) sw[qq][16 * (2 * lg + i) + l16] = red[qq][i];
}

template <int R>
__global__ __launch_bounds__(kThreads, 2) void bwd_adjoint_kernel(BwdArgs a) {
    __shared__ __align__(16) float sX[kTA][kR4][kPP];
    __shared__ __align__(16) float sBt[kTA][kR4][kNN];        // turned B (bpos order)
    __shared__ __align__(16) float sDY[kTA][kR4][kPP];
    __shared__ __align__(16) float sCt[kTA][kR4][kNN];        // turned C (bpos order)
    __shared__ float sV[kTA][kR4][kPP];         // v = G_{t+1} Bt_t
    __shared__ float sW[kTA][4][kR4][kNN];      // w = G_{t+1}^T X_t: each wave's partial (its 16 rows)
    __shared__ float sDot[kTA][kR4][8];         // [r][r'] = Ct[r'] . Bt[r], [r][4 + r'] = dy[r'] . X[r]
    __shared__ float sXV[kTA];                  // X_t . v
    __shared__ float sDPH[kTA][kR4][64];        // B side of the angle gradient, per rank
    __shared__ float sPC[kTA][64], sTh[kTA][64]; // C side (from the replay) and the rates, per pair
    __shared__ float sDLp[kTA];                 // <dy_t, y_t> (from the replay)
    __shared__ float sAl[kTA + 1], sBe[kTA + 1], sGa[kTA + 1], sDt[kTA + 1], sLm[kTA + 1], sRt[kTA + 1], sU[kTA + 1];

    const int bh = blockIdx.x, H = a.H, bi = bh / H, h = bh % H, g = h * a.G / H;
    const int L = a.L, P = a.P, N = a.N, np = a.np, io = a.io_bf16;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, l16 = lane & 15;
    const int r = w, j = lane;
    const bool pok = r < R && 2 * j < N, xok = r < R && j < P, turns = pok && j < np;
    const int prow = 16 * w + 4 * lg;

    float S[4][8];                             // G_{t+1}: the final state's sensitivity first
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int p = prow + v, n = 16 * nt + l16;
            S[v][nt] = (a.dh1 && p < P && n < N) ? a.dh1[((size_t)bh * P + p) * N + n] : 0.f;
        }
    float bb0 = 0.f, bb1 = 0.f, cb0 = 0.f, cb1 = 0.f;
    if (pok && a.Bb) { bb0 = a.Bb[((size_t)h * R + r) * N + 2 * j]; bb1 = a.Bb[((size_t)h * R + r) * N + 2 * j + 1]; }
    if (pok && a.Cb) { cb0 = a.Cb[((size_t)h * R + r) * N + 2 * j]; cb1 = a.Cb[((size_t)h * R + r) * N + 2 * j + 1]; }
    float gB0 = 0.f, gB1 = 0.f;                // B bias gradient partials
    // wave 0, lane j < np: the angle sensitivity sum_{k >= t} d loss / d phi_k
    float Phi = (w == 0 && j < np && a.dphi1) ? a.dphi1[(size_t)bh * np + j] : 0.f;
    // lane 0 of wave 0: the scalar chain (running log-decay sensitivity, token t+1's
    // pending step / blend gradients, the static rate's sum)
    float Sl = 0.f, pend_dt = 0.f, pend_lm = 0.f, dA_sum = 0.f;

    // The next group's raw inputs are loaded into registers while the current group computes:
    // its rows (every thread), the replay's angle terms and the rates (wave 0), the per-token
    // scalars and <dy, y> (threads 0 .. kTA).
    RawGroup<kTA> nrg;
    float npc[kTA], nth[kTA], ndt = 0.f, nlm = 0.f, nu = 0.f, ndl = 0.f;
    auto prefetch = [&](int t0n) {
        const int nvn = min(kTA, L - t0n);
        load_group_io<kTA>(nrg, a, bi, h, g, r, j, t0n, nvn, a.wphi, false);
        if (w == 0 && j < np) {
#pragma unroll
            for (int k = 0; k < kTA; ++k) {
                const size_t th = ((size_t)bi * L + t0n + min(k, nvn - 1)) * H + h;
                npc[k] = a.wdphi[th * np + j];
                nth[k] = a.theta[th * np + j];
            }
        }
        if (tid <= kTA && t0n + tid < L) {
            const size_t th = ((size_t)bi * L + t0n + tid) * H + h;
            ndt = a.dt[th];
            nlm = a.lam[th];
            nu = a.A[a.rate_law ? th : (size_t)h];
            ndl = a.wdl[th];
        }
    };
    if (L > 0) prefetch(((L - 1) / kTA) * kTA);

    for (int t0 = ((L - 1) / kTA) * kTA; t0 >= 0; t0 -= kTA) {
        const int nv = min(kTA, L - t0);
        float cs[kTA], sn[kTA];
        {
            const RawGroup<kTA> rg = nrg;
            float pc[kTA], thr[kTA];
#pragma unroll
            for (int k = 0; k < kTA; ++k) { pc[k] = npc[k]; thr[k] = nth[k]; }
            const float dtv0 = ndt, lm0 = nlm, u0 = nu, dl0 = ndl;
            if (t0 >= kTA) prefetch(t0 - kTA);
#pragma unroll
            for (int k = 0; k < kTA; ++k) {
                const bool valid = k < nv;
                cs[k] = 1.f; sn[k] = 0.f;
                if (valid && turns) phase_sincos(rg.ang[k], io, &sn[k], &cs[k]);   // phases wrapped into [0, 2 pi)
                const bool ok = valid && pok;
                const float2 bt = turn(rg.b0[k] + bb0, rg.b1[k] + bb1, turns, cs[k], sn[k]);
                const float2 ct = turn(rg.c0[k] + cb0, rg.c1[k] + cb1, turns, cs[k], sn[k]);
                sBt[k][r][bpos(2 * j)] = ok ? bt.x : 0.f;
                sBt[k][r][bpos(2 * j + 1)] = ok ? bt.y : 0.f;
                sCt[k][r][bpos(2 * j)] = ok ? ct.x : 0.f;
                sCt[k][r][bpos(2 * j + 1)] = ok ? ct.y : 0.f;
                sX[k][r][j] = (valid && xok) ? rg.x[k] : 0.f;
                sDY[k][r][j] = (valid && xok) ? rg.dy[k] : 0.f;
            }
            if (w == 0 && j < np) {
#pragma unroll
                for (int k = 0; k < kTA; ++k) {
                    sPC[k][j] = pc[k];
                    sTh[k][j] = thr[k];
                }
            }
            if (tid <= kTA) {
                // slot kTA is token t0 + kTA (the first of the group done before), or past the end:
                // there alpha = 1 and beta = 0 stand for the final carry
                float al = 1.f, be = 0.f, ga = 0.f, dtv = 0.f, lm = 0.f, rt = 0.f, u = 0.f;
                if (t0 + tid < L) {
                    dtv = dtv0; lm = lm0;
                    u = a.rate_law ? u0 : 0.f;
                    rt = a.rate_law ? heavy_tail_rate(u0) : -expf(u0);
                    al = expf(dtv * rt);
                    be = al * dtv * (1.f - lm);
                    ga = lm * dtv;
                }
                sAl[tid] = al; sBe[tid] = be; sGa[tid] = ga; sDt[tid] = dtv; sLm[tid] = lm; sRt[tid] = rt; sU[tid] = u;
                if (tid < kTA) {
                    sXV[tid] = 0.f;
                    sDLp[tid] = t0 + tid < L ? dl0 : 0.f;
                }
            }
        }
        __syncthreads();
        // ---- per token, last first (wave-local): v, w against G_{t+1}, then G_t ----
        for (int k = nv - 1; k >= 0; --k) {
            contract<R>(S, sX[k], sBt[k], sV[k], sW[k][w], prow, lg, l16);
            const float al1 = sAl[k + 1];
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) S[v][nt] *= al1;
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const float4 d = ld4(&sDY[k][q][prow]);
                const float dq[4] = {d.x, d.y, d.z, d.w};
                const float4 c0 = ld4(&sCt[k][q][l16 * 4]), c1 = ld4(&sCt[k][q][64 + l16 * 4]);
                const float cq[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) S[v][nt] = fmaf(dq[v], cq[nt], S[v][nt]);
            }
        }
        __syncthreads();
        // ---- per token R x R dot products and X . v ----
        // (these per-token loops and wave 0's run over the group's fixed size, tokens past the
        // valid ones skipped, so that the reductions and loads of different tokens interleave)
#pragma unroll
        for (int k = 0; k < kTA; ++k) {
            if (k < nv && r < R) {
                float d8[8];
                const float b0 = sBt[k][r][bpos(2 * j)], b1 = sBt[k][r][bpos(2 * j + 1)];
                const float xr = sX[k][r][j];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    d8[q] = (q < R && pok) ? sCt[k][q][bpos(2 * j)] * b0 + sCt[k][q][bpos(2 * j + 1)] * b1 : 0.f;
                    d8[4 + q] = (q < R && xok) ? sDY[k][q][j] * xr : 0.f;
                }
                const float d = rs_wave8(d8, lane);
                if ((lane & 7) == 0) sDot[k][r][lane >> 3] = d;
                const float xv = wave_sum(xok ? xr * sV[k][r][j] : 0.f);
                if (lane == 0) lds_add(&sXV[k], xv);
            }
        }
        __syncthreads();
        // ---- per token outputs: dx, dB (turned back), bias partials, angle terms ----
#pragma unroll
        for (int k = 0; k < kTA; ++k) {
            if (k >= nv) break;
            const int t = t0 + k;
            const size_t tok = (size_t)bi * L + t;
            const bool last = t == L - 1;
            const float ga = sGa[k], kap = ga * sAl[k + 1] + sBe[k + 1];
            float dph = 0.f;
            if (xok) {
                float dxv = kap * sV[k][r][j];
#pragma unroll
                for (int q = 0; q < R; ++q) dxv = fmaf(ga * sDY[k][q][j], sDot[k][r][q], dxv);
                if (last && a.dxp1) dxv += a.dxp1[((size_t)bh * R + r) * P + j];
                st_io(a.dx, ((tok * H + h) * R + r) * P + j, dxv, io);
            }
            if (pok) {
                const float w0 = sW[k][0][r][2 * j] + sW[k][1][r][2 * j] + sW[k][2][r][2 * j] + sW[k][3][r][2 * j];
                const float w1 = sW[k][0][r][2 * j + 1] + sW[k][1][r][2 * j + 1] + sW[k][2][r][2 * j + 1] +
                                 sW[k][3][r][2 * j + 1];
                float d0 = kap * w0, d1 = kap * w1;
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    const float m = ga * sDot[k][r][4 + q];
                    d0 = fmaf(m, sCt[k][q][bpos(2 * j)], d0);
                    d1 = fmaf(m, sCt[k][q][bpos(2 * j + 1)], d1);
                }
                if (last && a.dBp1) {
                    d0 += a.dBp1[((size_t)bh * R + r) * N + 2 * j];
                    d1 += a.dBp1[((size_t)bh * R + r) * N + 2 * j + 1];
                }
                float e0 = d0, e1 = d1;
                if (turns) {
                    const float b0 = sBt[k][r][bpos(2 * j)], b1 = sBt[k][r][bpos(2 * j + 1)];
                    dph = -d0 * b1 + d1 * b0;
                    e0 = d0 * cs[k] + d1 * sn[k];
                    e1 = -d0 * sn[k] + d1 * cs[k];
                }
                float* acc = a.accB + ((tok * a.G + g) * R + r) * N + 2 * j;
                unsafeAtomicAdd(acc, e0);
                unsafeAtomicAdd(acc + 1, e1);
                gB0 += e0;
                gB1 += e1;
            }
            sDPH[k][r][j] = dph;
        }
        __syncthreads();
        // ---- wave 0: angle sensitivities, then lane 0's scalar chain, last token first ----
        if (w == 0) {
#pragma unroll
            for (int k = kTA - 1; k >= 0; --k) {
                if (k >= nv) continue;
                const int t = t0 + k;
                const size_t th = ((size_t)bi * L + t) * H + h;
                float tp = 0.f;
                if (j < np) {
                    Phi += sDPH[k][0][j] + sDPH[k][1][j] + sDPH[k][2][j] + sDPH[k][3][j] + sPC[k][j];
                    a.dtheta[th * np + j] = sDt[k] * Phi;
                    tp = sTh[k][j] * Phi;
                }
                tp = wave_sum(tp);
                if (lane == 0) {
                    float dots = 0.f;
#pragma unroll
                    for (int q = 0; q < R; ++q)
#pragma unroll
                        for (int q2 = 0; q2 < R; ++q2) dots += sDot[k][q][q2] * sDot[k][q][4 + q2];
                    const bool has_next = t + 1 < L;
                    const float al1 = sAl[k + 1], be1 = sBe[k + 1];
                    const float dbe1 = has_next ? sXV[k] : 0.f;       // d beta_{t+1}
                    const float dga = al1 * sXV[k] + dots;             // d gamma_t
                    float dl = sDLp[k] - sGa[k] * dga - be1 * dbe1;
                    if (t == L - 1) dl += a.wdlf[bh];
                    Sl += dl;                                          // d loss / d log alpha_t
                    if (has_next) {
                        const float dde = al1 * dbe1;                  // beta = alpha delta
                        a.ddt[th + H] = pend_dt + (1.f - sLm[k + 1]) * dde;
                        a.dlam[th + H] = pend_lm - sDt[k + 1] * dde;
                    }
                    pend_dt = sRt[k] * Sl + sLm[k] * dga + tp;
                    pend_lm = sDt[k] * dga;
                    const float dA = sDt[k] * Sl;                      // log alpha = dt A
                    if (a.rate_law) a.dA[th] = dA * heavy_tail_rate_grad(sU[k]);
                    else dA_sum += dA;
                }
            }
        }
        __syncthreads();
    }
    // ---- the carried previous write at t = 0 (x_prev, turned B_prev) against G_0 ----
    if (L > 0) {
        sX[0][r][j] = (xok && a.xp0) ? ld_io(a.xp0, ((size_t)bh * R + r) * P + j, io) : 0.f;
        const bool ok = pok && a.Bp0;
        sBt[0][r][bpos(2 * j)] = ok ? ld_io(a.Bp0, ((size_t)bh * R + r) * N + 2 * j, io) : 0.f;
        sBt[0][r][bpos(2 * j + 1)] = ok ? ld_io(a.Bp0, ((size_t)bh * R + r) * N + 2 * j + 1, io) : 0.f;
        if (tid == 0) sXV[0] = 0.f;
        __syncthreads();
        contract<R>(S, sX[0], sBt[0], sV[0], sW[0][w], prow, lg, l16);
        __syncthreads();
        // sAl[0], sBe[0], ... still hold token 0 (the last group staged)
        const float al0 = sAl[0], be0 = sBe[0];
        if (r < R) {
            const float xv = wave_sum(xok ? sX[0][r][j] * sV[0][r][j] : 0.f);
            if (lane == 0) lds_add(&sXV[0], xv);
        }
        if (xok && a.dxp0) a.dxp0[((size_t)bh * R + r) * P + j] = be0 * sV[0][r][j];
        if (pok && a.dBp0) {
            a.dBp0[((size_t)bh * R + r) * N + 2 * j] =
                be0 * (sW[0][0][r][2 * j] + sW[0][1][r][2 * j] + sW[0][2][r][2 * j] + sW[0][3][r][2 * j]);
            a.dBp0[((size_t)bh * R + r) * N + 2 * j + 1] =
                be0 * (sW[0][0][r][2 * j + 1] + sW[0][1][r][2 * j + 1] + sW[0][2][r][2 * j + 1] + sW[0][3][r][2 * j + 1]);
        }
        if (a.dh0) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const int p = prow + v, n = 16 * nt + l16;
                    if (p < P && n < N) a.dh0[((size_t)bh * P + p) * N + n] = al0 * S[v][nt];
                }
        }
        __syncthreads();
        if (tid == 0) {
            const size_t th = (size_t)bi * L * H + h;                 // token 0
            const float dde = al0 * sXV[0];
            a.ddt[th] = pend_dt + (1.f - sLm[0]) * dde;
            a.dlam[th] = pend_lm - sDt[0] * dde;
            if (!a.rate_law) unsafeAtomicAdd(a.dA + h, dA_sum * -expf(a.A[h]));
        }
    }
    if (w == 0 && j < np && a.dphi0) a.dphi0[(size_t)bh * np + j] = Phi;
    if (pok && a.dBb) {
        unsafeAtomicAdd(a.dBb + ((size_t)h * R + r) * N + 2 * j, gB0);
        unsafeAtomicAdd(a.dBb + ((size_t)h * R + r) * N + 2 * j + 1, gB1);
    }
}

__global__ void fill_zero_kernel(float* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}
__global__ void copy_f32_kernel(const float* src, float* dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}
__global__ void acc_convert_kernel(const float* acc, void* out, size_t n, int io_bf16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        st_io(out, i, acc[i], io_bf16);
}
hipError_t fill_zero(float* p, size_t n, hipStream_t s) {
    if (!p || n == 0) return hipSuccess;
    const int blocks = (int)std::min<size_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

template <int R>
hipError_t launch_r(const BwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.b * a.H));
    hipLaunchKernelGGL(bwd_replay_kernel<R>, grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_adjoint_kernel<R>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool scan_bwd_supported(int P, int N, int R, int np) {
    return P >= 1 && P <= kPP && N >= 2 && N <= kNN && (N % 2) == 0 && R >= 1 && R <= kR4 && 2 * np <= N;
}

BwdWs scan_bwd_workspace(int b, int L, int H, int G, int R, int N, int np, bool chunked) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    BwdWs w{};
    size_t o = 0;
    const size_t tokbc = (size_t)b * L * G * R * N, tokh = (size_t)b * L * H;
    w.accB = o; o += up(tokbc * 4);
    w.accC = o; o += up(tokbc * 4);
    if (chunked) {
        // the chunked form's chunk states and phases replace the replay's per-token terms
        w.phi = w.dphi = w.dl = w.dlf = o;
        w.cws = o; o += up(scan_bwd_chunked_extra_bytes(b, L, H, np));
    } else {
        w.phi = o;  o += up(tokh * np * 4);
        w.dphi = o; o += up(tokh * np * 4);
        w.dl = o;   o += up(tokh * 4);
        w.dlf = o;  o += up((size_t)b * H * 4);
        w.cws = o;
    }
    w.total = o;
    return w;
}

hipError_t launch_scan_bwd(const BwdArgs& a, void* dB, void* dC, hipStream_t s) {
    if (a.L == 0) {
        // no token: the initial carry's gradients are the final carry's sensitivities
        hipError_t e = hipSuccess;
        if (!a.rate_law) e = fill_zero(a.dA, (size_t)a.H, s);
        if (e == hipSuccess) e = fill_zero(a.dBb, (size_t)a.H * a.R * a.N, s);
        if (e == hipSuccess) e = fill_zero(a.dCb, (size_t)a.H * a.R * a.N, s);
        const size_t bh = (size_t)a.b * a.H;
        const float* src[4] = {a.dh1, a.dphi1, a.dBp1, a.dxp1};
        float* dst[4] = {a.dh0, a.dphi0, a.dBp0, a.dxp0};
        const size_t n[4] = {bh * a.P * a.N, bh * a.np, bh * a.R * a.N, bh * a.R * a.P};
        for (int i = 0; i < 4 && e == hipSuccess; ++i) {
            if (!dst[i] || n[i] == 0) continue;
            const int blocks = (int)std::min<size_t>((n[i] + 255) / 256, 8192);
            hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks), dim3(256), 0, s, src[i], dst[i], n[i]);
            e = hipGetLastError();
        }
        return e;
    }
    const size_t nbc = (size_t)a.b * a.L * a.G * a.R * a.N;
    hipError_t e = fill_zero(a.accB, nbc, s);
    if (e == hipSuccess) e = fill_zero(a.accC, nbc, s);
    if (e == hipSuccess && !a.rate_law) e = fill_zero(a.dA, (size_t)a.H, s);
    if (e == hipSuccess) e = fill_zero(a.dBb, (size_t)a.H * a.R * a.N, s);
    if (e == hipSuccess) e = fill_zero(a.dCb, (size_t)a.H * a.R * a.N, s);
    if (e != hipSuccess) return e;
    if (a.cws) {
        e = launch_scan_bwd_chunked(a, a.cws, s);
    } else switch (a.R) {
        case 1: e = launch_r<1>(a, s); break;
        case 2: e = launch_r<2>(a, s); break;
        case 3: e = launch_r<3>(a, s); break;
        case 4: e = launch_r<4>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || nbc == 0) return e;
    const int blocks = (int)std::min<size_t>((nbc + 255) / 256, 8192);
    hipLaunchKernelGGL(acc_convert_kernel, dim3(blocks), dim3(256), 0, s, a.accB, dB, nbc, a.io_bf16);
    hipLaunchKernelGGL(acc_convert_kernel, dim3(blocks), dim3(256), 0, s, a.accC, dC, nbc, a.io_bf16);
    return hipGetLastError();
}

}  // namespace m3
