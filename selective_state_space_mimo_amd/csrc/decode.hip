// Single-token decode step, streaming a bf16 P x N state (P = 64, N = 128).
//
// The step is the decode listing of "Mamba-3: Improved Sequence Modeling
// using State Space Principles", section "Computing the rotation as a
// data-dependent RoPE", restricted to the scan core:
//   alpha = exp(-dt a), beta = alpha dt (1 - lam), gamma = lam dt
//   phi += dt theta;  Bt = rot(B + b_h, phi), Ct = rot(C + c_h, phi)
//   h = alpha h + beta X_prev^T Bt_prev + gamma X^T Bt;   y_r = h Ct_r
//   (Bt_prev, X_prev) <- (Bt, X)
// with the rank-R write of section "MIMO: a rank-4 state update ...".
//
// Section "Why a recurrent model's decode step is memory-bound" fixes the
// design: the state read and write-back are ~88% of the bytes, so the kernel
// is a stream.  One workgroup (256 threads) per (batch, head): every thread
// owns four 16-byte vectors of the state -- rows p = tid/16 + 16k, columns
// n0..n0+7 with n0 = 8 (tid % 16) -- which it loads before anything else
// (coalesced 128-bit loads, in flight during the per-head set-up).
// Arithmetic per state element: one multiply (alpha h) plus R dot2 ops
// (v_dot2_f32_bf16 fuses beta x_prev B_prev + gamma x B for one rank), the
// bf16 store, and R/2 dot2 ops for the readout.  The readout's 16-lane sums
// use a reduce-scatter butterfly so that each lane finishes one output.
//
// Rounding: the state is stored in bf16 (round to nearest even); Bt, Ct,
// beta x_prev and gamma x enter the dot products as bf16 (exact products,
// fp32 sums), and the readout uses the stored bf16 state.
#include "m3_internal.h"

namespace m3 {

namespace {

constexpr int kP = 64, kN = 128, kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v;
    v[0] = (bf16)lo;
    v[1] = (bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Cross-lane moves inside a row of 16 lanes (DPP, no LDS round trip).
// Each is an involution that pairs a lane of one half of the group with a
// lane of the other half: mirror (i <-> 15 - i) across the 8-lane halves,
// half-mirror (i <-> 7 - i) across 4-lane halves, then quad swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kRowMirror = 0x140, kRowHalfMirror = 0x141;
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
template <int LEVEL>
__device__ __forceinline__ float partner(float v) {
    if constexpr (LEVEL == 8) return dpp_mov<kRowMirror>(v);
    else if constexpr (LEVEL == 4) return dpp_mov<kRowHalfMirror>(v);
    else if constexpr (LEVEL == 2) return dpp_mov<kQuadSwap2>(v);
    else return dpp_mov<kQuadSwap1>(v);
}

// One reduce-scatter level: lanes in the upper half (lane & LEVEL) keep the
// upper half of the CNT values, the others the lower half; each adds its
// partner's copy of the half it keeps.
template <int LEVEL, int CNT, int V>
__device__ __forceinline__ void rs_level(float (&v)[V], bool up) {
    if constexpr (CNT > 1) {
        constexpr int HALF = CNT / 2;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const float keep = up ? v[i + HALF] : v[i];
            const float send = up ? v[i] : v[i + HALF];
            v[i] = keep + partner<LEVEL>(send);
        }
    } else {
        v[0] += partner<LEVEL>(v[0]);
    }
}

__device__ const float2 kZero2 = {0.f, 0.f};

template <int R>
__global__ __launch_bounds__(kThreads) void decode_fast_kernel(DecodeArgs a) {
    // (Bt_prev[n], Bt[n]) pairs per rank, Ct as bf16 pairs, (beta x_prev, gamma x) pairs
    __shared__ uint32_t sPair[R][kN];
    __shared__ uint32_t sC[R][kN / 2];
    __shared__ uint32_t sX[R][kP];

    const int bh = blockIdx.x, H = a.H, bi = bh / H, h = bh % H, g = h * a.G / H;
    const int tid = threadIdx.x, np = a.np;
    const int n0 = (tid & 15) * 8, prow = tid >> 4;

    // ---- 1. every global load this thread needs, issued before any use -------------
    // the rate input: A_log [H] (static) or the per-token input [b][H]
    const float dt = a.dt[bh], lam = a.lam[bh], alog = a.A_log[a.rate_law ? bh : h];
    // pair work (tid < R*N/2): rank r, pair i.  Addresses are clamped or
    // redirected to a zero word instead of branching, so that all loads are
    // in flight together.
    const bool has_pair = tid < R * kN / 2;
    const int q = tid % (R * kN / 2);
    const int r = q / (kN / 2), i = q % (kN / 2), k0 = 2 * i;
    const bool rot = i < np;
    const size_t bc = (((size_t)bi * a.G + g) * R + r) * kN + k0;
    const size_t bias_i = ((size_t)h * R + r) * kN + k0;
    const size_t bp_i = ((size_t)bh * R + r) * kN + k0;
    const size_t ph_i = (size_t)bh * np + (rot ? i : 0);
    const uint32_t braw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.B) + bc);
    const uint32_t craw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.C) + bc);
    const uint32_t bp_old = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.Bp) + bp_i);
    const float2 bbias = *(a.Bb ? reinterpret_cast<const float2*>(a.Bb + bias_i) : &kZero2);
    const float2 cbias = *(a.Cb ? reinterpret_cast<const float2*>(a.Cb + bias_i) : &kZero2);
    const float phi_old = *(rot ? a.phi + ph_i : &kZero2.x);
    const float th = *(rot ? a.theta + ph_i : &kZero2.x);
    // x work (tid < R*P)
    const bool has_x = tid < R * kP;
    const size_t xi = (size_t)bh * R * kP + tid % (R * kP);
    const uint16_t xraw = static_cast<const uint16_t*>(a.x)[xi];
    const uint16_t xpraw = static_cast<const uint16_t*>(a.xp)[xi];

    // The state's four 16-byte vectors go last: loads return in issue order,
    // so the set-up below can wait for the small loads while these stay in flight.
    u32x4* hs = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.h) + (size_t)bh * kP * kN);
    u32x4 st[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) st[k] = __builtin_nontemporal_load(&hs[((prow + 16 * k) * kN + n0) / 8]);

    // ---- 2. per-head scalars ------------------------------------------------------------
    const float alpha = expf(dt * (a.rate_law ? heavy_tail_rate(alog) : -expf(alog)));
    const float beta = alpha * dt * (1.f - lam), gamma = lam * dt;

    // ---- 3. biased, turned B and C (one adjacent pair per thread) -----------------------
    const float phi_new = phi_old + dt * th;
    if (has_pair) {
        float b0 = lo_f(braw) + bbias.x, b1 = hi_f(braw) + bbias.y;
        float c0 = lo_f(craw) + cbias.x, c1 = hi_f(craw) + cbias.y;
        if (rot) {
            float sn, cs;
            sincosf(phi_new, &sn, &cs);
            const float tb = b0 * cs - b1 * sn, tc = c0 * cs - c1 * sn;
            b1 = b0 * sn + b1 * cs; b0 = tb;
            c1 = c0 * sn + c1 * cs; c0 = tc;
        }
        const uint32_t nb = pack2(b0, b1);
        sPair[r][k0] = (bp_old & 0xffffu) | (nb << 16);
        sPair[r][k0 + 1] = (bp_old >> 16) | (nb & 0xffff0000u);
        sC[r][i] = pack2(c0, c1);
    }
    if (has_x) sX[tid / kP][tid % kP] = pack2(beta * bf16_bits_to_f32(xpraw), gamma * bf16_bits_to_f32(xraw));
    __syncthreads();
    // carries: every old value of this head has been read (loads above, before the barrier)
    if (has_pair) {
        const uint32_t nb = (sPair[r][k0] >> 16) | (sPair[r][k0 + 1] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.Bp) + bp_i) = nb;
        if (rot && r == 0) a.phi[ph_i] = wrap_2pi(phi_new);
    }
    if (has_x) static_cast<uint16_t*>(a.xp)[xi] = xraw;

    // ---- 4. state update, store, readout partials -------------------------------------
    uint32_t pr[R][8], cr[R][4];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pr[rr][j] = sPair[rr][n0 + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) cr[rr][j] = sC[rr][n0 / 2 + j];
    }
    constexpr int V = 4 * R;
    float v[V];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = prow + 16 * k;
        uint32_t xr[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) xr[rr] = sX[rr][p];
        const uint32_t w[4] = {st[k].x, st[k].y, st[k].z, st[k].w};
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float e0 = alpha * lo_f(w[m]), e1 = alpha * hi_f(w[m]);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                e0 = dot2(xr[rr], pr[rr][2 * m], e0);
                e1 = dot2(xr[rr], pr[rr][2 * m + 1], e1);
            }
            o[m] = pack2(e0, e1);
        }
        const u32x4 ov = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(ov, &hs[(p * kN + n0) / 8]);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc = dot2(o[m], cr[rr][m], acc);
            v[k * R + rr] = acc;
        }
    }

    // ---- 5. 16-lane reduce-scatter: after it lane l holds the full sum of one value ---
    const int lane = tid & 15;
    rs_level<8, V, V>(v, (lane & 8) != 0);
    rs_level<4, (V / 2 > 1 ? V / 2 : 1), V>(v, (lane & 4) != 0);
    rs_level<2, (V / 4 > 1 ? V / 4 : 1), V>(v, (lane & 2) != 0);
    rs_level<1, (V / 8 > 1 ? V / 8 : 1), V>(v, (lane & 1) != 0);
    // value index kept: one bit per halving level, most significant first
    int idx = 0, c2 = V;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
        if (c2 > 1) { c2 /= 2; if (lane & off) idx += c2; }
    constexpr int kLanesPerValue = 16 / V;
    if ((lane % kLanesPerValue) == 0) {
        const int k = idx / R, rr = idx % R, p = prow + 16 * k;
        static_cast<bf16*>(a.y)[((size_t)bh * R + rr) * kP + p] = (bf16)v[0];
    }
}

}  // namespace

bool decode_fast_supported(const DecodeArgs& a) {
    return a.P == kP && a.N == kN && (a.R == 1 || a.R == 2 || a.R == 4) && a.io_bf16 && a.st_bf16;
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(a.b * a.H), block(kThreads);
    switch (a.R) {
        case 1: hipLaunchKernelGGL(decode_fast_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(decode_fast_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(decode_fast_kernel<4>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace m3
