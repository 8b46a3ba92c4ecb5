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

template <int R>
__global__ __launch_bounds__(kThreads) void decode_fast_kernel(DecodeArgs a) {
    // (Bt_prev[n], Bt[n]) pairs per rank, Ct as bf16 pairs, (beta x_prev, gamma x) pairs
    __shared__ uint32_t sPair[R][kN];
    __shared__ uint32_t sC[R][kN / 2];
    __shared__ uint32_t sX[R][kP];

    const int bh = blockIdx.x, H = a.H, bi = bh / H, h = bh % H, g = h * a.G / H;
    const int tid = threadIdx.x, np = a.np;
    const int n0 = (tid & 15) * 8, prow = tid >> 4;

    // ---- 1. the state: four 16-byte vectors per thread, loaded first -------------
    u32x4* hs = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.h) + (size_t)bh * kP * kN);
    u32x4 st[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) st[k] = __builtin_nontemporal_load(&hs[((prow + 16 * k) * kN + n0) / 8]);

    // ---- 2. per-head scalars --------------------------------------------------------
    const float dt = a.dt[bh], lam = a.lam[bh];
    const float alpha = expf(-dt * expf(a.A_log[h]));
    const float beta = alpha * dt * (1.f - lam), gamma = lam * dt;

    // ---- 3. biased, turned B and C (one adjacent pair per thread) -------------------
    float phi_new = 0.f;
    if (tid < R * kN / 2) {
        const int r = tid / (kN / 2), i = tid % (kN / 2), k0 = 2 * i;
        const size_t bc = (((size_t)bi * a.G + g) * R + r) * kN + k0;
        const uint32_t braw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.B) + bc);
        const uint32_t craw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.C) + bc);
        float b0 = lo_f(braw), b1 = hi_f(braw), c0 = lo_f(craw), c1 = hi_f(craw);
        if (a.Bb) { const float2 v = *reinterpret_cast<const float2*>(a.Bb + ((size_t)h * R + r) * kN + k0); b0 += v.x; b1 += v.y; }
        if (a.Cb) { const float2 v = *reinterpret_cast<const float2*>(a.Cb + ((size_t)h * R + r) * kN + k0); c0 += v.x; c1 += v.y; }
        if (i < np) {
            phi_new = a.phi[(size_t)bh * np + i] + dt * a.theta[(size_t)bh * np + i];
            float sn, cs;
            sincosf(phi_new, &sn, &cs);
            const float tb = b0 * cs - b1 * sn, tc = c0 * cs - c1 * sn;
            b1 = b0 * sn + b1 * cs; b0 = tb;
            c1 = c0 * sn + c1 * cs; c0 = tc;
        }
        uint32_t* bp = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.Bp) + ((size_t)bh * R + r) * kN + k0);
        const uint32_t old = *bp;
        const uint32_t nb = pack2(b0, b1);
        sPair[r][k0] = (old & 0xffffu) | (nb << 16);
        sPair[r][k0 + 1] = (old >> 16) | (nb & 0xffff0000u);
        sC[r][i] = pack2(c0, c1);
        *bp = nb;                                   // new carry: this token's turned B
    }
    // ---- 4. (beta x_prev, gamma x) pairs ---------------------------------------------
    if (tid < R * kP) {
        const size_t xi = (size_t)bh * R * kP + tid;
        const float xn = bf16_bits_to_f32(static_cast<const uint16_t*>(a.x)[xi]);
        uint16_t* xp = static_cast<uint16_t*>(a.xp);
        const float xo = bf16_bits_to_f32(xp[xi]);
        sX[tid / kP][tid % kP] = pack2(beta * xo, gamma * xn);
        xp[xi] = static_cast<const uint16_t*>(a.x)[xi];
    }
    __syncthreads();
    if (tid < np) a.phi[(size_t)bh * np + tid] = wrap_2pi(phi_new);   // r == 0 owners; old values all read

    // ---- 5. state update, store, readout partials -------------------------------------
    uint32_t pr[R][8], cr[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pr[r][j] = sPair[r][n0 + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) cr[r][j] = sC[r][n0 / 2 + j];
    }
    float part[4 * R];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = prow + 16 * k;
        uint32_t xr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) xr[r] = sX[r][p];
        const uint32_t w[4] = {st[k].x, st[k].y, st[k].z, st[k].w};
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float e0 = alpha * lo_f(w[m]), e1 = alpha * hi_f(w[m]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                e0 = dot2(xr[r], pr[r][2 * m], e0);
                e1 = dot2(xr[r], pr[r][2 * m + 1], e1);
            }
            o[m] = pack2(e0, e1);
        }
        const u32x4 ov = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(ov, &hs[(p * kN + n0) / 8]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc = dot2(o[m], cr[r][m], acc);
            part[k * R + r] = acc;
        }
    }

    // ---- 6. 16-lane reduce-scatter: lane l ends with the sum of value (l % 16) ---------
    // (for 4R < 16 values the last steps are plain all-reduces)
    constexpr int V = 4 * R;
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = part[i];
    const int lane = tid & 15;
    int cnt = V;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        if (cnt > 1) {
            const int half = cnt / 2;
            const bool up = (lane & off) != 0;
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                if (i < half) {
                    const float keep = up ? v[i + half] : v[i];
                    const float send = up ? v[i] : v[i + half];
                    v[i] = keep + __shfl_xor(send, off);
                }
            }
            cnt = half;
        } else {
            v[0] += __shfl_xor(v[0], off);
        }
    }
    // value index held by this lane: bits of (off = 8, 4, 2, 1) while halving
    int idx = 0, c2 = V;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        if (c2 > 1) { c2 /= 2; if (lane & off) idx += c2; }
    }
    const int lanes_per_value = 16 / V;
    if ((lane % lanes_per_value) == 0) {
        const int k = idx / R, r = idx % R, p = prow + 16 * k;
        static_cast<bf16*>(a.y)[((size_t)bh * R + r) * kP + p] = (bf16)v[0];
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
