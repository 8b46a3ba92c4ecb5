// Per-coordinate selective scan (the Mamba 1 preset) on gfx950.
//
// "Diagonal Equivalence in State Space Models ..." (paperpeel.com), section 5.1
// "Per-coordinate scan" and the Mamba 1 row of its table of copied-weight
// presets; "Mamba-3: Improved Sequence Modeling using State Space Principles",
// section "How Mamba gets its recurrence from a differential equation".  For
// every batch b, channel d (group g = d G / D of the shared B, C) and state
// coordinate n, with the static rate a[d, n] = -exp(A_log[d, n]):
//     h[n] <- exp(dt a[d, n]) h[n] + dt B[g, n] x,      y = sum_n C[g, n] h[n].
//
// Work decomposition.  A workgroup (16 N threads) owns 64 consecutive channels
// of one batch (and one sequence segment); each lane holds
// four coordinates of one channel (a channel's lanes are consecutive), so the
// readout is a sum over the channel's N / 4 lanes (DPP within quads, lane swaps
// beyond).  Tokens go in blocks of 64: the block's x and dt tiles are fetched as
// whole rows (the channels of one token are contiguous), transposed into LDS
// (channel-major, so a lane reads four tokens per access), B and C rows are
// staged as fp32, and the outputs leave through an LDS tile as whole rows.  The
// next block's rows are fetched into registers while the current one computes.
// The recurrence itself is sequential in each lane (work-optimal: N / 4
// independent chains per lane, and enough channels to fill the chip on the
// training shapes).
//
// Few channels and long sequences: the sequence is split into segments.  Pass 1
// runs each segment from a zero state and records its local final state and the
// sum of its steps (a coordinate's decay over the segment is exp(a sum dt), the
// rates being static); pass 2 combines the segments' affine maps (decay, local
// state) with a wave-level inclusive scan (Kogge-Stone over lanes, DPP and
// lane swaps; [D] section 5.5) into each segment's incoming state; pass 3
// re-runs every segment from its true state.
#include <algorithm>

#include "m3_internal.h"

namespace m3 {

namespace {

constexpr int kPcsTB = 64;                 // tokens per block
constexpr int kPcsCW = 64;                 // channels per workgroup
constexpr float kPcsLog2e = 1.4426950408889634f;

enum PcsMode { kPcsFull = 0, kPcsSummary = 1 };

template <int N>
struct PcsLayout {
    static constexpr int LPC = N / 4;                          // lanes per channel
    static constexpr int CW = kPcsCW;                          // channels per workgroup
    static constexpr int NT = CW * LPC;                        // threads per workgroup
    static constexpr int XS = kPcsTB + 4;                      // row stride (floats) of the transposed tiles
    static constexpr int xs = 0;                               // float [CW][XS]: x, channel-major
    static constexpr int ds = xs + CW * XS * 4;                // float [CW][XS]: dt
    static constexpr int bs = ds + CW * XS * 4;                // float [TB][N]: B
    static constexpr int cs = bs + kPcsTB * N * 4;             // float [TB][N]: C
    static constexpr int ys = cs + kPcsTB * N * 4;             // float [TB][CW]: outputs, token-major
    static constexpr int total = ys + kPcsTB * CW * 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Sum over groups of W consecutive lanes (W a power of two <= 16), every lane of
// the group receiving the total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false));  // quad_perm 1,0,3,2
    if constexpr (W >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, false));  // quad_perm 2,3,0,1
    if constexpr (W >= 8) v += __shfl_xor(v, 4);
    if constexpr (W >= 16) v += __shfl_xor(v, 8);
    return v;
}

template <int N, int MODE, bool BF16>
__global__ __launch_bounds__(PcsLayout<N>::NT) void pcs_kernel(PcsArgs a) {
    using LY = PcsLayout<N>;
    constexpr int LPC = LY::LPC, CW = LY::CW, XS = LY::XS, TB = kPcsTB, kPcsThreads = LY::NT;
    constexpr bool kFull = MODE == kPcsFull;
    constexpr int ES = BF16 ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float* sX = reinterpret_cast<float*>(smem + LY::xs);
    float* sD = reinterpret_cast<float*>(smem + LY::ds);
    float* sB = reinterpret_cast<float*>(smem + LY::bs);
    float* sC = reinterpret_cast<float*>(smem + LY::cs);
    float* sY = reinterpret_cast<float*>(smem + LY::ys);

    const int tid = threadIdx.x;
    const int D = a.D, L = a.L, G = a.G, nseg = a.nseg;
    const int ntile = (D + CW - 1) / CW;
    int bid = blockIdx.x;
    const int seg = bid % nseg;
    bid /= nseg;
    const int tile = bid % ntile, bi = bid / ntile;
    const int d0 = tile * CW;
    const int g = d0 * G / D;                  // the tile's channels share one group (checked on the host)
    const int T0 = seg * a.seglen, T1 = min(L, T0 + a.seglen);

    // this lane: channel c of the tile, coordinates 4 q .. 4 q + 3
    const int c = tid / LPC, q = tid % LPC;
    const int d = d0 + c;
    const bool live = d < D;
    float a2[4], h[4];
    const size_t S = (size_t)a.b * D * nseg;
    const size_t chs = ((size_t)bi * D + (live ? d : 0)) * nseg + seg;    // (batch, channel, segment)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int n = 4 * q + m;
        a2[m] = live ? -expf(a.A_log[(size_t)d * N + n]) * kPcsLog2e : 0.f;
        float v = 0.f;
        if (kFull && live) {
            if (seg == 0) v = a.h0 ? a.h0[((size_t)bi * D + d) * N + n] : 0.f;
            else v = a.ws[S * N + chs * N + n];           // incoming state from the carry pass
        }
        h[m] = v;
    }
    float dsum = 0.f;                                      // sum of the segment's steps (summary)

    // ---- block fetch: rows of the block's tokens into registers ----
    // x: TB rows of CW * ES bytes; dt: TB rows of CW * 4 bytes; B, C: TB rows of N * ES bytes.
    constexpr int XP = TB * CW * ES / 16, DP = TB * CW * 4 / 16, BP = TB * N * ES / 16;   // 16-byte pieces
    constexpr int XV = (XP + kPcsThreads - 1) / kPcsThreads;     // ... per thread
    constexpr int DV = (DP + kPcsThreads - 1) / kPcsThreads;
    constexpr int BV = (BP + kPcsThreads - 1) / kPcsThreads;
    uint4 rX[XV], rD[DV], rB[BV], rC[BV];
    const uint8_t* xg = static_cast<const uint8_t*>(a.x);
    const uint8_t* dg = reinterpret_cast<const uint8_t*>(a.dt);
    const uint8_t* bg = static_cast<const uint8_t*>(a.B);
    const uint8_t* cg = static_cast<const uint8_t*>(a.C);
    auto fetch = [&](int t0) {
        constexpr int XPR = CW * ES / 16;                         // 16-byte pieces per x row
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int e = tid + kPcsThreads * v, r = e / XPR, k = e % XPR;
            const int t = t0 + r, dd = d0 + k * (16 / ES);
            uint4 z = {0u, 0u, 0u, 0u};
            if (e < XP && t < T1 && dd < D) z = *reinterpret_cast<const uint4*>(xg + (((size_t)bi * L + t) * D + dd) * ES);
            rX[v] = z;
        }
        constexpr int DPR = CW * 4 / 16;
#pragma unroll
        for (int v = 0; v < DV; ++v) {
            const int e = tid + kPcsThreads * v, r = e / DPR, k = e % DPR;
            const int t = t0 + r, dd = d0 + k * 4;
            uint4 z = {0u, 0u, 0u, 0u};
            if (e < DP && t < T1 && dd < D) z = *reinterpret_cast<const uint4*>(dg + (((size_t)bi * L + t) * D + dd) * 4);
            rD[v] = z;
        }
        constexpr int BPR = N * ES / 16;
#pragma unroll
        for (int v = 0; v < BV; ++v) {
            const int e = tid + kPcsThreads * v, r = e / BPR, k = e % BPR;
            const int t = t0 + r;
            uint4 zb = {0u, 0u, 0u, 0u}, zc = {0u, 0u, 0u, 0u};
            if (e < BP && t < T1) {
                const size_t o = ((((size_t)bi * L + t) * G + g) * N) * ES + 16 * k;
                zb = *reinterpret_cast<const uint4*>(bg + o);
                if (kFull) zc = *reinterpret_cast<const uint4*>(cg + o);
            }
            rB[v] = zb;
            rC[v] = zc;
        }
    };
    // the fetched rows into the LDS tiles: x and dt transposed (channel-major), B and C as fp32
    auto stage = [&]() {
        constexpr int XPR = CW * ES / 16;
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int e = tid + kPcsThreads * v, r = e / XPR, k = e % XPR;
            const int cc = k * (16 / ES);
            if (e >= XP) break;
            if constexpr (BF16) {
                const uint32_t w[4] = {rX[v].x, rX[v].y, rX[v].z, rX[v].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sX[(cc + 2 * i) * XS + r] = bf16_lo(w[i]);
                    sX[(cc + 2 * i + 1) * XS + r] = bf16_hi(w[i]);
                }
            } else {
                const float f[4] = {__uint_as_float(rX[v].x), __uint_as_float(rX[v].y), __uint_as_float(rX[v].z),
                                    __uint_as_float(rX[v].w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) sX[(cc + i) * XS + r] = f[i];
            }
        }
        constexpr int DPR = CW * 4 / 16;
#pragma unroll
        for (int v = 0; v < DV; ++v) {
            const int e = tid + kPcsThreads * v, r = e / DPR, k = e % DPR;
            const int cc = k * 4;
            if (e >= DP) break;
            sD[(cc + 0) * XS + r] = __uint_as_float(rD[v].x);
            sD[(cc + 1) * XS + r] = __uint_as_float(rD[v].y);
            sD[(cc + 2) * XS + r] = __uint_as_float(rD[v].z);
            sD[(cc + 3) * XS + r] = __uint_as_float(rD[v].w);
        }
        constexpr int BPR = N * ES / 16;
#pragma unroll
        for (int v = 0; v < BV; ++v) {
            const int e = tid + kPcsThreads * v, r = e / BPR, k = e % BPR;
            if (e < BP) {
                const int n0 = k * (16 / ES);
                if constexpr (BF16) {
                    const uint32_t wb[4] = {rB[v].x, rB[v].y, rB[v].z, rB[v].w};
                    const uint32_t wc[4] = {rC[v].x, rC[v].y, rC[v].z, rC[v].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sB[r * N + n0 + 2 * i] = bf16_lo(wb[i]);
                        sB[r * N + n0 + 2 * i + 1] = bf16_hi(wb[i]);
                        if (kFull) {
                            sC[r * N + n0 + 2 * i] = bf16_lo(wc[i]);
                            sC[r * N + n0 + 2 * i + 1] = bf16_hi(wc[i]);
                        }
                    }
                } else {
                    *reinterpret_cast<uint4*>(sB + r * N + n0) = rB[v];
                    if (kFull) *reinterpret_cast<uint4*>(sC + r * N + n0) = rC[v];
                }
            }
        }
    };
    // the block's outputs, whole rows of CW channels
    auto store_y = [&](int t0) {
        if constexpr (kFull) {
            constexpr int EPS = 16 / ES;                         // elements per 16-byte piece
            constexpr int YPR = CW / EPS;
#pragma unroll
            for (int v = 0; v < (TB * YPR + kPcsThreads - 1) / kPcsThreads; ++v) {
                const int e = tid + kPcsThreads * v, r = e / YPR, k = e % YPR;
                if (e >= TB * YPR) break;
                const int t = t0 + r, dd = d0 + k * EPS;
                const float* src = sY + r * CW + k * EPS;
                uint4 o;
                if constexpr (BF16) {
                    uint32_t w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        bf16x2 p;
                        p[0] = (bf16)src[2 * i];
                        p[1] = (bf16)src[2 * i + 1];
                        w[i] = __builtin_bit_cast(uint32_t, p);
                    }
                    o = uint4{w[0], w[1], w[2], w[3]};
                } else {
                    o = uint4{__float_as_uint(src[0]), __float_as_uint(src[1]), __float_as_uint(src[2]), __float_as_uint(src[3])};
                }
                if (t < T1 && dd < D) *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.y) + (((size_t)bi * L + t) * D + dd) * ES) = o;
            }
        }
    };

    if (T0 < T1) fetch(T0);
    for (int t0 = T0; t0 < T1; t0 += TB) {
        __syncthreads();                       // the previous block's tiles are consumed
        stage();
        __syncthreads();
        if (t0 + TB < T1) fetch(t0 + TB);      // the next block's rows, under this block's math
        const int nt = min(TB, T1 - t0);
        const float* xr = sX + c * XS;
        const float* dr = sD + c * XS;
#pragma unroll 1
        for (int t4 = 0; t4 < TB; t4 += 4) {
            if (t4 >= nt) break;
            const float4 xv = *reinterpret_cast<const float4*>(xr + t4);
            const float4 dv = *reinterpret_cast<const float4*>(dr + t4);
            const float xs4[4] = {xv.x, xv.y, xv.z, xv.w}, ds4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t4 + j;
                const float st = ds4[j];
                const float u = st * xs4[j];
                const float4 bv = *reinterpret_cast<const float4*>(sB + t * N + 4 * q);
                const float b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) h[m] = __builtin_amdgcn_exp2f(st * a2[m]) * h[m] + u * b4[m];
                if constexpr (kFull) {
                    const float4 cv = *reinterpret_cast<const float4*>(sC + t * N + 4 * q);
                    float acc = cv.x * h[0] + cv.y * h[1] + cv.z * h[2] + cv.w * h[3];
                    acc = group_sum<LPC>(acc);
                    if (q == 0) sY[t * CW + c] = acc;
                } else {
                    dsum += st;
                }
            }
        }
        if constexpr (kFull) {
            __syncthreads();
            store_y(t0);
        }
    }
    if (!live) return;
    if constexpr (kFull) {
        if (T1 == L && a.h1)
#pragma unroll
            for (int m = 0; m < 4; ++m) a.h1[((size_t)bi * D + d) * N + 4 * q + m] = h[m];
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) a.ws[chs * N + 4 * q + m] = h[m];
        if (q == 0) a.ws[2 * S * N + chs] = dsum;
    }
}

// Inclusive scan of the affine maps h -> A h + W over groups of W lanes (earlier lanes
// first): after it, lane k holds the composition of the maps of lanes 0 .. k of its group.
// Kogge-Stone: a lane combines with the lane o below it for o = 1, 2, 4, ...
template <int W>
__device__ __forceinline__ void affine_scan(float& A, float& B, int k) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
        const float Ap = __shfl_up(A, o, W), Bp = __shfl_up(B, o, W);
        if (k >= o) {
            B = A * Bp + B;
            A = A * Ap;
        }
    }
}

// Pass 2 of the segmented schedule: each (batch, channel, coordinate) owns a group of
// 64 lanes, lane k one segment (k < nseg; the others carry the identity map).  Segment
// k's map is (exp(a sum dt_k), local final state); its incoming state is the inclusive
// composition of segments 0 .. k - 1 applied to h0.
__global__ __launch_bounds__(256) void pcs_carry_kernel(PcsArgs a) {
    const int N = a.N, D = a.D, nseg = a.nseg;
    const int lane = threadIdx.x & 63;
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);       // (batch, channel, coordinate)
    if (item >= (long)a.b * D * N) return;
    const int n = item % N;
    const long bd = item / N;
    const int d = bd % D;
    const size_t S = (size_t)a.b * D * nseg;
    float A = 1.f, B = 0.f;
    if (lane < nseg) {
        const size_t chs = (size_t)bd * nseg + lane;
        const float rate = -expf(a.A_log[(size_t)d * N + n]);
        A = expf(rate * a.ws[2 * S * N + chs]);
        B = a.ws[chs * N + n];
    }
    affine_scan<64>(A, B, lane);
    const float h0 = a.h0 ? a.h0[(size_t)bd * N + n] : 0.f;
    // lane k holds segments 0 .. k composed: the incoming state of segment k + 1
    if (lane + 1 < nseg) a.ws[S * N + ((size_t)bd * nseg + lane + 1) * N + n] = A * h0 + B;
}

template <int N, bool BF16>
hipError_t launch_pcs_n(const PcsArgs& a, hipStream_t st) {
    using LY = PcsLayout<N>;
    const int ntile = (a.D + LY::CW - 1) / LY::CW;
    const int nblk = a.b * ntile * a.nseg;
    constexpr int kPcsThreads = LY::NT;
    hipError_t e;
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pcs_kernel<N, kPcsSummary, BF16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LY::total);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((pcs_kernel<N, kPcsSummary, BF16>), dim3(nblk), dim3(kPcsThreads), LY::total, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const long items = (long)a.b * a.D * a.N;
        hipLaunchKernelGGL(pcs_carry_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pcs_kernel<N, kPcsFull, BF16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LY::total);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pcs_kernel<N, kPcsFull, BF16>), dim3(nblk), dim3(kPcsThreads), LY::total, st, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_pcs_t(const PcsArgs& a, hipStream_t st) {
    switch (a.N) {
        case 8: return launch_pcs_n<8, BF16>(a, st);
        case 16: return launch_pcs_n<16, BF16>(a, st);
        case 32: return launch_pcs_n<32, BF16>(a, st);
        case 64: return launch_pcs_n<64, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool pcs_supported_state(int N) { return N == 8 || N == 16 || N == 32 || N == 64; }

int pcs_channels_per_group(int) { return kPcsCW; }

int pcs_groups_per_cu(int N) {
    auto fit = [](int lds, int threads) { return std::max(1, std::min(163840 / lds, 2048 / threads)); };
    switch (N) {
        case 8: return fit(PcsLayout<8>::total, PcsLayout<8>::NT);
        case 16: return fit(PcsLayout<16>::total, PcsLayout<16>::NT);
        case 32: return fit(PcsLayout<32>::total, PcsLayout<32>::NT);
        default: return fit(PcsLayout<64>::total, PcsLayout<64>::NT);
    }
}

int pcs_block_tokens() { return kPcsTB; }

size_t pcs_workspace_bytes(const PcsArgs& a) {
    if (a.nseg <= 1) return 0;
    const size_t S = (size_t)a.b * a.D * a.nseg;
    return (2 * S * a.N + S) * sizeof(float);
}

hipError_t launch_pcs(const PcsArgs& a, hipStream_t st) {
    return a.io_bf16 ? launch_pcs_t<true>(a, st) : launch_pcs_t<false>(a, st);
}

}  // namespace m3
