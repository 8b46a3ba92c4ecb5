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
// The recurrence is sequential in each lane (work-optimal: K independent chains
// per lane, and enough channels to fill the chip on the training shapes); the
// work decomposition is described at the kernel.
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

constexpr int kPcsCW = 64;                 // channels per workgroup
constexpr float kPcsLog2e = 1.4426950408889634f;

// Coordinates per lane and tokens per block (the schedule; the result does not
// depend on them beyond rounding).
#ifndef PCS_K
#define PCS_K 4
#endif
#ifndef PCS_TB
#define PCS_TB 32
#endif
#ifndef PCS_STREAM
#define PCS_STREAM 1
#endif
constexpr int kPcsK = PCS_K;
constexpr int kPcsTB = PCS_TB;

enum PcsMode { kPcsFull = 0, kPcsSummary = 1 };

// Floats of the segmented schedule's part of the workspace (local final states and
// incoming states [b, D, nseg, N], step sums [b, D, nseg]), rounded to 64 floats.
size_t pcs_seg_floats(const PcsArgs& a) {
    if (a.nseg <= 1) return 0;
    const size_t S = (size_t)a.b * a.D * a.nseg;
    return (2 * S * a.N + S + 63) & ~(size_t)63;
}

template <int N>
struct PcsLayout {
    static constexpr int K = kPcsK < N ? kPcsK : N;            // coordinates per lane
    static constexpr int LPC = N / K;                          // lanes per channel
    static constexpr int CW = kPcsCW;                          // channels per workgroup
    static constexpr int NT = CW * LPC;                        // threads per workgroup
    static constexpr int TB = kPcsTB;                          // tokens per block
    static constexpr int XS = TB + 4;                          // row stride (floats) of the transposed tiles
    static constexpr int xs = 0;                               // float [CW][XS]: x, channel-major; then y
    static constexpr int ds = xs + CW * XS * 4;                // float [CW][XS]: dt
    static constexpr int bs = ds + CW * XS * 4;                // float [TB][N]: B
    static constexpr int cs = bs + TB * N * 4;                 // float [TB][N]: C
    static constexpr int total = cs + TB * N * 4;
    static_assert(K % 4 == 0 && N % K == 0 && LPC <= 16 && NT <= 1024, "lane layout");
};

// A buffer resource over [base, base + bytes): loads past the end read zero and stores
// past it are dropped, so edge tiles need no branches (and the compiler can count
// the loads and stores in flight exactly instead of waiting for all of them).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pcs_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kPcsOob = 0x7ffffff0;        // an offset past every resource's end
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Sum over groups of W consecutive lanes (W a power of two <= 16), every lane of
// the group receiving the total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    // (the moves carry bound_ctrl, so the compiler folds each into its add as a DPP operand)
    if constexpr (W >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, true));  // quad_perm 1,0,3,2
    if constexpr (W >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, true));  // quad_perm 2,3,0,1
    if constexpr (W >= 8) v += __shfl_xor(v, 4);
    if constexpr (W >= 16) v += __shfl_xor(v, 8);
    return v;
}

// Work decomposition.  A workgroup of 64 N / K threads owns 64 consecutive
// channels of one batch (and one sequence segment); each lane holds K coordinates
// of one channel (a channel's N / K lanes are consecutive), so the readout is a
// sum over the channel's lanes (DPP within quads, lane swaps beyond).  Tokens go
// in blocks of TB: the block's x and dt tiles are fetched as whole rows (the
// channels of one token are contiguous) and transposed into LDS (channel-major,
// so a lane reads four tokens per access); B and C rows are staged as fp32.  Each
// channel's readout overwrites the x entry of the same token, already consumed, and
// the block's outputs leave from that tile as whole rows.  The next block's rows
// are fetched into registers while the current one computes.
template <int N, int MODE, bool BF16>
__global__ __launch_bounds__(PcsLayout<N>::NT) void pcs_kernel(PcsArgs a) {
    using LY = PcsLayout<N>;
    constexpr int K = LY::K, LPC = LY::LPC, CW = LY::CW, XS = LY::XS, TB = LY::TB, NT = LY::NT;
    constexpr bool kFull = MODE == kPcsFull;
    constexpr int ES = BF16 ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float* sX = reinterpret_cast<float*>(smem + LY::xs);
    float* sD = reinterpret_cast<float*>(smem + LY::ds);
    float* sB = reinterpret_cast<float*>(smem + LY::bs);
    float* sC = reinterpret_cast<float*>(smem + LY::cs);

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

    // this lane: channel c of the tile, coordinates K q .. K q + K - 1
    const int c = tid / LPC, q = tid % LPC;
    const int d = d0 + c;
    const bool live = d < D;
    float a2[K], h[K];
    const size_t S = (size_t)a.b * D * nseg;
    const size_t chs = ((size_t)bi * D + (live ? d : 0)) * nseg + seg;    // (batch, channel, segment)
#pragma unroll
    for (int m = 0; m < K; ++m) {
        const int n = K * q + m;
        a2[m] = live ? -expf(a.A_log[(size_t)d * N + n]) * kPcsLog2e : 0.f;
        float v = 0.f;
        if (kFull && live) {
            if (seg == 0) v = a.h0 ? a.h0[((size_t)bi * D + d) * N + n] : 0.f;
            else v = a.ws[S * N + chs * N + n];           // incoming state from the carry pass
        }
        h[m] = v;
    }
    float dsum = 0.f;                                      // sum of the segment's steps (summary)
    // The state and rate loads land before the first block: otherwise the wait for them,
    // merged over the block loop, also waits for each block's prefetch as its math starts.
    __builtin_amdgcn_s_waitcnt(0x0f70);                    // vmcnt(0)

    // ---- block fetch: rows of the block's tokens into registers ----
    // x: TB rows of CW * ES bytes; dt: TB rows of CW * 4 bytes (16-byte pieces); B, C: TB
    // rows of N * ES bytes (4-byte pieces).  Where a tile divides evenly among the threads
    // (the common shapes) no thread is idle and no check is compiled.
    constexpr int XP = TB * CW * ES / 16, DP = TB * CW * 4 / 16, BP = TB * N * ES / 4;
    constexpr int XV = (XP + NT - 1) / NT;     // ... per thread
    constexpr int DV = (DP + NT - 1) / NT;
    constexpr int BV = (BP + NT - 1) / NT;
    constexpr bool kXe = XP % NT == 0, kDe = DP % NT == 0, kBe = BP % NT == 0;
    uint4 rX[XV], rD[DV];
    uint32_t rB[BV], rC[BV];
    // resources over the segment's rows (the host keeps each under 2 GiB): a row at or past
    // T1 reads zero, and an output row there is dropped
    const size_t row0 = (size_t)bi * L + T0;
    const uint32_t nrow = (uint32_t)(T1 - T0);
    const auto rx = pcs_rsrc(static_cast<const uint8_t*>(a.x) + row0 * D * ES, nrow * (uint32_t)D * ES);
    const auto rd = pcs_rsrc(reinterpret_cast<const uint8_t*>(a.dt) + row0 * D * 4, nrow * (uint32_t)D * 4);
    const auto rb = pcs_rsrc(static_cast<const uint8_t*>(a.B) + row0 * G * N * ES, nrow * (uint32_t)(G * N * ES));
    const auto rc = pcs_rsrc(static_cast<const uint8_t*>(a.C) + row0 * G * N * ES, nrow * (uint32_t)(G * N * ES));
    const auto ry = pcs_rsrc(static_cast<uint8_t*>(a.y) + row0 * D * ES, nrow * (uint32_t)D * ES);
    auto fetch = [&](int t0) {
        const int tr = t0 - T0;                                   // the block's first row in the segment
        constexpr int XPR = CW * ES / 16;                         // 16-byte pieces per x row
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int e = tid + NT * v, r = e / XPR, k = e % XPR;
            const int dd = d0 + k * (16 / ES);
            const int o = ((kXe || e < XP) && dd < D) ? ((tr + r) * D + dd) * ES : kPcsOob;
            rX[v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
        }
        constexpr int DPR = CW * 4 / 16;
#pragma unroll
        for (int v = 0; v < DV; ++v) {
            const int e = tid + NT * v, r = e / DPR, k = e % DPR;
            const int dd = d0 + k * 4;
            const int o = ((kDe || e < DP) && dd < D) ? ((tr + r) * D + dd) * 4 : kPcsOob;
            rD[v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, o, 0, 0));
        }
        constexpr int BPR = N * ES / 4;
#pragma unroll
        for (int v = 0; v < BV; ++v) {
            const int e = tid + NT * v, r = e / BPR, k = e % BPR;
            const int o = (kBe || e < BP) ? ((tr + r) * G + g) * N * ES + 4 * k : kPcsOob;
            rB[v] = __builtin_amdgcn_raw_buffer_load_b32(rb, o, 0, 0);
            if (kFull) rC[v] = __builtin_amdgcn_raw_buffer_load_b32(rc, o, 0, 0);
        }
    };
    // the fetched rows into the LDS tiles: x and dt transposed (channel-major), B and C as fp32
    auto stage = [&]() {
        constexpr int XPR = CW * ES / 16;
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int e = tid + NT * v, r = e / XPR, k = e % XPR;
            const int cc = k * (16 / ES);
            if constexpr (!kXe) if (e >= XP) break;
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
            const int e = tid + NT * v, r = e / DPR, k = e % DPR;
            const int cc = k * 4;
            if constexpr (!kDe) if (e >= DP) break;
            sD[(cc + 0) * XS + r] = __uint_as_float(rD[v].x);
            sD[(cc + 1) * XS + r] = __uint_as_float(rD[v].y);
            sD[(cc + 2) * XS + r] = __uint_as_float(rD[v].z);
            sD[(cc + 3) * XS + r] = __uint_as_float(rD[v].w);
        }
        constexpr int BPR = N * ES / 4;
#pragma unroll
        for (int v = 0; v < BV; ++v) {
            const int e = tid + NT * v, r = e / BPR, k = e % BPR;
            if constexpr (!kBe) if (e >= BP) break;
            const int n0 = k * (4 / ES);
            if constexpr (BF16) {
                *reinterpret_cast<float2*>(sB + r * N + n0) = float2{bf16_lo(rB[v]), bf16_hi(rB[v])};
                if (kFull) *reinterpret_cast<float2*>(sC + r * N + n0) = float2{bf16_lo(rC[v]), bf16_hi(rC[v])};
            } else {
                sB[r * N + n0] = __uint_as_float(rB[v]);
                if (kFull) sC[r * N + n0] = __uint_as_float(rC[v]);
            }
        }
    };
    // the block's outputs (in the x tile, channel-major) as whole rows of CW channels
    auto store_y = [&](int t0) {
        if constexpr (kFull) {
            constexpr int EPS = 16 / ES;                         // elements per 16-byte piece
            constexpr int YPR = CW / EPS;
            constexpr int YP = TB * YPR;
#pragma unroll
            for (int v = 0; v < (YP + NT - 1) / NT; ++v) {
                const int e = tid + NT * v, r = e / YPR, k = e % YPR;
                if constexpr (YP % NT != 0) if (e >= YP) break;
                const int dd = d0 + k * EPS;
                const float* src = sX + (k * EPS) * XS + r;
                uint4 o;
                if constexpr (BF16) {
                    uint32_t w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        bf16x2 p;
                        p[0] = (bf16)src[(2 * i) * XS];
                        p[1] = (bf16)src[(2 * i + 1) * XS];
                        w[i] = __builtin_bit_cast(uint32_t, p);
                    }
                    o = uint4{w[0], w[1], w[2], w[3]};
                } else {
                    o = uint4{__float_as_uint(src[0]), __float_as_uint(src[XS]), __float_as_uint(src[2 * XS]),
                              __float_as_uint(src[3 * XS])};
                }
                const int off = dd < D ? ((t0 - T0 + r) * D + dd) * ES : kPcsOob;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), ry, off, 0, 0);
            }
        }
    };

    if (T0 < T1) fetch(T0);
    if constexpr (kFull) {
        // as many dropped stores (past the resource's end) as a block stores, so that the
        // stores in flight at the first block's staging match those of every later block
        // and the wait there covers only the fetch
        constexpr int YV = (TB * CW * ES / 16 + NT - 1) / NT;
#pragma unroll
        for (int v = 0; v < YV; ++v) __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, ry, kPcsOob, 0, 0);
    }
    for (int t0 = T0; t0 < T1; t0 += TB) {
        __syncthreads();                       // the previous block's tiles are consumed
        stage();
        __syncthreads();
        if (t0 + TB < T1) fetch(t0 + TB);      // the next block's rows, under this block's math
        const int nt = min(TB, T1 - t0);
        float* xr = sX + c * XS;
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
                float bk[K];
#pragma unroll
                for (int m4 = 0; m4 < K; m4 += 4) {
                    const float4 bv = *reinterpret_cast<const float4*>(sB + t * N + K * q + m4);
                    bk[m4] = bv.x; bk[m4 + 1] = bv.y; bk[m4 + 2] = bv.z; bk[m4 + 3] = bv.w;
                }
#pragma unroll
                for (int m = 0; m < K; ++m) h[m] = __builtin_amdgcn_exp2f(st * a2[m]) * h[m] + u * bk[m];
                if constexpr (kFull) {
                    float acc;
#pragma unroll
                    for (int m4 = 0; m4 < K; m4 += 4) {
                        const float4 cv = *reinterpret_cast<const float4*>(sC + t * N + K * q + m4);
                        const float part = cv.x * h[m4] + cv.y * h[m4 + 1] + cv.z * h[m4 + 2] + cv.w * h[m4 + 3];
                        acc = m4 == 0 ? part : acc + part;
                    }
                    acc = group_sum<LPC>(acc);
                    // x[t] of this channel was read above by every lane of the channel (one
                    // wave); the channel's lanes all hold the sum and write the same value
                    xr[t] = acc;
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
            for (int m = 0; m < K; ++m) a.h1[((size_t)bi * D + d) * N + K * q + m] = h[m];
    } else {
#pragma unroll
        for (int m = 0; m < K; ++m) a.ws[chs * N + K * q + m] = h[m];
        if (q == 0) a.ws[2 * S * N + chs] = dsum;
    }
}

// ---- streaming form, N = 16 -------------------------------------------------------
// A workgroup of NW waves owns 64 channels: lane c of every wave holds channel d0 + c,
// wave w the coordinates w N / NW .. (w + 1) N / NW - 1.  Two waves when the channels
// alone set the parallelism (a lone wave issues a vector instruction only every fourth
// cycle or so; two interleave on the SIMD), one when sequence segments already give
// every SIMD several waves (no exchange, no duplicated x and dt reads).  Per token a
// wave reads one 64-channel row piece of x (128 bytes in bf16) and of dt, whole cache
// lines, PF tokens ahead of the math through a ring of registers.  B and C come in tiles
// of PF tokens (one vector load per lane, a tile ahead, in the same ring), each wave
// widening its own half of the coordinates to fp32 into one of two LDS tiles, from which
// each token's row is a uniform (broadcast) read.  LDS reads complete in order, so their
// waits stay exact.  (Scalar loads would deliver the rows as scalar operands, but they
// complete out of order: each wait for one drains all of them, defeating any prefetch.)
// Each wave keeps its (partial) readouts of a group of PF tokens; at the group's end two
// waves swap halves through LDS (one barrier) and each completes and stores half the
// group's outputs; a lone wave stores them all.
constexpr int kPcsPF = 16;                 // tokens in flight (the ring), and tokens per B, C tile
constexpr int kPcsHalf = kPcsPF / 2;

template <int N, int NW, int MODE, bool BF16>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4))) void pcs_stream_kernel(PcsArgs a) {
    static_assert(NW == 1 || NW == 2, "one or two waves");
    constexpr bool kFull = MODE == kPcsFull;
    constexpr int ES = BF16 ? 2 : 4, PF = kPcsPF, HF = kPcsHalf;
    constexpr int K = N / NW;                              // coordinates per lane
    const int lane = threadIdx.x & 63;
    const int w = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int D = a.D, L = a.L, G = a.G, nseg = a.nseg;
    const int ntile = (D + 63) / 64;
    int bid = blockIdx.x;
    const int seg = bid % nseg;
    bid /= nseg;
    const int tile = bid % ntile, bi = bid / ntile;
    const int d0 = tile * 64, d = d0 + lane;
    const int g = d0 * G / D;                  // the tile's channels share one group (checked on the host)
    const int T0 = seg * a.seglen, T1 = min(L, T0 + a.seglen);
    const bool live = d < D;
    const int n0 = w * K;                      // this wave's first coordinate

    float a2[K], h[K];
    const size_t S = (size_t)a.b * D * nseg;
    const size_t chs = ((size_t)bi * D + (live ? d : 0)) * nseg + seg;
#pragma unroll
    for (int m = 0; m < K; ++m) {
        a2[m] = live ? -expf(a.A_log[(size_t)d * N + n0 + m]) * kPcsLog2e : 0.f;
        float v = 0.f;
        if (kFull && live) {
            if (seg == 0) v = a.h0 ? a.h0[((size_t)bi * D + d) * N + n0 + m] : 0.f;
            else v = a.ws[S * N + chs * N + n0 + m];
        }
        h[m] = v;
    }
    float dsum = 0.f;
    // The state and rate loads land before the loop: otherwise the wait for them, merged
    // over the loop, would also wait for the ring's loads.
    __builtin_amdgcn_s_waitcnt(0x0f70);                    // vmcnt(0)

    // resources over the segment's rows (the host keeps each under 2 GiB); rows at or past
    // T1 read zero (dt = 0 leaves the state unchanged) and their outputs are dropped
    const size_t row0 = (size_t)bi * L + T0;
    const uint32_t nrow = (uint32_t)(T1 - T0);
    const auto rx = pcs_rsrc(static_cast<const uint8_t*>(a.x) + row0 * D * ES, nrow * (uint32_t)D * ES);
    const auto rd = pcs_rsrc(reinterpret_cast<const uint8_t*>(a.dt) + row0 * D * 4, nrow * (uint32_t)D * 4);
    const auto ry = pcs_rsrc(static_cast<uint8_t*>(a.y) + row0 * D * ES, nrow * (uint32_t)D * ES);
    const int lo = live ? d * ES : kPcsOob, lod = live ? d * 4 : kPcsOob;
    // the ring holds the loaded bits; they are converted where used, PF tokens later (a
    // conversion at the load would wait for the load at once)
    // (the lane's channel as the vector offset, the token row as the scalar offset)
    // x stays in the ring as the loaded bits (a 16-bit value for bf16: widening it to 32 bits
    // would mask its upper half at the loop's head, where that masking waits for every load)
    // (typed as a 16-bit float only so that no integer widening is asked for; no arithmetic
    // is done on it)
    using XRaw = typename std::conditional<BF16, _Float16, uint32_t>::type;
    auto ld_x = [&](int r) -> XRaw {
        if constexpr (BF16)
            return __builtin_bit_cast(_Float16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(rx, lo, r * D * ES, 0));
        else return __builtin_amdgcn_raw_buffer_load_b32(rx, lo, r * D * 4, 0);
    };
    auto ld_dt = [&](int r) -> uint32_t { return __builtin_amdgcn_raw_buffer_load_b32(rd, lod, r * D * 4, 0); };

    // B, C tiles: PF rows of this wave's K values; 16-byte pieces
    const auto rb = pcs_rsrc(static_cast<const uint8_t*>(a.B) + row0 * G * N * ES, nrow * (uint32_t)(G * N * ES));
    const auto rc = pcs_rsrc(static_cast<const uint8_t*>(a.C) + row0 * G * N * ES, nrow * (uint32_t)(G * N * ES));
    constexpr int PPR = K * ES / 16;                       // pieces per row
    static_assert(PPR >= 1, "a wave's half row is at least 16 bytes");
    constexpr int TP = PF * PPR;                           // pieces per tile (<= 64)
    constexpr int NTEN = kFull ? 2 : 1;                    // B, and C when the readout is made
    static_assert(TP <= 64, "tile pieces");
    __shared__ __attribute__((aligned(16))) float sBC[NW][2][2][PF][K];  // [wave][buffer][B, C][token][m]
    __shared__ __attribute__((aligned(16))) float sY[NW == 2 ? 2 : 1][2][64][PF];   // [buffer][from wave][lane][token]
    uint4 tq[NTEN];
    // with fewer pieces than lanes, lanes past them repeat a piece (same value to the same
    // address): no lane is masked off, so no branch splits the token loop's block
    auto fetch_tile = [&](int rt) {                        // rows rt .. rt + PF - 1
        const int e = lane % TP, row = e / PPR, part = e % PPR;
        const int o = ((rt + row) * G + g) * N * ES + n0 * ES + part * 16;
#pragma unroll
        for (int ten = 0; ten < NTEN; ++ten)
            tq[ten] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ten ? rc : rb, o, 0, 0));
    };
    auto stage_tile = [&](int buf) {
        const int e = lane % TP, row = e / PPR, part = e % PPR;
#pragma unroll
        for (int ten = 0; ten < NTEN; ++ten) {
            const uint4 t = tq[ten];
            float* dst = &sBC[w][buf][ten][row][part * (16 / ES)];
            if constexpr (BF16) {
                reinterpret_cast<float4*>(dst)[0] = float4{bf16_lo(t.x), bf16_hi(t.x), bf16_lo(t.y), bf16_hi(t.y)};
                reinterpret_cast<float4*>(dst)[1] = float4{bf16_lo(t.z), bf16_hi(t.z), bf16_lo(t.w), bf16_hi(t.w)};
            } else {
                *reinterpret_cast<uint4*>(dst) = t;
            }
        }
    };

    // Prologue, in the order the loop issues the same kinds of operations, so that what is
    // in flight at the loop's head is the same on entry and on every later pass and the
    // compiler's waits stay a ring deep: the first tile, the ring, a group's worth of
    // dropped stores (past the resource's end), the second tile.
    fetch_tile(0);
    XRaw xq[PF];
    uint32_t dq[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        xq[j] = ld_x(j);
        dq[j] = ld_dt(j);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kFull) {
#pragma unroll
        for (int j = 0; j < PF / NW; ++j) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)0, ry, kPcsOob, 0, 0);
    }
    stage_tile(0);
    fetch_tile(PF);

    float bn[K], cn[K];
    float yp[PF];                              // this wave's partial readouts of the group
    for (int r0 = 0; r0 < (int)nrow; r0 += PF) {
        const int buf = (r0 / PF) & 1;
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int r = r0 + j;
            // take this token's x and dt out of the ring before the slot is reloaded, so that
            // each slot keeps one register (a slot whose old and new values overlapped would
            // be copied at the loop's end, and the copy would wait for the load)
            // (for bf16 the copy is the widening shift: the value's bits to the upper half)
            uint32_t dcur, xcur;
            asm("v_mov_b32 %0, %1" : "=v"(dcur) : "v"(dq[j]));
            if constexpr (BF16) asm("v_lshlrev_b32 %0, 16, %1" : "=v"(xcur) : "v"(xq[j]));
            else asm("v_mov_b32 %0, %1" : "=v"(xcur) : "v"(xq[j]));
            __builtin_amdgcn_sched_barrier(0);
            xq[j] = ld_x(r + PF);              // the ring: this slot's next token
            dq[j] = ld_dt(r + PF);
#pragma unroll                                 // this token's rows, before the exponentials
            for (int m4 = 0; m4 < K; m4 += 4) {
                const float4 bv = *reinterpret_cast<const float4*>(&sBC[w][buf][0][j][m4]);
                bn[m4] = bv.x; bn[m4 + 1] = bv.y; bn[m4 + 2] = bv.z; bn[m4 + 3] = bv.w;
                if constexpr (kFull) {
                    const float4 cv = *reinterpret_cast<const float4*>(&sBC[w][buf][1][j][m4]);
                    cn[m4] = cv.x; cn[m4 + 1] = cv.y; cn[m4 + 2] = cv.z; cn[m4 + 3] = cv.w;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            const float st = __uint_as_float(dcur);
            const float u = st * __uint_as_float(xcur);
#pragma unroll
            for (int m = 0; m < K; ++m) h[m] = __builtin_amdgcn_exp2f(st * a2[m]) * h[m] + u * bn[m];
            if constexpr (kFull) {
                // partial sums: short dependency chains (four of N / 4 terms for a lone wave,
                // whose instructions issue in order; two at half the coordinates)
                constexpr int NP = NW == 1 ? 4 : 2;
                float p[NP];
#pragma unroll
                for (int k = 0; k < NP; ++k) p[k] = cn[k] * h[k];
#pragma unroll
                for (int m = NP; m < K; ++m) p[m % NP] += cn[m] * h[m];
                if constexpr (NP == 4) yp[j] = (p[0] + p[1]) + (p[2] + p[3]);
                else yp[j] = p[0] + p[1];
            } else {
                dsum += st;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        auto store_y = [&](int j, float acc) {
            const int r = r0 + j;
            if constexpr (BF16) {
                const bf16 yb = (bf16)acc;
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, yb), ry, lo, r * D * ES, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), ry, lo, r * D * 4, 0);
            }
        };
        if constexpr (kFull && NW == 1) {
#pragma unroll
            for (int j = 0; j < PF; ++j) store_y(j, yp[j]);
        } else if constexpr (kFull) {
            // both waves post all their partials; wave 0 completes tokens 0 .. HF - 1, wave 1
            // the rest, reading both halves back at an offset of its own (the wave index is
            // not a compile-time constant, and indexing the partials' registers by it
            // would take a register-indexing mode switch per value)
            float4* dst = reinterpret_cast<float4*>(&sY[buf][w][lane][0]);
#pragma unroll
            for (int i = 0; i < PF; i += 4) dst[i / 4] = float4{yp[i], yp[i + 1], yp[i + 2], yp[i + 3]};
            __syncthreads();
            const int keep = w * HF;
            const float4* s0 = reinterpret_cast<const float4*>(&sY[buf][0][lane][keep]);
            const float4* s1 = reinterpret_cast<const float4*>(&sY[buf][1][lane][keep]);
#pragma unroll
            for (int i = 0; i < HF; i += 4) {
                const float4 u = s0[i / 4], v = s1[i / 4];
                store_y(keep + i + 0, u.x + v.x);
                store_y(keep + i + 1, u.y + v.y);
                store_y(keep + i + 2, u.z + v.z);
                store_y(keep + i + 3, u.w + v.w);
            }
        }
        // the next tile (loaded through this group) into the other buffer, and the one after
        // it on its way; each wave stages only the rows it reads: no barrier
        stage_tile(buf ^ 1);
        fetch_tile(r0 + 2 * PF);
    }
    if (!live) return;
    if constexpr (kFull) {
        if (T1 == L && a.h1)
#pragma unroll
            for (int m = 0; m < K; ++m) a.h1[((size_t)bi * D + d) * N + n0 + m] = h[m];
    } else {
#pragma unroll
        for (int m = 0; m < K; ++m) a.ws[chs * N + n0 + m] = h[m];
        if (w == 0) a.ws[2 * S * N + chs] = dsum;
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
hipError_t launch_pcs_stream(const PcsArgs& a, hipStream_t st) {
    const int nblk = a.b * ((a.D + 63) / 64) * a.nseg;
    hipError_t e;
    if (a.nseg > 1) {
        // segments give the parallelism: one wave per 64 channels
        hipLaunchKernelGGL((pcs_stream_kernel<N, 1, kPcsSummary, BF16>), dim3(nblk), dim3(64), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const long items = (long)a.b * a.D * a.N;
        hipLaunchKernelGGL(pcs_carry_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((pcs_stream_kernel<N, 1, kPcsFull, BF16>), dim3(nblk), dim3(64), 0, st, a);
    } else {
        hipLaunchKernelGGL((pcs_stream_kernel<N, 2, kPcsFull, BF16>), dim3(nblk), dim3(128), 0, st, a);
    }
    return hipGetLastError();
}

template <int N, bool BF16>
hipError_t launch_pcs_n(const PcsArgs& a, hipStream_t st) {
    using LY = PcsLayout<N>;
    const int ntile = (a.D + LY::CW - 1) / LY::CW;
    const int nblk = a.b * ntile * a.nseg;
    constexpr int kThreads = LY::NT;
    hipError_t e;
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pcs_kernel<N, kPcsSummary, BF16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LY::total);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((pcs_kernel<N, kPcsSummary, BF16>), dim3(nblk), dim3(kThreads), LY::total, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const long items = (long)a.b * a.D * a.N;
        hipLaunchKernelGGL(pcs_carry_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pcs_kernel<N, kPcsFull, BF16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LY::total);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pcs_kernel<N, kPcsFull, BF16>), dim3(nblk), dim3(kThreads), LY::total, st, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_pcs_t(const PcsArgs& a, hipStream_t st) {
    switch (a.N) {
        case 8: return launch_pcs_n<8, BF16>(a, st);
        case 16: return PCS_STREAM ? launch_pcs_stream<16, BF16>(a, st) : launch_pcs_n<16, BF16>(a, st);
        case 32: return launch_pcs_n<32, BF16>(a, st);
        case 64: return launch_pcs_n<64, BF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool pcs_supported_state(int N) { return N == 8 || N == 16 || N == 32 || N == 64; }

int pcs_channels_per_group(int) { return kPcsCW; }

int pcs_waves_per_group(int N, bool segmented) {
    if (PCS_STREAM && N == 16) return segmented ? 1 : 2;   // waves per 64 channels
    switch (N) {
        case 8: return PcsLayout<8>::NT / 64;
        case 16: return PcsLayout<16>::NT / 64;
        case 32: return PcsLayout<32>::NT / 64;
        default: return PcsLayout<64>::NT / 64;
    }
}

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

size_t pcs_workspace_bytes(const PcsArgs& a) { return pcs_seg_floats(a) * sizeof(float); }

hipError_t launch_pcs(const PcsArgs& a, hipStream_t st) {
    return a.io_bf16 ? launch_pcs_t<true>(a, st) : launch_pcs_t<false>(a, st);
}

}  // namespace m3
