// Chunked scan for one rank without rotation or bias (the Mamba-2-equivalent SISO
// workload), bf16 I/O, fp32 state, P = 64, N = 128, chunks of 64 tokens.
//
// The same chunked form as the matrix-core scan ("The trapezoid term as a two-tap
// filter", "Mamba-3: Improved Sequence Modeling using State Space Principles"; chunk-local
// cumulative log-decays, "Diagonal Equivalence in State Space Models ...", section 2.4),
// with the folded carry Hf = H + d_next x_e B_e^T:
//   y_t    = exp(l_t) Hf_in C_t + sum_{u<=t} W(t,u) (C_t . B_u) x_u,
//   W(t,u) = exp(l_t - l_u) (g_u + [u<t] d_{u+1}),
//   Hf_out = exp(l_e) Hf_in + sum_u v_u x_u B_u^T,  v_u = exp(l_e - l_u)(g_u + d_{u+1}).
// With one rank, no bias and no rotation the scores C_t . B_u of a chunk depend on the
// (batch, group) only, not on the head ("MIMO: a rank-4 state update ...": B and C are
// shared by a group's heads).  So the work splits in two kernels:
//   * siso_prep_kernel, one workgroup per (batch, group, chunk): the chunk's causal score
//     tiles S^T = B C^T (fp32, in the MFMA result layout the scan reads them back in) and
//     the B^T operands of the state update (B's key rows as the k dimension, in the
//     permuted key order below), into the workspace;
//   * siso_scan_kernel, one workgroup of 4 waves per (batch, head, half of P): wave q owns
//     query tile q of each chunk (16 tokens) and a quarter of the state's N columns; it
//     weights its score tiles by W, multiplies by X^T (Y^T += X^T S'^T), adds the carry
//     readout (Y^T += exp(l_t) Hf C^T, the A operand a bf16 snapshot of the state in LDS),
//     and updates its state columns (Hf^T += B^T (v x)); x tiles come through LDS (the
//     only operand that needs a transpose), everything else straight from memory into
//     registers a chunk ahead.
// Key order inside a 32-key MFMA step (k slots of lane group g = lane / 16): keys 4 g ..
// 4 g + 3, then 16 + 4 g .. 16 + 4 g + 3: the order in which two 16 x 16 score tiles hold
// them (a lane's four rows of each), so weighted score tiles are B operands as they stand.
#include "scan_common.h"


namespace m3 {

namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSQ = 64;                                    // tokens per chunk
constexpr int kSTiles = 10;                                // causal score tiles (q >= kt) of a chunk
constexpr int kSTileBytes = 64 * 16;                       // one 16 x 16 fp32 tile, 16 bytes a lane
constexpr int kBTBytes = 8 * 2 * 64 * 16;                  // B^T operands: 8 n-tiles x 2 key steps
constexpr size_t kPrepChunkBytes = (size_t)kSTiles * kSTileBytes + kBTBytes;   // 26 KiB

__device__ __forceinline__ int stile(int q, int kt) { return q * (q + 1) / 2 + kt; }   // kt <= q

// Workgroup i of a launch runs on XCD i % 8; consecutive logical indices (one batch's score
// tiles, and the heads of one batch that read them) are placed on the same XCD, so that
// each XCD's L2 holds one batch's shared operands.
__device__ __forceinline__ int xcd_logical(int bid, int nblk) {
    return (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
}

// key of slot e (0..7) of lane group g in a 32-key step
__device__ __forceinline__ int slot_key(int g, int e) { return (e < 4 ? 4 * g : 16 + 4 * g) + (e & 3); }

// ---- pass 1: scores and B^T operands per (batch, group, chunk) ----------------------------
__global__ __launch_bounds__(256) void siso_prep_kernel(ScanArgs a) {
    const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int L = a.L, G = a.G;
    const int nch = (L + kSQ - 1) / kSQ;
    const int lb = xcd_logical(blockIdx.x, gridDim.x);
    const int c = lb % nch, bg = lb / nch;
    const int g = bg % G, bi = bg / G;
    const int c0 = c * kSQ;
    const int nv = min(kSQ, L - c0);
    const uint32_t rowb = (uint32_t)G * kN * 2u;               // bytes from one token's row to the next
    const size_t base = ((size_t)bi * L + c0) * G + g;          // row of the chunk's first token
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const uint16_t*>(a.B) + base * kN, (uint32_t)nv * rowb);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(static_cast<const uint16_t*>(a.C) + base * kN, (uint32_t)nv * rowb);
    char* const out = reinterpret_cast<char*>(a.ws) + ((size_t)bg * nch + c) * kPrepChunkBytes;

    // C rows of query tile q as B operands (column t, k = n) and the score tiles kt <= q
    bf16x8 cop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        cop[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rc, (int)((16 * q + l16) * rowb + (32 * ks + 8 * g4) * 2), 0, 0));
    for (int kt = 0; kt <= q; ++kt) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                              rb, (int)((16 * kt + l16) * rowb + (32 * ks + 8 * g4) * 2), 0, 0));
            s = mfma(bop, cop[ks], s);
        }
        *reinterpret_cast<f32x4*>(out + stile(q, kt) * kSTileBytes + lane * 16) = s;
    }
    // B^T operands (row n, k = the step's keys in slot order) of n-tiles 2 q, 2 q + 1
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int nt = 2 * q + j;
#pragma unroll
        for (int us = 0; us < 2; ++us) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int u0 = 32 * us + slot_key(g4, e), u1 = 32 * us + slot_key(g4, e + 1);
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(u0 * rowb + (16 * nt + l16) * 2), 0, 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(u1 * rowb + (16 * nt + l16) * 2), 0, 0);
                w[e / 2] = (lo & 0xffffu) | (hi << 16);
            }
            *reinterpret_cast<uint4*>(out + kSTiles * kSTileBytes + ((nt * 2 + us) * 64 + lane) * 16) =
                uint4{w[0], w[1], w[2], w[3]};
        }
    }
}

// ---- pass 2: the scan per (batch, head, half of P) ----------------------------------------
// Eight waves in two roles, so that each SIMD holds one of each and their dependency chains
// overlap instead of adding up:
//   * output waves 0-3 (wave q: query tile q): weight the score tiles, the carry readout
//     from the state snapshot, Y^T += X^T S'^T, the output stores;
//   * state waves 4-7 (wave 4 + q: the state's n-tiles 2 q, 2 q + 1, both P tiles): the
//     state update Hf^T = exp(l_e) Hf^T + B^T (v x) and its bf16 snapshot for the next
//     chunk's readout; wave 4 also scans the next chunk's decays into the token tables.
// LDS: x tiles [2][64 keys][32 p] bf16 (64-byte rows), the state snapshot [2][32 p][128 n]
// bf16 (256-byte rows, 16-byte groups swizzled by p), token tables [2][4][64] fp32 + the
// chunk's total log-decay.  One barrier per chunk.
constexpr int kPS = 32;                                    // P columns per workgroup
constexpr int kSXBytes = kSQ * kPS * 2;                    // 4 KiB
constexpr int kSHBytes = kPS * kN * 2;                     // 8 KiB
constexpr int kSTBytes = 4 * kSQ * 4 + 16;                 // l2, g1, gam, v; then l2 at the chunk end
constexpr int kSiLds = 2 * kSXBytes + 2 * kSHBytes + 2 * kSTBytes;
constexpr int kSiThreads = 512;

__device__ __forceinline__ int sh_off(int p, int grp) { return p * 256 + ((grp ^ (p & 15)) << 4); }

// the x operand (column p = c0 + lane % 16, the 32-key step us in slot order) from a row-major
// x tile by transposed reads: lane s of a 16-lane group points at key row kb + s / 4, columns
// c0 + 4 (s % 4) .. + 3, and receives column c0 + s at keys kb .. kb + 3
__device__ __forceinline__ bf16x8 x_operand(const char* tile, int c0, int us, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int kr = 32 * us + 4 * g + (s >> 2);
    const int col = c0 + 4 * (s & 3);
    const uint2 lo = ds_tr(tile + kr * (kPS * 2) + col * 2);
    const uint2 hi = ds_tr(tile + (kr + 16) * (kPS * 2) + col * 2);
    return __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
}

__global__ __launch_bounds__(kSiThreads) void siso_scan_kernel(ScanArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool state_role = w >= 4;
    const int q = w & 3;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int L = a.L, H = a.H, G = a.G;
    const int nch = (L + kSQ - 1) / kSQ;
    const int nloop = (nch + 1) & ~1;                          // (an even count: see below)
    const int lb = xcd_logical(blockIdx.x, gridDim.x);
    const int ph = lb % (kP / kPS);
    const int bh = lb / (kP / kPS);
    const int h = bh % H, bi = bh / H;
    const int g = h * G / H;
    const int p0 = ph * kPS;
    const bool dyn_rate = a.rate_law != 0;
    const float ah = dyn_rate ? 0.f : expf(a.A_log[h]);

    // buffer resources over the whole (batch, head) stream; tokens at or past L read zero
    // and their stores are dropped (the host keeps every offset below 2^31).  A chunk past
    // the sequence (the loop runs an even count) reads zero everywhere: dt = 0 leaves the
    // state as it is, and its stores are dropped.
    const uint32_t xrow = (uint32_t)H * kP * 2u, brow = (uint32_t)G * kN * 2u;
    const size_t tok0 = (size_t)bi * L;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const uint16_t*>(a.x) + (tok0 * H + h) * kP + p0,
                                                (uint32_t)(L - 1) * xrow + kPS * 2);
    const char* const prep = reinterpret_cast<const char*>(a.ws) + ((size_t)bi * G + g) * nch * kPrepChunkBytes;
    auto prep_rsrc = [&](int c) { return make_rsrc(prep + (size_t)min(c, nch - 1) * kPrepChunkBytes, (uint32_t)kPrepChunkBytes); };

    char* const sX = smem;
    char* const sH = smem + 2 * kSXBytes;
    float* const sT = reinterpret_cast<float*>(smem + 2 * kSXBytes + 2 * kSHBytes);
    constexpr int kTF = kSTBytes / 4;                          // floats per table set

    // every wave: 8 bytes of the chunk's x tile (key tid / 8, bytes 8 (tid % 8) ..)
    auto fetch_x = [&](int c) -> u32x2 {
        return __builtin_amdgcn_raw_buffer_load_b64(rx, (int)((c * kSQ + (tid >> 3)) * xrow + 8 * (tid & 7)), 0, 0);
    };
    auto stage_x = [&](int c, const u32x2& v) {
        *reinterpret_cast<u32x2*>(sX + (c & 1) * kSXBytes + (tid >> 3) * (kPS * 2) + 8 * (tid & 7)) = v;
    };

    if (!state_role) {
        // =========================== output waves ===========================
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<uint16_t*>(a.y) + (tok0 * H + h) * kP + p0,
                                                    (uint32_t)(L - 1) * xrow + kPS * 2);
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(static_cast<const uint16_t*>(a.C) + (tok0 * G + g) * kN,
                                                    (uint32_t)(L - 1) * brow + kN * 2);
        struct In {
            u32x2 x;
            f32x4 s[4];          // score tiles kt = 0 .. q of query tile q (past q: the diagonal again)
            bf16x8 c[4];         // C rows of query tile q (B operands, k = n)
        };
        auto fetch = [&](int c, In& in) {
            const int c0 = c * kSQ;
            in.x = fetch_x(c);
            const __amdgpu_buffer_rsrc_t rp = prep_rsrc(c);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                in.s[kt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rp, stile(q, min(kt, q)) * kSTileBytes + lane * 16, 0, 0));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                in.c[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rc, (int)((c0 + 16 * q + l16) * brow + (32 * ks + 8 * g4) * 2), 0, 0));
        };
        auto chunk = [&](int c, In& cur, In& nxt) {
            const int buf = c & 1, c0 = c * kSQ;
            const char* const xt = sX + buf * kSXBytes;
            const float* const tb = sT + buf * kTF;
            stage_x(c, cur.x);
            fetch(c + 1, nxt);
            __syncthreads();
            // weights: S'^T(u, t) = S^T(u, t) W(t, u), lane: column t = 16 q + l16, rows u
            const float l2t = tb[16 * q + l16];
            bf16x8 sop[2];
#pragma unroll
            for (int us = 0; us < 2; ++us) {
                uint32_t wv[4];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int kt = 2 * us + half;
                    const int u0 = 16 * kt + 4 * g4;
                    const float4 lu = *reinterpret_cast<const float4*>(tb + u0);
                    const float4 g1 = *reinterpret_cast<const float4*>(tb + kSQ + u0);
                    const float4 gm = *reinterpret_cast<const float4*>(tb + 2 * kSQ + u0);
                    const float lv[4] = {lu.x, lu.y, lu.z, lu.w}, g1v[4] = {g1.x, g1.y, g1.z, g1.w},
                                gmv[4] = {gm.x, gm.y, gm.z, gm.w};
                    float sv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // W from 0 / 1 masks (selects of constants): no branch per lane
                        const int u = u0 + i, t = 16 * q + l16;
                        const float below = u < t ? 1.f : 0.f, diag = u == t ? 1.f : 0.f;
                        const float e = __builtin_amdgcn_exp2f(fminf(l2t - lv[i], 0.f));
                        const float wt = fmaf(e * g1v[i], below, gmv[i] * diag);
                        sv[i] = kt <= q ? cur.s[kt][i] * wt : 0.f;
                    }
                    wv[2 * half] = pack2(sv[0], sv[1]);
                    wv[2 * half + 1] = pack2(sv[2], sv[3]);
                }
                sop[us] = __builtin_bit_cast(bf16x8, uint4{wv[0], wv[1], wv[2], wv[3]});
            }
            // Y^T (p-tile pt, lane: column t, rows p 4 g4 ..) = exp(l_t) Hf C^T + X^T S'^T
            const char* const hsn = sH + buf * kSHBytes;
            const float sc = __builtin_amdgcn_exp2f(l2t);
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 hop = *reinterpret_cast<const bf16x8*>(hsn + sh_off(16 * pt + l16, 4 * ks + g4));
                    r = mfma(hop, cur.c[ks], r);
                }
                f32x4 y = {r[0] * sc, r[1] * sc, r[2] * sc, r[3] * sc};
#pragma unroll
                for (int us = 0; us < 2; ++us)
                    if (2 * us <= q) y = mfma(x_operand(xt, 16 * pt, us, lane), sop[us], y);
                // 4 consecutive p of token t per lane (rows of tokens past L are dropped)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])}, ry,
                                                      (int)((c0 + 16 * q + l16) * xrow + (16 * pt + 4 * g4) * 2), 0, 0);
            }
        };
        In ia, ib;
        fetch(0, ia);
        for (int c = 0; c < nloop; c += 2) {
            chunk(c, ia, ib);
            chunk(c + 1, ib, ia);
        }
        return;
    }

    // =========================== state waves ===========================
    const __amdgpu_buffer_rsrc_t rdt = make_rsrc(a.dt + tok0 * H + h, (uint32_t)((L - 1) * H + 1) * 4u);
    const __amdgpu_buffer_rsrc_t rlm = make_rsrc(a.lam + tok0 * H + h, (uint32_t)((L - 1) * H + 1) * 4u);
    // (static rates: the rate loads read dt again, unused)
    const __amdgpu_buffer_rsrc_t rra = dyn_rate ? make_rsrc(a.A_log + tok0 * H + h, (uint32_t)((L - 1) * H + 1) * 4u) : rdt;
    struct In {
        u32x2 x;
        float dt, lm, ra;        // token 64 (c + 1) + lane: the next chunk's (dt, lambda, rate input)
        float dtn, lmn;          // the token after the next chunk
        bf16x8 bt[2][2];         // B^T operands of n-tiles 2 q + j, key steps us
    };
    // the scalars of chunk cs (the wave that scans them is a chunk ahead of the rest)
    auto fetch_scalars = [&](int cs, In& in) {
        const int o = (cs * kSQ + lane) * H * 4, on = (cs * kSQ + kSQ) * H * 4;
        in.dt = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdt, o, 0, 0));
        in.lm = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rlm, o, 0, 0));
        in.ra = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rra, o, 0, 0));
        in.dtn = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdt, on, 0, 0));
        in.lmn = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rlm, on, 0, 0));
    };
    auto fetch = [&](int c, In& in) {
        in.x = fetch_x(c);
        fetch_scalars(c + 1, in);
        const __amdgpu_buffer_rsrc_t rp = prep_rsrc(c);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int us = 0; us < 2; ++us)
                in.bt[j][us] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                              rp, kSTiles * kSTileBytes + (((2 * q + j) * 2 + us) * 64 + lane) * 16, 0, 0));
    };
    // the token tables of a chunk into set tset (wave 4 only; every lane one token)
    auto tables = [&](const In& in, int tset) {
        float* const tb = sT + tset * kTF;
        // (branch-free: both sides of the heavy-tail law are formed, then one is taken)
        float inv = 1.f / (1.f - fminf(in.ra, 0.f));
        asm volatile("" : "+v"(inv));
        const float ht = in.ra >= 0.f ? 1.f + in.ra : inv;
        const float rate = dyn_rate ? fminf(-ht, -1e-4f) : -ah;
        const float la = in.dt * rate;
        const float gm = in.lm * in.dt, dl = in.dt * (1.f - in.lm);
        const float l = group_scan<64>(la, lane);                 // inclusive
        const float le = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 63));
        const float dnn = in.dtn * (1.f - in.lmn);
        const float dn1 = __shfl_down(dl, 1, 64);
        const float dn = lane == 63 ? dnn : dn1;
        const float l2 = l * kLog2e, le2 = le * kLog2e;
        tb[lane] = l2;
        tb[kSQ + lane] = gm + dn;
        tb[2 * kSQ + lane] = gm;
        tb[3 * kSQ + lane] = __builtin_amdgcn_exp2f(le2 - l2) * (gm + dn);
        tb[4 * kSQ] = le2;                                        // (every lane, the same value)
    };

    // the state: Hf^T tiles (n-tile 2 q + j, p-tile pt), lane: column p, rows n 4 g4 ..
    f32x4 hs[2][2];
    {
        float d0 = 0.f;
        if (a.Bp0 && a.xp0) d0 = a.dt[tok0 * H + h] * (1.f - a.lam[tok0 * H + h]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int p = p0 + 16 * pt + l16, n = 16 * (2 * q + j) + 4 * g4;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (a.h0) {
                    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.h0) +
                                                                      ((size_t)bh * kP + p) * kN + n);
                    v = f32x4{f.x, f.y, f.z, f.w};
                }
                if (a.Bp0 && a.xp0) {
                    const float xv = d0 * bf16_bits_to_f32(static_cast<const uint16_t*>(a.xp0)[(size_t)bh * kP + p]);
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        v[m] += xv * bf16_bits_to_f32(static_cast<const uint16_t*>(a.Bp0)[(size_t)bh * kN + n + m]);
                }
                hs[j][pt] = v;
            }
    }
    // snapshot of the state at a chunk's start (bf16, row p, 16-byte groups swizzled)
    auto snapshot = [&](int sbuf) {
        char* dst = sH + sbuf * kSHBytes;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int p = 16 * pt + l16, n = 16 * (2 * q + j) + 4 * g4;
                *reinterpret_cast<uint2*>(dst + sh_off(p, n >> 3) + (n & 7) * 2) =
                    uint2{pack2(hs[j][pt][0], hs[j][pt][1]), pack2(hs[j][pt][2], hs[j][pt][3])};
            }
    };
    snapshot(0);
    {
        In i0;
        fetch_scalars(0, i0);
        if (q == 0) tables(i0, 0);
    }
    auto chunk = [&](int c, In& cur, In& nxt) {
        const int buf = c & 1;
        const char* const xt = sX + buf * kSXBytes;
        const float* const tb = sT + buf * kTF;
        stage_x(c, cur.x);
        fetch(c + 1, nxt);
        __syncthreads();
        // Hf^T = exp(l_e) Hf^T + B^T (v x), the B operand x scaled by v per key
        const float fe = __builtin_amdgcn_exp2f(tb[4 * kSQ]);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            bf16x8 vx[2];
#pragma unroll
            for (int us = 0; us < 2; ++us) {
                const float4 va = *reinterpret_cast<const float4*>(tb + 3 * kSQ + 32 * us + 4 * g4);
                const float4 vb = *reinterpret_cast<const float4*>(tb + 3 * kSQ + 32 * us + 16 + 4 * g4);
                const float vv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
                const uint4 raw = __builtin_bit_cast(uint4, x_operand(xt, 16 * pt, us, lane));
                const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = pack2(lo_f(rw[k]) * vv[2 * k], hi_f(rw[k]) * vv[2 * k + 1]);
                vx[us] = __builtin_bit_cast(bf16x8, uint4{o[0], o[1], o[2], o[3]});
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 v = {hs[j][pt][0] * fe, hs[j][pt][1] * fe, hs[j][pt][2] * fe, hs[j][pt][3] * fe};
#pragma unroll
                for (int us = 0; us < 2; ++us) v = mfma(cur.bt[j][us], vx[us], v);
                hs[j][pt] = v;
            }
        }
        // the snapshot for the next chunk (the other buffer: this one may still be read), and
        // the next chunk's tables (the other set: this one may still be read)
        snapshot(buf ^ 1);
        if (q == 0) tables(cur, buf ^ 1);
    };
    In ia, ib;
    fetch(0, ia);
    for (int c = 0; c < nloop; c += 2) {
        chunk(c, ia, ib);
        chunk(c + 1, ib, ia);
    }

    // ---- the final carry: the state after the last token (folded with d_L = 0) ----
    if (a.h1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int p = p0 + 16 * pt + l16, n = 16 * (2 * q + j) + 4 * g4;
                *reinterpret_cast<float4*>(static_cast<float*>(a.h1) + ((size_t)bh * kP + p) * kN + n) =
                    float4{hs[j][pt][0], hs[j][pt][1], hs[j][pt][2], hs[j][pt][3]};
            }
    }
    if (a.Bp1 && a.xp1) {
        const int st = tid - 256;                                  // state-wave thread index
        const size_t t = tok0 + L - 1;
        if (ph == 0 && st < kN)
            static_cast<uint16_t*>(a.Bp1)[(size_t)bh * kN + st] =
                static_cast<const uint16_t*>(a.B)[(t * G + g) * kN + st];
        if (st < kPS)
            static_cast<uint16_t*>(a.xp1)[(size_t)bh * kP + p0 + st] =
                static_cast<const uint16_t*>(a.x)[(t * H + h) * kP + p0 + st];
    }
}

}  // namespace

bool scan_siso_supported(const ScanArgs& a) {
    if (!a.io_bf16 || a.st_bf16 || a.R != 1 || a.np != 0 || a.P != kP || a.N != kN) return false;
    if (a.Bb || a.Cb || a.lift) return false;
    if (a.L < 1 || a.Q != kSQ) return false;
    // every buffer offset of a stream below 2^31
    const double xb = (double)a.L * a.H * kP * 2, bb = (double)a.L * a.G * kN * 2;
    return xb < 2147483000.0 && bb < 2147483000.0;
}

size_t scan_siso_workspace_bytes(const ScanArgs& a) {
    const size_t nch = (a.L + kSQ - 1) / kSQ;
    return (size_t)a.b * a.G * nch * kPrepChunkBytes;
}

hipError_t launch_scan_siso(const ScanArgs& a, hipStream_t st) {
    const int nch = (a.L + kSQ - 1) / kSQ;
    hipLaunchKernelGGL(siso_prep_kernel, dim3((unsigned)((size_t)a.b * a.G * nch)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&siso_scan_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kSiLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(siso_scan_kernel, dim3((unsigned)((size_t)a.b * a.H * (kP / kPS))), dim3(kSiThreads), kSiLds, st, a);
    return hipGetLastError();
}

}  // namespace m3
