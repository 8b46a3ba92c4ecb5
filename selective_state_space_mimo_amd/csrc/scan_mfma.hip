// Chunked scan on bf16 MFMA (gfx950), P = 64, N = 128, R in {1, 2, 4}.
//
// The chunked (SSD) form follows "The trapezoid term as a two-tap filter"
// of "Mamba-3: Improved Sequence Modeling using State Space Principles": inside
// a chunk the output is the masked product (L o C B^T) X, whose mask is the
// decay mask times a band with gamma on the diagonal and beta one below; the
// state is carried between chunks ("Diagonal Equivalence in State Space
// Models ...", section 2.4: chunk-local cumulative log-decays, so every
// decay factor is exp of a non-positive difference).  The rotation enters
// only through B and C, turned by the running angle ("Computing the rotation
// as a data-dependent RoPE"), and a chunk holds Q tokens x R ranks = M rows
// ("MIMO: a rank-4 state update ...": every write reaches every read).
//
// The carried state is "folded": Hf = H + d_next X_e^T Bt_e (H after the
// chunk's last token e plus the lagged share of e's write that the next token
// delivers, d_u = dt_u (1 - lam_u)).  Then, with l the chunk-local cumulative
// log-decay, g_s = lam_s dt_s and dS_s = d_{s+1}:
//   y_(t,r)  = exp(l_t) Hf_in Ct_(t,r)
//            + sum_{s<=t} exp(l_t - l_s) (g_s + [s<t] dS_s) sum_r' (Ct_(t,r).Bt_(s,r')) x_(s,r')
//   Hf_out   = exp(l_e) Hf_in + sum_s exp(l_e - l_s)(g_s + dS_s) X_s^T Bt_s
//
// Work decomposition (one workgroup = 8 waves per (batch, head, segment)):
//   * query rows of a chunk are split into 16-row tiles, dealt to the waves
//     in a zig-zag so that causal work is balanced; each wave keeps its C
//     tiles (biased, turned, bf16) in registers as MFMA B operands and its
//     output tiles Y^T (P x 16) as fp32 accumulators;
//   * key rows stream through LDS in blocks of 64 (double-buffered): every
//     wave turns 8 rows of B into Bt (row-major, for the scores) and into
//     (v * Bt)^T (for the state update), and stores X^T -- all swizzled so
//     that the 16-byte MFMA operand reads are bank-conflict free;
//   * scores S^T = Bt C^T come out of the MFMA with each lane holding one
//     query column and four key rows; masked and rounded to bf16 they are
//     directly the B operand of Y^T += X^T S'^T (the two key tiles of a pair
//     give the 8 k-slots; X^T is read with the same k permutation);
//   * the P x N state lives in MFMA accumulators (as H^T: each wave owns 16
//     state columns), updated by Hf^T += (v Bt)^T X; a bf16 copy in LDS is
//     the A operand of the carry readout Y^T = Hf Ct^T.
//   * per-chunk prefix sums (log-decay, angles) use wave shuffles.
// Segmented schedule (few streams, long sequences): pass 1 computes, per
// segment, the folded state from a zero carry in a local angle frame; pass 2
// runs the affine carry recurrence across segments (turning each summary into
// the global frame); pass 3 evaluates every segment from its true carry.
#include "m3_internal.h"

namespace m3 {

namespace {

constexpr int kP = 64, kN = 128, kWaves = 8, kThreads = 64 * kWaves, kKB = 64;
constexpr float kLog2e = 1.4426950408889634f;

enum Mode { kFull = 0, kSummary = 1 };

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v;
    v[0] = (bf16)lo;
    v[1] = (bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// ---- LDS layout ------------------------------------------------------------------
// Per key-block buffer: Bn [64 j][128 n] bf16, BvT [128 n][64 j] bf16, XT [64 p][64 j] bf16.
constexpr int kBnBytes = kKB * kN * 2;           // 16 KiB
constexpr int kBvBytes = kN * kKB * 2;           // 16 KiB
constexpr int kXtBytes = kP * kKB * 2;           //  8 KiB
constexpr int kBufBytes = kBnBytes + kBvBytes + kXtBytes;
constexpr int kHsBytes = kP * kN * 2;            // bf16 snapshot of the folded state

// 16-byte-group swizzles.  Bn and Hs rows hold 16 groups (256 B); BvT and XT
// rows hold 8 groups (128 B).
__device__ __forceinline__ int sw16(int row) { return row & 15; }
__device__ __forceinline__ int sw8(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int bn_off(int j, int grp) { return j * 256 + ((grp ^ sw16(j)) << 4); }
__device__ __forceinline__ int hs_off(int p, int grp) { return p * 256 + ((grp ^ sw16(p)) << 4); }
__device__ __forceinline__ int bv_off(int n, int grp) { return n * 128 + ((grp ^ sw8(n)) << 4); }
__device__ __forceinline__ int xt_off(int p, int grp) { return p * 128 + ((grp ^ sw8(p)) << 4); }

template <int Q, int NPMAX>
struct Layout {
    static constexpr int buf0 = 0;
    static constexpr int hs = 2 * kBufBytes;
    static constexpr int cs = hs + kHsBytes;                  // float2 [Q][NPMAX]
    static constexpr int cbias = cs + Q * NPMAX * 8;          // float [4][128]
    static constexpr int l2 = cbias + 4 * kN * 4;             // float [Q]
    static constexpr int gam = l2 + Q * 4;
    static constexpr int dels = gam + Q * 4;
    static constexpr int vs = dels + Q * 4;
    static constexpr int phic = vs + Q * 4;                   // float [64]
    static constexpr int misc = phic + 64 * 4;                // float [16]
    static constexpr int total = misc + 16 * 4;
};

struct Smem {
    char* base;
    __device__ char* buf(int i) const { return base + i * kBufBytes; }
};

// Query tile k of wave w (chunk-level tile index), or -1.
template <int M>
__device__ __forceinline__ int query_tile(int w, int k) {
    constexpr int NT = M / 16;
    if constexpr (NT >= 16) {
        const int g = k >> 1;
        return (k & 1) == 0 ? 16 * g + w : 16 * g + 15 - w;
    } else {
        return (k == 0 && w < NT) ? w : -1;
    }
}

// Inclusive scan of v over lanes [0, W) groups of a wave (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_scan(float v, int lane_in_group) {
#pragma unroll
    for (int off = 1; off < W; off <<= 1) {
        const float u = __shfl_up(v, off, W);
        if (lane_in_group >= off) v += u;
    }
    return v;
}

template <int R, int Q, int MODE>
__global__ __launch_bounds__(kThreads) void scan_mfma_kernel(ScanArgs a) {
    constexpr int M = Q * R;                 // rows per chunk
    constexpr int NKB = M / kKB;             // key blocks per chunk
    constexpr int NT = M / 16;               // query tiles per chunk
    constexpr int TPW = NT >= 16 ? NT / 8 : 1;
    constexpr int NPMAX = 4096 / Q > 64 ? 64 : 4096 / Q;
    using LY = Layout<Q, NPMAX>;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    Smem sm{smem_raw};
    float* sL2 = reinterpret_cast<float*>(smem_raw + LY::l2);
    float* sGam = reinterpret_cast<float*>(smem_raw + LY::gam);
    float* sDelS = reinterpret_cast<float*>(smem_raw + LY::dels);
    float* sV = reinterpret_cast<float*>(smem_raw + LY::vs);
    float* sPhic = reinterpret_cast<float*>(smem_raw + LY::phic);
    float2* sCS = reinterpret_cast<float2*>(smem_raw + LY::cs);
    float* sCb = reinterpret_cast<float*>(smem_raw + LY::cbias);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int H = a.H, L = a.L, np = a.np, nseg = a.nseg;

    // ---- which (batch, head, segment): consecutive logical ids share an XCD --------
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
    // logical order: batch, then segment, then head (heads of one batch and
    // segment read the same B, C rows)
    const int h = logical % H;
    const int rest = logical / H;
    const int seg = rest % nseg, bi = rest / nseg;
    const int bh = bi * H + h;
    const int g = h * a.G / H;
    const int T0 = seg * a.seglen;
    const int T1 = min(L, T0 + a.seglen);
    const bool last_seg = (T1 == L);
    const float ah = expf(a.A_log[h]);
    const size_t ss = (size_t)bh * nseg + seg;          // workspace slot
    const size_t S = (size_t)a.b * H * nseg;
    float* wsHloc = a.ws;
    float* wsHin = a.ws ? a.ws + S * kP * kN : nullptr;
    float* wsLam = a.ws ? a.ws + 2 * S * kP * kN : nullptr;
    float* wsDphi = a.ws ? wsLam + S : nullptr;
    float* wsPhi = a.ws ? wsDphi + S * np : nullptr;

    const uint16_t* Bg = static_cast<const uint16_t*>(a.B);
    const uint16_t* Cg = static_cast<const uint16_t*>(a.C);
    const uint16_t* Xg = static_cast<const uint16_t*>(a.x);

    // ---- per-workgroup set-up ------------------------------------------------------------
    // B bias pair of this lane for every rank (producer lanes own n-pair (2 lane, 2 lane + 1))
    float2 bb[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        bb[r] = a.Bb ? *reinterpret_cast<const float2*>(a.Bb + ((size_t)h * R + r) * kN + 2 * lane) : float2{0.f, 0.f};
    if (MODE == kFull)
        for (int e = tid; e < R * kN; e += kThreads) sCb[e] = a.Cb ? a.Cb[(size_t)h * R * kN + e] : 0.f;
    // running angle at the segment start
    for (int i = tid; i < np; i += kThreads) {
        float v = 0.f;
        if (MODE == kFull) {
            if (seg == 0) v = a.phi0 ? a.phi0[(size_t)bh * np + i] : 0.f;
            else v = wsPhi[ss * np + i];
        }
        sPhic[i] = v;
    }
    // folded state: this wave owns state columns n in [16w, 16w + 16), all P rows,
    // as four H^T tiles (lane: p = 16 pt + l16, n = 16 w + 4 g4 + m)
    f32x4 hacc[4];
    {
        const int nb = 16 * w + 4 * g4;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int p = 16 * pt + l16;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (MODE == kFull) {
                if (seg == 0) {
                    if (a.h0) {
                        const size_t o = ((size_t)bh * kP + p) * kN + nb;
                        if (a.st_bf16) {
                            const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.h0) + o);
                            v = f32x4{lo_f(u.x), hi_f(u.x), lo_f(u.y), hi_f(u.y)};
                        } else {
                            const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.h0) + o);
                            v = f32x4{f.x, f.y, f.z, f.w};
                        }
                    }
                    if (a.Bp0 && a.xp0 && L > 0) {
                        const size_t t0 = (size_t)bi * L * H + h;     // token 0 of this stream
                        const float d0 = a.dt[t0] * (1.f - a.lam[t0]);
                        const uint16_t* bp = static_cast<const uint16_t*>(a.Bp0) + (size_t)bh * R * kN;
                        const uint16_t* xp = static_cast<const uint16_t*>(a.xp0) + (size_t)bh * R * kP;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float xv = d0 * bf16_bits_to_f32(xp[r * kP + p]);
#pragma unroll
                            for (int m = 0; m < 4; ++m) v[m] += xv * bf16_bits_to_f32(bp[r * kN + nb + m]);
                        }
                    }
                } else {
                    const float4 f = *reinterpret_cast<const float4*>(wsHin + (ss * kP + p) * kN + nb);
                    v = f32x4{f.x, f.y, f.z, f.w};
                }
            }
            hacc[pt] = v;
        }
    }
    float lam_sum = 0.f;                                        // summary: sum of log alpha

    // ---- chunk loop ------------------------------------------------------------------------
    for (int c0 = T0; c0 < T1; c0 += Q) {
        const int nvalid = min(Q, T1 - c0);
        // (A) the folded state snapshot (bf16) for the carry readout, and the
        //     per-token angle increments staged in buffer 1
        if (MODE == kFull) {
            const int nb = 16 * w + 4 * g4;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = 16 * pt + l16;
                const uint2 u = {pack2(hacc[pt][0], hacc[pt][1]), pack2(hacc[pt][2], hacc[pt][3])};
                *reinterpret_cast<uint2*>(smem_raw + LY::hs + hs_off(p, nb >> 3) + ((nb >> 2) & 1) * 8) = u;
            }
        }
        float* stage = reinterpret_cast<float*>(sm.buf(1));
        for (int e = tid; e < Q * np; e += kThreads) {
            const int t = e / np, i = e - t * np;
            float v = 0.f;
            if (t < nvalid) {
                const size_t ti = ((size_t)bi * L + c0 + t) * H + h;
                v = a.dt[ti] * a.theta[ti * np + i];
            }
            stage[e] = v;
        }
        // (B) scalars: wave 0 scans log alpha over the chunk's tokens
        if (w == 0) {
            constexpr int TPL = Q > 64 ? Q / 64 : 1;          // tokens per lane
            float la[TPL], gm[TPL], dl[TPL];
            float lsum = 0.f;
#pragma unroll
            for (int k = 0; k < TPL; ++k) {
                const int t = lane * TPL + k;
                la[k] = 0.f; gm[k] = 0.f; dl[k] = 0.f;
                if (t < Q && t < nvalid) {
                    const size_t ti = ((size_t)bi * L + c0 + t) * H + h;
                    const float dt = a.dt[ti], lm = a.lam[ti];
                    la[k] = -dt * ah;
                    gm[k] = lm * dt;
                    dl[k] = dt * (1.f - lm);
                }
                lsum += la[k];
                la[k] = lsum;                                  // lane-local inclusive prefix
            }
            const float incl = group_scan<64>(lsum, lane);
            const float excl = incl - lsum;
            // look-ahead: d of the token after the chunk (0 past the sequence end)
            float dnext = 0.f;
            if (c0 + Q < L) {
                const size_t ti = ((size_t)bi * L + c0 + Q) * H + h;
                dnext = a.dt[ti] * (1.f - a.lam[ti]);
            }
            const float le = __shfl(incl, 63) * kLog2e;         // l_e (padded tokens add 0)
#pragma unroll
            for (int k = 0; k < TPL; ++k) {
                const int t = lane * TPL + k;
                if (t < Q) {
                    sL2[t] = (excl + la[k]) * kLog2e;
                    sGam[t] = gm[k];
                }
            }
            // dS_t = d_{t+1}
#pragma unroll
            for (int k = 0; k < TPL; ++k) {
                const int t = lane * TPL + k;
                float dn;
                if (k + 1 < TPL) dn = dl[k + 1];
                else {
                    const float nx = __shfl_down(dl[0], 1);
                    dn = (t + 1 < Q) ? nx : dnext;
                }
                if (t < Q) {
                    sDelS[t] = dn;
                    sV[t] = exp2f(le - (excl + la[k]) * kLog2e) * (gm[k] + dn);
                }
            }
            if (lane == 0) reinterpret_cast<float*>(smem_raw + LY::misc)[0] = le;
            lam_sum += le * (1.f / kLog2e);                    // wave 0 keeps the segment total
        }
        __syncthreads();
        // (C) angles: threads (pair i, part k) scan the staged increments
        {
            constexpr int TPP_BIG = 16;                        // threads per pair when np <= 32
            const int tpp = np <= 32 ? TPP_BIG : 8;
            const int i = tid / tpp, k = tid % tpp;
            if (i < np) {
                const int tpt = Q / tpp;                       // tokens per thread (>= 1)
                float loc = 0.f;
                for (int t = k * tpt; t < (k + 1) * tpt; ++t) loc += stage[t * np + i];
                float incl = tpp == 16 ? group_scan<16>(loc, k) : group_scan<8>(loc, k);
                const float base = sPhic[i];
                float run = base + incl - loc;
                for (int t = k * tpt; t < (k + 1) * tpt; ++t) {
                    run += stage[t * np + i];
                    float sn, cs;
                    __sincosf(run, &sn, &cs);
                    sCS[t * np + i] = float2{cs, sn};
                }
                if (k == tpp - 1) sPhic[i] = wrap_2pi(run);
            }
        }
        __syncthreads();
        const float le2 = reinterpret_cast<float*>(smem_raw + LY::misc)[0];

        // (D) per-wave query tiles: C (biased, turned, bf16) and the carry readout
        bf16x8 cq[TPW][4];
        f32x4 yacc[TPW][4];
        if (MODE == kFull) {
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int qt = query_tile<M>(w, k);
                const int qi = 16 * (qt < 0 ? 0 : qt) + l16;      // chunk row
                const int t = qi / R, r = qi % R;
                const bool valid = qt >= 0 && t < nvalid;
                const size_t crow = ((((size_t)bi * L + c0 + (valid ? t : 0)) * a.G + g) * R + r) * kN;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int n0 = 32 * ks + 8 * g4;
                    uint4 raw = valid ? *reinterpret_cast<const uint4*>(Cg + crow + n0) : uint4{0, 0, 0, 0};
                    const float4 b0 = *reinterpret_cast<const float4*>(sCb + r * kN + n0);
                    const float4 b1 = *reinterpret_cast<const float4*>(sCb + r * kN + n0 + 4);
                    float v[8] = {lo_f(raw.x) + b0.x, hi_f(raw.x) + b0.y, lo_f(raw.y) + b0.z, hi_f(raw.y) + b0.w,
                                  lo_f(raw.z) + b1.x, hi_f(raw.z) + b1.y, lo_f(raw.w) + b1.z, hi_f(raw.w) + b1.w};
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
                        const int ip = n0 / 2 + pp;
                        if (ip < np) {
                            const float2 c = sCS[t * np + ip];
                            const float e = v[2 * pp], o = v[2 * pp + 1];
                            v[2 * pp] = e * c.x - o * c.y;
                            v[2 * pp + 1] = e * c.y + o * c.x;
                        }
                    }
                    bf16x8 q;
#pragma unroll
                    for (int m = 0; m < 8; ++m) q[m] = valid ? (bf16)v[m] : (bf16)0.f;
                    cq[k][ks] = q;
                }
                // Y^T = exp(l_t) * (Hf Ct^T)
                const float sc = exp2f(sL2[t < Q ? t : Q - 1]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const int p = 16 * pt + l16;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 av = *reinterpret_cast<const bf16x8*>(smem_raw + LY::hs + hs_off(p, 4 * ks + g4));
                        acc = mfma(av, cq[k][ks], acc);
                    }
                    yacc[k][pt] = acc * sc;
                }
            }
        }
        // the state decays over the whole chunk before this chunk's writes land
        {
            const float f = exp2f(le2);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) hacc[pt] = hacc[pt] * f;
        }

        // (E) key blocks: produce block J into buffer J % 2, consume it
        auto produce = [&](int J) {
            char* buf = sm.buf(J & 1);
            // wave w turns rows 8w .. 8w+7 of block J; lane owns n-pair (2 lane, 2 lane + 1)
            uint32_t bvt0[4], bvt1[4];                      // 8 rows of (v Bt) for n = 2 lane, 2 lane + 1
            uint32_t xt0[4], xt1[4];                        // 8 rows of x for p = 2 lane, 2 lane + 1 (lane < 32)
            const int ip = lane;                            // pair index
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int j = kKB * J + 8 * w + rr;          // chunk row
                const int t = j / R, r = j % R;
                const int s = c0 + t;                        // token
                const bool valid = t < nvalid;
                const size_t tok = (size_t)bi * L + (valid ? s : c0);
                uint32_t braw = 0, xraw = 0;
                if (valid) {
                    braw = *reinterpret_cast<const uint32_t*>(Bg + (((tok * a.G + g) * R + r) * kN + 2 * lane));
                    if (lane < 32) xraw = *reinterpret_cast<const uint32_t*>(Xg + (((tok * H + h) * R + r) * kP + 2 * lane));
                }
                float b0 = valid ? lo_f(braw) + bb[r].x : 0.f;
                float b1 = valid ? hi_f(braw) + bb[r].y : 0.f;
                if (ip < np) {
                    const float2 c = sCS[t * np + ip];
                    const float e = b0, o = b1;
                    b0 = e * c.x - o * c.y;
                    b1 = e * c.y + o * c.x;
                }
                const uint32_t bt = pack2(b0, b1);
                if (MODE == kFull) {
                    *reinterpret_cast<uint32_t*>(buf + bn_off(8 * w + rr, lane >> 2) + (lane & 3) * 4) = bt;
                    if (valid && s == L - 1 && last_seg && a.Bp1) {
                        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.Bp1) + ((size_t)bh * R + r) * kN + 2 * lane) = bt;
                        if (lane < 32 && a.xp1)
                            *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.xp1) + ((size_t)bh * R + r) * kP + 2 * lane) = xraw;
                    }
                }
                const float vv = sV[t];
                const uint32_t bv = pack2(b0 * vv, b1 * vv);
                // transpose in registers: (row rr) -> k-slot rr of the n = 2 lane / 2 lane + 1 rows
                if (rr & 1) {
                    bvt0[rr >> 1] |= bv << 16;
                    bvt1[rr >> 1] |= bv & 0xffff0000u;
                    xt0[rr >> 1] |= xraw << 16;
                    xt1[rr >> 1] |= xraw & 0xffff0000u;
                } else {
                    bvt0[rr >> 1] = bv & 0xffffu;
                    bvt1[rr >> 1] = bv >> 16;
                    xt0[rr >> 1] = xraw & 0xffffu;
                    xt1[rr >> 1] = xraw >> 16;
                }
            }
            *reinterpret_cast<uint4*>(buf + kBnBytes + bv_off(2 * lane, w)) = uint4{bvt0[0], bvt0[1], bvt0[2], bvt0[3]};
            *reinterpret_cast<uint4*>(buf + kBnBytes + bv_off(2 * lane + 1, w)) = uint4{bvt1[0], bvt1[1], bvt1[2], bvt1[3]};
            if (lane < 32) {
                *reinterpret_cast<uint4*>(buf + kBnBytes + kBvBytes + xt_off(2 * lane, w)) = uint4{xt0[0], xt0[1], xt0[2], xt0[3]};
                *reinterpret_cast<uint4*>(buf + kBnBytes + kBvBytes + xt_off(2 * lane + 1, w)) = uint4{xt1[0], xt1[1], xt1[2], xt1[3]};
            }
        };

        auto consume = [&](int J) {
            const char* buf = sm.buf(J & 1);
            const char* bvb = buf + kBnBytes;
            const char* xtb = buf + kBnBytes + kBvBytes;
            if (MODE == kFull) {
#pragma unroll
                for (int k = 0; k < TPW; ++k) {
                    const int qt = query_tile<M>(w, k);
                    if (qt < 0) continue;
                    const int qi = 16 * qt + l16;
                    const int t = qi / R;
                    const float l2t = sL2[t];
#pragma unroll
                    for (int kp = 0; kp < 2; ++kp) {
                        const int ka = 4 * J + 2 * kp;          // chunk-level key tiles ka, ka + 1
                        if (ka > qt) continue;
                        const bool has_b = ka + 1 <= qt;
                        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            const bf16x8 av = *reinterpret_cast<const bf16x8*>(buf + bn_off(32 * kp + l16, 4 * ks + g4));
                            s0 = mfma(av, cq[k][ks], s0);
                        }
                        if (has_b) {
#pragma unroll
                            for (int ks = 0; ks < 4; ++ks) {
                                const bf16x8 av = *reinterpret_cast<const bf16x8*>(buf + bn_off(32 * kp + 16 + l16, 4 * ks + g4));
                                s1 = mfma(av, cq[k][ks], s1);
                            }
                        }
                        // mask: key rows 16 ka + 4 g4 + m (tile a) and 16 (ka+1) + 4 g4 + m (tile b)
                        bf16x8 bop;
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const int sa = (16 * ka + 4 * g4 + m) / R;
                            const int sb = (16 * ka + 16 + 4 * g4 + m) / R;
                            float wa = 0.f, wb = 0.f;
                            if (sa <= t) wa = exp2f(l2t - sL2[sa]) * (sGam[sa] + (sa < t ? sDelS[sa] : 0.f));
                            if (has_b && sb <= t) wb = exp2f(l2t - sL2[sb]) * (sGam[sb] + (sb < t ? sDelS[sb] : 0.f));
                            bop[m] = (bf16)(s0[m] * wa);
                            bop[4 + m] = (bf16)(s1[m] * wb);
                        }
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt) {
                            const int p = 16 * pt + l16;
                            // k-slots: keys 4 g4 + 0..3 of tile a, then of tile b
                            const int j0 = 32 * kp + 4 * g4, j1 = j0 + 16;
                            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(xtb + xt_off(p, j0 >> 3) + ((j0 >> 2) & 1) * 8);
                            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(xtb + xt_off(p, j1 >> 3) + ((j1 >> 2) & 1) * 8);
                            const bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                            yacc[k][pt] = mfma(av, bop, yacc[k][pt]);
                        }
                    }
                }
            }
            // state: Hf^T[n-tile w] += (v Bt)^T X over the block's 64 rows
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(bvb + bv_off(16 * w + l16, 4 * ks + g4));
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x8 bv = *reinterpret_cast<const bf16x8*>(xtb + xt_off(16 * pt + l16, 4 * ks + g4));
                    hacc[pt] = mfma(av, bv, hacc[pt]);
                }
            }
        };

        produce(0);
        __syncthreads();
        for (int J = 0; J < NKB; ++J) {
            if (J + 1 < NKB) produce(J + 1);
            consume(J);
            __syncthreads();
        }

        // (F) outputs of this chunk
        if (MODE == kFull) {
            bf16* yg = static_cast<bf16*>(a.y);
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int qt = query_tile<M>(w, k);
                if (qt < 0) continue;
                const int qi = 16 * qt + l16;
                const int t = qi / R, r = qi % R;
                if (t >= nvalid) continue;
                bf16* yrow = yg + ((((size_t)bi * L + c0 + t) * H + h) * R + r) * kP;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    bf16x4 o;
#pragma unroll
                    for (int m = 0; m < 4; ++m) o[m] = (bf16)yacc[k][pt][m];
                    *reinterpret_cast<bf16x4*>(yrow + 16 * pt + 4 * g4) = o;
                }
            }
        }
    }

    // ---- end of the stream / segment ----------------------------------------------------------
    const int nb = 16 * w + 4 * g4;
    if (MODE == kSummary) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int p = 16 * pt + l16;
            *reinterpret_cast<float4*>(wsHloc + (ss * kP + p) * kN + nb) = float4{hacc[pt][0], hacc[pt][1], hacc[pt][2], hacc[pt][3]};
        }
        if (tid == 0) wsLam[ss] = lam_sum;
        for (int i = tid; i < np; i += kThreads) wsDphi[ss * np + i] = sPhic[i];
    } else if (last_seg) {
        if (a.h1) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = 16 * pt + l16;
                const size_t o = ((size_t)bh * kP + p) * kN + nb;
                if (a.st_bf16) {
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h1) + o) =
                        uint2{pack2(hacc[pt][0], hacc[pt][1]), pack2(hacc[pt][2], hacc[pt][3])};
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(a.h1) + o) = float4{hacc[pt][0], hacc[pt][1], hacc[pt][2], hacc[pt][3]};
                }
            }
        }
        if (a.phi1)
            for (int i = tid; i < np; i += kThreads) a.phi1[(size_t)bh * np + i] = sPhic[i];
    }
}

// Pass 2 of the segmented schedule: the affine carry recurrence over segments.
// Thread = one (p, n-pair) of one stream; loops over the segments in order.
//   Hin[0]   = h0 + d_0 X_prev0^T Bt_prev0                (folded initial carry)
//   Hin[k+1] = exp(Lam_k) Hin[k] + rot(Hloc_k, Phi_k),    Phi_{k+1} = Phi_k + dphi_k
__global__ __launch_bounds__(256) void carry_pass_kernel(ScanArgs a) {
    const int bh = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;     // pair element index in [0, P*N/2)
    if (e >= kP * kN / 2) return;
    const int p = e / (kN / 2), ip = e % (kN / 2), n = 2 * ip;
    const int nseg = a.nseg, np = a.np, H = a.H, L = a.L;
    const int bi = bh / H;
    const size_t S = (size_t)a.b * H * nseg;
    float* wsHloc = a.ws;
    float* wsHin = a.ws + S * kP * kN;
    float* wsLam = a.ws + 2 * S * kP * kN;
    float* wsDphi = wsLam + S;
    float* wsPhi = wsDphi + S * np;
    float h0 = 0.f, h1 = 0.f;
    if (a.h0) {
        const size_t o = ((size_t)bh * kP + p) * kN + n;
        h0 = ld_io(a.h0, o, a.st_bf16);
        h1 = ld_io(a.h0, o + 1, a.st_bf16);
    }
    if (a.Bp0 && a.xp0) {
        const size_t t0 = (size_t)bi * L * H + (bh % H);
        const float d0 = a.dt[t0] * (1.f - a.lam[t0]);
        for (int r = 0; r < a.R; ++r) {
            const float xv = d0 * ld_io(a.xp0, ((size_t)bh * a.R + r) * kP + p, 1);
            h0 += xv * ld_io(a.Bp0, ((size_t)bh * a.R + r) * kN + n, 1);
            h1 += xv * ld_io(a.Bp0, ((size_t)bh * a.R + r) * kN + n + 1, 1);
        }
    }
    float phi = (ip < np && a.phi0) ? a.phi0[(size_t)bh * np + ip] : 0.f;
    for (int k = 0; k < nseg; ++k) {
        const size_t ss = (size_t)bh * nseg + k;
        const size_t o = (ss * kP + p) * kN + n;
        wsHin[o] = h0;
        wsHin[o + 1] = h1;
        if (ip < np && p == 0) wsPhi[ss * np + ip] = phi;
        const float dec = expf(wsLam[ss]);
        float u0 = wsHloc[o], u1 = wsHloc[o + 1];
        if (ip < np) {
            float sn, cs;
            sincosf(phi, &sn, &cs);
            const float t0 = u0 * cs - u1 * sn;
            u1 = u0 * sn + u1 * cs;
            u0 = t0;
            phi = wrap_2pi(phi + wsDphi[ss * np + ip]);
        }
        h0 = dec * h0 + u0;
        h1 = dec * h1 + u1;
    }
}

template <int R, int Q>
hipError_t launch_rq(const ScanArgs& a, hipStream_t st) {
    constexpr int NPMAX = 4096 / Q > 64 ? 64 : 4096 / Q;
    const size_t lds = Layout<Q, NPMAX>::total;
    const int nblk = a.b * a.H * a.nseg;
    hipError_t e;
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_mfma_kernel<R, Q, kSummary>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((scan_mfma_kernel<R, Q, kSummary>), dim3(nblk), dim3(kThreads), lds, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(carry_pass_kernel, dim3((kP * kN / 2 + 255) / 256, a.b * a.H), dim3(256), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_mfma_kernel<R, Q, kFull>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_mfma_kernel<R, Q, kFull>), dim3(nblk), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

bool scan_mfma_supported(const ScanArgs& a) {
    if (!a.io_bf16 || a.P != kP || a.N != kN) return false;
    const int M = a.Q * a.R;
    if (!(a.R == 1 || a.R == 2 || a.R == 4)) return false;
    if (!(a.Q == 16 || a.Q == 32 || a.Q == 64 || a.Q == 128)) return false;
    if (M < 64 || M > 512) return false;
    const int npmax = 4096 / a.Q > 64 ? 64 : 4096 / a.Q;
    return a.np <= npmax;
}

size_t scan_mfma_workspace_bytes(const ScanArgs& a) {
    if (a.nseg <= 1) return 0;
    const size_t S = (size_t)a.b * a.H * a.nseg;
    return S * (2 * (size_t)kP * kN + 1 + 2 * (size_t)a.np) * sizeof(float);
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t st) {
    switch (a.R * 1000 + a.Q) {
        case 1064: return launch_rq<1, 64>(a, st);
        case 1128: return launch_rq<1, 128>(a, st);
        case 2032: return launch_rq<2, 32>(a, st);
        case 2064: return launch_rq<2, 64>(a, st);
        case 2128: return launch_rq<2, 128>(a, st);
        case 4016: return launch_rq<4, 16>(a, st);
        case 4032: return launch_rq<4, 32>(a, st);
        case 4064: return launch_rq<4, 64>(a, st);
        case 4128: return launch_rq<4, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace m3
