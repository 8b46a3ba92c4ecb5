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
//            + sum_{s<=t} W(t,s) sum_r' (Ct_(t,r).Bt_(s,r')) x_(s,r'),
//     W(t,s) = exp(l_t - l_s) (g_s + [s<t] dS_s)
//   Hf_out   = exp(l_e) Hf_in + sum_s v_s X_s^T Bt_s,  v_s = exp(l_e - l_s)(g_s + dS_s)
//
// Work decomposition: one workgroup of 8 waves per (batch, head, segment),
// chunks of M = Q R <= 256 rows, split by role so that each SIMD holds one wave
// of each kind and vector work overlaps matrix work:
//   * 4 consumer waves own the chunk's query tiles (16 rows each, dealt so
//     that the causal work is equal).  Each keeps its C tiles (biased, turned,
//     bf16) in registers as MFMA B operands and its output tiles Y^T (P x 16) as
//     fp32 accumulators; per key block it forms the scores S^T = Bt C^T (each
//     lane: one query column, four key rows), weights them with W -- computed
//     per lane from the tabled log-decays, exact, never factored -- and feeds
//     them as bf16 B operands straight into Y^T += X^T S'^T.  The tiles a key
//     block meets are a suffix of the wave's (ascending) tiles, so each block
//     runs a straight-line body chosen by that suffix.
//   * 4 producer waves stream key rows: raw B and x rows are fetched with
//     bounded buffer loads into a register ring DP blocks ahead (across chunk
//     boundaries); each producer turns 8 rows of every 32-row block into Bt
//     (row-major, for the scores) and (v Bt)^T, and stores X^T, in LDS tiles
//     swizzled for conflict-free 16-byte operand reads.  The producers own the
//     P x N state as MFMA accumulators (H^T, 32 columns each) and update it with
//     Hf^T += (v Bt)^T X; a bf16 snapshot in LDS is the consumers' A operand for
//     the carry readout Y^T = Hf Ct^T.
//   * per chunk, all waves compute the running angles into a table of bf16
//     pairs (the B and C rows are turned with packed-bf16 dot products, fp32
//     sums); one producer scans the log-decays with DPP.
//   * key blocks are double-buffered in LDS with one barrier per block; both
//     roles pass the same barriers.
// Segmented schedule (few streams, long sequences): pass 1 computes, per
// segment, the folded state from a zero carry in a local angle frame; pass 2
// runs the affine carry recurrence across segments (turning each summary into
// the global frame); pass 3 evaluates every segment from its true carry.
#include "scan_common.h"

#include <type_traits>

namespace m3 {

namespace {

template <int R, int Q>
struct Layout {
    static constexpr int hs = 2 * kBufBytes;
    // [Q][64] two bf16 pairs, (cos, -sin) and (sin, cos); pair i of token t sits in column
    // i ^ (t & 60), which keeps aligned groups of four pairs together and spreads the angle
    // writes (one token row per lane group) over the banks
    static constexpr int cs = hs + kHsBytes;
    static constexpr int cbias = cs + Q * 64 * 8;             // bf16 pairs [4][64]: C bias
    static constexpr int l2 = cbias + 4 * 64 * 4;             // float [Q] each below
    static constexpr int g1 = l2 + Q * 4;
    static constexpr int gam = g1 + Q * 4;
    static constexpr int vs = gam + Q * 4;
    // raw per-token inputs of the chunk, staged by the consumers: dt and lambda of its Q
    // tokens and of the token after it ([Q + 4], 16-byte multiples), the rate input [Q]
    static constexpr int dtv = vs + Q * 4;
    static constexpr int lmv = dtv + (Q + 4) * 4;
    static constexpr int arv = lmv + (Q + 4) * 4;
    static constexpr int phic = arv + Q * 4;                  // float [64]
    static constexpr int misc = phic + 64 * 4;                // float [16]
    // float [64][Q + 1]: theta, pair-major.  It shares the key-block buffers, which hold
    // nothing from the last key block of a chunk to the next chunk's block-0 tiles (the
    // theta staging and the angles fall in between).
    static constexpr int stg = 0;
    static_assert(64 * (Q + 1) * 4 <= 2 * kBufBytes, "theta staging fits the key-block buffers");
    // Output tiles leave through LDS so that every store writes whole rows.  With Q <= 64 a
    // chunk's outputs are staged (rows of 144 bytes, query row q at q * 144) at its end and
    // stored during the next chunk's key blocks; with Q = 128 (no room) each consumer stores
    // a tile at a time through a 4 KiB scratch.
    static constexpr bool kYStage = Q <= 64;
    static constexpr int cmb = misc + 16 * 4;                 // float [R][64]: readout weights (layer)
    static constexpr int xsc = cmb + R * 64 * 4;              // per consumer 4 KiB (Q = 128)
    static constexpr int ysg = xsc + (kYStage ? 0 : 4 * 4096);
    static constexpr int total = ysg + (kYStage ? R * Q * 144 : 0);
};

// ---- warp-specialised variant (chunks of at most 256 rows) ----------------------------------
// Waves 0-3 are consumers: each keeps a quarter of the chunk's query tiles (C tiles in
// registers, Y^T accumulators) and runs the scores, their weighting and Y^T += X^T S'^T.
// The last 4 waves are producers: each turns 8 of every key block's 32 rows into the LDS
// tiles and owns 32 columns of the state (Hf^T += (v Bt)^T X).  Every SIMD holds producer
// and consumer waves, so that the producers' vector work overlaps the consumers' matrix work.
// Both kinds pass the same barriers: one after each chunk section, one per key block.
//
// Consumer waves: 4, or 8 at R = 4, Q = 64 (256 rows): there each consumer keeps two query
// tiles, which fits 168 registers per lane, and the workgroup's 12 waves put three on each
// SIMD (two consumers and a producer) to hide more of the latency of a wave's LDS reads,
// fetches and barriers.
template <int R, int Q>
constexpr int n_consumers() { return (R == 4 && Q == 64) ? 8 : 4; }
template <int R, int Q>
constexpr int n_threads() { return 64 * (n_consumers<R, Q>() + kNP); }

// Query tile k of consumer c (NC consumers): tiles are dealt in groups of 2 NC, consumer c
// taking tile c and tile 2 NC - 1 - c of each group (equal causal work per consumer).
template <int NC>
__host__ __device__ constexpr int ctile(int c, int k) {
    return 2 * NC * (k >> 1) + ((k & 1) ? 2 * NC - 1 - c : c);
}
// Query tile t meets key blocks 0 .. t / 2 and reaches the diagonal in the last of them.  A
// consumer's tiles end in strictly increasing blocks, so in any key block at most one of its
// tiles is on the diagonal: the first active one, in the last block before it retires.
template <int NC, int TPC>
constexpr bool ctile_blocks_increase() {
    for (int c = 0; c < NC; ++c)
        for (int k = 0; k + 1 < TPC; ++k)
            if (ctile<NC>(c, k + 1) / 2 <= ctile<NC>(c, k) / 2) return false;
    return true;
}
static_assert(ctile_blocks_increase<4, 4>() && ctile_blocks_increase<8, 2>(), "one diagonal tile per key block and consumer");

// Waves per SIMD the kernel is built for.  Chunks of 16 tokens at R = 4 (64 rows: the
// small-chunk MIMO schedule) fit two workgroups per CU: at most 128 registers per lane (four
// waves per SIMD) and half the LDS; the extra waves hide the latencies that one workgroup's
// two waves per SIMD leave exposed.  R = 4, Q = 64 runs 12 waves (three per SIMD).
template <int R, int Q>
constexpr int waves_per_simd() { return (R == 4 && Q == 16) ? 4 : n_threads<R, Q>() / 256; }

// LAYER: the kernel runs inside the layer entry point, so x is un-lifted (lift applied as
// the rows are fetched) and dt, lam, theta are the raw projections (activated as they are
// staged); a compile-time switch, so the scan on its own carries none of it.
template <int R, int Q, int MODE, bool LAYER>
__global__ __launch_bounds__((n_threads<R, Q>()), (waves_per_simd<R, Q>())) void scan_ws_kernel(ScanArgs a) {
    constexpr int kNC = n_consumers<R, Q>();                // consumer waves
    constexpr int kThreads = n_threads<R, Q>();
    constexpr int M = Q * R;                 // rows per chunk
    constexpr int NKB = M / kKB;             // key blocks per chunk
    constexpr int NT = M / 16;               // query tiles per chunk
    constexpr int TPC = NT / kNC;            // query tiles per consumer
    constexpr int RPB = 32 / kNC;            // staged output rows a consumer stores per key block
    static_assert(RPB * NKB == 16 * TPC, "a chunk's staged rows leave over its key blocks");
    static_assert(RPB % R == 0, "a key block's staged rows are whole tokens");
    constexpr int TPL = Q > 64 ? Q / 64 : 1; // tokens per lane of the scanning wave
    constexpr int KT = R >= 4 ? 1 : 4 / R;   // key tokens among a lane's 4 rows of a score tile
    constexpr bool kEarlyExp = KT == 1;      // decay exps ahead of the score MFMAs (registers allow)
    constexpr bool kFullMode = MODE == kFull;
    static_assert(TPC >= 1 && TPC <= 4 && NKB >= 2 && NKB % 2 == 0, "chunk shape");
    using LY = Layout<R, Q>;
    static_assert(!LAYER || LY::kYStage, "the layer variant stages its outputs");
    static_assert(waves_per_simd<R, Q>() != 4 || LY::total <= 80 * 1024, "two workgroups per CU fit the LDS");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float* sL2 = reinterpret_cast<float*>(smem + LY::l2);
    float* sG1 = reinterpret_cast<float*>(smem + LY::g1);
    float* sGam = reinterpret_cast<float*>(smem + LY::gam);
    float* sV = reinterpret_cast<float*>(smem + LY::vs);
    float* sDt = reinterpret_cast<float*>(smem + LY::dtv);
    float* sLm = reinterpret_cast<float*>(smem + LY::lmv);
    float* sAr = reinterpret_cast<float*>(smem + LY::arv);
    float* sPhic = reinterpret_cast<float*>(smem + LY::phic);
    uint2* sCS = reinterpret_cast<uint2*>(smem + LY::cs);
    uint32_t* sCb = reinterpret_cast<uint32_t*>(smem + LY::cbias);
    float* sMisc = reinterpret_cast<float*>(smem + LY::misc);
    float* stage = reinterpret_cast<float*>(smem + LY::stg);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int H = a.H, L = a.L, np = a.np, nseg = a.nseg;

    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int logical = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
    const int h = logical % H;
    const int rest = logical / H;
    const int seg = rest % nseg, bi = rest / nseg;
    const int bh = bi * H + h;
    const int g = h * a.G / H;
    const int T0 = seg * a.seglen;
    const int T1 = min(L, T0 + a.seglen);
    const bool last_seg = (T1 == L);
    const bool dyn_rate = a.rate_law != 0;               // A_log holds the per-token rate input
    const float ah = dyn_rate ? 0.f : expf(a.A_log[h]);
    const float dtb = LAYER && a.dt_bias ? a.dt_bias[h] : 0.f;   // raw projections: step bias
    const size_t ss = (size_t)bh * nseg + seg;
    const size_t S = (size_t)a.b * H * nseg;
    float* const wsHloc = a.ws;
    float* const wsHin = a.ws + S * kP * kN;
    float* const wsLam = a.ws + 2 * S * kP * kN;
    float* const wsDphi = wsLam + S;
    float* const wsPhi = wsDphi + S * np;

    const size_t tokbase = (size_t)bi * L;
    const uint16_t* const Bg = static_cast<const uint16_t*>(a.B) + (tokbase * a.G + g) * R * kN;
    const uint16_t* const Cg = static_cast<const uint16_t*>(a.C) + (tokbase * a.G + g) * R * kN;
    constexpr bool lifted = LAYER;                        // x rows lifted as they are fetched
    const int xrows = lifted ? 1 : R;                      // x rows per (token, head) in memory
    const uint16_t* const Xg = static_cast<const uint16_t*>(a.x) + (tokbase * H + h) * xrows * kP;
    const size_t bstride = (size_t)a.G * R * kN;
    const size_t xstride = (size_t)H * xrows * kP;
    const uint32_t bsb = (uint32_t)bstride * 2u, xsb = (uint32_t)xstride * 2u;   // bytes per token
    const uint32_t ysb = (uint32_t)H * R * kP * 2u;                               // y: bytes per token
    const float* const dtg = a.dt + tokbase * H + h;
    const float* const lamg = a.lam + tokbase * H + h;
    const float* const rateg = a.A_log + (dyn_rate ? tokbase * H + h : 0);
    const float* const thg = np ? a.theta + (tokbase * H + h) * np : a.dt;

    // ---- shared set-up ------------------------------------------------------------------------
    if (kFullMode)
        for (int e = tid; e < R * kN / 2; e += kThreads)
            sCb[e] = a.Cb ? pack2(a.Cb[(size_t)h * R * kN + 2 * e], a.Cb[(size_t)h * R * kN + 2 * e + 1]) : 0u;
    for (int i = tid; i < np; i += kThreads) {
        float v = 0.f;
        if (kFullMode) v = seg == 0 ? (a.phi0 ? a.phi0[(size_t)bh * np + i] : 0.f) : wsPhi[ss * np + i];
        sPhic[i] = v;
    }
    for (int e = tid; e < Q * 64; e += kThreads)
        if ((e & 63) >= np) sCS[(e & ~63) + ((e & 63) ^ ((e >> 6) & 60))] = cs_entry(1.f, 0.f);
    if constexpr (LAYER)
        if (kFullMode)
            for (int e = tid; e < R * kP; e += kThreads)
                reinterpret_cast<float*>(smem + LY::cmb)[e] = a.comb[(size_t)h * R * kP + e];

    // theta of the chunk at cstart (all threads: THU consecutive pairs of one token each,
    // THP times), one buffer load per value.  Token t's np angles of this head start t H np after the
    // chunk's first; the record count ends at this head's last angle of the last valid
    // token, so nothing past the segment end or past the tensor is read.  Lanes of pairs
    // at or past np read zero (those values are never used).
    constexpr int THP = (Q + 63) / 64;                    // token rounds
    constexpr int THU = Q >= 64 ? 8 : Q / 8;              // pairs per thread and round
    constexpr int THG = 64 / THU;                         // threads per token
    auto load_theta = [&](int cstart, float (&th)[THP][THU]) {
        int tt = tid;                                         // opaque: offsets formed here
        asm volatile("" : "+v"(tt));
            tt &= 1023;                                      // a thread index: non-negative
        const int th_t = tt / THG, th_i = (tt % THG) * THU;
        const int nt = __builtin_amdgcn_readfirstlane(min(max(T1 - cstart, 0), Q));
        const uint32_t nrec = nt > 0 ? (uint32_t)((nt - 1) * H * np + np) * 4u : 0u;
        const __amdgpu_buffer_rsrc_t rt = make_rsrc(thg + (size_t)cstart * H * np, nrec);
#pragma unroll
        for (int pp = 0; pp < THP; ++pp) {
            // a group wholly past np gets an offset beyond every record count
            const int vo = th_i < np ? ((th_t + 64 * pp) * H * np + th_i) * 4 : 0x7fffff00;
#pragma unroll
            for (int u = 0; u < THU; ++u) th[pp][u] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rt, vo + 4 * u, 0, 0));
        }
    };
    auto stage_theta = [&](const float (&th)[THP][THU]) {
        int tt = tid;
        asm volatile("" : "+v"(tt));
            tt &= 1023;                                      // a thread index: non-negative
        const int th_t = tt / THG, th_i = (tt % THG) * THU;
#pragma unroll
        for (int pp = 0; pp < THP; ++pp) {
            const int t = th_t + 64 * pp;
            if (t < Q) {
#pragma unroll
                for (int u = 0; u < THU; ++u)
                    stage[(th_i + u) * (Q + 1) + t] = LAYER ? kPiF * tanh_f(th[pp][u]) : th[pp][u];
            }
        }
    };
    // (B) angles, all threads: TPP threads per pair scan dt * theta over the chunk
    auto angles = [&]() {
        auto run = [&](auto tpp_c) {
            constexpr int TPP = decltype(tpp_c)::value;
            constexpr int TPT = Q / TPP;
            int tt = tid;                                     // opaque: offsets formed here
            asm volatile("" : "+v"(tt));
            tt &= 1023;                                      // a thread index: non-negative
            const int k = tt % TPP, i = tt / TPP;
            if (i < np) {
                float inc[TPT];
                float loc = 0.f;
#pragma unroll
                for (int u = 0; u < TPT; ++u) {
                    const int t = k * TPT + u;
                    loc += sDt[t] * stage[i * (Q + 1) + t];
                    inc[u] = loc;
                }
                const float incl = group_scan<TPP>(loc, k);
                const float base = sPhic[i] + incl - loc;
#pragma unroll
                for (int u = 0; u < TPT; ++u) {
                    float sn, cs;
                    __sincosf(base + inc[u], &sn, &cs);
                    const int t = k * TPT + u;
                    sCS[t * 64 + (i ^ (t & 60))] = cs_entry(cs, sn);
                }
                if (k == TPP - 1) sPhic[i] = wrap_2pi(base + inc[TPT - 1]);
            }
        };
        if (np <= 32) run(std::integral_constant<int, 16>{});
        else run(std::integral_constant<int, 8>{});
    };
    // A chunk's raw per-token inputs (dt and lambda of its tokens and of the next one, the
    // rate input), loaded by the producer threads at the previous chunk's start (value e:
    // dt of token e, then lambda, then the rate input) and staged in LDS at its first key
    // block ahead of that block's row fetches, when they have long arrived; the wave that
    // scans them then reads LDS only and never waits on the row fetches.
    constexpr int NSV = (3 * Q + 2 + kNP * 64 - 1) / (kNP * 64);
    float rgS[NSV];
    auto load_scalars = [&](int cstart) {
#pragma unroll
        for (int j = 0; j < NSV; ++j) {
            const int e = tid - kNC * 64 + kNP * 64 * j;
            float v = 0.f;
            if (e < 2 * Q + 2) {
                const int t = e <= Q ? e : e - (Q + 1);
                const bool ok = t < Q ? cstart + t < T1 : cstart + Q < L;
                if (ok) v = (e <= Q ? dtg : lamg)[(size_t)(cstart + t) * H];
            } else if (e < 3 * Q + 2 && dyn_rate) {
                const int t = e - (2 * Q + 2);
                if (cstart + t < T1) v = rateg[(size_t)(cstart + t) * H];
            }
            rgS[j] = v;
        }
    };
    // (raw projections: the step and the blend are activated here, for valid tokens only;
    // the others stay 0)
    auto stage_scalars = [&](int cstart) {
        int tt = tid;                                         // opaque: the LDS addresses are
        asm volatile("" : "+v"(tt));                          // formed here, not kept live
        tt &= 1023;
#pragma unroll
        for (int j = 0; j < NSV; ++j) {
            const int e = tt - kNC * 64 + kNP * 64 * j;
            float v = rgS[j];
            if (LAYER && e < 2 * Q + 2) {
                const int t = e <= Q ? e : e - (Q + 1);
                const bool ok = t < Q ? cstart + t < T1 : cstart + Q < L;
                if (ok) v = e <= Q ? softplus_f(v + dtb) : sigmoid_f(v);
            }
            if (e <= Q) sDt[e] = v;
            else if (e < 2 * Q + 2) sLm[e - (Q + 1)] = v;
            else if (e < 3 * Q + 2) sAr[e - (2 * Q + 2)] = v;
        }
    };
    float rgTh[THP][THU];
    load_theta(T0, rgTh);
    if (w >= kNC) {
        load_scalars(T0);
        stage_scalars(T0);
    }
    __syncthreads();

    if (w < kNC) {
        // =============================== consumers ===============================
        const int c = w;
        bf16x8 cq[TPC][4];
        f32x4 yacc[TPC][4];
        char* const xs = smem + LY::xsc + c * 4096;          // this wave's scratch (Q = 128)
        char* const ys = smem + LY::ysg;                      // output staging (Q <= 64)
        // outputs of the chunk at cst (nv valid tokens), through the scratch (rows of
        // 144 bytes) so that every store writes whole rows
        auto store_y = [&](int cst, int nv) {
            // rows of tokens at or past nv fall outside the record count: dropped
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<uint16_t*>(a.y) + ((tokbase + cst) * H + h) * R * kP,
                                                        (uint32_t)nv * ysb);
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
#pragma unroll
            for (int k = 0; k < TPC; ++k) {
                const int qt = ctile<kNC>(c, k);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    *reinterpret_cast<uint2*>(xs + (ln & 15u) * 144 + (16 * pt + 4 * (ln >> 4)) * 2) =
                        uint2{pack2(yacc[k][pt][0], yacc[k][pt][1]), pack2(yacc[k][pt][2], yacc[k][pt][3])};
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const unsigned j = 8 * i + (ln >> 3);
                    const u32x4 v = *reinterpret_cast<const u32x4*>(xs + j * 144 + (ln & 7u) * 16);
                    const unsigned qi = 16 * qt + j;
                    const unsigned t = qi / R, r = qi % R;
                    __builtin_amdgcn_raw_buffer_store_b128(v, ry, (int)(t * ysb + r * (kP * 2) + 16 * (ln & 7u)), 0, 0);
                }
            }
        };

        // (Q <= 64) this wave's output tiles into their staging rows
        auto stage_y = [&]() {
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
#pragma unroll
            for (int k = 0; k < TPC; ++k) {
                const unsigned qt = ctile<kNC>(c, k);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    *reinterpret_cast<uint2*>(ys + (16 * qt + (ln & 15u)) * 144 + (16 * pt + 4 * (ln >> 4)) * 2) =
                        uint2{pack2(yacc[k][pt][0], yacc[k][pt][1]), pack2(yacc[k][pt][2], yacc[k][pt][3])};
            }
        };
        // (Q <= 64) NR staged rows 16 qt + r0 .. + NR - 1 (of a tile of this wave; NR = 8 or
        // 4, eight lanes a row) to the outputs of the chunk at cst with nv valid tokens; rows of
        // later tokens fall outside the record count
        auto store_rows = [&](int cst, int nv, int qt, int r0, auto nrc) {
            constexpr unsigned NR = decltype(nrc)::value;
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<uint16_t*>(a.y) + ((tokbase + cst) * H + h) * R * kP,
                                                        (uint32_t)nv * ysb);
            if (NR == 8 || ln < 8 * NR) {
                const unsigned qi = 16 * (unsigned)qt + (unsigned)r0 + (ln >> 3);
                const u32x4 v = *reinterpret_cast<const u32x4*>(ys + qi * 144 + (ln & 7u) * 16);
                const unsigned t = qi / R, r = qi % R;
                __builtin_amdgcn_raw_buffer_store_b128(v, ry, (int)(t * ysb + r * (kP * 2) + 16 * (ln & 7u)), 0, 0);
            }
        };
        // (layer) Outputs leave as one P-wide row per token: the R staged readout rows
        // recombined, sum_r comb[r] y_r, and with a gate, (that + dskip x) silu(gate).  The
        // 16-byte pieces of a chunk's outputs of this wave are dealt to lanes: piece p (token u
        // = p / 8 of the wave, its rows R u .. R u + R - 1 in tile order; eight pieces a token)
        // to lane p % 64, slot p / 64.  Each lane loads the x and gate pieces of its slots
        // with the chunk's C rows, finishes its pieces once those have landed (all lanes at
        // once, in place: piece k of a token replaces piece k of its first staged row), and
        // the key blocks store the finished pieces.
        constexpr unsigned kXU = TPC * 16 / R;                // tokens of this wave's tiles
        constexpr int kXS = (8 * kXU + 63) / 64;             // pieces per lane
        u32x4 xpc[kXS], zpc[kXS];
        const bool gated = LAYER && a.gate != nullptr;
        const float dsk = LAYER && a.dskip ? a.dskip[h] : 0.f;
        // query row of piece p's first rank
        auto piece_row = [&](unsigned p) -> unsigned {
            const unsigned rr = R * (p >> 3);
            return 16u * (unsigned)ctile<kNC>(c, (int)(rr >> 4)) + (rr & 15u);
        };
        // x and gate pieces of the chunk at cst (nv valid tokens); pieces past the wave's
        // outputs, rows of later tokens and every piece without a gate read zero
        auto load_xz = [&](int cst, int nv) {
            const uint32_t nb = gated ? (uint32_t)nv * (uint32_t)(H * kP * 2) : 0u;
            const size_t rb = ((tokbase + cst) * H + h) * kP;
            const __amdgpu_buffer_rsrc_t rxs = make_rsrc(static_cast<const uint16_t*>(a.x) + rb, nb);
            const __amdgpu_buffer_rsrc_t rzs = make_rsrc(static_cast<const uint16_t*>(gated ? a.gate : a.x) + rb, nb);
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
#pragma unroll
            for (int sl = 0; sl < kXS; ++sl) {
                const unsigned p = 64u * sl + ln;
                const int off = p < 8u * kXU ? (int)((piece_row(p) / R) * (unsigned)(H * kP * 2) + 16u * (p & 7u)) : (int)nb;
                xpc[sl] = __builtin_amdgcn_raw_buffer_load_b128(rxs, off, 0, 0);
                zpc[sl] = __builtin_amdgcn_raw_buffer_load_b128(rzs, off, 0, 0);
            }
        };
        // every piece of the staged chunk, in place
        auto finish_pieces = [&]() {
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
            const float* cw = reinterpret_cast<const float*>(smem + LY::cmb);
#pragma unroll
            for (int sl = 0; sl < kXS; ++sl) {
                const unsigned p = 64u * sl + ln;
                const unsigned qi0 = piece_row(p < 8u * kXU ? p : 0u), k = p & 7u;
                float acc[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(ys + (qi0 + r) * 144 + k * 16);
                    const float4 w0 = *reinterpret_cast<const float4*>(cw + r * kP + 8 * k);
                    const float4 w1 = *reinterpret_cast<const float4*>(cw + r * kP + 8 * k + 4);
                    acc[0] += w0.x * lo_f(v[0]); acc[1] += w0.y * hi_f(v[0]);
                    acc[2] += w0.z * lo_f(v[1]); acc[3] += w0.w * hi_f(v[1]);
                    acc[4] += w1.x * lo_f(v[2]); acc[5] += w1.y * hi_f(v[2]);
                    acc[6] += w1.z * lo_f(v[3]); acc[7] += w1.w * hi_f(v[3]);
                }
                if (gated) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float xi = (i & 1) ? hi_f(xpc[sl][i / 2]) : lo_f(xpc[sl][i / 2]);
                        const float zi = (i & 1) ? hi_f(zpc[sl][i / 2]) : lo_f(zpc[sl][i / 2]);
                        // silu(z) = z / (1 + exp(-z)) with the hardware exp2 and reciprocal
                        // (rounded to bf16 next); a large |z| gives z or -0
                        const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zi * kLog2e));
                        acc[i] = (acc[i] + dsk * xi) * (zi * sg);
                    }
                }
                // (the row reads of all lanes precede these writes: a wave's LDS accesses
                // complete in order)
                if (p < 8u * kXU)
                    *reinterpret_cast<u32x4*>(ys + qi0 * 144 + k * 16) =
                        u32x4{pack2(acc[0], acc[1]), pack2(acc[2], acc[3]), pack2(acc[4], acc[5]), pack2(acc[6], acc[7])};
            }
        };
        // finished pieces pbeg .. pbeg + NPC - 1 (one slot) of the chunk at cst (nv valid
        // tokens; rows of later tokens fall outside the record count)
        auto layer_store = [&](int cst, int nv, unsigned pbeg, auto npc) {
            constexpr unsigned NPC = decltype(npc)::value;
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
            const unsigned p = (pbeg & ~63u) + ln;
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<uint16_t*>(a.y) + ((tokbase + cst) * H + h) * kP,
                                                        (uint32_t)nv * (uint32_t)(H * kP * 2));
            if (ln - (pbeg & 63u) < NPC && p < 8u * kXU) {
                const unsigned qi0 = piece_row(p), k = p & 7u;
                const u32x4 o = *reinterpret_cast<const u32x4*>(ys + qi0 * 144 + k * 16);
                __builtin_amdgcn_raw_buffer_store_b128(o, ro, (int)((qi0 / R) * (unsigned)(H * kP * 2) + 16 * k), 0, 0);
            }
        };

        // raw C rows of tiles KB .. KE - 1 of the chunk at cst straight into the operand layout
        // (tile k, slice ks: row 16 qt + lane % 16, n = 32 ks + 8 (lane / 16) ...); rows of
        // tokens past the segment end read zero (their outputs are never stored)
        auto load_c = [&](int cst, auto kbc, auto kec) {
            constexpr int KB = decltype(kbc)::value, KE = decltype(kec)::value;
            // (uniform; stated, so that the resource stays scalar on every path)
            const int nv = __builtin_amdgcn_readfirstlane(max(0, min(Q, T1 - cst)));
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cg + (size_t)(nv > 0 ? cst : 0) * bstride, (uint32_t)nv * bsb);
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
#pragma unroll
            for (int k = KB; k < KE; ++k) {
                const int qt = ctile<kNC>(c, k);
                const unsigned qi = 16 * qt + (ln & 15u);
                const unsigned t = qi / R, r = qi % R;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    cq[k][ks] = __builtin_bit_cast(
                        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(t * bsb + r * (kN * 2) + 64 * ks + 16 * (ln >> 4)), 0, 0));
            }
        };

        // Tiles 0 .. TPC - 2 of a chunk are retired before its last phase of key blocks; their
        // C rows for the next chunk are loaded then (for the first chunk, here), and only tile
        // TPC - 1 at the chunk start.  Every chunk issues the same global loads and stores in
        // the same order (rows past the segment end fall outside the record counts), so a wait
        // for a load counts exactly the later ones and never the output stores just issued.
        if (kFullMode && TPC > 1) load_c(T0, std::integral_constant<int, 0>{}, std::integral_constant<int, TPC - 1>{});
        int cidx = 0;
        for (int c0 = T0; c0 < T1; c0 += Q, ++cidx) {
            // (A) theta into LDS (loaded a chunk ago), then the chunk's C rows, the next
            //     chunk's theta and per-token inputs
            stage_theta(rgTh);
            if (kFullMode) load_c(c0, std::integral_constant<int, TPC - 1>{}, std::integral_constant<int, TPC>{});
            // (layer, one tile per consumer) x and gate pieces of the previous chunk's
            // outputs, stored over this chunk's key blocks (none before the first chunk: zero
            // records); with more tiles they are loaded in the previous chunk's last phase
            if constexpr (LAYER && TPC == 1)
                if (kFullMode) load_xz(c0 > T0 ? c0 - Q : c0, c0 > T0 ? Q : 0);
            load_theta(c0 + Q, rgTh);
            __syncthreads();
            angles();
            // the previous chunk's outputs: staged (stored during this chunk's key blocks) or stored
            if (kFullMode && c0 > T0) {
                if constexpr (LY::kYStage) stage_y();
                else store_y(c0 - Q, Q);
            }
            __syncthreads();
            // (layer) the previous chunk's output pieces, finished in place
            if constexpr (LAYER)
                if (kFullMode && c0 > T0) finish_pieces();
            // (C) C tiles: bias and turn; carry readout Y^T = exp(l_t) Hf Ct^T
            int tq[TPC];
            float l2q[TPC];
            if (kFullMode) {
                int ln = lane;                                // opaque: offsets formed here
                asm volatile("" : "+v"(ln));
                ln &= 63;
                const int l16 = ln & 15, g4 = ln >> 4;
#pragma unroll
                for (int k = 0; k < TPC; ++k) {
                    const int qi = 16 * ctile<kNC>(c, k) + l16;
                    const int t = qi / R;
                    tq[k] = t;
                    l2q[k] = sL2[t];
                    // Pairs at or past np have identity table entries, so every slice takes the
                    // same path (a per-slice branch on np serialised the table reads); where the
                    // registers allow, all of the tile's table and bias reads are issued first.
                    constexpr int RG = waves_per_simd<R, Q>() < 4 ? 4 : 1;      // slices per read group
                    uint4 ce[4][2], bi[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        if (ks % RG == 0) {
#pragma unroll
                            for (int u = ks; u < ks + RG; ++u) {
                                const int i0 = 16 * u + 4 * g4;             // first pair
                                const uint2* e = sCS + t * 64 + (i0 ^ (t & 60));   // pairs i0 .. i0 + 3
                                ce[u][0] = *reinterpret_cast<const uint4*>(e);
                                ce[u][1] = *reinterpret_cast<const uint4*>(e + 2);
                                // a lane's rows have rank l16 % R in every tile (16 % R == 0)
                                bi[u] = *reinterpret_cast<const uint4*>(sCb + (l16 % R) * 64 + i0);
                            }
                        }
                        const uint4 raw = __builtin_bit_cast(uint4, cq[k][ks]);
                        const float2 p0 = rot_pair(raw.x, bi[ks].x, uint2{ce[ks][0].x, ce[ks][0].y});
                        const float2 p1 = rot_pair(raw.y, bi[ks].y, uint2{ce[ks][0].z, ce[ks][0].w});
                        const float2 p2 = rot_pair(raw.z, bi[ks].z, uint2{ce[ks][1].x, ce[ks][1].y});
                        const float2 p3 = rot_pair(raw.w, bi[ks].w, uint2{ce[ks][1].z, ce[ks][1].w});
                        cq[k][ks] = __builtin_bit_cast(
                            bf16x8, uint4{pack2(p0.x, p0.y), pack2(p1.x, p1.y), pack2(p2.x, p2.y), pack2(p3.x, p3.y)});
                    }
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = 16 * pt + l16;
                    bf16x8 av[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        av[ks] = *reinterpret_cast<const bf16x8*>(smem + LY::hs + hs_off(p, 4 * ks + g4));
#pragma unroll
                    for (int k = 0; k < TPC; ++k) yacc[k][pt] = mfma(av[0], cq[k][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int ks = 1; ks < 4; ++ks)
#pragma unroll
                        for (int k = 0; k < TPC; ++k) yacc[k][pt] = mfma(av[ks], cq[k][ks], yacc[k][pt]);
                }
#pragma unroll
                for (int k = 0; k < TPC; ++k) {
                    const float sc = __builtin_amdgcn_exp2f(l2q[k]);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) yacc[k][pt] = yacc[k][pt] * sc;
                }
            }
            __syncthreads();
            // (D) key blocks: scores against this wave's query tiles, weights, Y^T += X^T S'^T.
            //     A wave's tiles ascend with k, so the tiles that meet key block J are those
            //     from some K0 on; the blocks run in phases of constant K0, each phase a loop
            //     over one straight-line body.
            auto block_body = [&](auto k0c, auto dgc, int J) {
                constexpr int K0 = decltype(k0c)::value;
                // 0: no tile on the diagonal; 1: tile K0 on it; 2: every tile checks
                constexpr int kDiag = decltype(dgc)::value;
                const int ka = 2 * J;
                const char* buf = smem + (J & 1) * kBufBytes;
                const char* xtb = buf + kBnBytes + kBvBytes;
                float kl2[2][KT], kg1[2][KT], kgm[2][KT];
#pragma unroll
                for (int ab = 0; ab < 2; ++ab)
#pragma unroll
                    for (int j = 0; j < KT; ++j) {
                        const int ts = (16 * (ka + ab) + 4 * g4) / R + j;
                        kl2[ab][j] = sL2[ts];
                        kg1[ab][j] = sG1[ts];
                        if (kDiag) kgm[ab][j] = sGam[ts];
                    }
                // The decay factors of W: they need only the tabled log-decays, so with one
                // key token per lane and key tile (R = 4) their exps go before the score
                // MFMAs and overlap them; with more they stay after (registers).
                float ex[TPC][2][KT];
                auto decays = [&]() {
#pragma unroll
                    for (int k = K0; k < TPC; ++k)
#pragma unroll
                        for (int ab = 0; ab < 2; ++ab)
#pragma unroll
                            for (int j = 0; j < KT; ++j) ex[k][ab][j] = __builtin_amdgcn_exp2f(l2q[k] - kl2[ab][j]);
                };
                if constexpr (kEarlyExp) decays();
                f32x4 s0[TPC], s1[TPC];
                {
                    bf16x8 op[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) op[ks] = *reinterpret_cast<const bf16x8*>(buf + bn_off(l16, 4 * ks + g4));
#pragma unroll
                    for (int k = K0; k < TPC; ++k) {
                        s0[k] = mfma(op[0], cq[k][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int ks = 1; ks < 4; ++ks) s0[k] = mfma(op[ks], cq[k][ks], s0[k]);
                    }
                }
                {
                    bf16x8 op[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        op[ks] = *reinterpret_cast<const bf16x8*>(buf + bn_off(16 + l16, 4 * ks + g4));
#pragma unroll
                    for (int k = K0; k < TPC; ++k) {
                        s1[k] = mfma(op[0], cq[k][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int ks = 1; ks < 4; ++ks) s1[k] = mfma(op[ks], cq[k][ks], s1[k]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!kEarlyExp) decays();
                // S'^T = W o S^T as bf16 B operands.  The tile on the block's diagonal
                // (query tile ka or ka + 1) masks per element; key rows after its query
                // rows get weight 0 (also the whole of key tile b when the query tile is ka).
                bf16x8 bop[TPC];
#pragma unroll
                for (int k = K0; k < TPC; ++k) {
                    const bool diag = kDiag == 2 ? ctile<kNC>(c, k) <= ka + 1 : (kDiag == 1 && k == K0);   // uniform
                    float wgt[2][KT];
#pragma unroll
                    for (int ab = 0; ab < 2; ++ab) {
#pragma unroll
                        for (int j = 0; j < KT; ++j) {
                            const float e = ex[k][ab][j];
                            wgt[ab][j] = e * kg1[ab][j];
                            if (kDiag) {             // selects (the key token's g was read with the tables)
                                const int ts = (16 * (ka + ab) + 4 * g4) / R + j;
                                const float wd = ts < tq[k] ? wgt[ab][j] : (ts == tq[k] ? e * kgm[ab][j] : 0.f);
                                wgt[ab][j] = diag ? wd : wgt[ab][j];
                            }
                        }
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        bop[k][m] = (bf16)(s0[k][m] * wgt[0][m * KT / 4]);
                        bop[k][4 + m] = (bf16)(s1[k][m] * wgt[1][m * KT / 4]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // X^T in the k order of S'^T: keys 4 g4 + 0..3 of tile a, then of tile b
                bf16x8 xo[4];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) xo[pt] = *reinterpret_cast<const bf16x8*>(xtb + q4_off(16 * pt + l16, g4));
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                    for (int k = K0; k < TPC; ++k) yacc[k][pt] = mfma(xo[pt], bop[k], yacc[k][pt]);
            };
            // per key block (Q <= 64): rows RPB J .. RPB J + RPB - 1 of this wave's staged outputs
            // of the previous chunk (tile RPB J / 16)
            // (none before the first chunk: a record count of 0 drops the stores)
            const int nprev = c0 > T0 ? Q : 0;
            auto block_end = [&](int J) {
                if constexpr (LAYER) {
                    // the tokens of rows RPB J .. RPB J + RPB - 1: pieces 8 RPB J / R ..
                    if (kFullMode)
                        layer_store(nprev ? c0 - Q : c0, nprev, 8u * RPB * J / R,
                                    std::integral_constant<unsigned, 8 * RPB / R>{});
                } else if constexpr (LY::kYStage) {
                    if (kFullMode)
                        store_rows(nprev ? c0 - Q : c0, nprev, ctile<kNC>(c, RPB * J / 16), RPB * J % 16,
                                   std::integral_constant<unsigned, RPB>{});
                }
                __syncthreads();
            };
            int Jb = 0;
            auto phase = [&](auto mc) {
                constexpr int K0 = decltype(mc)::value;
                const int Je = K0 < TPC ? min(NKB, ctile<kNC>(c, K0 < TPC ? K0 : 0) / 2 + 1) : NKB;
                if constexpr (TPC > 1 && K0 == TPC - 1)
                    if (kFullMode) {             // (none after the last chunk: zero records)
                        load_c(c0 + Q, std::integral_constant<int, 0>{}, std::integral_constant<int, TPC - 1>{});
                        // (layer) x and gate pieces of this chunk's outputs, finished at the
                        // next chunk's start: a phase of key blocks hides their latency
                        if constexpr (LAYER) load_xz(c0, min(Q, T1 - c0));
                    }
                if constexpr (K0 < TPC && kEarlyExp) {
                    // blocks before the last of tile K0, then its diagonal block
#pragma unroll 1
                    for (int J = Jb; J < Je - 1; ++J) {
                        if (kFullMode) block_body(mc, std::integral_constant<int, 0>{}, J);
                        block_end(J);
                    }
                    if (Je > Jb) {
                        if (kFullMode) block_body(mc, std::integral_constant<int, 1>{}, Je - 1);
                        block_end(Je - 1);
                    }
                } else if constexpr (K0 < TPC) {
#pragma unroll 1
                    for (int J = Jb; J < Je; ++J) {
                        if (kFullMode) block_body(mc, std::integral_constant<int, 2>{}, J);
                        block_end(J);
                    }
                } else {
#pragma unroll 1
                    for (int J = Jb; J < Je; ++J) block_end(J);
                }
                Jb = max(Jb, Je);
            };
            phase(std::integral_constant<int, 0>{});
            if constexpr (TPC >= 1) phase(std::integral_constant<int, 1>{});
            if constexpr (TPC >= 2) phase(std::integral_constant<int, 2>{});
            if constexpr (TPC >= 3) phase(std::integral_constant<int, 3>{});
            if constexpr (TPC >= 4) phase(std::integral_constant<int, 4>{});
        }
        // the last chunk's outputs
        if (kFullMode && T1 > T0) {
            const int cst = T0 + (T1 - T0 - 1) / Q * Q, nv = (T1 - T0 - 1) % Q + 1;
            if constexpr (LAYER) {
                stage_y();
                if constexpr (TPC == 1) load_xz(cst, nv);     // (else loaded in its last phase)
                finish_pieces();
#pragma unroll
                for (int sl = 0; sl < kXS; ++sl) layer_store(cst, nv, 64u * sl, std::integral_constant<unsigned, 64>{});
            } else if constexpr (LY::kYStage) {
                stage_y();
#pragma unroll
                for (int k = 0; k < TPC; ++k)
#pragma unroll
                    for (int i = 0; i < 2; ++i) store_rows(cst, nv, ctile<kNC>(c, k), 8 * i, std::integral_constant<unsigned, 8>{});
            } else {
                store_y(cst, nv);
            }
        }
    } else {
        // =============================== producers ===============================
        const int pw = w - kNC;
        // Key rows of producer pw in a block: key group pw of both key tiles.  For B, half-wave
        // hh = lane / 32 takes rows 16 hh + 4 pw + i (i < 4): token offset hh 16 / R + i / R
        // from the token of row 4 pw, rank i % R, and lane lq = lane % 32 its n = 4 lq ..
        // 4 lq + 3 (pairs 2 lq, 2 lq + 1).  For x, lane lq takes p = 2 lq, 2 lq + 1 of all 8
        // rows rr = 4 hh' + i (both half-waves load the same).
        constexpr int NTK = 16 / R + 3 / R + 1;              // tokens spanned by the 8 rows
        const int hh = lane >> 5, lq = lane & 31;
        // B bias of this lane's two pairs, per rank (bf16 pairs)
        uint32_t bb[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            bb[r][0] = bb[r][1] = 0u;
            if (a.Bb) {
                const float4 v = *reinterpret_cast<const float4*>(a.Bb + ((size_t)h * R + r) * kN + 4 * lq);
                bb[r][0] = pack2(v.x, v.y);
                bb[r][1] = pack2(v.z, v.w);
            }
        }
        // lift factors of this lane's two x elements p = 2 lq, 2 lq + 1, per rank
        float lf[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            lf[r][0] = lifted ? a.lift[((size_t)h * R + r) * kP + 2 * lq] : 0.f;
            lf[r][1] = lifted ? a.lift[((size_t)h * R + r) * kP + 2 * lq + 1] : 0.f;
        }
        // state columns [32 pw, 32 pw + 32): H^T tiles (n-tile 2 pw + u, p-tile pt), lane:
        // p = 16 pt + l16, n = 32 pw + 16 u + 4 g4 + m
        f32x4 hacc[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int nb = 32 * pw + 16 * u + 4 * g4;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p = 16 * pt + l16;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (kFullMode) {
                    if (seg == 0) {
                        if (a.h0) {
                            const size_t o = ((size_t)bh * kP + p) * kN + nb;
                            if (a.st_bf16) {
                                const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.h0) + o);
                                v = f32x4{lo_f(q.x), hi_f(q.x), lo_f(q.y), hi_f(q.y)};
                            } else {
                                const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.h0) + o);
                                v = f32x4{f.x, f.y, f.z, f.w};
                            }
                        }
                        if (a.Bp0 && a.xp0) {
                            const float dt0 = LAYER ? softplus_f(dtg[0] + dtb) : dtg[0];
                            const float d0 = dt0 * (1.f - (LAYER ? sigmoid_f(lamg[0]) : lamg[0]));
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
                hacc[u][pt] = v;
            }
        }
        float lam_sum = 0.f;

        // raw key rows of block gb of the segment, through buffer loads bounded at the
        // segment end (rows of later tokens read zero)
        // prefetch ring: slot J % DP holds block J's raw rows, fetched DP blocks ahead
        constexpr int DP = (NKB >= 4 && kNC == 4) ? 4 : 2;      // 12 waves: 168 registers
        static_assert(NKB % DP == 0, "whole ring groups per chunk");
        uint2 rgB[DP][4];
        uint32_t rgX[DP][8];
        // Blocks are fetched in order; consecutive blocks (also across a chunk boundary)
        // start 32 / R tokens apart, so the fetch keeps running row pointers.
        constexpr int TPB = kKB / R;                         // tokens per block
        int f_rem = T1 - (T0 + 4 * pw / R);                  // tokens from row 4 pw to the segment end
        const uint16_t* f_b = Bg + (size_t)(T0 + 4 * pw / R) * bstride;
        const uint16_t* f_x = Xg + (size_t)(T0 + 4 * pw / R) * xstride;
        auto fetch = [&](uint2 (&pb)[4], uint32_t (&px)[8]) {
            const int nt = __builtin_amdgcn_readfirstlane(min(max(f_rem, 0), NTK));
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(f_b, (uint32_t)nt * bsb);
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(f_x, (uint32_t)nt * xsb);
            unsigned ln = lane;                               // opaque: offsets formed here
            asm volatile("" : "+v"(ln));
            ln &= 63u;
            const unsigned h2 = ln >> 5, l2 = ln & 31u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned u = h2 * (16 / R) + i / R, r = i % R;
                pb[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rb, (int)(u * bsb + 256 * r + 8 * l2), 0, 0));
            }
            // row rr = (token u, rank r); an un-lifted x has one row per token, which every
            // rank's slot loads (the lift is applied when the rows are turned into tiles)
            const unsigned rstride = lifted ? 0u : 128u;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const unsigned u = (rr >> 2) * (16 / R) + (rr & 3) / R, r = (rr & 3) % R;
                px[rr] = __builtin_amdgcn_raw_buffer_load_b32(rx, (int)(u * xsb + rstride * r + 4 * l2), 0, 0);
            }
            f_rem -= TPB;
            f_b += (size_t)TPB * bstride;
            f_x += (size_t)TPB * xstride;
        };
        // turn the rows of block J and write its tiles, row-major over the key rows: Bn (the
        // scores' operand), Bv = v Bt and X (read back by transposed reads).  Rows of tokens
        // past the chunk's valid ones need no masking: their raw rows read zero and their v is
        // zero (dt = 0), so only finite values (the turned bias) reach the tiles.
        // per-row angle table entries (this lane's two pairs) and v of block J (rows of one
        // token share the reads); read ahead of the block's state MFMAs
        auto block_scalars = [&](int J, uint4 (&csr)[4], float (&vvr)[4]) {
            const int tb = (kKB * J + 4 * pw) / R;              // token of row 4 pw
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tb + hh * (16 / R) + i / R;
                csr[i] = *reinterpret_cast<const uint4*>(sCS + t * 64 + ((2 * lq) ^ (t & 60)));
                vvr[i] = sV[t];
            }
        };
        auto store_block = [&](int J, const uint2 (&pb)[4], const uint32_t (&px)[8], const uint4 (&csr)[4],
                               const float (&vvr)[4]) {
            char* buf = smem + (J & 1) * kBufBytes;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * hh + 4 * pw + i;
                const int o = bn_off(row, lq >> 1) + (lq & 1) * 8;
                const float2 p0 = rot_pair(pb[i].x, bb[i % R][0], uint2{csr[i].x, csr[i].y});
                const float2 p1 = rot_pair(pb[i].y, bb[i % R][1], uint2{csr[i].z, csr[i].w});
                if (kFullMode) *reinterpret_cast<uint2*>(buf + o) = uint2{pack2(p0.x, p0.y), pack2(p1.x, p1.y)};
                const float v = vvr[i];
                *reinterpret_cast<uint2*>(buf + kBnBytes + o) = uint2{pack2(p0.x * v, p0.y * v), pack2(p1.x * v, p1.y * v)};
            }
            // the 8 x rows (lifted here when x is un-lifted: row rr of rank r is lift[r] * x)
            uint32_t xv[8];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int r = (rr & 3) % R;
                xv[rr] = lifted ? pack2(lf[r][0] * lo_f(px[rr]), lf[r][1] * hi_f(px[rr])) : px[rr];
            }
            // XT rows p = 2 lq, 2 lq + 1, key group pw (lanes of the first half-wave)
            uint32_t xt0[4], xt1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xt0[q] = __builtin_amdgcn_perm(xv[2 * q + 1], xv[2 * q], 0x05040100u);
                xt1[q] = __builtin_amdgcn_perm(xv[2 * q + 1], xv[2 * q], 0x07060302u);
            }
            char* xtt = buf + kBnBytes + kBvBytes;
            if (hh == 0) {
                *reinterpret_cast<uint4*>(xtt + q4_off(2 * lq, pw)) = uint4{xt0[0], xt0[1], xt0[2], xt0[3]};
                *reinterpret_cast<uint4*>(xtt + q4_off(2 * lq + 1, pw)) = uint4{xt1[0], xt1[1], xt1[2], xt1[3]};
            }
        };
#pragma unroll
        for (int d = 0; d < DP; ++d) fetch(rgB[d], rgX[d]);

        int cidx = 0;
        for (int c0 = T0; c0 < T1; c0 += Q, ++cidx) {
            // (A) state snapshot (bf16, the carry readout's operand); theta staging
            if (kFullMode) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int nb = 32 * pw + 16 * u + 4 * g4;
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const int p = 16 * pt + l16;
                        *reinterpret_cast<uint2*>(smem + LY::hs + hs_off(p, nb >> 3) + ((nb >> 2) & 1) * 8) =
                            uint2{pack2(hacc[u][pt][0], hacc[u][pt][1]), pack2(hacc[u][pt][2], hacc[u][pt][3])};
                    }
                }
            }
            stage_theta(rgTh);
            load_theta(c0 + Q, rgTh);
            load_scalars(c0 + Q);
            // wave 4 scans the log-decays from the staged inputs and tables the per-token scalars
            if (pw == 0) {
                // lane index made opaque here: the table addresses are formed per chunk rather
                // than kept live (or spilled) across the chunk loop
                int lns = lane;
                asm volatile("" : "+v"(lns));
                lns &= 63;
                float la[TPL], gm[TPL], dl[TPL];
                float lsum = 0.f;
#pragma unroll
                for (int k = 0; k < TPL; ++k) {
                    const int t = lns * TPL + k;
                    const bool in = t < Q;
                    const float dt = in ? sDt[t] : 0.f, lm = in ? sLm[t] : 0.f;
                    float rate = -ah;
                    if (dyn_rate) rate = heavy_tail_rate(in ? sAr[t] : 0.f);
                    la[k] = dt * rate;
                    gm[k] = lm * dt;
                    dl[k] = dt * (1.f - lm);
                    lsum += la[k];
                    la[k] = lsum;
                }
                const float incl = group_scan<64>(lsum, lane);
                const float excl = incl - lsum;
                const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
                const float le = tot * kLog2e;
                const float nx = dpp_read<0x130>(dl[0]);           // wave_shl:1
                const float dnext = sDt[Q] * (1.f - sLm[Q]);
#pragma unroll
                for (int k = 0; k < TPL; ++k) {
                    const int t = lns * TPL + k;
                    const float dn = (k + 1 < TPL) ? dl[k + 1] : ((t + 1 < Q) ? nx : dnext);
                    if (t < Q) {
                        const float l2t = (excl + la[k]) * kLog2e;
                        sL2[t] = l2t;
                        sG1[t] = gm[k] + dn;
                        sGam[t] = gm[k];
                        sV[t] = __builtin_amdgcn_exp2f(le - l2t) * (gm[k] + dn);
                    }
                }
                if (lane == 0) sMisc[0] = le;
                lam_sum += tot;
            }
            __syncthreads();
            angles();
            __syncthreads();
            // (C) the next chunk's inputs (the angles no longer read this chunk's); the state
            //     decays over the whole chunk before its writes land; block 0
            stage_scalars(c0 + Q);
            {
                const float f = exp2f(sMisc[0]);
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) hacc[u][pt] = hacc[u][pt] * f;
            }
            {
                uint4 csr[4];
                float vvr[4];
                block_scalars(0, csr, vvr);
                store_block(0, rgB[0], rgX[0], csr, vvr);
            }
            __syncthreads();
            // (D) per block: the state update from block J; block J + 1's tiles; refill
#pragma unroll 1
            for (int J0 = 0; J0 < NKB; J0 += DP) {
#pragma unroll
                for (int d = 0; d < DP; ++d) {
                    const int J = J0 + d;
                    fetch(rgB[d], rgX[d]);
                    // every LDS read of the iteration first (block J's operands, block J + 1's
                    // angles and v), then the state MFMAs, then block J + 1's tiles
                    const char* buf = smem + (J & 1) * kBufBytes;
                    const char* bvb = buf + kBnBytes;
                    const char* xtb = buf + kBnBytes + kBvBytes;
                    // A: (v Bt)^T rows n = 32 pw + 16 u + l16; B: XT row p = 16 pt + l16
                    bf16x8 av[2], bv[4];
#pragma unroll
                    for (int u = 0; u < 2; ++u) av[u] = key_operand_256(bvb, 32 * pw + 16 * u, lane);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) bv[pt] = *reinterpret_cast<const bf16x8*>(xtb + q4_off(16 * pt + l16, g4));
                    // a next block exists within the ring group (d < DP - 1: NKB % DP == 0)
                    const bool more = d + 1 < DP || J + 1 < NKB;
                    uint4 csr[4];
                    float vvr[4];
                    if (more) block_scalars(J + 1, csr, vvr);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                        for (int u = 0; u < 2; ++u) hacc[u][pt] = mfma(av[u], bv[pt], hacc[u][pt]);
                    if (more) store_block(J + 1, rgB[(d + 1) % DP], rgX[(d + 1) % DP], csr, vvr);
                    // schedule: the LDS reads, then the row fetches, then the MFMAs each
                    // followed by a share of the row turning, then the tile writes
                    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 12, 0);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x200, 12, 0);
                    __syncthreads();
                }
            }
        }
        // ---- end of the stream / segment: the state ----
        if (!kFullMode) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int nb = 32 * pw + 16 * u + 4 * g4;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = 16 * pt + l16;
                    *reinterpret_cast<float4*>(wsHloc + (ss * kP + p) * kN + nb) =
                        float4{hacc[u][pt][0], hacc[u][pt][1], hacc[u][pt][2], hacc[u][pt][3]};
                }
            }
            if (pw == 0 && lane == 0) wsLam[ss] = lam_sum;
        } else if (last_seg && a.h1) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int nb = 32 * pw + 16 * u + 4 * g4;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int p = 16 * pt + l16;
                    const size_t o = ((size_t)bh * kP + p) * kN + nb;
                    if (a.st_bf16)
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h1) + o) =
                            uint2{pack2(hacc[u][pt][0], hacc[u][pt][1]), pack2(hacc[u][pt][2], hacc[u][pt][3])};
                    else
                        *reinterpret_cast<float4*>(static_cast<float*>(a.h1) + o) =
                            float4{hacc[u][pt][0], hacc[u][pt][1], hacc[u][pt][2], hacc[u][pt][3]};
                }
            }
        }
    }

    // ---- end of the stream / segment: phase and previous write (all threads; sPhic holds
    //      the final phase since the last chunk's angle section) ----
    if (!kFullMode) {
        for (int i = tid; i < np; i += kThreads) wsDphi[ss * np + i] = sPhic[i];
    } else if (last_seg) {
        if (a.phi1)
            for (int i = tid; i < np; i += kThreads) a.phi1[(size_t)bh * np + i] = sPhic[i];
        if (a.Bp1 && a.xp1) {
            const int t = L - 1;
            for (int e = tid; e < R * kN / 2; e += kThreads) {
                const int r = e / (kN / 2), i = e % (kN / 2);
                const uint32_t raw = *reinterpret_cast<const uint32_t*>(Bg + (size_t)t * bstride + r * kN + 2 * i);
                float b0 = lo_f(raw) + (a.Bb ? a.Bb[((size_t)h * R + r) * kN + 2 * i] : 0.f);
                float b1 = hi_f(raw) + (a.Bb ? a.Bb[((size_t)h * R + r) * kN + 2 * i + 1] : 0.f);
                if (i < np) {
                    float sn, cs;
                    sincosf(sPhic[i], &sn, &cs);
                    const float e0 = b0;
                    b0 = e0 * cs - b1 * sn;
                    b1 = e0 * sn + b1 * cs;
                }
                *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.Bp1) + ((size_t)bh * R + r) * kN + 2 * i) = pack2(b0, b1);
            }
            for (int e = tid; e < R * kP; e += kThreads) {
                uint16_t v = Xg[(size_t)t * xstride + (lifted ? e % kP : e)];
                if (lifted) v = __builtin_bit_cast(uint16_t, (bf16)(a.lift[(size_t)h * R * kP + e] * bf16_bits_to_f32(v)));
                static_cast<uint16_t*>(a.xp1)[(size_t)bh * R * kP + e] = v;
            }
        }
    }
}

// Pass 2 of the segmented schedule: the affine carry recurrence over segments,
//   Hin[0]   = h0 + d_0 X_prev0^T Bt_prev0                (folded initial carry)
//   Hin[k+1] = exp(Lam_k) Hin[k] + rot(Hloc_k, Phi_k),    Phi_{k+1} = Phi_k + dphi_k,
// as wave-level prefix scans ("Diagonal Equivalence in State Space Models ...", section 2.5:
// the recurrence is an associative scan of (decay, write) pairs).  A group of W lanes (W a
// power of two, at least the number of segments up to 64) owns one (p, n-pair) element of
// one stream, lane k its segment k: an inclusive Kogge-Stone sum of the angle steps gives
// each segment's Phi, the rotated local states become the writes, and an inclusive
// Kogge-Stone composition of the affine maps (a lane combines with the lane o below it,
// o = 1, 2, 4, ...) gives every segment's incoming state at once.  More than 64 segments
// run as blocks of 64, each block's composition applied to the state carried out of the
// one before.
template <int W>
__device__ __forceinline__ void seg_sum_scan(float& v, int k) {       // inclusive sum, angles mod 2 pi
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
        const float u = __shfl_up(v, o, W);
        if (k >= o) v = wrap_2pi(v + u);
    }
}
template <int W>
__device__ __forceinline__ void seg_affine_scan(float& A, float& B0, float& B1, int k) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
        const float Au = __shfl_up(A, o, W), B0u = __shfl_up(B0, o, W), B1u = __shfl_up(B1, o, W);
        if (k >= o) {                          // (earlier maps first): x -> A (Au x + Bu) + B
            B0 = A * B0u + B0;
            B1 = A * B1u + B1;
            A = A * Au;
        }
    }
}

template <int W>
__global__ __launch_bounds__(256) void carry_scan_kernel(ScanArgs a) {
    constexpr int GPW = 64 / W;                                  // elements per wave
    const int lane = threadIdx.x & 63, k_in = lane % W, grp = lane / W;
    const long elem = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * GPW + grp;   // (stream, pair element)
    constexpr int EPS = kP * kN / 2;                             // pair elements per stream
    if (elem >= (long)a.b * a.H * EPS) return;                   // whole groups leave together
    const int bh = (int)(elem / EPS), e = (int)(elem % EPS);
    const int p = e / (kN / 2), ip = e % (kN / 2), n = 2 * ip;
    const int nseg = a.nseg, np = a.np, H = a.H, L = a.L;
    const int bi = bh / H;
    const size_t S = (size_t)a.b * H * nseg;
    const float* wsHloc = a.ws;
    float* wsHin = a.ws + S * kP * kN;
    const float* wsLam = a.ws + 2 * S * kP * kN;
    const float* wsDphi = wsLam + S;
    float* wsPhi = a.ws + 2 * S * kP * kN + S + S * np;
    // the folded initial carry of this element (each lane of the group computes it)
    float h0 = 0.f, h1 = 0.f;
    if (a.h0) {
        const size_t o = ((size_t)bh * kP + p) * kN + n;
        h0 = ld_io(a.h0, o, a.st_bf16);
        h1 = ld_io(a.h0, o + 1, a.st_bf16);
    }
    if (a.Bp0 && a.xp0) {
        const size_t t0 = (size_t)bi * L * H + (bh % H);
        const bool raw = a.lift != nullptr;                      // the layer's raw projections
        const float dt0 = raw ? softplus_f(a.dt[t0] + (a.dt_bias ? a.dt_bias[bh % H] : 0.f)) : a.dt[t0];
        const float d0 = dt0 * (1.f - (raw ? sigmoid_f(a.lam[t0]) : a.lam[t0]));
        for (int r = 0; r < a.R; ++r) {
            const float xv = d0 * ld_io(a.xp0, ((size_t)bh * a.R + r) * kP + p, 1);
            h0 += xv * ld_io(a.Bp0, ((size_t)bh * a.R + r) * kN + n, 1);
            h1 += xv * ld_io(a.Bp0, ((size_t)bh * a.R + r) * kN + n + 1, 1);
        }
    }
    const bool turns = ip < np;
    float phi_in = (turns && a.phi0) ? a.phi0[(size_t)bh * np + ip] : 0.f;    // angle entering the block
    for (int k0 = 0; k0 < nseg; k0 += W) {
        const int k = k0 + k_in;
        const bool valid = k < nseg;
        const size_t ss = (size_t)bh * nseg + (valid ? k : 0);
        // segment k's angle: the carried angle plus the steps of the block's earlier segments
        float dphi = (valid && turns) ? wsDphi[ss * np + ip] : 0.f;
        seg_sum_scan<W>(dphi, k_in);                             // inclusive
        float before = __shfl_up(dphi, 1, W);
        if (k_in == 0) before = 0.f;
        const float phi = wrap_2pi(phi_in + before);
        // segment k's map: x -> exp(Lam_k) x + rot(Hloc_k, Phi_k)  (identity past the last segment)
        float A = 1.f, B0 = 0.f, B1 = 0.f;
        if (valid) {
            const size_t o = (ss * kP + p) * kN + n;
            A = expf(wsLam[ss]);
            B0 = wsHloc[o];
            B1 = wsHloc[o + 1];
            if (turns) {
                float sn, cs;
                sincosf(phi, &sn, &cs);
                const float t0 = B0 * cs - B1 * sn;
                B1 = B0 * sn + B1 * cs;
                B0 = t0;
            }
        }
        seg_affine_scan<W>(A, B0, B1, k_in);                     // lane k: segments k0 .. k composed
        // incoming state of segment k: segments k0 .. k - 1 applied to the carried state
        float Ae = __shfl_up(A, 1, W), E0 = __shfl_up(B0, 1, W), E1 = __shfl_up(B1, 1, W);
        if (k_in == 0) { Ae = 1.f; E0 = 0.f; E1 = 0.f; }
        if (valid) {
            const size_t o = (ss * kP + p) * kN + n;
            wsHin[o] = Ae * h0 + E0;
            wsHin[o + 1] = Ae * h1 + E1;
            if (turns && p == 0) wsPhi[ss * np + ip] = phi;
        }
        // the state and angle carried out of the block: its last lane's composition
        const int last = (lane / W) * W + W - 1;
        const float c0 = A * h0 + B0, c1 = A * h1 + B1;
        h0 = __shfl(c0, last);
        h1 = __shfl(c1, last);
        phi_in = wrap_2pi(phi_in + __shfl(dphi, last));
    }
}

template <int R, int Q, bool LAYER>
hipError_t launch_rql(const ScanArgs& a, hipStream_t st) {
    const size_t lds = Layout<R, Q>::total;
    const int nblk = a.b * a.H * a.nseg;
    hipError_t e;
    if (a.nseg > 1) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_ws_kernel<R, Q, kSummary, LAYER>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((scan_ws_kernel<R, Q, kSummary, LAYER>), dim3(nblk), dim3(n_threads<R, Q>()), lds, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_carry_pass(a, st)) != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_ws_kernel<R, Q, kFull, LAYER>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_ws_kernel<R, Q, kFull, LAYER>), dim3(nblk), dim3(n_threads<R, Q>()), lds, st, a);
    return hipGetLastError();
}

template <int R, int Q>
hipError_t launch_rq(const ScanArgs& a, hipStream_t st) {
    if constexpr (Q <= 64) {                 // the layer variant stages its outputs (Q <= 64)
        if (a.lift) return launch_rql<R, Q, true>(a, st);
    } else {
        if (a.lift) return hipErrorInvalidValue;
    }
    return launch_rql<R, Q, false>(a, st);
}

}  // namespace

hipError_t launch_carry_pass(const ScanArgs& a, hipStream_t st) {
    const long elems = (long)a.b * a.H * (kP * kN / 2);
    auto go = [&](auto kernel, int w) {
        const long groups_per_block = 4 * (64 / w);
        hipLaunchKernelGGL(kernel, dim3((unsigned)((elems + groups_per_block - 1) / groups_per_block)), dim3(256), 0,
                           st, a);
        return hipGetLastError();
    };
    if (a.nseg <= 2) return go(carry_scan_kernel<2>, 2);
    if (a.nseg <= 4) return go(carry_scan_kernel<4>, 4);
    if (a.nseg <= 8) return go(carry_scan_kernel<8>, 8);
    if (a.nseg <= 16) return go(carry_scan_kernel<16>, 16);
    if (a.nseg <= 32) return go(carry_scan_kernel<32>, 32);
    return go(carry_scan_kernel<64>, 64);
}

int scan_mfma_chunk(int io_bf16, int P, int N, int R, int Q) {
    if (!io_bf16 || P != kP || N != kN || !(R == 1 || R == 2 || R == 4)) return Q;
    const bool built = (Q == 16 || Q == 32 || Q == 64 || Q == 128) && Q * R >= 64 && Q * R <= kMaxRows;
    return built ? Q : 64 / R;                   // otherwise the small-chunk schedule
}

int scan_mfma_groups_per_cu(int R, int Q) { return (R == 4 && Q == 16) ? 2 : 1; }

bool scan_mfma_supported(const ScanArgs& a) {
    if (!a.io_bf16 || a.P != kP || a.N != kN) return false;
    if (!(a.R == 1 || a.R == 2 || a.R == 4)) return false;
    if (!(a.Q == 16 || a.Q == 32 || a.Q == 64 || a.Q == 128)) return false;
    const int M = a.Q * a.R;
    return M >= 64 && M <= kMaxRows;
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
        default: return hipErrorInvalidValue;
    }
}

}  // namespace m3
