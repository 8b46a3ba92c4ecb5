// Backward pass of the scan in chunked form on the matrix cores, for bf16 I/O at
// P = 64, N = 128, rank 4 (the shapes of the rank-4 prefill workload).
//
// "Diagonal Equivalence in State Space Models: Characterization, Retrieval Rank, and
// Selective Extensions" (paperpeel.com): section 2.4 (the chunked, state-space-duality
// form: within a chunk the recurrence is a masked product, across chunks a state is
// passed), section 2.5 (the adjoint recurrence: the state sensitivity runs backward
// through the transposed transition) and appendix D.3 (a backward that keeps the
// chunk-boundary states of the forward sweep).  The recurrence is the three-term update
// of "Mamba-3: Improved Sequence Modeling using State Space Principles"
// (intuitivepapers.ai), sections "How the exponential-trapezoidal update works",
// "Computing the rotation as a data-dependent RoPE" and "MIMO: a rank-4 state update".
//
// Folded carry.  With delta_t = dt_t (1 - lambda_t) (so beta_t = alpha_t delta_t), the
// folded state Hf_t = H_t + delta_{t+1} X_t^T Bt_t obeys, over a chunk of tokens c0 .. e
// with chunk-local cumulative log-decays l_t (l_t = sum_{c0 <= k <= t} log alpha_k):
//   H_t  = exp(l_t) Hf_in + sum_{u <= t} W(t,u) X_u^T Bt_u,
//   W(t,u) = exp(l_t - l_u) (gamma_u + [u < t] delta_{u+1}),
//   Hf_e = exp(l_e) Hf_in + sum_u v_u X_u^T Bt_u,   v_u = exp(l_e - l_u)(gamma_u + delta_{u+1}),
// and y_t[r] = H_t Ct_t[r].  Its adjoint over the chunk, given Gf_out = d loss / d Hf_e
// (from the later chunks) and dy, with rows m = (t, r), u' = (u, r'):
//   S^T(u', m) = Bt_u' . Ct_m,  S2^T(u', m) = X_u' . dy_m,  P(t,u) = sum_{r,r'} S^T S2^T,
//   dCt_m  = exp(l_t) Hf_in^T dy_m + sum_u' W S2^T(u', m) Bt_u',
//   dBt_u' = v_u Gf_out^T X_u'    + sum_m  W S2^T(u', m) Ct_m,
//   dX_u'  = v_u Gf_out Bt_u'     + sum_m  W S^T(u', m)  dy_m,
//   Gf_in  = exp(l_e) Gf_out + sum_m exp(l_t) dy_m (x) Ct_m,
// and the coefficient sensitivities, with Q_u = sum_r' X_u' . (Gf_out Bt_u'):
//   d gamma_u       = sum_{t >= u} exp(l_t - l_u) P(t,u) + exp(l_e - l_u) Q_u,
//   d delta_{u+1}   = sum_{t >  u} exp(l_t - l_u) P(t,u) + exp(l_e - l_u) Q_u,
//   d log alpha_t   = <G_t, alpha_t Hf_{t-1}>     (G_t = d loss / d H_t)
//                   = sum_{t' >= t} exp(l_t') <dy_t' (x) Ct_t', Hf_in> + exp(l_e) <Gf_out, Hf_in>
//                     + sum_{t' >= t} sum_{u < t} exp(l_t' - l_u)(gamma_u + delta_{u+1}) P(t',u)
//                     + sum_{u < t} v_u Q_u,
// every term an inner product of the chunk's own reads and writes (the difference of all
// reads and all writes at a token gives the same value but cancels in bf16 operands).
// The angle's sensitivity Phi_t (the reverse running sum of each token's rotation term)
// cancels across the sequence: the scores see only angle differences.  Rotating every
// token from t on by eps equals turning the incoming folded state by -eps and the final
// carry by +eps, so, per pair j (J_j a quarter turn of the pair's two columns),
//   Phi_t[j] = Phi_L[j] - <Gf_{t-1}, J_j Hf_{t-1}>,
//   Phi_L[j] = d phi_L[j] + <d h_L, J_j H_L> + <d B_prev,L, J_j Bt_{L-1}>.
// The kernel sums the rotation terms inside a chunk and takes Phi at each chunk's start
// from this identity, so rounding does not accumulate along the sequence.
//
// Two kernels per call, one workgroup of 8 waves per (batch, head) stream:
//   * bwdc_state_kernel walks the chunks forward and stores each chunk's incoming folded
//     state Hf_in (bf16, n-major) and its starting phases (fp32, wrapped into [0, 2 pi));
//   * bwdc_main_kernel walks them backward with Gf (fp32) in matrix-core accumulators:
//     per chunk, the score tiles S^T and S2^T, the weighted tiles (bf16 in LDS), the
//     products above, then the per-token scalar gradients (waves 0 and 1; meanwhile
//     waves 2..7 load the next chunk's x, dy, B, C rows and start phases into LDS); the
//     chunk's phase table is built by waves 1..4, four tokens each.
// Shared B and C gradients are summed over a group's heads by fp32 atomic adds into the
// workspace (as the token-serial backward does), converted to bf16 afterwards.
#include "scan_common.h"

namespace m3 {

namespace {

constexpr int kBQ = 16;                       // tokens per chunk
constexpr int kBR = 4;                        // ranks
constexpr int kBM = kBQ * kBR;                // rows (token, rank) per chunk
constexpr int kBT = 512;                      // threads: 8 waves
constexpr int kMaxPairs = 64;
constexpr size_t kHfChunkBytes = (size_t)kN * kP * 2;   // one chunk's Hf_in, [n][p] bf16

// ---- LDS layout of the main kernel (bytes) ----
constexpr int oX = 0;                         // X    [64 m][64 p]   bf16, 128-byte rows
constexpr int oDY = oX + kBM * kP * 2;        // dy   [64 m][64 p]
constexpr int oB = oDY + kBM * kP * 2;        // Bt   [64 m][128 n]  256-byte rows
constexpr int oC = oB + kBM * kN * 2;         // Ct   [64 m][128 n]
constexpr int oG = oC + kBM * kN * 2;         // Gf_out [128 n][64 p] (bf16 copy)
constexpr int oM1 = oG + kN * kP * 2;         // W S2^T stored as [64 m][64 u']
constexpr int oM2 = oM1 + kBM * kBM * 2;      // W S^T  stored as [64 m][64 u']
constexpr int oPH = oM2 + kBM * kBM * 2;      // (cos, sin) of the phases [16 t][64 pair]
constexpr int oDPB = oPH + kBQ * kMaxPairs * 8;   // B side of d phi [16][64]
constexpr int oDPC = oDPB + kBQ * kMaxPairs * 4;  // C side of d phi [16][64]
constexpr int oPM = oDPC + kBQ * kMaxPairs * 4;   // P(t, u) [16][16]
constexpr int oTAB = oPM + kBQ * kBQ * 4;

struct Tab {
    float l[kBQ], E[kBQ], gam[kBQ], v[kBQ], a[kBQ], u[kBQ];
    float dl[kBQ + 1], dt[kBQ + 1], lam[kBQ + 1];   // delta, dt, lambda of tokens c0 .. c0 + 16
    float RHp[8][kBQ];                              // per wave: <dy_t (x) Ct_t, Hf_in> of each token
    float Qp[4][kBQ];                               // per p tile: Q_u
    float GH[8];                                    // per wave: <Gf_out, Hf_in>
    float TP[kBQ];                                  // sum over pairs of theta_t Phi_t
    float dgam[kBQ], ddl[kBQ], dla[kBQ];
    alignas(16) float K[kBQ][kBQ];                              // [t][u]: sum_{t' >= t} of the corner terms of column u
    float ddl_next;                                 // d delta of token c0 + 16 from this chunk
    float phb[kMaxPairs];                           // <Gf_in, J_j Hf_in> of each pair
    float pend_dt, pend_lam;                        // token c0's gradients without its delta term
    float le;
};
constexpr int oRAW = oTAB + (int)((sizeof(Tab) + 15) / 16 * 16);

// ---- LDS layout of the state kernel ----
constexpr int sX_ = 0;                        // X  [64 m][64 p]
constexpr int sV_ = sX_ + kBM * kP * 2;       // v Bt [64 m][128 n]
constexpr int sPH_ = sV_ + kBM * kN * 2;      // (cos, sin) of the phases [16][64]
constexpr int sTAB_ = sPH_ + kBQ * kMaxPairs * 8;
constexpr int sRAW_ = sTAB_ + (int)((sizeof(Tab) + 15) / 16 * 16);

// Byte offset of element (row, col) of a bf16 tile with 128- or 256-byte rows.  The 16-byte
// groups of a row are XOR-permuted by the row (256-byte rows: by row mod 16; 128-byte rows,
// two to a bank cycle: by (row / 2) mod 8), so that 16 consecutive rows reading one group,
// and 4 rows reading a pair of groups (the transposing reads), fall on distinct banks.
__device__ __forceinline__ int swz(int pitch, int row, int col) {
    const int grp = col >> 3;
    const int x = pitch == 256 ? (row & 15) : ((row >> 1) & 7);
    return row * pitch + ((grp ^ x) << 4) + (col & 7) * 2;
}
// A-style operand: lane (g, s) reads row row0 + s, columns kbase + 8 g .. + 7 (16 bytes).
__device__ __forceinline__ bf16x8 row_op(const char* base, int pitch, int row0, int kbase, int lane) {
    const int g = lane >> 4, s = lane & 15;
    return *reinterpret_cast<const bf16x8*>(base + swz(pitch, row0 + s, kbase + 8 * g));
}
// B-style operand from a row-major tile by transposing reads: lane (g, s) receives column
// c0 + s at rows kbase + 8 g .. + 7 (two reads of four rows).
__device__ __forceinline__ bf16x8 tr_op(const char* base, int pitch, int kbase, int c0, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int row = kbase + 8 * g + (s >> 2), col = c0 + 4 * (s & 3);
    const uint2 lo = ds_tr(base + swz(pitch, row, col));
    const uint2 hi = ds_tr(base + swz(pitch, row + 4, col));
    return __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
}
// Four rows kb .. kb + 3 of column c0 + s (lane (g, s); kb chosen per lane group).
__device__ __forceinline__ void tr4(const char* base, int pitch, int kb, int c0, int lane, float out[4]) {
    const int s = lane & 15;
    const uint2 v = ds_tr(base + swz(pitch, kb + (s >> 2), c0 + 4 * (s & 3)));
    out[0] = lo_f(v.x); out[1] = hi_f(v.x); out[2] = lo_f(v.y); out[3] = hi_f(v.y);
}
// Workgroup barrier for LDS traffic only.  A __syncthreads() is also a release fence for
// global memory, which waits for every store and atomic in flight; the chunk loops write
// global memory that no wave of the workgroup reads back, so they wait for LDS only.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ float quad_swap(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a lane group, complete in the group's lane 15 (DPP scan).
__device__ __forceinline__ float sum16_at15(float v) { return group_scan<16>(v, 0); }
// Sum over the wave, in every lane.
__device__ __forceinline__ float sum64(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_scan<64>(v, 0)), 63));
}
__device__ __forceinline__ uint2 pack4(const f32x4& v) { return uint2{pack2(v[0], v[1]), pack2(v[2], v[3])}; }

// A chunk's raw per-token inputs, staged in LDS a chunk ahead of their use: dt, lambda and
// the rate input of tokens c0 .. c0 + 16 and theta of tokens c0 .. c0 + 15 (zero past L).
struct Raw {
    float th[kBQ][kMaxPairs];
    float dt[kBQ + 1], lam[kBQ + 1], ra[kBQ + 1];
    float phs[kMaxPairs];              // the chunk's start phases (main kernel)
};
struct RawRegs {
    float th0, th1, sdt, slm, sra;     // (kept apart: summing them here would wait for the loads)
};
// Global memory goes through buffer resources whose record counts end at the last valid
// token, with every load, store and atomic issued unconditionally: a token past L reads
// zero and its writes are dropped (an offset of kOOB is always out of range).  A memory
// operation under a lane-dependent branch would make the compiler wait for every
// operation in flight (the memory counter counts in issue order).
constexpr int kOOB = 0x7ffffff0;
__device__ __forceinline__ float ldf(__amdgpu_buffer_rsrc_t r, int off) {
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void stf(__amdgpu_buffer_rsrc_t r, int off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
// rows of tokens c0 .. c0 + n - 1 of a [.., L, S, ...] tensor at one (batch, slot): base
// element e0, `row` elements a token, `w` elements read per token
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tok_rsrc(const void* base, size_t e0, int esize, int n, int row, int w) {
    const char* p = base ? static_cast<const char*>(base) + e0 * esize : nullptr;
    return make_rsrc(p, base && n > 0 ? (uint32_t)(((n - 1) * row + w) * esize) : 0u);
}

__device__ __forceinline__ RawRegs load_raw(const BwdArgs& a, int bi, int h, int c0, int tid) {
    const int L = a.L, H = a.H, np = a.np;
    const int nv = min(kBQ, L - c0), ns = min(kBQ + 1, L - c0);
    const size_t t0 = ((size_t)bi * L + c0) * H + h;
    RawRegs r{0.f, 0.f, 0.f, 0.f, 0.f};
    if (np > 0) {
        const __amdgpu_buffer_rsrc_t rth = tok_rsrc(a.theta, t0 * np, 4, nv, H * np, np);
        const int e0 = tid, e1 = tid + kBT;
        const int ta = e0 / np, tb_ = e1 / np;
        r.th0 = ldf(rth, e0 < kBQ * np ? (ta * H * np + e0 - ta * np) * 4 : kOOB);
        r.th1 = ldf(rth, e1 < kBQ * np ? (tb_ * H * np + e1 - tb_ * np) * 4 : kOOB);
    }
    const int kind = tid / (kBQ + 1), t = tid - kind * (kBQ + 1);
    const int off = tid < 3 * (kBQ + 1) ? t * H * 4 : kOOB;
    const float vdt = ldf(tok_rsrc(a.dt, t0, 4, ns, H, 1), kind == 0 ? off : kOOB);
    const float vlm = ldf(tok_rsrc(a.lam, t0, 4, ns, H, 1), kind == 1 ? off : kOOB);
    const float vra = ldf(tok_rsrc(a.rate_law ? a.A : nullptr, t0, 4, ns, H, 1), kind == 2 ? off : kOOB);
    r.sdt = vdt;
    r.slm = vlm;
    r.sra = vra;
    return r;
}
__device__ __forceinline__ void store_raw(const RawRegs& r, int np, int tid, Raw* raw) {
    if (np > 0) {
        const int e0 = tid, e1 = tid + kBT;
        if (e0 < kBQ * np) { const int t = e0 / np; raw->th[t][e0 - t * np] = r.th0; }
        if (e1 < kBQ * np) { const int t = e1 / np; raw->th[t][e1 - t * np] = r.th1; }
    }
    if (tid < 3 * (kBQ + 1)) {
        const int kind = tid / (kBQ + 1), t = tid - kind * (kBQ + 1);
        (kind == 0 ? raw->dt : kind == 1 ? raw->lam : raw->ra)[t] = r.sdt + r.slm + r.sra;
    }
}

constexpr int oPRE = oRAW + (int)((sizeof(Raw) + 15) / 16 * 16);   // next chunk's rows: 6 pieces x 512 threads x 16 B
constexpr int kPreBytes = 6 * kBT * 16;
constexpr int oBIAS = oPRE + kPreBytes;                               // B and C biases of the head [2][4][128] fp32
constexpr int kMainLds = oBIAS + 2 * kBR * kN * 4;
static_assert(kMainLds <= 160 * 1024, "the main kernel's LDS exceeds a compute unit's");

// The rows of chunk [c0, c0 + 16) that thread tid stages (row m = tid / 8: token m / 4, rank
// m % 4; piece tid % 8), loaded straight into LDS (buffer loads to LDS; lane i of a wave
// writes 16 bytes at the wave's base + 16 i): x, dy (16 bytes each), B, C (32 bytes each).
// Rows past L read zero.  Completion is awaited with the memory counter before the reads.
// Buffer-to-LDS loads written out, so that the compiler does not hold every later LDS access
// of the issuing wave until they land; their waits are explicit (vmcnt(0) of the issuing waves,
// then a barrier, before the data is read).  lds: a uniform LDS byte address (m0); each lane
// writes its piece at lds + 16 lane (4 lane for the 4-byte form).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(r), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" :: "v"(voff), "s"(r), "{m0}"(lds) : "memory");
}

// The next chunk's x, dy, B and C rows as 3072 16-byte pieces, piece q landing at pre + 16 q:
// [0, 512) x, [512, 1024) dy, [1024, 2048) B and [2048, 3072) C (piece k of thread j of a kind
// is row j / 8, 16-byte group j % 8, first or second half of a 256-byte row).  Issued by waves
// 2..7 (eight pieces per lane; a wave's 64 pieces of one instruction lie in one kind), while
// waves 0 and 1 work alone on the chunk's per-token sensitivities.  Wave 2 first brings the
// chunk's np start phases (phs, from the state pass) into raw->phs: it is its oldest load, so
// vmcnt(8) in that wave means it has landed.
__device__ __forceinline__ void prefetch_rows(const BwdArgs& a, int bi, int h, int gg, int c0, int tid, char* pre,
                                              const float* phs, Raw* raw) {
    const int L = a.L, H = a.H, G = a.G;
    const int nv = min(kBQ, L - c0);
    const size_t t0 = (size_t)bi * L + c0;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6) - 2, lane = tid & 63;
    const uint32_t xb = (uint32_t)(((nv - 1) * H + 1) * kBR * kP * 2), bb = (uint32_t)(((nv - 1) * G + 1) * kBR * kN * 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const uint16_t*>(a.x) + (t0 * H + h) * kBR * kP, xb);
    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(static_cast<const uint16_t*>(a.dy) + (t0 * H + h) * kBR * kP, xb);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const uint16_t*>(a.B) + (t0 * G + gg) * kBR * kN, bb);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(static_cast<const uint16_t*>(a.C) + (t0 * G + gg) * kBR * kN, bb);
    const uint32_t pre_lds = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)pre);
    if (wv == 0)
        lds_dma4(make_rsrc(phs, (uint32_t)a.np * 4u),
                 __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const float*)raw->phs)),
                 lane * 4);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int q0 = k * 384 + wv * 64;                 // the wave's first piece (uniform)
        const int kind = q0 >> 9;
        const int j = (q0 & 511) + lane;
        const int m = j >> 3, q8 = j & 7, t = m >> 2, r = m & 3;
        const int xo = (t * H * kBR * kP + r * kP + 8 * q8) * 2;
        const int bo_ = (t * G * kBR * kN + r * kN + 16 * q8) * 2 + ((kind & 1) ? 16 : 0);
        const __amdgpu_buffer_rsrc_t rs = kind == 0 ? rx : kind == 1 ? rdy : kind < 4 ? rb : rc;
        lds_dma16(rs, __builtin_amdgcn_readfirstlane(pre_lds + q0 * 16), kind < 2 ? xo : bo_);
    }
}
// The state pass's next-chunk rows: x (512 16-byte pieces), then B's first and second
// halves (512 each); piece j of a kind is row j / 8, 16-byte group j % 8 (as above).  All
// eight waves issue three buffer-to-LDS loads each (instruction k of wave w: pieces
// 512 k + 64 w ..), during the chunk before the one that reads them.
constexpr int sPRE_ = sRAW_ + (int)((sizeof(Raw) + 15) / 16 * 16);
constexpr int sBIAS_ = sPRE_ + 3 * kBT * 16;                         // the head's B bias [4][128] fp32
constexpr int kStateLds = sBIAS_ + kBR * kN * 4;
static_assert(2 * kStateLds <= 160 * 1024, "two state-pass workgroups share a compute unit");
static_assert(kBT == kBR * kN, "one bias element per thread");
__device__ __forceinline__ void prefetch_xb(const BwdArgs& a, int bi, int h, int gg, int c0, int tid, char* pre) {
    const int L = a.L, H = a.H, G = a.G;
    const int nv = min(kBQ, L - c0);
    const size_t t0 = (size_t)bi * L + c0;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const uint32_t xb = (uint32_t)(((nv - 1) * H + 1) * kBR * kP * 2), bb = (uint32_t)(((nv - 1) * G + 1) * kBR * kN * 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const uint16_t*>(a.x) + (t0 * H + h) * kBR * kP, xb);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const uint16_t*>(a.B) + (t0 * G + gg) * kBR * kN, bb);
    const uint32_t pre_lds = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)pre);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int j = wv * 64 + lane;                      // piece of kind k
        const int m = j >> 3, q8 = j & 7, t = m >> 2, r = m & 3;
        const int xo = (t * H * kBR * kP + r * kP + 8 * q8) * 2;
        const int bo_ = (t * G * kBR * kN + r * kN + 16 * q8) * 2 + (k == 2 ? 16 : 0);
        lds_dma16(k == 0 ? rx : rb, __builtin_amdgcn_readfirstlane(pre_lds + (k * kBT + wv * 64) * 16), k == 0 ? xo : bo_);
    }
}

// The per-token scalars of the chunk into the table (wave 0; lane t: token c0 + t, lane 16
// the token after the chunk).  Tokens at or past L have dt = 0: no decay, no write.
__device__ void chunk_scalars(const BwdArgs& a, const Raw* raw, float rateA, int lane, Tab* tb) {
    const bool in = lane <= kBQ;
    const int li = in ? lane : 0;
    const float dt = in ? raw->dt[li] : 0.f;
    const float lam = in ? raw->lam[li] : 0.f;
    float rate = 0.f, u = 0.f;
    if (a.rate_law) {
        u = in ? raw->ra[li] : 0.f;
        rate = -heavy_tail_rate(u);
    } else {
        rate = rateA;
    }
    const float la = -dt * rate;
    const float gam = lam * dt, dl = dt * (1.f - lam);
    const float l = group_scan<16>(lane < kBQ ? la : 0.f, lane);
    const float le = __shfl(l, kBQ - 1, 64);
    const float dn = __shfl_down(dl, 1, 64);
    if (lane < kBQ) {
        tb->l[lane] = l;
        tb->E[lane] = __expf(l);
        tb->gam[lane] = gam;
        tb->v[lane] = __expf(fminf(le - l, 0.f)) * (gam + dn);
        tb->a[lane] = rate;
        tb->u[lane] = u;
    }
    if (in) {
        tb->dl[lane] = dl;
        tb->dt[lane] = dt;
        tb->lam[lane] = lam;
    }
    if (lane == 0) tb->le = le;
}

// Phases of the chunk's tokens (wave 1, lane j < np: pair j) from the chunk's starting
// phase phi (wrapped): phi_t[j] = phi + sum_{k <= t} dt_k theta_k[j]; their cos and sin
// (hardware forms of the phase wrapped into [0, 2 pi)) into the table.  Returns the phase
// after the chunk.
__device__ float chunk_phases(const Raw* raw, int j, float phi, float2* cst) {
    float dtv[kBQ], thv[kBQ];                 // the chunk's reads first
#pragma unroll
    for (int t = 0; t < kBQ; ++t) { dtv[t] = raw->dt[t]; thv[t] = raw->th[t][j]; }
#pragma unroll
    for (int t = 0; t < kBQ; ++t) {
        phi = fmaf(dtv[t], thv[t], phi);
        float sn, cs;
        __sincosf(wrap_2pi(phi), &sn, &cs);
        cst[t * kMaxPairs + j] = float2{cs, sn};
    }
    return phi;
}

// Tokens T0 .. T0 + 3 of chunk_phases, for one of four waves sharing the table: the same
// running sum up to token T0 + 3 (so the same values), the cos and sin of its last four.
template <int T0>
__device__ void chunk_phases4(const Raw* raw, int j, float phi, float2* cst) {
    constexpr int TE = T0 + 4;
    float dtv[TE], thv[TE];
#pragma unroll
    for (int t = 0; t < TE; ++t) { dtv[t] = raw->dt[t]; thv[t] = raw->th[t][j]; }
#pragma unroll
    for (int t = 0; t < TE; ++t) {
        phi = fmaf(dtv[t], thv[t], phi);
        if (t >= T0) {
            float sn, cs;
            __sincosf(wrap_2pi(phi), &sn, &cs);
            cst[t * kMaxPairs + j] = float2{cs, sn};
        }
    }
}

// 16 turned values of a row at columns n0 .. n0 + 15 from loaded data: raw (two 16-byte
// pieces) + bias (16 floats), pairs (2 j, 2 j + 1) with j < np turned by the token's table
// entries, times scale; bf16 pairs out.
__device__ __forceinline__ void turn_loaded(const uint4& r0, const uint4& r1, const float* bias, const float2* cst, int np,
                                            int n0, float scale, uint32_t out[8]) {
    float v[16];
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) { v[2 * k] = lo_f(w[k]); v[2 * k + 1] = hi_f(w[k]); }
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
        const float4 b4 = *reinterpret_cast<const float4*>(bias + n0 + k);
        v[k] += b4.x; v[k + 1] += b4.y; v[k + 2] += b4.z; v[k + 3] += b4.w;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = (n0 >> 1) + k;
        float e = v[2 * k], o = v[2 * k + 1];
        if (j < np) {
            const float2 c = cst[j];
            const float e2 = e * c.x - o * c.y, o2 = e * c.y + o * c.x;
            e = e2; o = o2;
        }
        out[k] = pack2(e * scale, o * scale);
    }
}

// 16 turned values of row (token, rank) at columns n0 .. n0 + 15: raw + bias, pairs
// (2 j, 2 j + 1) with j < np rotated by the token's phases, times scale; bf16 pairs out.
__device__ __forceinline__ void turn_piece(const uint16_t* raw, const float* bias, const float2* cst, int np, int n0,
                                           float scale, uint32_t out[8]) {
    float v[16];
    if (raw) {
        const uint4 r0 = *reinterpret_cast<const uint4*>(raw + n0);
        const uint4 r1 = *reinterpret_cast<const uint4*>(raw + n0 + 8);
        const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) { v[2 * k] = lo_f(w[k]); v[2 * k + 1] = hi_f(w[k]); }
        if (bias) {
#pragma unroll
            for (int k = 0; k < 16; k += 4) {
                const float4 b4 = *reinterpret_cast<const float4*>(bias + n0 + k);
                v[k] += b4.x; v[k + 1] += b4.y; v[k + 2] += b4.z; v[k + 3] += b4.w;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = (n0 >> 1) + k;
        float e = v[2 * k], o = v[2 * k + 1];
        if (j < np) {
            const float2 c = cst[j];
            const float e2 = e * c.x - o * c.y, o2 = e * c.y + o * c.x;
            e = e2; o = o2;
        }
        out[k] = pack2(e * scale, o * scale);
    }
}

// ---------------------------------------------------------------------------------------
// Forward sweep: each chunk's incoming folded state and starting phases.
__global__ __launch_bounds__(kBT) void bwdc_state_kernel(BwdArgs a, char* hfws, float* phws, float* phl) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, s = lane & 15;
    const int L = a.L, H = a.H, G = a.G, np = a.np;
    const int bh = blockIdx.x, h = bh % H, bi = bh / H, gg = h * G / H;
    const int nch = (L + kBQ - 1) / kBQ;
    const float rateA = a.rate_law ? 0.f : expf(a.A[h]);   // the static rate law's rate
    char* const sX = smem + sX_;
    char* const sV = smem + sV_;
    float2* const ph = reinterpret_cast<float2*>(smem + sPH_);
    Tab* const tb = reinterpret_cast<Tab*>(smem + sTAB_);

    // Hf_{-1} = H0 + delta_0 x_prev^T B_prev (the initial carry, folded); wave w owns n-tile w
    f32x4 hf[4];
    {
        const int n = 16 * w + s;
        float d0 = 0.f;
        if (a.Bp0 && a.xp0) {
            const size_t t0 = (size_t)bi * L * H + h;
            d0 = a.dt[t0] * (1.f - a.lam[t0]);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 16 * pt + 4 * g4 + i;
                float v = a.h0 ? ld_io(a.h0, ((size_t)bh * kP + p) * kN + n, a.st_bf16) : 0.f;
                if (a.Bp0 && a.xp0)
#pragma unroll
                    for (int r = 0; r < kBR; ++r)
                        v += d0 * ld_io(a.xp0, ((size_t)bh * kBR + r) * kP + p, a.io_bf16) *
                             ld_io(a.Bp0, ((size_t)bh * kBR + r) * kN + n, a.io_bf16);
                hf[pt][i] = v;
            }
    }
    float phi = (w == 1 && lane < np && a.phi0) ? a.phi0[(size_t)bh * np + lane] : 0.f;
    Raw* const raw = reinterpret_cast<Raw*>(smem + sRAW_);
    char* const pre = smem + sPRE_;
    float* const sBias = reinterpret_cast<float*>(smem + sBIAS_);
    store_raw(load_raw(a, bi, h, 0, tid), np, tid, raw);
    sBias[tid] = a.Bb ? a.Bb[(size_t)h * kBR * kN + tid] : 0.f;     // kBT == kBR * kN
    prefetch_xb(a, bi, h, gg, 0, tid, pre);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int c0 = c * kBQ;
        if (w == 0) chunk_scalars(a, raw, rateA, lane, tb);
        if (w == 1 && lane < np) {
            phi = wrap_2pi(phi);
            phws[((size_t)bh * nch + c) * np + lane] = phi;
            phi = chunk_phases(raw, lane, phi, ph);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");             // the chunk's rows in LDS
        lds_barrier();
        const bool more = c + 1 < nch;
        RawRegs nx{0.f, 0.f, 0.f, 0.f, 0.f};
        if (more) nx = load_raw(a, bi, h, c0 + kBQ, tid);
        {
            // X rows and v-scaled turned B rows (row m = tid / 8, piece tid % 8); rows past L
            // read zero and their scale v is zero
            const int m = tid >> 3, q8 = tid & 7, t = m >> 2, r = m & 3;
            const uint4 xv = *reinterpret_cast<const uint4*>(pre + 0 * kBT * 16 + tid * 16);
            const uint4 b0 = *reinterpret_cast<const uint4*>(pre + 1 * kBT * 16 + tid * 16);
            const uint4 b1 = *reinterpret_cast<const uint4*>(pre + 2 * kBT * 16 + tid * 16);
            *reinterpret_cast<uint4*>(sX + swz(kP * 2, m, 8 * q8)) = xv;
            uint32_t o[8];
            turn_loaded(b0, b1, sBias + r * kN, ph + t * kMaxPairs, np, 16 * q8, tb->v[t], o);
            *reinterpret_cast<uint4*>(sV + swz(kN * 2, m, 16 * q8)) = uint4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<uint4*>(sV + swz(kN * 2, m, 16 * q8 + 8)) = uint4{o[4], o[5], o[6], o[7]};
        }
        // the chunk's incoming state, n-major: lane writes p = 16 pt + 4 g4 .. + 3 of column n
        {
            char* dst = hfws + ((size_t)bh * nch + c) * kHfChunkBytes;
            const int n = 16 * w + s;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                *reinterpret_cast<uint2*>(dst + (n * kP + 16 * pt + 4 * g4) * 2) = pack4(hf[pt]);
        }
        lds_barrier();
        if (more) store_raw(nx, np, tid, raw);
        if (more) prefetch_xb(a, bi, h, gg, c0 + kBQ, tid, pre);     // the staging reads are done
        // Hf = exp(l_e) Hf + X^T (v Bt): rows p (A = X^T by transposing reads), columns n
        const float fe = __expf(tb->le);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            f32x4 acc = {hf[pt][0] * fe, hf[pt][1] * fe, hf[pt][2] * fe, hf[pt][3] * fe};
#pragma unroll
            for (int km = 0; km < 2; ++km)
                acc = mfma(tr_op(sX, kP * 2, 32 * km, 16 * pt, lane), tr_op(sV, kN * 2, 32 * km, 16 * w, lane), acc);
            hf[pt] = acc;
        }
        lds_barrier();
    }

    // Phi_L[j] = d phi_L[j] + <d h_L, J_j H_L> + <d B_prev,L, J_j Bt_{L-1}> (hf is H_L: delta_L = 0)
    if (np == 0) return;
    float* const hterm = reinterpret_cast<float*>(sV);          // [64 pairs]
    {
        const int n = 16 * w + s;
        const bool odd = (s & 1) != 0;
        float acc = 0.f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float partner = quad_swap(hf[pt][i]);
                const float d = a.dh1 ? a.dh1[((size_t)bh * kP + 16 * pt + 4 * g4 + i) * kN + n] : 0.f;
                acc = fmaf(d, odd ? partner : -partner, acc);
            }
        acc += quad_swap(acc);
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        if (g4 == 0 && !odd) hterm[n >> 1] = acc;
    }
    __syncthreads();
    if (tid < np) {
        const int j = tid, tl = (L - 1) - (nch - 1) * kBQ;
        float v = hterm[j] + (a.dphi1 ? a.dphi1[(size_t)bh * np + j] : 0.f);
        if (a.dBp1) {
            const float sn = ph[tl * kMaxPairs + j].y, cs = ph[tl * kMaxPairs + j].x;
            const size_t tok = (size_t)bi * L + (L - 1);
#pragma unroll
            for (int r = 0; r < kBR; ++r) {
                const uint16_t* raw = static_cast<const uint16_t*>(a.B) + (tok * G + gg) * kBR * kN + r * kN;
                float e = bf16_bits_to_f32(raw[2 * j]), o = bf16_bits_to_f32(raw[2 * j + 1]);
                if (a.Bb) {
                    e += a.Bb[((size_t)h * kBR + r) * kN + 2 * j];
                    o += a.Bb[((size_t)h * kBR + r) * kN + 2 * j + 1];
                }
                const float e2 = e * cs - o * sn, o2 = e * sn + o * cs;
                v += a.dBp1[((size_t)bh * kBR + r) * kN + 2 * j] * (-o2) + a.dBp1[((size_t)bh * kBR + r) * kN + 2 * j + 1] * e2;
            }
        }
        phl[(size_t)bh * np + j] = v;
    }
}

// ---------------------------------------------------------------------------------------
// Reverse sweep over the chunks.
__global__ __launch_bounds__(kBT) void bwdc_main_kernel(BwdArgs a, const char* hfws, const float* phws, const float* phl) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, s = lane & 15;
    const int L = a.L, H = a.H, G = a.G, np = a.np;
    const int bh = blockIdx.x, h = bh % H, bi = bh / H, gg = h * G / H;
    const int nch = (L + kBQ - 1) / kBQ;
    const float rateA = a.rate_law ? 0.f : expf(a.A[h]);   // the static rate law's rate
    const size_t bo = (size_t)bi * L;
    char* const sX = smem + oX;
    char* const sDY = smem + oDY;
    char* const sB = smem + oB;
    char* const sC = smem + oC;
    char* const sG = smem + oG;
    char* const sM1 = smem + oM1;
    char* const sM2 = smem + oM2;
    float2* const ph = reinterpret_cast<float2*>(smem + oPH);
    float* const dphB = reinterpret_cast<float*>(smem + oDPB);
    float* const dphC = reinterpret_cast<float*>(smem + oDPC);
    float* const sPM = reinterpret_cast<float*>(smem + oPM);
    Tab* const tb = reinterpret_cast<Tab*>(smem + oTAB);

    // Gf = d loss / d Hf at the sequence end: the final state's sensitivity (wave w: n-tile w)
    f32x4 gf[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            gf[pt][i] = a.dh1 ? a.dh1[((size_t)bh * kP + 16 * pt + 4 * g4 + i) * kN + 16 * w + s] : 0.f;
    // Phi: the angle's sensitivity (wave 1, lane j < np), and its constant Phi_L
    float Phi = (w == 1 && lane < np && a.dphi1) ? a.dphi1[(size_t)bh * np + lane] : 0.f;
    const float PhiL = (w == 1 && lane < np) ? phl[(size_t)bh * np + lane] : 0.f;
    float bbias[4] = {0.f, 0.f, 0.f, 0.f}, cbias[4] = {0.f, 0.f, 0.f, 0.f};
    float dA_acc = 0.f;                       // static rate law: sum of d A over tokens (wave 0)
    float pend_dt = 0.f, pend_lam = 0.f;      // token c0 + 16 of the previous iteration (wave 0, lane 0)

    Raw* const raw = reinterpret_cast<Raw*>(smem + oRAW);
    char* const pre = smem + oPRE;
    float* const sBias = reinterpret_cast<float*>(smem + oBIAS);
    store_raw(load_raw(a, bi, h, (nch - 1) * kBQ, tid), np, tid, raw);
    for (int i = tid; i < 2 * kBR * kN; i += kBT) {
        const float* src = i < kBR * kN ? a.Bb : a.Cb;
        sBias[i] = src ? src[(size_t)h * kBR * kN + (i % (kBR * kN))] : 0.f;
    }
    if (w >= 2) {
        prefetch_rows(a, bi, h, gg, (nch - 1) * kBQ, tid, pre, phws + ((size_t)bh * nch + nch - 1) * np, raw);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();

    for (int c = nch - 1; c >= 0; --c) {
        const int c0 = c * kBQ;
        // ---- S0a: scalars, phases ----
        if (w == 0) chunk_scalars(a, raw, rateA, lane, tb);
        if (w >= 1 && w <= 4 && lane < np) {                       // four tokens a wave
            const float phi0 = raw->phs[lane];
            if (w == 1) chunk_phases4<0>(raw, lane, phi0, ph);
            else if (w == 2) chunk_phases4<4>(raw, lane, phi0, ph);
            else if (w == 3) chunk_phases4<8>(raw, lane, phi0, ph);
            else chunk_phases4<12>(raw, lane, phi0, ph);
        }
        if (w >= 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the rows' loads into LDS
        lds_barrier();
        // Hf_in pieces (loaded first: they are used two phases later): B operands of dy Hf_in (column n = 16 w + s, k = p) and the lane's
        // own elements of the state tiles (for <Gf_out, Hf_in>)
        const char* const hin = hfws + ((size_t)bh * nch + c) * kHfChunkBytes;
        bf16x8 hop[2];
        uint2 hown[4];
        {
            const int n = 16 * w + s;
#pragma unroll
            for (int kp = 0; kp < 2; ++kp)
                hop[kp] = *reinterpret_cast<const bf16x8*>(hin + (n * kP + 32 * kp + 8 * g4) * 2);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) hown[pt] = *reinterpret_cast<const uint2*>(hin + (n * kP + 16 * pt + 4 * g4) * 2);
        }
        // ---- S0b: staging (the rows were prefetched into LDS) ----
        {
            const int m = tid >> 3, q8 = tid & 7, t = m >> 2, r = m & 3;
            const uint4 xv = *reinterpret_cast<const uint4*>(pre + 0 * kBT * 16 + tid * 16);
            const uint4 dv = *reinterpret_cast<const uint4*>(pre + 1 * kBT * 16 + tid * 16);
            const uint4 b0 = *reinterpret_cast<const uint4*>(pre + 2 * kBT * 16 + tid * 16);
            const uint4 b1 = *reinterpret_cast<const uint4*>(pre + 3 * kBT * 16 + tid * 16);
            const uint4 cc0 = *reinterpret_cast<const uint4*>(pre + 4 * kBT * 16 + tid * 16);
            const uint4 cc1 = *reinterpret_cast<const uint4*>(pre + 5 * kBT * 16 + tid * 16);
            *reinterpret_cast<uint4*>(sX + swz(kP * 2, m, 8 * q8)) = xv;
            *reinterpret_cast<uint4*>(sDY + swz(kP * 2, m, 8 * q8)) = dv;
            const float keep = c0 + t < L ? 1.f : 0.f;       // rows past L: zero (the bias too)
            uint32_t o[8];
            turn_loaded(b0, b1, sBias + r * kN, ph + t * kMaxPairs, np, 16 * q8, keep, o);
            *reinterpret_cast<uint4*>(sB + swz(kN * 2, m, 16 * q8)) = uint4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<uint4*>(sB + swz(kN * 2, m, 16 * q8 + 8)) = uint4{o[4], o[5], o[6], o[7]};
            turn_loaded(cc0, cc1, sBias + kBR * kN + r * kN, ph + t * kMaxPairs, np, 16 * q8, keep, o);
            *reinterpret_cast<uint4*>(sC + swz(kN * 2, m, 16 * q8)) = uint4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<uint4*>(sC + swz(kN * 2, m, 16 * q8 + 8)) = uint4{o[4], o[5], o[6], o[7]};
        }
        {
            const int n = 16 * w + s;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                *reinterpret_cast<uint2*>(sG + swz(kP * 2, n, 16 * pt + 4 * g4)) = pack4(gf[pt]);
        }
        lds_barrier();
        // the next chunk's raw inputs, staged in LDS once this chunk's are used (S3b)
        RawRegs nx{0.f, 0.f, 0.f, 0.f, 0.f};
        // ---- S1: score tiles S^T, S2^T (rows u', columns m), weights, P(t, u) ----
        {
            const int mt = w & 3;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int ut = 2 * (w >> 2) + k2;
                f32x4 st = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < 4; ++kn)
                    st = mfma(row_op(sB, kN * 2, 16 * ut, 32 * kn, lane), row_op(sC, kN * 2, 16 * mt, 32 * kn, lane), st);
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
                    s2 = mfma(row_op(sX, kP * 2, 16 * ut, 32 * kp, lane), row_op(sDY, kP * 2, 16 * mt, 32 * kp, lane), s2);
                const int t = 4 * mt + (s >> 2), u = 4 * ut + g4;
                float wt = 0.f;
                if (u <= t)
                    wt = __expf(fminf(tb->l[t] - tb->l[u], 0.f)) * (tb->gam[u] + (u < t ? tb->dl[u + 1] : 0.f));
                const f32x4 m1 = {wt * s2[0], wt * s2[1], wt * s2[2], wt * s2[3]};
                const f32x4 m2 = {wt * st[0], wt * st[1], wt * st[2], wt * st[3]};
                const int m = 16 * mt + s;
                *reinterpret_cast<uint2*>(sM1 + swz(kBM * 2, m, 16 * ut + 4 * g4)) = pack4(m1);
                *reinterpret_cast<uint2*>(sM2 + swz(kBM * 2, m, 16 * ut + 4 * g4)) = pack4(m2);
                float pr = st[0] * s2[0] + st[1] * s2[1] + st[2] * s2[2] + st[3] * s2[3];
                pr += quad_swap(pr);
                pr += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(pr), 0x4E, 0xf, 0xf, false));
                if ((s & 3) == 0) sPM[t * kBQ + u] = pr;
            }
        }
        lds_barrier();
        // ---- S2: the products ----
        const int nt = w, n = 16 * nt + s;
        const bool odd = (s & 1) != 0;
        const int pair = n >> 1;
        const bool turns = pair < np;
        const bool wturn = 8 * nt < np;                        // any turning pair in this wave's n-tile
        // (a) dCt = W S2 Bt + exp(l_t) dy Hf_in   (rows m, column n)
#pragma unroll 1
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (2 * ks <= mt) a1 = mfma(row_op(sM1, kBM * 2, 16 * mt, 32 * ks, lane), tr_op(sB, kN * 2, 32 * ks, 16 * nt, lane), a1);
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) a2 = mfma(row_op(sDY, kP * 2, 16 * mt, 32 * kp, lane), hop[kp], a2);
            const int t = 4 * mt + g4, tok = c0 + t;
            const float E = tb->E[t];
            float dc[4], cv[4];
            tr4(sC, kN * 2, 16 * mt + 4 * g4, 16 * nt, lane, cv);
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { dc[i] = fmaf(E, a2[i], a1[i]); rs = fmaf(cv[i], a2[i], rs); }
            rs = sum16_at15(rs);
            if (s == 15) tb->RHp[w][t] = rs;
            float outv[4];
            if (wturn) {
                const float2 cq = ph[t * kMaxPairs + pair];
                const float cs = turns ? cq.x : 1.f, sn = turns ? cq.y : 0.f;
                float dpp = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = quad_swap(cv[i]), pd = quad_swap(dc[i]);
                    const float e = odd ? pv : cv[i], o = odd ? cv[i] : pv;
                    const float de = odd ? pd : dc[i], dO = odd ? dc[i] : pd;
                    dpp += -de * o + dO * e;
                    outv[i] = odd ? -de * sn + dO * cs : de * cs + dO * sn;
                }
                if (turns && !odd) dphC[t * kMaxPairs + pair] = dpp;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) outv[i] = dc[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) cbias[i] += outv[i];
            if (tok < L) {
                float* acc = a.accC + ((bo + tok) * G + gg) * kBR * kN + n;
#pragma unroll
                for (int i = 0; i < 4; ++i) unsafeAtomicAdd(acc + i * kN, outv[i]);
            }
        }
        // (b) dBt = (W S2)^T Ct + v_u X Gf_out   (rows u', column n)
#pragma unroll 1
        for (int ut = 0; ut < 4; ++ut) {
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (2 * ks + 1 >= ut) a1 = mfma(tr_op(sM1, kBM * 2, 32 * ks, 16 * ut, lane), tr_op(sC, kN * 2, 32 * ks, 16 * nt, lane), a1);
#pragma unroll
            for (int kp = 0; kp < 2; ++kp)
                a2 = mfma(row_op(sX, kP * 2, 16 * ut, 32 * kp, lane), row_op(sG, kP * 2, 16 * nt, 32 * kp, lane), a2);
            const int u = 4 * ut + g4, tok = c0 + u;
            const float v = tb->v[u];
            float db[4], bv[4];
            tr4(sB, kN * 2, 16 * ut + 4 * g4, 16 * nt, lane, bv);
#pragma unroll
            for (int i = 0; i < 4; ++i) db[i] = fmaf(v, a2[i], a1[i]);
            if (tok == L - 1 && a.dBp1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) db[i] += a.dBp1[((size_t)bh * kBR + i) * kN + n];
            }
            float outv[4];
            if (wturn) {
                const float2 cq = ph[u * kMaxPairs + pair];
                const float cs = turns ? cq.x : 1.f, sn = turns ? cq.y : 0.f;
                float dpp = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = quad_swap(bv[i]), pd = quad_swap(db[i]);
                    const float e = odd ? pv : bv[i], o = odd ? bv[i] : pv;
                    const float de = odd ? pd : db[i], dO = odd ? db[i] : pd;
                    dpp += -de * o + dO * e;
                    outv[i] = odd ? -de * sn + dO * cs : de * cs + dO * sn;
                }
                if (turns && !odd) dphB[u * kMaxPairs + pair] = dpp;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) outv[i] = db[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) bbias[i] += outv[i];
            if (tok < L) {
                float* acc = a.accB + ((bo + tok) * G + gg) * kBR * kN + n;
#pragma unroll
                for (int i = 0; i < 4; ++i) unsafeAtomicAdd(acc + i * kN, outv[i]);
            }
        }
        // (c) dX = (W S)^T dy + v_u Z, Z = Bt Gf_out^T   (rows u', column p)
        {
            const int pt = w & 3, p = 16 * pt + s;
#pragma unroll 1
            for (int k2 = 0; k2 < 2; ++k2) {
                const int ut = 2 * (w >> 2) + k2;
                f32x4 z = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < 4; ++kn)
                    z = mfma(row_op(sB, kN * 2, 16 * ut, 32 * kn, lane), tr_op(sG, kP * 2, 32 * kn, 16 * pt, lane), z);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (2 * ks + 1 >= ut) a1 = mfma(tr_op(sM2, kBM * 2, 32 * ks, 16 * ut, lane), tr_op(sDY, kP * 2, 32 * ks, 16 * pt, lane), a1);
                const int u = 4 * ut + g4, tok = c0 + u;
                const float v = tb->v[u];
                float xv[4];
                tr4(sX, kP * 2, 16 * ut + 4 * g4, 16 * pt, lane, xv);
                float q = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) q = fmaf(xv[i], z[i], q);
                q = sum16_at15(q);
                if (s == 15) tb->Qp[pt][u] = q;
                if (tok < L) {
                    const size_t row = ((bo + tok) * H + h) * kBR * kP + p;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float dxv = fmaf(v, z[i], a1[i]);
                        if (tok == L - 1 && a.dxp1) dxv += a.dxp1[((size_t)bh * kBR + i) * kP + p];
                        static_cast<bf16*>(a.dx)[row + i * kP] = (bf16)dxv;
                    }
                }
            }
        }
        // (d) <Gf_out, Hf_in>, then Gf_in = exp(l_e) Gf_out + (E dy)^T Ct
        {
            float gh = 0.f;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                gh = fmaf(gf[pt][0], lo_f(hown[pt].x), gh);
                gh = fmaf(gf[pt][1], hi_f(hown[pt].x), gh);
                gh = fmaf(gf[pt][2], lo_f(hown[pt].y), gh);
                gh = fmaf(gf[pt][3], hi_f(hown[pt].y), gh);
            }
            gh = sum64(gh);
            if (lane == 0) tb->GH[w] = gh;
            const float fe = __expf(tb->le);
#pragma unroll 2
            for (int pt = 0; pt < 4; ++pt) {
                f32x4 acc = {gf[pt][0] * fe, gf[pt][1] * fe, gf[pt][2] * fe, gf[pt][3] * fe};
#pragma unroll
                for (int km = 0; km < 2; ++km) {
                    // A = dy^T (rows p, k = m) scaled by E of each key's token: k slots 0-3 are
                    // token 8 km + 2 g4, slots 4-7 token 8 km + 2 g4 + 1
                    const uint4 raw = __builtin_bit_cast(uint4, tr_op(sDY, kP * 2, 32 * km, 16 * pt, lane));
                    const float e0 = tb->E[8 * km + 2 * g4], e1 = tb->E[8 * km + 2 * g4 + 1];
                    const uint4 sc = {pack2(lo_f(raw.x) * e0, hi_f(raw.x) * e0), pack2(lo_f(raw.y) * e0, hi_f(raw.y) * e0),
                                      pack2(lo_f(raw.z) * e1, hi_f(raw.z) * e1), pack2(lo_f(raw.w) * e1, hi_f(raw.w) * e1)};
                    acc = mfma(__builtin_bit_cast(bf16x8, sc), tr_op(sC, kN * 2, 32 * km, 16 * nt, lane), acc);
                }
                gf[pt] = acc;
            }
            // <Gf_in, J_j Hf_in> of pair j = n / 2 (the chunk's starting Phi is Phi_L minus it)
            float jt = 0.f;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const float hv[4] = {lo_f(hown[pt].x), hi_f(hown[pt].x), lo_f(hown[pt].y), hi_f(hown[pt].y)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float partner = quad_swap(hv[i]);
                    jt = fmaf(gf[pt][i], odd ? partner : -partner, jt);
                }
            }
            jt += quad_swap(jt);
            jt += __shfl_xor(jt, 16, 64);
            jt += __shfl_xor(jt, 32, 64);
            if (g4 == 0 && !odd && turns) tb->phb[pair] = jt;
        }
        lds_barrier();
        // ---- S3a: coefficient sensitivities (wave 0), the angle's (wave 1) ----
        // (this chunk's rows were staged in S0b, so the prefetch buffer is free)
        if (c > 0) nx = load_raw(a, bi, h, c0 - kBQ, tid);
        if (w >= 2 && c > 0) prefetch_rows(a, bi, h, gg, c0 - kBQ, tid, pre, phws + ((size_t)bh * nch + c - 1) * np, raw);
        if (w == 0) {
            // every LDS read of the phase is issued before the arithmetic that needs it
            const int u = lane & 15;
            const bool ul = lane < kBQ;
            float lt[kBQ], pm[kBQ];
#pragma unroll
            for (int t = 0; t < kBQ; t += 4) {
                const float4 q = *reinterpret_cast<const float4*>(tb->l + t);
                lt[t] = q.x; lt[t + 1] = q.y; lt[t + 2] = q.z; lt[t + 3] = q.w;
            }
#pragma unroll
            for (int t = 0; t < kBQ; ++t) pm[t] = sPM[t * kBQ + u];
            const float lu = tb->l[u], le = tb->le;
            const float Qu = tb->Qp[0][u] + tb->Qp[1][u] + tb->Qp[2][u] + tb->Qp[3][u];
            float RH = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) RH += tb->RHp[k][u];
            float GH = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) GH += tb->GH[k];
            const float wv = tb->gam[u] + tb->dl[u + 1];
            const float diagP = sPM[u * kBQ + u];
            const float Eu = tb->E[u], vu = tb->v[u];
            // column u: tail = sum_{t > u} exp(l_t - l_u) P(t, u); the corner terms
            // exp(l_t' - l_u) wv_u P(t', u) summed over t' >= t, for every t > u (entries with
            // t <= u are written too and never read)
            float tail = 0.f, cs = 0.f, kc[kBQ];
#pragma unroll
            for (int t = kBQ - 1; t >= 1; --t) {
                const float ep = t > u ? __expf(fminf(lt[t] - lu, 0.f)) * pm[t] : 0.f;
                tail += ep;
                cs = fmaf(wv, ep, cs);
                kc[t] = cs;
            }
            if (ul) {
#pragma unroll
                for (int t = 1; t < kBQ; ++t) tb->K[t][u] = kc[t];
            }
            const float endq = __expf(fminf(le - lu, 0.f)) * Qu;
            const float vq = vu * Qu;
            // d log alpha_t (lane t = u): suffix of exp(l) RH (a scan of the lanes mirrored
            // within the row of 16), prefix of v Q, row t of K over u < t
            const float rv = dpp_read<0x140>(Eu * RH);
            const float sc = group_scan<16>(ul ? rv : 0.f, lane);
            const float suf = dpp_read<0x140>(sc);
            const float pre = group_scan<16>(ul ? vq : 0.f, lane) - vq;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float corner = 0.f;
#pragma unroll
            for (int k = 0; k < kBQ; k += 4) {
                const float4 q = *reinterpret_cast<const float4*>(&tb->K[u][k]);
                corner += (k < u ? q.x : 0.f) + (k + 1 < u ? q.y : 0.f) + (k + 2 < u ? q.z : 0.f) + (k + 3 < u ? q.w : 0.f);
            }
            const float dla = suf + __expf(le) * GH + pre + corner;
            const float dnext = tail + endq;                    // d delta of token u + 1
            const float dprev = dpp_read<0x111>(dnext);         // lane u: d delta of token u (u >= 1)
            if (ul) {
                tb->dgam[u] = diagP + tail + endq;
                tb->ddl[u] = u >= 1 ? dprev : 0.f;
                tb->dla[u] = dla;
            }
            if (lane == kBQ - 1) tb->ddl_next = dnext;
        }
        if (w == 1) {
            // Phi from the chunk's end back to its start (lane j < np: pair j), eight tokens'
            // LDS reads issued at a time; theta_t . Phi_t per pair into the B-side table (lanes
            // past np write 0; the table's rows of tokens t8 .. t8 + 7 are read before they are
            // overwritten), d theta through a resource that ends at the last token
            const bool pl = lane < np;
            float* const tpt = dphB;
            const int dvo = pl ? lane * 4 : kOOB;                // the token's offset goes in soffset
            const __amdgpu_buffer_rsrc_t rdt = tok_rsrc(a.dtheta, ((bo + c0) * H + h) * np, 4, min(kBQ, L - c0), H * np, np);
            float* const dpl = dphB + lane;             // [t][pair]: B side; rows kBQ + t: C side
            const float* const thl = &raw->th[0][lane];
#pragma unroll
            for (int t8 = kBQ - 8; t8 >= 0; t8 -= 8) {
                // the eight tokens' reads first (rows t8 .. t8 + 7 are overwritten only after)
                float ds[8], thv[8], dtv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    ds[i] = dpl[(t8 + i) * kMaxPairs] + dpl[(kBQ + t8 + i) * kMaxPairs];
                    thv[i] = thl[(t8 + i) * kMaxPairs];
                    dtv[i] = tb->dt[t8 + i];
                }
                asm volatile("" : "+v"(thv[0]), "+v"(thv[1]), "+v"(thv[2]), "+v"(thv[3]),
                                  "+v"(thv[4]), "+v"(thv[5]), "+v"(thv[6]), "+v"(thv[7]));   // loaded on every lane
#pragma unroll
                for (int i = 7; i >= 0; --i) {
                    const int t = t8 + i;
                    Phi += pl ? ds[i] : 0.f;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dtv[i] * Phi), rdt, dvo, t * H * np * 4, 0);
                    dpl[t * kMaxPairs] = pl ? thv[i] * Phi : 0.f;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < kBQ) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < kMaxPairs; j += 4) {
                    const float4 q = *reinterpret_cast<const float4*>(tpt + lane * kMaxPairs + j);
                    acc += (q.x + q.y) + (q.z + q.w);
                }
                tb->TP[lane] = acc;
            }
            if (pl) Phi = PhiL - tb->phb[lane];                 // Phi at the chunk's first token
        }
        lds_barrier();
        // ---- S3b: per-token outputs (wave 0, lane t) ----
        if (w == 0) {
            const int t = lane & 15, tok = c0 + t;
            const float dtt = tb->dt[t], lamt = tb->lam[t], dla = tb->dla[t], dg = tb->dgam[t], dd = tb->ddl[t];
            const float d_dt = dla * (-tb->a[t]) + dg * lamt + dd * (1.f - lamt) + tb->TP[t];
            const float d_lam = (dg - dd) * dtt;
            const float d_A = dla * dtt;
            const bool valid = lane < kBQ && tok < L;
            const size_t ti = (bo + (valid ? tok : 0)) * H + h;
            if (valid) {
                if (a.rate_law) {
                    const float uu = tb->u[t];
                    const float ht = uu >= 0.f ? 1.f + uu : 1.f / (1.f - uu);
                    const float dht = uu >= 0.f ? 1.f : 1.f / ((1.f - uu) * (1.f - uu));
                    a.dA[ti] = (-ht < -1e-4f) ? -d_A * dht : 0.f;
                } else {
                    dA_acc += d_A;
                }
                if (t >= 1) {
                    a.ddt[ti] = d_dt;
                    a.dlam[ti] = d_lam;
                }
            }
            // token c0 + 16 (finished but for the delta term from this chunk's last token)
            const float pdt = __shfl(d_dt, 0, 64), plam = __shfl(d_lam, 0, 64);
            if (lane == 0) {
                const int tn = c0 + kBQ;
                if (tn < L) {
                    const float dn = tb->ddl_next;
                    const size_t tin = (bo + tn) * H + h;
                    a.ddt[tin] = pend_dt + dn * (1.f - tb->lam[kBQ]);
                    a.dlam[tin] = pend_lam - dn * tb->dt[kBQ];
                }
                pend_dt = pdt;
                pend_lam = plam;
            }
        }
        if (c > 0) store_raw(nx, np, tid, raw);
        if (w == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");     // the next chunk's start phases
        lds_barrier();
    }

    // ---- the initial carry: Hf_{-1} = H0 + delta_0 x_prev^T B_prev ----
    const float d0 = tb->dl[0];
    const int n = 16 * w + s;
    if (a.dh0) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dh0[((size_t)bh * kP + 16 * pt + 4 * g4 + i) * kN + n] = gf[pt][i];
    }
    float gdot = 0.f;                          // <Gf_in, x_prev^T B_prev>
    if (a.Bp0 && a.xp0) {
        float bp[kBR];
#pragma unroll
        for (int r = 0; r < kBR; ++r) bp[r] = ld_io(a.Bp0, ((size_t)bh * kBR + r) * kN + n, a.io_bf16);
        float xb[kBR] = {0.f, 0.f, 0.f, 0.f};  // sum_p x_prev[r][p] Gf[p][n] over the lane's p
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 16 * pt + 4 * g4 + i;
#pragma unroll
                for (int r = 0; r < kBR; ++r) {
                    const float xp = ld_io(a.xp0, ((size_t)bh * kBR + r) * kP + p, a.io_bf16);
                    xb[r] = fmaf(xp, gf[pt][i], xb[r]);
                }
            }
#pragma unroll
        for (int r = 0; r < kBR; ++r) {
            gdot = fmaf(xb[r], bp[r], gdot);
            // d B_prev[r][n] = delta_0 sum_p x_prev[r][p] Gf[p][n]: sum over the lane groups
            float tot = xb[r] + __shfl_xor(xb[r], 16, 64);
            tot += __shfl_xor(tot, 32, 64);
            if (a.dBp0 && g4 == 0) a.dBp0[((size_t)bh * kBR + r) * kN + n] = d0 * tot;
        }
    } else if (a.dBp0) {
        if (g4 == 0)
#pragma unroll
            for (int r = 0; r < kBR; ++r) a.dBp0[((size_t)bh * kBR + r) * kN + n] = 0.f;
    }
    // d x_prev[r][p] = delta_0 sum_n Gf[p][n] B_prev[r][n]: per-wave partial rows in LDS
    float* const red = reinterpret_cast<float*>(smem + oB);    // [8 waves][4 r][64 p]
    if (a.Bp0 && a.xp0) {
        float bp[kBR];
#pragma unroll
        for (int r = 0; r < kBR; ++r) bp[r] = ld_io(a.Bp0, ((size_t)bh * kBR + r) * kN + n, a.io_bf16);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < kBR; ++r) {
                    const float v = sum16_at15(gf[pt][i] * bp[r]);
                    if (s == 15) red[(w * kBR + r) * kP + 16 * pt + 4 * g4 + i] = v;
                }
    }
    gdot = sum64(gdot);
    if (lane == 0) tb->GH[w] = gdot;
    __syncthreads();
    if (a.dxp0 && tid < kBR * kP) {
        float v = 0.f;
        if (a.Bp0 && a.xp0)
#pragma unroll
            for (int k = 0; k < 8; ++k) v += red[k * kBR * kP + tid];
        a.dxp0[(size_t)bh * kBR * kP + tid] = d0 * v;
    }
    if (w == 0 && lane == 0) {
        float GD = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) GD += tb->GH[k];
        const size_t t0 = bo * H + h;
        a.ddt[t0] = pend_dt + GD * (1.f - tb->lam[0]);
        a.dlam[t0] = pend_lam - GD * tb->dt[0];
    }
    if (w == 0 && !a.rate_law) {
        const float tot = sum64(lane < kBQ ? dA_acc : 0.f);
        if (lane == 0) unsafeAtomicAdd(a.dA + h, tot * -expf(a.A[h]));
    }
    if (w == 1 && lane < np && a.dphi0) a.dphi0[(size_t)bh * np + lane] = Phi;
    // bias gradients: sum over the lane groups (tokens), then over batches
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float vb = bbias[i] + __shfl_xor(bbias[i], 16, 64);
        vb += __shfl_xor(vb, 32, 64);
        float vc = cbias[i] + __shfl_xor(cbias[i], 16, 64);
        vc += __shfl_xor(vc, 32, 64);
        if (g4 == 0) {
            if (a.dBb) unsafeAtomicAdd(a.dBb + ((size_t)h * kBR + i) * kN + n, vb);
            if (a.dCb) unsafeAtomicAdd(a.dCb + ((size_t)h * kBR + i) * kN + n, vc);
        }
    }
}

}  // namespace

bool scan_bwd_chunked_eligible(int io_bf16, int P, int N, int R, int np, int L) {
    return io_bf16 && P == kP && N == kN && R == kBR && np >= 0 && np <= kMaxPairs && L >= 1;
}

size_t scan_bwd_chunked_extra_bytes(int b, int L, int H, int np) {
    const size_t nch = (size_t)(L + kBQ - 1) / kBQ;
    return (size_t)b * H * nch * (kHfChunkBytes + (size_t)np * 4) + (size_t)b * H * np * 4;
}

hipError_t launch_scan_bwd_chunked(const BwdArgs& a, char* extra, hipStream_t s) {
    const size_t nch = (size_t)(a.L + kBQ - 1) / kBQ;
    char* hfws = extra;
    float* phws = reinterpret_cast<float*>(extra + (size_t)a.b * a.H * nch * kHfChunkBytes);
    float* phl = phws + (size_t)a.b * a.H * nch * a.np;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwdc_state_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kStateLds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwdc_main_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMainLds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.b * a.H));
    hipLaunchKernelGGL(bwdc_state_kernel, grid, dim3(kBT), kStateLds, s, a, hfws, phws, phl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwdc_main_kernel, grid, dim3(kBT), kMainLds, s, a, hfws, phws, phl);
    return hipGetLastError();
}

}  // namespace m3
