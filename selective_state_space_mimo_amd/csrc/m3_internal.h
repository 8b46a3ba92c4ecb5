// Internal declarations shared by the host entry points and the kernels of
// libm3scan.  Not part of the public ABI (include/m3scan.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr float kTwoPi = 6.283185307179586f;

// Everything a scan launch needs; passed by value to the kernels.
struct ScanArgs {
    int b, L, H, G, P, N, R, np, Q;
    int io_bf16, st_bf16;
    const void* x; const void* B; const void* C;
    const float* dt; const float* lam; const float* theta; const float* A_log;
    int rate_law;   // 0: A_log [H] static rates; 1: A_log holds the per-token rate input [b,L,H]
    const float* Bb; const float* Cb;
    // initial carry (each may be null = zero)
    const void* h0; const float* phi0; const void* Bp0; const void* xp0;
    void* y;
    // final carry (each may be null = not written)
    void* h1; float* phi1; void* Bp1; void* xp1;
    // segmented schedule: nseg segments of seglen tokens (seglen % Q == 0)
    int nseg, seglen;
    float* ws;   // workspace (segmented schedule only)
    // Matrix-core path only, the layer entry point: when lift is non-null, x is the
    // un-lifted [b, L, H, P] and key row (t, r) is lift[h, r, :] * x[t] (the layer's P x R
    // lift, applied as the rows are fetched), and dt, lam, theta hold the layer's raw
    // projections, activated as they are staged: dt = softplus(dt + dt_bias[h]),
    // lam = sigmoid(lam), theta = pi tanh(theta).
    const float* lift;
    const float* dt_bias;
    // with lift: the readout weights [H, R, P]; y is then the recombined readout
    // sum_r comb[h, r] y_r, [b, L, H, P] (chunks of at most 64 tokens only)
    const float* comb;
    // with comb and a non-null gate [b, L, H, P]: y is the layer's output, the recombined
    // readout plus the skip dskip[h] x (dskip null: none), times silu(gate)
    const void* gate;
    const float* dskip;
};

// Decode-step arguments (one token, carry in place).
struct DecodeArgs {
    int b, H, G, P, N, R, np;
    int io_bf16, st_bf16;
    const void* x; const void* B; const void* C;
    const float* dt; const float* lam; const float* theta; const float* A_log;
    int rate_law;   // 0: A_log [H]; 1: A_log holds the per-token rate input [b,H]
    const float* Bb; const float* Cb;
    void* h; float* phi; void* Bp; void* xp;
    void* y;
};

// The layer steps around the scan (block.hip): raw projections and parameters in,
// the scan's inputs (lifted x, normalised B and C, dt, lambda, angular rates) out
// (prologue); the scan's readouts in, the gated layer output out (epilogue).
struct BlockArgs {
    int b, L, H, G, P, N, R, np;
    int io_bf16;
    const void* z; const void* x; const void* Braw; const void* Craw;
    const float* dt_raw; const float* lam_raw; const float* th_raw;
    const float* dt_bias; const float* Bg; const float* Cg;
    const float* lift; const float* comb; const float* D;
    float eps;
    void* xl; void* Bn; void* Cn; float* dt; float* lam; float* th;   // prologue outputs
    const void* y;                                                    // scan readouts [.., R, P]
    void* out;                                                        // layer output [.., P]
};

// Backward pass of the scan (bwd.hip): forward inputs, output sensitivities in, the
// gradients out; fp32 workspace for the shared B / C sums and the replay's per-token terms.
struct BwdArgs {
    int b, L, H, G, P, N, R, np;
    int io_bf16, st_bf16, rate_law;
    const void* x; const void* B; const void* C;
    const float* dt; const float* lam; const float* theta; const float* A;
    const float* Bb; const float* Cb;
    const void* h0; const float* phi0; const void* Bp0; const void* xp0;   // initial carry (null = 0)
    const void* dy;                                                        // [b, L, H, R, P] io
    const float* dh1; const float* dphi1; const float* dBp1; const float* dxp1;   // final-carry sensitivities
    void* dx; float* ddt; float* dlam; float* dtheta; float* dA; float* dBb; float* dCb;
    float* dh0; float* dphi0; float* dBp0; float* dxp0;                    // initial-carry gradients
    float* accB; float* accC;          // [b, L, G, R, N] fp32 sums over the heads of a group
    float* wphi; float* wdphi;         // [b, L, H, np] running angles, C side of the angle gradient
    float* wdl;                        // [b, L, H] <dy_t, y_t>
    float* wdlf;                       // [b, H] <dh_L, h_L>
    char* cws;                         // chunked form: chunk states and phases (null: token-serial form)
};
struct BwdWs {
    size_t accB, accC, phi, dphi, dl, dlf, cws, total;   // byte offsets of the workspace parts
};
bool scan_bwd_supported(int P, int N, int R, int np);
// The chunked (matrix-core) form of the backward: bf16 I/O, P 64, N 128, rank 4, at most
// 64 rotated pairs, at least one token.  Other shapes take the token-serial form.
bool scan_bwd_chunked_eligible(int io_bf16, int P, int N, int R, int np, int L);
size_t scan_bwd_chunked_extra_bytes(int b, int L, int H, int np);
hipError_t launch_scan_bwd_chunked(const BwdArgs& a, char* extra, hipStream_t s);
BwdWs scan_bwd_workspace(int b, int L, int H, int G, int R, int N, int np, bool chunked);
hipError_t launch_scan_bwd(const BwdArgs& a, void* dB, void* dC, hipStream_t s);

// ---- host-side launchers (return hipSuccess or the launch error) ----------
hipError_t launch_block_prologue(const BlockArgs& a, hipStream_t s);
hipError_t launch_block_epilogue(const BlockArgs& a, hipStream_t s);
hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t s);
size_t scan_generic_lds_bytes(int P, int N, int R, int np, int qg);
int scan_generic_chunk(int P, int N, int R, int np, int Q);

// The chunk the MFMA path runs for a requested chunk Q: at most 256 rows (Q R) per
// chunk; a longer request is split, which changes rounding only.
int scan_mfma_chunk(int io_bf16, int P, int N, int R, int Q);
// Workgroups of the matrix-core scan that one compute unit holds at once for (R, Q).
int scan_mfma_groups_per_cu(int R, int Q);
bool scan_mfma_supported(const ScanArgs& a);
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t s);
size_t scan_mfma_workspace_bytes(const ScanArgs& a);
// Pass 2 of the segmented schedule (the carry recurrence across segments).
hipError_t launch_carry_pass(const ScanArgs& a, hipStream_t s);
// One rank, no rotation, no bias, bf16 I/O, fp32 state, P 64, N 128, chunks of 64 tokens:
// head-shared scores per (batch, group, chunk), then the scan per (batch, head, half of P).
bool scan_siso_supported(const ScanArgs& a);
size_t scan_siso_workspace_bytes(const ScanArgs& a);
hipError_t launch_scan_siso(const ScanArgs& a, hipStream_t s);

// Per-coordinate selective scan (pcs.hip): x, dt [b, L, D], A_log [D, N], B, C
// [b, L, G, N], state [b, D, N] fp32; x, B, C and y in the io dtype, dt fp32.
struct PcsArgs {
    int b, L, D, G, N;
    int io_bf16;
    const void* x; const float* dt; const float* A_log; const void* B; const void* C;
    const float* h0;        // initial state (null = zero)
    void* y;
    float* h1;              // final state (null = not written)
    int nseg, seglen;       // segmented schedule: nseg segments of seglen tokens
    float* ws;              // workspace (segmented schedule only)
};
bool pcs_supported_state(int N);
int pcs_channels_per_group(int N);   // channels per workgroup
int pcs_groups_per_cu(int N);        // workgroups one compute unit holds at once
int pcs_waves_per_group(int N, bool segmented);
int pcs_block_tokens();              // tokens per block (segments are whole blocks)
size_t pcs_workspace_bytes(const PcsArgs& a);
hipError_t launch_pcs(const PcsArgs& a, hipStream_t s);

bool decode_fast_supported(const DecodeArgs& a);
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t s);

// ---- device helpers --------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
    return __uint_as_float(((uint32_t)u) << 16);
}
__device__ __forceinline__ float ld_io(const void* p, size_t i, int is_bf16) {
    if (is_bf16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}
__device__ __forceinline__ void st_io(void* p, size_t i, float v, int is_bf16) {
    if (is_bf16) ((bf16*)p)[i] = (bf16)v;           // round to nearest even
    else ((float*)p)[i] = v;
}
// Decay rate (< 0) from a per-token input u: the heavy-tail activation, negated and
// kept at or below -1e-4 (1 + u for u >= 0, 1 / (1 - u) for u < 0).
__device__ __forceinline__ float heavy_tail_rate(float u) {
    const float ht = u >= 0.f ? 1.f + u : 1.f / (1.f - u);
    return fminf(-ht, -1e-4f);
}
// The layer's activations of its raw step, blend and angle projections.
__device__ __forceinline__ float softplus_f(float v) { return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v))); }
__device__ __forceinline__ float sigmoid_f(float v) { return 1.f / (1.f + expf(-v)); }
// tanh from the hardware base-2 exponential and reciprocal: tanh x = 1 - 2 / (e^{2x} + 1)
// (exactly +-1 at the ends, where e^{2x} is 0 or infinite); below |x| = 1/16, where that
// form cancels, the odd Taylor series x - x^3/3 + 2 x^5/15 (truncation below 3e-10).
__device__ __forceinline__ float tanh_f(float x) {
    const float e = __builtin_amdgcn_exp2f(x * 2.8853900817779268f);        // e^{2x} = 2^{2x log2 e}
    const float big = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
    const float x2 = x * x;
    const float small = x * fmaf(x2, fmaf(x2, 2.f / 15.f, -1.f / 3.f), 1.f);
    return fabsf(x) < 0.0625f ? small : big;
}
constexpr float kPiF = 3.14159265358979f;
// Reduce an angle into [0, 2 pi).
__device__ __forceinline__ float wrap_2pi(float v) {
    float w = v - kTwoPi * floorf(v * (1.0f / kTwoPi));
    return (w >= kTwoPi || w < 0.f) ? 0.f : w;
}

}  // namespace m3
