// The Mamba-3 layer steps on either side of the scan ("Mamba-3: Improved
// Sequence Modeling using State Space Principles", the decode listing of
// "Computing the rotation as a data-dependent RoPE", "MIMO: a rank-4 state
// update" and "The Mamba-3 block, layer by layer"):
//   before the scan: step dt = softplus(dt_raw + dt_bias), lambda = sigmoid(lam_raw),
//     angular rate pi tanh(th_raw), BCNorm (RMSNorm of B and C over the state axis,
//     times a gain; the per-head bias is added inside the scan, after the norm), and
//     the lift of the P-wide x into R copies, x_r = lift[h, r] * x;
//   after it: the R readouts recombined as y = sum_r comb[h, r] * y_r, the skip
//     D[h] x (un-lifted x) and the gate silu(z).
// The decay rate (static or heavy-tail) is the scan's own.  These kernels are
// bandwidth-bound element maps: one wave per row (norm) or per (token, head), lanes
// over the contiguous axis, fp32 arithmetic, io stores rounded to nearest even.
#include "m3_internal.h"

namespace m3 {

namespace {

constexpr int kWaves = 4;                // waves per workgroup
constexpr float kPi = 3.14159265358979f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float softplus(float v) { return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v))); }
__device__ __forceinline__ float sigmoid(float v) { return 1.f / (1.f + expf(-v)); }

// BCNorm: row (token, group, rank) of B (which = 0) or C (which = 1).
__global__ __launch_bounds__(64 * kWaves) void bcnorm_kernel(BlockArgs a) {
    const int lane = threadIdx.x & 63;
    const long long rows = (long long)a.b * a.L * a.G * a.R;
    const long long ri = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (ri >= 2 * rows) return;
    const int which = (int)(ri & 1);
    const size_t row = (size_t)(ri >> 1);
    const void* src = which ? a.Craw : a.Braw;
    void* dst = which ? a.Cn : a.Bn;
    const float* gain = which ? a.Cg : a.Bg;
    const int N = a.N;
    float v[4];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int n = lane + 64 * k;
        v[k] = n < N ? ld_io(src, row * N + n, a.io_bf16) : 0.f;
        ss += v[k] * v[k];
    }
    ss = wave_sum(ss);
    const float sc = 1.f / sqrtf(ss / (float)N + a.eps);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int n = lane + 64 * k;
        if (n < N) st_io(dst, row * N + n, v[k] * sc * (gain ? gain[n] : 1.f), a.io_bf16);
    }
}

// Per (token, head): the scalars, the angular rates and the lifted x.
__global__ __launch_bounds__(64 * kWaves) void prologue_kernel(BlockArgs a) {
    const int lane = threadIdx.x & 63;
    const long long th_ = (long long)a.b * a.L * a.H;
    const long long ti = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);     // token * H + head
    if (ti >= th_) return;
    const int h = (int)(ti % a.H);
    if (lane == 0) {
        a.dt[ti] = softplus(a.dt_raw[ti] + (a.dt_bias ? a.dt_bias[h] : 0.f));
        a.lam[ti] = sigmoid(a.lam_raw[ti]);
    }
    for (int i = lane; i < a.np; i += 64) a.th[(size_t)ti * a.np + i] = kPi * tanhf(a.th_raw[(size_t)ti * a.np + i]);
    for (int p = lane; p < a.P; p += 64) {
        const float xv = ld_io(a.x, (size_t)ti * a.P + p, a.io_bf16);
        for (int r = 0; r < a.R; ++r)
            st_io(a.xl, ((size_t)ti * a.R + r) * a.P + p, a.lift[((size_t)h * a.R + r) * a.P + p] * xv, a.io_bf16);
    }
}

// Per (token, head): recombine the R readouts, add the skip, gate.
__global__ __launch_bounds__(64 * kWaves) void epilogue_kernel(BlockArgs a) {
    const int lane = threadIdx.x & 63;
    const long long th_ = (long long)a.b * a.L * a.H;
    const long long ti = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (ti >= th_) return;
    const int h = (int)(ti % a.H);
    const float dh = a.D ? a.D[h] : 0.f;
    for (int p = lane; p < a.P; p += 64) {
        float acc = 0.f;
        for (int r = 0; r < a.R; ++r)
            acc += a.comb[((size_t)h * a.R + r) * a.P + p] * ld_io(a.y, ((size_t)ti * a.R + r) * a.P + p, a.io_bf16);
        acc += dh * ld_io(a.x, (size_t)ti * a.P + p, a.io_bf16);
        const float zz = ld_io(a.z, (size_t)ti * a.P + p, a.io_bf16);
        st_io(a.out, (size_t)ti * a.P + p, acc * zz * sigmoid(zz), a.io_bf16);
    }
}

unsigned blocks_for(long long waves) { return (unsigned)((waves + kWaves - 1) / kWaves); }

}  // namespace

hipError_t launch_block_prologue(const BlockArgs& a, hipStream_t s) {
    const long long rows = 2LL * a.b * a.L * a.G * a.R;
    const long long toks = (long long)a.b * a.L * a.H;
    if (rows > 0) {
        hipLaunchKernelGGL(bcnorm_kernel, dim3(blocks_for(rows)), dim3(64 * kWaves), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (toks > 0) hipLaunchKernelGGL(prologue_kernel, dim3(blocks_for(toks)), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_block_epilogue(const BlockArgs& a, hipStream_t s) {
    const long long toks = (long long)a.b * a.L * a.H;
    if (toks > 0) hipLaunchKernelGGL(epilogue_kernel, dim3(blocks_for(toks)), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace m3
