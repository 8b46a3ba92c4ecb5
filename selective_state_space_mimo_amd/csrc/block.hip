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

__device__ __forceinline__ float softplus(float v) { return softplus_f(v); }
__device__ __forceinline__ float sigmoid(float v) { return sigmoid_f(v); }

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
    for (int i = lane; i < a.np; i += 64) a.th[(size_t)ti * a.np + i] = kPi * tanh_f(a.th_raw[(size_t)ti * a.np + i]);
    for (int p = lane; p < a.P && a.xl; p += 64) {
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
            acc += (a.comb ? a.comb[((size_t)h * a.R + r) * a.P + p] : 1.f) *
                   ld_io(a.y, ((size_t)ti * a.R + r) * a.P + p, a.io_bf16);
        acc += dh * ld_io(a.x, (size_t)ti * a.P + p, a.io_bf16);
        const float zz = ld_io(a.z, (size_t)ti * a.P + p, a.io_bf16);
        st_io(a.out, (size_t)ti * a.P + p, acc * zz * sigmoid(zz), a.io_bf16);
    }
}

// ---- vectorised forms: 16-byte pieces of V io elements (V = 8 bf16 or 4 f32) per lane ----
template <int V> struct Vec;
template <> struct Vec<8> {          // bf16
    typedef uint4 T;
    __device__ static void unpack(const T& t, float (&f)[8]) {
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static T pack(const float (&f)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x2 v;
            v[0] = (bf16)f[2 * i];
            v[1] = (bf16)f[2 * i + 1];
            w[i] = __builtin_bit_cast(uint32_t, v);
        }
        return T{w[0], w[1], w[2], w[3]};
    }
};
template <> struct Vec<4> {          // f32
    typedef float4 T;
    __device__ static void unpack(const T& t, float (&f)[4]) { f[0] = t.x; f[1] = t.y; f[2] = t.z; f[3] = t.w; }
    __device__ static T pack(const float (&f)[4]) { return T{f[0], f[1], f[2], f[3]}; }
};

// BCNorm, vectorised: G = N / V lanes per row, 64 / G rows per wave pass (N / V a power
// of two dividing 64), kBcPasses passes per wave over consecutive rows.  B and C rows
// alternate, and every pass covers an even number of rows, so a lane keeps one tensor
// and one piece of the row throughout: its gains are loaded once, and all of its row
// pieces are in flight together before any is reduced.
constexpr int kBcPasses = 4;
template <int V>
__global__ __launch_bounds__(64 * kWaves) void bcnorm_vec_kernel(BlockArgs a) {
    typedef typename Vec<V>::T T;
    const int lane = threadIdx.x & 63;
    const int G = a.N / V, RPW = 64 / G;
    const long long rows = (long long)a.b * a.L * a.G * a.R;
    const long long r0 = ((long long)blockIdx.x * kWaves + (threadIdx.x >> 6)) * RPW * kBcPasses + lane / G;
    const int which = (int)(r0 & 1);                          // RPW is even: the same every pass
    const int j = lane % G;                                   // piece of the row
    const T* src = reinterpret_cast<const T*>(which ? a.Craw : a.Braw);
    T* dst = reinterpret_cast<T*>(which ? a.Cn : a.Bn);
    const float* gain = which ? a.Cg : a.Bg;
    float gv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) gv[i] = gain ? gain[j * V + i] : 1.f;
    T raw[kBcPasses];
#pragma unroll
    for (int k = 0; k < kBcPasses; ++k) {
        const long long ri = r0 + (long long)k * RPW;
        raw[k] = ri < 2 * rows ? src[(size_t)(ri >> 1) * G + j] : T{};
    }
#pragma unroll
    for (int k = 0; k < kBcPasses; ++k) {
        const long long ri = r0 + (long long)k * RPW;
        float f[V];
        Vec<V>::unpack(raw[k], f);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) ss += f[i] * f[i];
        for (int o = G >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);    // within the row's lanes
        const float sc = 1.f / sqrtf(ss / (float)a.N + a.eps);
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] *= sc * gv[i];
        if (ri < 2 * rows) dst[(size_t)(ri >> 1) * G + j] = Vec<V>::pack(f);
    }
}

// Per (token, head), vectorised: the lifted x (G = P / V lanes per token-head); the
// scalars and angular rates by the first lane of each token-head.
template <int V>
__global__ __launch_bounds__(64 * kWaves) void prologue_vec_kernel(BlockArgs a) {
    typedef typename Vec<V>::T T;
    const int lane = threadIdx.x & 63;
    const int G = a.P / V, TPW = 64 / G;
    const long long nth = (long long)a.b * a.L * a.H;
    const long long ti = ((long long)blockIdx.x * kWaves + (threadIdx.x >> 6)) * TPW + lane / G;
    if (ti >= nth) return;
    const int h = (int)(ti % a.H), j = lane % G;
    if (a.dt) {                                          // (else the scan activates them itself)
        if (j == 0) {
            a.dt[ti] = softplus(a.dt_raw[ti] + (a.dt_bias ? a.dt_bias[h] : 0.f));
            a.lam[ti] = sigmoid(a.lam_raw[ti]);
        }
        for (int i = j; i < a.np; i += G) a.th[(size_t)ti * a.np + i] = kPi * tanh_f(a.th_raw[(size_t)ti * a.np + i]);
    }
    if (!a.xl) return;                                   // the scan lifts x itself
    float xv[V];
    Vec<V>::unpack(reinterpret_cast<const T*>(a.x)[(size_t)ti * G + j], xv);
    for (int r = 0; r < a.R; ++r) {
        const float* l = a.lift + ((size_t)h * a.R + r) * a.P + j * V;
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = l[i] * xv[i];
        reinterpret_cast<T*>(a.xl)[((size_t)ti * a.R + r) * G + j] = Vec<V>::pack(o);
    }
}

// Per (token, head), vectorised epilogue.
template <int V>
__global__ __launch_bounds__(64 * kWaves) void epilogue_vec_kernel(BlockArgs a) {
    typedef typename Vec<V>::T T;
    const int lane = threadIdx.x & 63;
    const int G = a.P / V, TPW = 64 / G;
    const long long nth = (long long)a.b * a.L * a.H;
    const long long ti = ((long long)blockIdx.x * kWaves + (threadIdx.x >> 6)) * TPW + lane / G;
    if (ti >= nth) return;
    const int h = (int)(ti % a.H), j = lane % G;
    const float dh = a.D ? a.D[h] : 0.f;
    float acc[V], t[V];
    Vec<V>::unpack(reinterpret_cast<const T*>(a.x)[(size_t)ti * G + j], t);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = dh * t[i];
    for (int r = 0; r < a.R; ++r) {
        Vec<V>::unpack(reinterpret_cast<const T*>(a.y)[((size_t)ti * a.R + r) * G + j], t);
        if (a.comb) {
            const float* w = a.comb + ((size_t)h * a.R + r) * a.P + j * V;
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] += w[i] * t[i];
        } else {                                         // y already recombined (R = 1)
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] += t[i];
        }
    }
    Vec<V>::unpack(reinterpret_cast<const T*>(a.z)[(size_t)ti * G + j], t);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] *= t[i] * sigmoid(t[i]);
    reinterpret_cast<T*>(a.out)[(size_t)ti * G + j] = Vec<V>::pack(acc);
}

// The vectorised forms need the row (N) and token-head (P) widths to be whole numbers
// of 16-byte pieces whose count per row divides the wave.
bool pow2_divides_64(int g) { return g >= 1 && g <= 64 && (g & (g - 1)) == 0; }
int vec_width(const BlockArgs& a) { return a.io_bf16 ? 8 : 4; }
bool vec_ok(const BlockArgs& a, int n) {
    const int v = vec_width(a);
    return n % v == 0 && pow2_divides_64(n / v);
}

unsigned blocks_for(long long waves) { return (unsigned)((waves + kWaves - 1) / kWaves); }

}  // namespace

hipError_t launch_block_prologue(const BlockArgs& a, hipStream_t s) {
    const long long rows = 2LL * a.b * a.L * a.G * a.R;
    const long long toks = (long long)a.b * a.L * a.H;
    const int v = vec_width(a);
    if (rows > 0) {
        if (vec_ok(a, a.N) && a.N / v <= 32) {          // (an even number of rows per pass)
            const long long rpw = (64 / (a.N / v)) * kBcPasses;    // rows (B and C) per wave
            const long long waves = (rows + rpw - 1) / rpw;
            if (v == 8) hipLaunchKernelGGL(bcnorm_vec_kernel<8>, dim3(blocks_for(waves)), dim3(64 * kWaves), 0, s, a);
            else hipLaunchKernelGGL(bcnorm_vec_kernel<4>, dim3(blocks_for(waves)), dim3(64 * kWaves), 0, s, a);
        } else {
            hipLaunchKernelGGL(bcnorm_kernel, dim3(blocks_for(rows)), dim3(64 * kWaves), 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (toks > 0 && (a.dt || a.xl)) {
        if (vec_ok(a, a.P)) {
            const int tpw = 64 / (a.P / v);
            if (v == 8) hipLaunchKernelGGL(prologue_vec_kernel<8>, dim3(blocks_for((toks + tpw - 1) / tpw)), dim3(64 * kWaves), 0, s, a);
            else hipLaunchKernelGGL(prologue_vec_kernel<4>, dim3(blocks_for((toks + tpw - 1) / tpw)), dim3(64 * kWaves), 0, s, a);
        } else {
            hipLaunchKernelGGL(prologue_kernel, dim3(blocks_for(toks)), dim3(64 * kWaves), 0, s, a);
        }
    }
    return hipGetLastError();
}

hipError_t launch_block_epilogue(const BlockArgs& a, hipStream_t s) {
    const long long toks = (long long)a.b * a.L * a.H;
    const int v = vec_width(a);
    if (toks > 0) {
        if (vec_ok(a, a.P)) {
            const int tpw = 64 / (a.P / v);
            if (v == 8) hipLaunchKernelGGL(epilogue_vec_kernel<8>, dim3(blocks_for((toks + tpw - 1) / tpw)), dim3(64 * kWaves), 0, s, a);
            else hipLaunchKernelGGL(epilogue_vec_kernel<4>, dim3(blocks_for((toks + tpw - 1) / tpw)), dim3(64 * kWaves), 0, s, a);
        } else {
            hipLaunchKernelGGL(epilogue_kernel, dim3(blocks_for(toks)), dim3(64 * kWaves), 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace m3
