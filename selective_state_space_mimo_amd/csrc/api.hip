// Host side of the C ABI declared in include/m3scan.h: argument checking,
// schedule choice and kernel dispatch.  Every check runs before the first
// HIP call, so a call that returns an argument error has launched nothing.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/m3scan.h"
#include "m3_internal.h"

using namespace m3;

namespace {

constexpr uintptr_t kAlign = 16;

// Device scratch of m3_scan_fwd_noalloc: the segmented schedule's workspace for
// callers that cannot allocate.  Each GPU the library runs on holds one copy until
// the process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not a device address): scratch_address() looks up each
// device's address once with hipGetSymbolAddress and keeps it.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// The current device's address of `scratch` (looked up on the first call on that device).
m3_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return M3_ERR_HIP;
    if (dev >= kMaxDevices) return M3_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return M3_ERR_HIP;
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return M3_OK;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) % kAlign) != 0; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};
Range rng(const void* p, size_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

size_t esize(m3_dtype t) { return t == M3_BF16 ? 2 : 4; }

m3_status check_desc(const m3_desc* d, bool scan) {
    if (!d) return M3_ERR_INVALID_ARG;
    if (d->batch < 1 || d->nheads < 1 || d->ngroups < 1 || d->nheads % d->ngroups) return M3_ERR_INVALID_ARG;
    if (d->headdim < 1 || d->dstate < 2 || (d->dstate & 1) || d->rank < 1) return M3_ERR_INVALID_ARG;
    if (d->npairs < 0 || 2 * d->npairs > d->dstate) return M3_ERR_INVALID_ARG;
    if ((d->io_dtype != M3_F32 && d->io_dtype != M3_BF16) ||
        (d->state_dtype != M3_F32 && d->state_dtype != M3_BF16))
        return M3_ERR_INVALID_ARG;
    if (scan && (d->seqlen < 0 || d->chunk < 1 || d->nsegments < 0)) return M3_ERR_INVALID_ARG;
    if (d->rate_law != M3_RATE_STATIC && d->rate_law != M3_RATE_HEAVY_TAIL) return M3_ERR_INVALID_ARG;
    if (d->headdim > 256 || d->dstate > 256 || d->rank > 8) return M3_ERR_UNSUPPORTED;
    if (scan && d->chunk > 256) return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

// Tensor sizes (bytes) of one call.
struct Sizes {
    size_t x, bc, tok, theta, alog, bias, h, phi, bp, xp;
};
Sizes sizes(const m3_desc* d, long long L) {
    const size_t b = d->batch, H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, R = d->rank,
                 np = d->npairs, io = esize(d->io_dtype), st = esize(d->state_dtype);
    Sizes s;
    s.x = b * L * H * R * P * io;
    s.bc = b * L * G * R * N * io;
    s.tok = b * L * H * 4;
    s.theta = b * L * H * np * 4;
    s.alog = d->rate_law == M3_RATE_HEAVY_TAIL ? b * L * H * 4 : H * 4;
    s.bias = H * R * N * 4;
    s.h = b * H * P * N * st;
    s.phi = b * H * np * 4;
    s.bp = b * H * R * N * io;
    s.xp = b * H * R * P * io;
    return s;
}

m3_status check_carry(const m3_carry* c, const m3_desc* d) {
    if (!c->h || !c->B_prev || !c->x_prev) return M3_ERR_INVALID_ARG;
    if (d->npairs > 0 && !c->phi) return M3_ERR_INVALID_ARG;
    if (misaligned(c->h) || misaligned(c->phi) || misaligned(c->B_prev) || misaligned(c->x_prev))
        return M3_ERR_ALIGNMENT;
    return M3_OK;
}

void carry_ranges(const m3_carry* c, const Sizes& s, Range out[4]) {
    out[0] = rng(c->h, s.h);
    out[1] = rng(c->phi, c->phi ? s.phi : 0);
    out[2] = rng(c->B_prev, s.bp);
    out[3] = rng(c->x_prev, s.xp);
}

// Schedule: number of sequence segments per (batch, head) stream and their
// length in tokens (a multiple of the chunk).
void choose_segments(const m3_desc* d, int Q, int* nseg, int* seglen) {
    const int L = d->seqlen;
    const int nchunks = (L + Q - 1) / Q;
    int k = d->nsegments;
    if (k == 0) {
        // When the (batch, head) streams alone cannot fill the compute units' workgroup
        // slots (256 units, each holding one or two of the scan's workgroups), split each
        // stream into just enough segments to fill them: every further segment costs a
        // summary pass and a re-evaluation, and a partial wave of workgroups a tail.
        const long long streams = (long long)d->batch * d->nheads;
        const long long slots = 256LL * scan_mfma_groups_per_cu(d->rank, Q);
        k = streams >= slots ? 1 : (int)((slots + streams - 1) / streams);
    }
    k = std::max(1, std::min(k, std::max(1, nchunks)));
    const int cps = (nchunks + k - 1) / k;       // chunks per segment
    *seglen = cps * Q;
    *nseg = std::max(1, (L + *seglen - 1) / *seglen);
}

ScanArgs make_scan_args(const m3_desc* d, const void* x, const void* B, const void* C, const float* dt,
                        const float* lam, const float* theta, const float* A_log, const float* Bb,
                        const float* Cb, const m3_carry* init, void* y, const m3_carry* fin) {
    ScanArgs a{};
    a.b = d->batch; a.L = d->seqlen; a.H = d->nheads; a.G = d->ngroups; a.P = d->headdim;
    a.N = d->dstate; a.R = d->rank; a.np = d->npairs;
    a.io_bf16 = d->io_dtype == M3_BF16; a.st_bf16 = d->state_dtype == M3_BF16;
    a.Q = scan_mfma_chunk(a.io_bf16, a.P, a.N, a.R, d->chunk);
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.lam = lam; a.theta = d->npairs ? theta : nullptr;
    a.A_log = A_log; a.rate_law = d->rate_law; a.Bb = Bb; a.Cb = Cb;
    if (init) { a.h0 = init->h; a.phi0 = d->npairs ? init->phi : nullptr; a.Bp0 = init->B_prev; a.xp0 = init->x_prev; }
    a.y = y;
    if (fin) { a.h1 = fin->h; a.phi1 = d->npairs ? fin->phi : nullptr; a.Bp1 = fin->B_prev; a.xp1 = fin->x_prev; }
    choose_segments(d, a.Q, &a.nseg, &a.seglen);
    return a;
}

// ---- L == 0: final carry = initial carry (zeros without one) -----------------------
__global__ void copy_or_zero_kernel(const uint16_t* src, uint16_t* dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : (uint16_t)0;
}
hipError_t copy_or_zero(const void* src, void* dst, size_t bytes, hipStream_t s) {
    if (!dst || bytes == 0) return hipSuccess;
    const size_t n = bytes / 2;   // every carry tensor holds whole 2-byte units
    const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)src, (uint16_t*)dst, n);
    return hipGetLastError();
}

// Workspace of the layer entry points: the scan's inputs (lifted x, normalised B
// and C, dt, lambda, angular rates), its readouts and its own workspace, each part
// starting on a 256-byte boundary.
struct BlockWs {
    bool fused;     // the matrix-core scan runs the layer steps itself (see m3_block_fwd)
    size_t xl, bn, cn, dt, lam, th, y, scan, scan_bytes, total;
};
// Whether m3_block_fwd takes the fused path for *d: the matrix-core scan lifts x and
// activates dt, lambda, theta as it stages them and writes the recombined readout.
bool block_fused(const m3_desc* d) {
    if (d->seqlen < 1) return false;
    const ScanArgs a = make_scan_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      nullptr, nullptr, nullptr, nullptr);
    return a.io_bf16 && scan_mfma_supported(a) && a.Q <= 64;
}
BlockWs block_ws(const m3_desc* d, int decode) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t L = decode ? 1 : (size_t)d->seqlen;
    const size_t b = d->batch, H = d->nheads, G = d->ngroups, P = d->headdim, N = d->dstate, R = d->rank,
                 np = d->npairs, io = esize(d->io_dtype);
    BlockWs w{};
    w.fused = !decode && block_fused(d);
    // the fused path needs neither the lifted rows nor the activated inputs nor the readouts
    // (the scan writes the layer's output)
    const size_t Rl = w.fused ? 0 : R, Ry = w.fused ? 0 : R, Lt = w.fused ? 0 : L;
    size_t o = 0;
    w.xl = o;  o += up(b * L * H * Rl * P * io);
    w.bn = o;  o += up(b * L * G * R * N * io);
    w.cn = o;  o += up(b * L * G * R * N * io);
    w.dt = o;  o += up(b * Lt * H * 4);
    w.lam = o; o += up(b * Lt * H * 4);
    w.th = o;  o += up(b * Lt * H * np * 4);
    w.y = o;   o += up(b * L * H * Ry * P * io);
    w.scan = o;
    w.scan_bytes = 0;
    if (!decode && L > 0) {
        ScanArgs a = make_scan_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, nullptr);
        if (a.io_bf16 && scan_mfma_supported(a)) w.scan_bytes = scan_mfma_workspace_bytes(a);
    }
    w.total = o + w.scan_bytes;
    return w;
}

// Checks shared by the two layer entry points (pointers, alignment, parameters,
// workspace size, overlaps of the output and the workspace with the inputs).
m3_status check_block(const m3_desc* d, const m3_block_params* p, int decode, const void* z, const void* x,
                      const void* Braw, const void* Craw, const float* dt_raw, const float* A,
                      const float* lam_raw, const float* th_raw, const void* out, const void* ws, size_t wsb) {
    if (!p || !p->lift || !p->comb || !(p->eps > 0.f) || !(p->eps < 1e30f)) return M3_ERR_INVALID_ARG;
    if (!z || !x || !Braw || !Craw || !dt_raw || !A || !lam_raw || !out) return M3_ERR_INVALID_ARG;
    if (d->npairs > 0 && !th_raw) return M3_ERR_INVALID_ARG;
    const void* ptrs[] = {z, x, Braw, Craw, dt_raw, A, lam_raw, d->npairs ? th_raw : nullptr, out, ws,
                          p->dt_bias, p->B_gain, p->C_gain, p->B_bias, p->C_bias, p->lift, p->comb, p->D};
    for (const void* q : ptrs)
        if (misaligned(q)) return M3_ERR_ALIGNMENT;
    const BlockWs w = block_ws(d, decode);
    if (w.total > 0 && (!ws || wsb < w.total)) return M3_ERR_INVALID_ARG;
    const Sizes s = sizes(d, decode ? 1 : d->seqlen);
    const size_t io = esize(d->io_dtype);
    const size_t zx = s.x / d->rank;                      // [b, L, H, P]
    (void)io;
    const Range ro = rng(out, zx), rw = rng(ws, w.total);
    const Range ins[] = {rng(z, zx), rng(x, zx), rng(Braw, s.bc), rng(Craw, s.bc), rng(dt_raw, s.tok), rng(A, s.alog),
                         rng(lam_raw, s.tok), rng(d->npairs ? th_raw : nullptr, d->npairs ? s.theta : 0)};
    for (const Range& r : ins)
        if (overlap(ro, r) || overlap(rw, r)) return M3_ERR_INVALID_ARG;
    if (overlap(ro, rw)) return M3_ERR_INVALID_ARG;
    return M3_OK;
}

BlockArgs make_block_args(const m3_desc* d, const m3_block_params* p, int L, const void* z, const void* x,
                          const void* Braw, const void* Craw, const float* dt_raw, const float* lam_raw,
                          const float* th_raw, void* out, void* ws, const BlockWs& w) {
    BlockArgs a{};
    a.b = d->batch; a.L = L; a.H = d->nheads; a.G = d->ngroups; a.P = d->headdim; a.N = d->dstate;
    a.R = d->rank; a.np = d->npairs; a.io_bf16 = d->io_dtype == M3_BF16;
    a.z = z; a.x = x; a.Braw = Braw; a.Craw = Craw; a.dt_raw = dt_raw; a.lam_raw = lam_raw;
    a.th_raw = d->npairs ? th_raw : nullptr;
    a.dt_bias = p->dt_bias; a.Bg = p->B_gain; a.Cg = p->C_gain; a.lift = p->lift; a.comb = p->comb; a.D = p->D;
    a.eps = p->eps;
    char* base = static_cast<char*>(ws);
    a.xl = base + w.xl; a.Bn = base + w.bn; a.Cn = base + w.cn;
    a.dt = reinterpret_cast<float*>(base + w.dt); a.lam = reinterpret_cast<float*>(base + w.lam);
    a.th = reinterpret_cast<float*>(base + w.th);
    a.y = base + w.y;
    a.out = out;
    return a;
}

}  // namespace

extern "C" {

const char* m3_status_string(m3_status s) {
    switch (s) {
        case M3_OK: return "ok";
        case M3_ERR_INVALID_ARG: return "invalid argument";
        case M3_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case M3_ERR_ALIGNMENT: return "tensor base not 16-byte aligned";
        case M3_ERR_HIP: return "HIP runtime error";
        case M3_ERR_TOO_LARGE: return "schedule needs more than the no-allocation scratch (64 MiB per GPU)";
    }
    return "unknown status";
}

int m3_version(void) { return (0 << 16) | (1 << 8) | 0; }

m3_status m3_scan_workspace_size(const m3_desc* d, size_t* bytes) {
    if (!bytes) return M3_ERR_INVALID_ARG;
    m3_status st = check_desc(d, true);
    if (st != M3_OK) return st;
    *bytes = 0;
    if (d->seqlen == 0) return M3_OK;
    ScanArgs a = make_scan_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr);
    // (the biases are not part of the descriptor: a shape the single-rank path takes
    // without them gets room for either path)
    if (a.io_bf16 && scan_mfma_supported(a)) *bytes = scan_mfma_workspace_bytes(a);
    if (scan_siso_supported(a)) *bytes = std::max(*bytes, scan_siso_workspace_bytes(a));
    return M3_OK;
}

}  // extern "C"

namespace {

// m3_scan_fwd, or with use_scratch m3_scan_fwd_noalloc (the workspace argument is
// ignored and the segmented schedule runs in the device scratch).
m3_status scan_fwd_impl(const m3_desc* d, const void* x, const void* B, const void* C, const float* dt,
                        const float* lam, const float* theta, const float* A_log, const float* B_bias,
                        const float* C_bias, const m3_carry* init, void* y, const m3_carry* final_,
                        void* workspace, size_t workspace_bytes, m3_stream_t stream, bool use_scratch) {
    m3_status st = check_desc(d, true);
    if (st != M3_OK) return st;
    const int L = d->seqlen;
    if (init && (st = check_carry(init, d)) != M3_OK) return st;
    if (final_ && (st = check_carry(final_, d)) != M3_OK) return st;
    const Sizes s = sizes(d, L);
    Range ri[4], rf[4];
    if (init) carry_ranges(init, s, ri);
    if (final_) {
        carry_ranges(final_, s, rf);
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j)
                if (init && overlap(rf[i], ri[j])) return M3_ERR_INVALID_ARG;
        for (int i = 0; i < 4; ++i)
            for (int j = i + 1; j < 4; ++j)
                if (overlap(rf[i], rf[j])) return M3_ERR_INVALID_ARG;
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (L == 0) {
        if (!final_) return M3_OK;
        const Sizes s1 = sizes(d, 0);
        hipError_t e = copy_or_zero(init ? init->h : nullptr, final_->h, s1.h, hs);
        if (e == hipSuccess && d->npairs) e = copy_or_zero(init ? init->phi : nullptr, final_->phi, s1.phi, hs);
        if (e == hipSuccess) e = copy_or_zero(init ? init->B_prev : nullptr, final_->B_prev, s1.bp, hs);
        if (e == hipSuccess) e = copy_or_zero(init ? init->x_prev : nullptr, final_->x_prev, s1.xp, hs);
        return e == hipSuccess ? M3_OK : M3_ERR_HIP;
    }
    if (!x || !B || !C || !dt || !lam || !A_log || !y) return M3_ERR_INVALID_ARG;
    if (d->npairs > 0 && !theta) return M3_ERR_INVALID_ARG;
    const void* ptrs[] = {x, B, C, dt, lam, d->npairs ? theta : nullptr, A_log, B_bias, C_bias, y, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return M3_ERR_ALIGNMENT;
    const Range ry = rng(y, s.x);
    const Range ins[] = {rng(x, s.x), rng(B, s.bc), rng(C, s.bc), rng(dt, s.tok), rng(lam, s.tok),
                         rng(d->npairs ? theta : nullptr, d->npairs ? s.theta : 0), rng(A_log, s.alog),
                         rng(B_bias, B_bias ? s.bias : 0), rng(C_bias, C_bias ? s.bias : 0)};
    for (const Range& r : ins)
        if (overlap(ry, r)) return M3_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i) {
        if (init && overlap(ry, ri[i])) return M3_ERR_INVALID_ARG;
        if (final_ && overlap(ry, rf[i])) return M3_ERR_INVALID_ARG;
        // the final carry is written while other workgroups still read the inputs
        if (final_)
            for (const Range& r : ins)
                if (overlap(rf[i], r)) return M3_ERR_INVALID_ARG;
    }

    ScanArgs a = make_scan_args(d, x, B, C, dt, lam, theta, A_log, B_bias, C_bias, init, y, final_);
    hipError_t e;
    const bool siso = scan_siso_supported(a);
    if (siso || (a.io_bf16 && scan_mfma_supported(a))) {
        const size_t need = siso ? scan_siso_workspace_bytes(a) : scan_mfma_workspace_bytes(a);
        if (use_scratch) {
            // every summary, incoming state and phase is written before it is read, so the
            // scratch needs no clearing; what a previous call left there does not matter
            if (need > kScratchBytes) return M3_ERR_TOO_LARGE;
            workspace = nullptr;
            if (need > 0 && (st = scratch_address(&workspace)) != M3_OK) return st;
        } else if (need > 0) {
            if (!workspace || workspace_bytes < need) return M3_ERR_INVALID_ARG;
            const Range rw = rng(workspace, need);
            for (const Range& r : ins)
                if (overlap(rw, r)) return M3_ERR_INVALID_ARG;
            if (overlap(rw, ry)) return M3_ERR_INVALID_ARG;
            for (int i = 0; i < 4; ++i)
                if ((init && overlap(rw, ri[i])) || (final_ && overlap(rw, rf[i]))) return M3_ERR_INVALID_ARG;
        }
        a.ws = static_cast<float*>(workspace);
        e = siso ? launch_scan_siso(a, hs) : launch_scan_mfma(a, hs);
    } else {
        if (scan_generic_chunk(a.P, a.N, a.R, a.np, a.Q) < 1) return M3_ERR_UNSUPPORTED;
        e = launch_scan_generic(a, hs);
    }
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // namespace

extern "C" {

m3_status m3_scan_fwd(const m3_desc* d, const void* x, const void* B, const void* C, const float* dt,
                      const float* lam, const float* theta, const float* A_log, const float* B_bias,
                      const float* C_bias, const m3_carry* init, void* y, const m3_carry* final_,
                      void* workspace, size_t workspace_bytes, m3_stream_t stream) {
    return scan_fwd_impl(d, x, B, C, dt, lam, theta, A_log, B_bias, C_bias, init, y, final_, workspace,
                         workspace_bytes, stream, false);
}

m3_status m3_scan_fwd_noalloc(const m3_desc* d, const void* x, const void* B, const void* C, const float* dt,
                              const float* lam, const float* theta, const float* A_log, const float* B_bias,
                              const float* C_bias, const m3_carry* init, void* y, const m3_carry* final_,
                              m3_stream_t stream) {
    return scan_fwd_impl(d, x, B, C, dt, lam, theta, A_log, B_bias, C_bias, init, y, final_, nullptr, 0, stream,
                         true);
}

size_t m3_scan_noalloc_max_workspace(void) { return kScratchBytes; }

m3_status m3_decode_step(const m3_desc* d, const void* x, const void* B, const void* C, const float* dt,
                         const float* lam, const float* theta, const float* A_log, const float* B_bias,
                         const float* C_bias, const m3_carry* carry, void* y, m3_stream_t stream) {
    m3_status st = check_desc(d, false);
    if (st != M3_OK) return st;
    if (!carry || !x || !B || !C || !dt || !lam || !A_log || !y) return M3_ERR_INVALID_ARG;
    if (d->npairs > 0 && !theta) return M3_ERR_INVALID_ARG;
    if ((st = check_carry(carry, d)) != M3_OK) return st;
    const void* ptrs[] = {x, B, C, dt, lam, d->npairs ? theta : nullptr, A_log, B_bias, C_bias, y};
    for (const void* p : ptrs)
        if (misaligned(p)) return M3_ERR_ALIGNMENT;
    const Sizes s = sizes(d, 1);
    Range rc[4];
    carry_ranges(carry, s, rc);
    const Range ry = rng(y, s.x);
    const Range ins[] = {rng(x, s.x), rng(B, s.bc), rng(C, s.bc), rng(dt, s.tok), rng(lam, s.tok),
                         rng(d->npairs ? theta : nullptr, d->npairs ? s.theta : 0), rng(A_log, s.alog),
                         rng(B_bias, B_bias ? s.bias : 0), rng(C_bias, C_bias ? s.bias : 0)};
    for (const Range& r : ins) {
        if (overlap(ry, r)) return M3_ERR_INVALID_ARG;
        for (int i = 0; i < 4; ++i)
            if (overlap(rc[i], r)) return M3_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 4; ++i) {
        if (overlap(ry, rc[i])) return M3_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(rc[i], rc[j])) return M3_ERR_INVALID_ARG;
    }

    DecodeArgs a{};
    a.b = d->batch; a.H = d->nheads; a.G = d->ngroups; a.P = d->headdim; a.N = d->dstate; a.R = d->rank;
    a.np = d->npairs; a.io_bf16 = d->io_dtype == M3_BF16; a.st_bf16 = d->state_dtype == M3_BF16;
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.lam = lam; a.theta = d->npairs ? theta : nullptr; a.A_log = A_log;
    a.rate_law = d->rate_law;
    a.Bb = B_bias; a.Cb = C_bias;
    a.h = carry->h; a.phi = d->npairs ? carry->phi : nullptr; a.Bp = carry->B_prev; a.xp = carry->x_prev;
    a.y = y;
    hipError_t e;
    if (decode_fast_supported(a)) {
        e = launch_decode_fast(a, reinterpret_cast<hipStream_t>(stream));
    } else {
        if (scan_generic_chunk(a.P, a.N, a.R, a.np, 1) < 1) return M3_ERR_UNSUPPORTED;
        e = launch_decode_generic(a, reinterpret_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status m3_block_workspace_size(const m3_desc* d, int decode, size_t* bytes) {
    if (!bytes) return M3_ERR_INVALID_ARG;
    m3_status st = check_desc(d, !decode);
    if (st != M3_OK) return st;
    *bytes = block_ws(d, decode).total;
    return M3_OK;
}

m3_status m3_block_fwd(const m3_desc* d, const m3_block_params* p, const void* z, const void* x,
                       const void* B_raw, const void* C_raw, const float* dt_raw, const float* A,
                       const float* lam_raw, const float* th_raw, const m3_carry* init, void* out,
                       const m3_carry* final_, void* workspace, size_t workspace_bytes, m3_stream_t stream) {
    m3_status st = check_desc(d, true);
    if (st != M3_OK) return st;
    if (d->seqlen == 0)      // nothing but the carry copy
        return m3_scan_fwd(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           init, nullptr, final_, nullptr, 0, stream);
    if ((st = check_block(d, p, 0, z, x, B_raw, C_raw, dt_raw, A, lam_raw, th_raw, out, workspace,
                          workspace_bytes)) != M3_OK)
        return st;
    if (init && (st = check_carry(init, d)) != M3_OK) return st;
    if (final_) {
        if ((st = check_carry(final_, d)) != M3_OK) return st;
        const Sizes cs = sizes(d, d->seqlen);
        Range ri[4], rf[4];
        carry_ranges(final_, cs, rf);
        if (init) carry_ranges(init, cs, ri);
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j)
                if ((init && overlap(rf[i], ri[j])) || (j > i && overlap(rf[i], rf[j]))) return M3_ERR_INVALID_ARG;
        // nor the raw inputs, the output or the workspace (written while they are read)
        const size_t zx = cs.x / d->rank;
        const Range others[] = {rng(z, zx), rng(x, zx), rng(B_raw, cs.bc), rng(C_raw, cs.bc), rng(dt_raw, cs.tok),
                                rng(A, cs.alog), rng(lam_raw, cs.tok), rng(d->npairs ? th_raw : nullptr,
                                                                             d->npairs ? cs.theta : 0),
                                rng(out, zx), rng(workspace, block_ws(d, 0).total)};
        for (int i = 0; i < 4; ++i)
            for (const Range& r : others)
                if (overlap(rf[i], r)) return M3_ERR_INVALID_ARG;
    }
    const BlockWs w = block_ws(d, 0);
    BlockArgs a = make_block_args(d, p, d->seqlen, z, x, B_raw, C_raw, dt_raw, lam_raw, th_raw, out, workspace, w);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    // The matrix-core scan lifts x as it fetches the rows and activates the raw step,
    // blend and angle inputs as it stages them; elsewhere the prologue writes the lifted
    // rows and the activated inputs and the scan reads them.  BCNorm always runs first
    // (B and C are shared by the heads of a group).
    ScanArgs sa = make_scan_args(d, x, a.Bn, a.Cn, dt_raw, lam_raw, d->npairs ? th_raw : nullptr, A, p->B_bias,
                                 p->C_bias, init, base + w.y, final_);
    const bool fused = w.fused;
    if (fused) {
        a.xl = nullptr;
        a.dt = a.lam = a.th = nullptr;
    }
    if (launch_block_prologue(a, hs) != hipSuccess) return M3_ERR_HIP;
    if (fused) {
        // the scan recombines the readouts, adds the skip and applies the gate as it stores
        // each token's row: it writes the layer's output, and no epilogue runs
        sa.lift = p->lift;
        sa.dt_bias = p->dt_bias;
        sa.comb = p->comb;
        sa.gate = z;
        sa.dskip = p->D;
        sa.y = out;
        sa.ws = w.scan_bytes ? reinterpret_cast<float*>(base + w.scan) : nullptr;
        return launch_scan_mfma(sa, hs) == hipSuccess ? M3_OK : M3_ERR_HIP;
    } else {
        st = m3_scan_fwd(d, a.xl, a.Bn, a.Cn, a.dt, a.lam, d->npairs ? a.th : nullptr, A, p->B_bias, p->C_bias,
                         init, base + w.y, final_, w.scan_bytes ? base + w.scan : nullptr, w.scan_bytes, stream);
        if (st != M3_OK) return st;
    }
    return launch_block_epilogue(a, hs) == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status m3_block_decode_step(const m3_desc* d, const m3_block_params* p, const void* z, const void* x,
                               const void* B_raw, const void* C_raw, const float* dt_raw, const float* A,
                               const float* lam_raw, const float* th_raw, const m3_carry* carry, void* out,
                               void* workspace, size_t workspace_bytes, m3_stream_t stream) {
    m3_status st = check_desc(d, false);
    if (st != M3_OK) return st;
    if (!carry) return M3_ERR_INVALID_ARG;
    if ((st = check_block(d, p, 1, z, x, B_raw, C_raw, dt_raw, A, lam_raw, th_raw, out, workspace,
                          workspace_bytes)) != M3_OK)
        return st;
    const BlockWs w = block_ws(d, 1);
    const BlockArgs a = make_block_args(d, p, 1, z, x, B_raw, C_raw, dt_raw, lam_raw, th_raw, out, workspace, w);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (launch_block_prologue(a, hs) != hipSuccess) return M3_ERR_HIP;
    char* base = static_cast<char*>(workspace);
    st = m3_decode_step(d, a.xl, a.Bn, a.Cn, a.dt, a.lam, d->npairs ? a.th : nullptr, A, p->B_bias, p->C_bias,
                        carry, base + w.y, stream);
    if (st != M3_OK) return st;
    return launch_block_epilogue(a, hs) == hipSuccess ? M3_OK : M3_ERR_HIP;
}

m3_status m3_scan_bwd_workspace_size(const m3_desc* d, size_t* bytes) {
    if (!bytes) return M3_ERR_INVALID_ARG;
    m3_status st = check_desc(d, true);
    if (st != M3_OK) return st;
    if (!scan_bwd_supported(d->headdim, d->dstate, d->rank, d->npairs)) return M3_ERR_UNSUPPORTED;
    const bool chunked = scan_bwd_chunked_eligible(d->io_dtype == M3_BF16, d->headdim, d->dstate, d->rank, d->npairs,
                                                   d->seqlen);
    *bytes = d->seqlen == 0 ? 0
                            : scan_bwd_workspace(d->batch, d->seqlen, d->nheads, d->ngroups, d->rank, d->dstate,
                                                 d->npairs, chunked).total;
    return M3_OK;
}

m3_status m3_scan_bwd(const m3_desc* d, const void* x, const void* B, const void* C, const float* dt,
                      const float* lam, const float* theta, const float* A_log, const float* B_bias,
                      const float* C_bias, const m3_carry* init, const void* dy, const m3_carry_grad* dfinal,
                      const m3_scan_grads* g, void* workspace, size_t workspace_bytes, m3_stream_t stream) {
    m3_status st = check_desc(d, true);
    if (st != M3_OK) return st;
    if (!scan_bwd_supported(d->headdim, d->dstate, d->rank, d->npairs)) return M3_ERR_UNSUPPORTED;
    if (!g) return M3_ERR_INVALID_ARG;
    const int L = d->seqlen;
    const size_t b = d->batch, H = d->nheads, P = d->headdim, N = d->dstate, R = d->rank, np = d->npairs;
    const Sizes s = sizes(d, L);
    if (init && (st = check_carry(init, d)) != M3_OK) return st;
    if (L > 0) {
        if (!x || !B || !C || !dt || !lam || !A_log || !dy) return M3_ERR_INVALID_ARG;
        if (np > 0 && !theta) return M3_ERR_INVALID_ARG;
        if (!g->dx || !g->dB || !g->dC || !g->ddt || !g->dlam || !g->dA) return M3_ERR_INVALID_ARG;
        if (np > 0 && !g->dtheta) return M3_ERR_INVALID_ARG;
    }
    const m3_carry_grad zero{};
    const m3_carry_grad& df = dfinal ? *dfinal : zero;
    const void* ptrs[] = {x, B, C, dt, lam, np ? theta : nullptr, A_log, B_bias, C_bias, dy, workspace,
                          g->dx, g->dB, g->dC, g->ddt, g->dlam, np ? g->dtheta : nullptr, g->dA, g->dB_bias,
                          g->dC_bias, g->dinit.h, g->dinit.phi, g->dinit.B_prev, g->dinit.x_prev,
                          df.h, df.phi, df.B_prev, df.x_prev};
    for (const void* p : ptrs)
        if (misaligned(p)) return M3_ERR_ALIGNMENT;
    // inputs (forward inputs, init carry, dy, dfinal) and outputs (every gradient, workspace)
    const size_t f4 = 4;
    const bool chunked = scan_bwd_chunked_eligible(d->io_dtype == M3_BF16, d->headdim, d->dstate, d->rank, np, L);
    const BwdWs w = scan_bwd_workspace(d->batch, L, d->nheads, d->ngroups, d->rank, d->dstate, d->npairs, chunked);
    const size_t wsb = L > 0 ? w.total : 0;
    if (wsb > 0 && (!workspace || workspace_bytes < wsb)) return M3_ERR_INVALID_ARG;
    Range ri[4] = {};
    if (init) carry_ranges(init, s, ri);
    const Range ins[] = {rng(x, s.x), rng(B, s.bc), rng(C, s.bc), rng(dt, s.tok), rng(lam, s.tok),
                         rng(np ? theta : nullptr, np ? s.theta : 0), rng(A_log, s.alog),
                         rng(B_bias, B_bias ? s.bias : 0), rng(C_bias, C_bias ? s.bias : 0), rng(dy, s.x),
                         ri[0], ri[1], ri[2], ri[3],
                         rng(df.h, df.h ? b * H * P * N * f4 : 0), rng(df.phi, df.phi ? b * H * np * f4 : 0),
                         rng(df.B_prev, df.B_prev ? b * H * R * N * f4 : 0),
                         rng(df.x_prev, df.x_prev ? b * H * R * P * f4 : 0)};
    const Range outs[] = {rng(g->dx, g->dx ? s.x : 0), rng(g->dB, g->dB ? s.bc : 0), rng(g->dC, g->dC ? s.bc : 0),
                          rng(g->ddt, g->ddt ? s.tok : 0), rng(g->dlam, g->dlam ? s.tok : 0),
                          rng(np ? g->dtheta : nullptr, np && g->dtheta ? s.theta : 0),
                          rng(g->dA, g->dA ? s.alog : 0), rng(g->dB_bias, g->dB_bias ? s.bias : 0),
                          rng(g->dC_bias, g->dC_bias ? s.bias : 0),
                          rng(g->dinit.h, g->dinit.h ? b * H * P * N * f4 : 0),
                          rng(g->dinit.phi, g->dinit.phi ? b * H * np * f4 : 0),
                          rng(g->dinit.B_prev, g->dinit.B_prev ? b * H * R * N * f4 : 0),
                          rng(g->dinit.x_prev, g->dinit.x_prev ? b * H * R * P * f4 : 0), rng(workspace, wsb)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return M3_ERR_INVALID_ARG;
        for (size_t k = i + 1; k < sizeof(outs) / sizeof(outs[0]); ++k)
            if (overlap(outs[i], outs[k])) return M3_ERR_INVALID_ARG;
    }

    BwdArgs a{};
    a.b = d->batch; a.L = L; a.H = d->nheads; a.G = d->ngroups; a.P = d->headdim; a.N = d->dstate;
    a.R = d->rank; a.np = d->npairs;
    a.io_bf16 = d->io_dtype == M3_BF16; a.st_bf16 = d->state_dtype == M3_BF16; a.rate_law = d->rate_law;
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.lam = lam; a.theta = np ? theta : nullptr; a.A = A_log;
    a.Bb = B_bias; a.Cb = C_bias;
    if (init) { a.h0 = init->h; a.phi0 = np ? init->phi : nullptr; a.Bp0 = init->B_prev; a.xp0 = init->x_prev; }
    a.dy = dy;
    a.dh1 = df.h; a.dphi1 = np ? df.phi : nullptr; a.dBp1 = df.B_prev; a.dxp1 = df.x_prev;
    a.dx = g->dx; a.ddt = g->ddt; a.dlam = g->dlam; a.dtheta = np ? g->dtheta : nullptr; a.dA = g->dA;
    a.dBb = g->dB_bias; a.dCb = g->dC_bias;
    a.dh0 = g->dinit.h; a.dphi0 = np ? g->dinit.phi : nullptr; a.dBp0 = g->dinit.B_prev; a.dxp0 = g->dinit.x_prev;
    if (L > 0) {
        char* base = static_cast<char*>(workspace);
        a.accB = reinterpret_cast<float*>(base + w.accB);
        a.accC = reinterpret_cast<float*>(base + w.accC);
        a.wphi = reinterpret_cast<float*>(base + w.phi);
        a.wdphi = reinterpret_cast<float*>(base + w.dphi);
        a.wdl = reinterpret_cast<float*>(base + w.dl);
        a.wdlf = reinterpret_cast<float*>(base + w.dlf);
        a.cws = chunked ? base + w.cws : nullptr;
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    return launch_scan_bwd(a, g->dB, g->dC, hs) == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // extern "C"

namespace {

// Tokens per segment whose rows of x, dt, y (D elements) and of B, C (G N elements)
// stay under 2 GiB, the reach of the kernel's 32-bit buffer offsets.
long long pcs_max_segment_rows(const m3_pcs_desc* d) {
    const long long row = std::max<long long>((long long)d->channels, (long long)d->ngroups * d->dstate) * 4;
    return (1LL << 31) / row - 64;            // 64 rows of margin for the prefetch past a segment's end
}

// Checks of an m3_pcs_desc: M3_ERR_INVALID_ARG for an invalid one, M3_ERR_UNSUPPORTED
// outside the kernels' range (state widths, channel alignment, groups split by a
// workgroup's channel tile, more than 64 segments).
m3_status check_pcs_desc(const m3_pcs_desc* d) {
    if (!d) return M3_ERR_INVALID_ARG;
    if (d->batch < 1 || d->seqlen < 0 || d->channels < 1 || d->ngroups < 1 || d->channels % d->ngroups ||
        d->dstate < 1 || d->nsegments < 0)
        return M3_ERR_INVALID_ARG;
    if (d->io_dtype != M3_F32 && d->io_dtype != M3_BF16) return M3_ERR_INVALID_ARG;
    if (!pcs_supported_state(d->dstate)) return M3_ERR_UNSUPPORTED;
    // x, dt and y rows move in 16-byte pieces
    if (d->channels % (d->io_dtype == M3_BF16 ? 8 : 4)) return M3_ERR_UNSUPPORTED;
    // a workgroup's channels read one group's B and C
    if (d->ngroups > 1 && (d->channels / d->ngroups) % pcs_channels_per_group(d->dstate)) return M3_ERR_UNSUPPORTED;
    if (d->nsegments > 64) return M3_ERR_UNSUPPORTED;
    // every segment's rows must fit the kernel's 32-bit offsets
    const long long max_rows = pcs_max_segment_rows(d);
    if (max_rows < 1 || (d->seqlen + max_rows - 1) / max_rows > 64) return M3_ERR_UNSUPPORTED;
    return M3_OK;
}

// Segments per (batch, channel).  A segmented run costs a second pass over the
// sequence (the summary), so it is chosen only when the (batch, channel tile) waves
// alone would leave SIMDs idle (fewer than one wave per SIMD, 1024 SIMDs); then enough
// segments for about four waves per SIMD, at most 64 (one wave's lanes in the carry
// pass) and at most the number of token blocks.  Each segment is a whole number of
// blocks, and its rows of x, dt and y stay under 2 GiB (the kernel's 32-bit offsets).
void pcs_segments(const m3_pcs_desc* d, int* nseg, int* seglen) {
    const int TB = pcs_block_tokens();
    const int nblocks = (d->seqlen + TB - 1) / TB;
    int k = d->nsegments;
    if (k == 0) {
        const int cw = pcs_channels_per_group(d->dstate);
        const long long tiles = (long long)d->batch * ((d->channels + cw - 1) / cw);
        const long long waves = tiles * pcs_waves_per_group(d->dstate, false);
        const long long seg_waves = tiles * pcs_waves_per_group(d->dstate, true);   // per segment
        k = waves >= 1024 ? 1 : (int)std::min<long long>(64, (4096 + seg_waves - 1) / seg_waves);
    }
    const long long max_rows = pcs_max_segment_rows(d);
    k = std::max<long long>(k, (d->seqlen + max_rows - 1) / max_rows);
    k = std::max(1, std::min(k, std::max(1, nblocks)));
    const int bps = (nblocks + k - 1) / k;   // blocks per segment
    *seglen = std::max(1, bps) * TB;
    *nseg = std::max(1, (d->seqlen + *seglen - 1) / *seglen);
}

PcsArgs make_pcs_args(const m3_pcs_desc* d) {
    PcsArgs a{};
    a.b = d->batch; a.L = d->seqlen; a.D = d->channels; a.G = d->ngroups; a.N = d->dstate;
    a.io_bf16 = d->io_dtype == M3_BF16;
    pcs_segments(d, &a.nseg, &a.seglen);
    return a;
}

}  // namespace

extern "C" {

m3_status m3_pcs_workspace_size(const m3_pcs_desc* d, size_t* bytes) {
    if (!bytes) return M3_ERR_INVALID_ARG;
    m3_status st = check_pcs_desc(d);
    if (st != M3_OK) return st;
    *bytes = d->seqlen > 0 ? pcs_workspace_bytes(make_pcs_args(d)) : 0;
    return M3_OK;
}

m3_status m3_pcs_fwd(const m3_pcs_desc* d, const void* x, const float* dt, const float* A_log, const void* B,
                     const void* C, const float* h0, void* y, float* h1, void* workspace, size_t workspace_bytes,
                     m3_stream_t stream) {
    m3_status st = check_pcs_desc(d);
    if (st != M3_OK) return st;
    const size_t b = d->batch, L = d->seqlen, D = d->channels, G = d->ngroups, N = d->dstate,
                 io = esize(d->io_dtype);
    const size_t sx = b * L * D * io, sdt = b * L * D * 4, sa = D * N * 4, sbc = b * L * G * N * io, sh = b * D * N * 4;
    if (misaligned(h0) || misaligned(h1)) return M3_ERR_ALIGNMENT;
    const Range rh0 = rng(h0, h0 ? sh : 0), rh1 = rng(h1, h1 ? sh : 0);
    if (overlap(rh0, rh1)) return M3_ERR_INVALID_ARG;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (L == 0) {
        if (!h1) return M3_OK;
        return copy_or_zero(h0, h1, sh, hs) == hipSuccess ? M3_OK : M3_ERR_HIP;
    }
    if (!x || !dt || !A_log || !B || !C || !y) return M3_ERR_INVALID_ARG;
    const void* ptrs[] = {x, dt, A_log, B, C, y, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return M3_ERR_ALIGNMENT;
    const Range ry = rng(y, sx);
    const Range ins[] = {rng(x, sx), rng(dt, sdt), rng(A_log, sa), rng(B, sbc), rng(C, sbc), rh0};
    for (const Range& r : ins)
        if (overlap(ry, r) || overlap(rh1, r)) return M3_ERR_INVALID_ARG;
    if (overlap(ry, rh1)) return M3_ERR_INVALID_ARG;
    PcsArgs a = make_pcs_args(d);
    const size_t need = pcs_workspace_bytes(a);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return M3_ERR_INVALID_ARG;
        const Range rw = rng(workspace, need);
        for (const Range& r : ins)
            if (overlap(rw, r)) return M3_ERR_INVALID_ARG;
        if (overlap(rw, ry) || overlap(rw, rh1)) return M3_ERR_INVALID_ARG;
    }
    a.x = x; a.dt = dt; a.A_log = A_log; a.B = B; a.C = C; a.h0 = h0; a.y = y; a.h1 = h1;
    a.ws = static_cast<float*>(workspace);
    return launch_pcs(a, hs) == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // extern "C"
