// Device helpers shared by the matrix-core scan kernels (scan_mfma.hip,
// scan_mx.hip): buffer resources, bf16 packing, the packed-bf16 rotation of a
// pair by a tabled angle, DPP scans, swizzled LDS tile offsets.  Each includer
// gets its own copies (anonymous namespace).
#pragma once

#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kP = 64, kN = 128, kKB = 32;
constexpr int kNP = 4;                   // producer waves
constexpr int kMaxRows = 256;            // rows (tokens x ranks) per chunk
constexpr float kLog2e = 1.4426950408889634f;

enum Mode { kFull = 0, kSummary = 1 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
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
// Per key-block buffer: Bn [32 j][128 n] (turned B) and Bv [32 j][128 n] (v times turned B),
// row-major over the block's 32 key rows j; XT [64 p][32 j] bf16, keys in the scores'
// permuted order (group q: keys 4 q .. 4 q + 3, then 16 + 4 q ..).
constexpr int kBnBytes = kKB * kN * 2;           // 8 KiB
constexpr int kBvBytes = kKB * kN * 2;           // 8 KiB
constexpr int kXtBytes = kP * kKB * 2;           // 4 KiB
constexpr int kBufBytes = kBnBytes + kBvBytes + kXtBytes;
constexpr int kHsBytes = kP * kN * 2;            // bf16 snapshot of the folded state

// 16-byte-group swizzles.  Bn, Bv and Hs rows hold 16 groups (256 B); XT rows 4 (64 B).
__device__ __forceinline__ int bn_off(int j, int grp) { return j * 256 + ((grp ^ (j & 15)) << 4); }
__device__ __forceinline__ int hs_off(int p, int grp) { return p * 256 + ((grp ^ (p & 15)) << 4); }
__device__ __forceinline__ int q4_off(int row, int grp) { return row * 64 + ((grp ^ ((row >> 1) & 3)) << 4); }

// The state update's A operand, (v Bt)^T (k over a block's keys), comes from the row-major
// Bv tile by transposed reads (ds_read_b64_tr_b16).  Within each 16-lane group the instruction treats
// the lanes' 8-byte chunks as a 16 x 4 matrix M (lane s: M[s][0..3]) and returns to lane i
// the column M[4 j + i / 4][i % 4], j = 0..3.  So when lane s points at key row kb + s / 4,
// columns c0 + 4 (s % 4) .. + 3, lane i receives column c0 + i at keys kb .. kb + 3.
// The operand's k order is the scores' permuted one (lane group g: keys 4 g .. 4 g + 3 of
// key tile a, then of key tile b), so each operand is two reads, kb = 4 g and 16 + 4 g.
typedef short tr_v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ds_tr(const char* p) {
    const tr_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) tr_v4i16*)(p));
    return __builtin_bit_cast(uint2, v);
}
// operand over (16 columns from c0) x (the block's 32 keys) of a 256-byte-row tile (Bv)
__device__ __forceinline__ bf16x8 key_operand_256(const char* tile, int c0, int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int col = c0 + 4 * (s & 3), kr = 4 * g + (s >> 2);
    const int off = (col & 7) * 2;
    const uint2 lo = ds_tr(tile + bn_off(kr, col >> 3) + off);
    const uint2 hi = ds_tr(tile + bn_off(16 + kr, col >> 3) + off);
    return __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
}

// Rotation of an (even, odd) pair by a tabled angle, on packed-bf16 dot products with fp32
// sums.  An angle's table entry holds two bf16 pairs, (cos, -sin) and (sin, cos); a bias is
// a bf16 pair; rot(v + b) = rot(v) + rot(b), each half of the result two dot products.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float2 rot_pair(uint32_t v, uint32_t bias, uint2 cs) {
    return float2{dot2(v, cs.x, dot2(bias, cs.x, 0.f)), dot2(v, cs.y, dot2(bias, cs.y, 0.f))};
}
__device__ __forceinline__ uint2 cs_entry(float c, float s) { return uint2{pack2(c, -s), pack2(s, c)}; }

// DPP read of v from another lane; lanes whose source is outside the pattern (or
// whose row is masked off) read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_read(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}

// Inclusive scan of v over groups of W lanes of a wave (W a power of two, 8 <= W <= 64):
// shifts within 16-lane rows, then the row broadcasts of lane 15 and lane 31.
template <int W>
__device__ __forceinline__ float group_scan(float v, int lane_in_group) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
    if constexpr (W == 8) {
        float u = dpp_read<0x111>(v); v = lane_in_group >= 1 ? v + u : v;
        u = dpp_read<0x112>(v); v = lane_in_group >= 2 ? v + u : v;
        u = dpp_read<0x114>(v); v = lane_in_group >= 4 ? v + u : v;
    } else {
        v += dpp_read<0x111>(v);        // row_shr:1, 2, 4, 8 (zero-filled at the row start)
        v += dpp_read<0x112>(v);
        v += dpp_read<0x114>(v);
        v += dpp_read<0x118>(v);
        if constexpr (W >= 32) v += dpp_read<0x142, 0xa>(v);   // row_bcast:15 into rows 1, 3
        if constexpr (W == 64) v += dpp_read<0x143, 0xc>(v);   // row_bcast:31 into rows 2, 3
    }
    return v;
}

}  // namespace
}  // namespace m3
