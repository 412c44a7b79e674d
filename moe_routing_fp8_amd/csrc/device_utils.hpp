// Device helpers shared by the gfx950 kernels: wave64 cross-lane reductions
// through DPP, bf16 unpacking, the e4m3 group scale and packed e4m3 stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// DPP16 controls (GCN/CDNA data-parallel primitives, one 16-lane row).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each half row
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within each row

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
}

// Maximum over each aligned 16-lane row; every lane of the row receives it.
// After the two quad steps each quad holds its maximum; the half-row mirror
// pairs quad 0 with quad 1 (and 2 with 3); the row mirror pairs the halves.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
    x = max(x, dpp_u32<kDppQuadXor1>(x));
    x = max(x, dpp_u32<kDppQuadXor2>(x));
    x = max(x, dpp_u32<kDppRowHalfMirror>(x));
    x = max(x, dpp_u32<kDppRowMirror>(x));
    return x;
}

// Maximum over each aligned 8-lane half row; every lane of it receives it.
__device__ __forceinline__ uint32_t row8_max_u32(uint32_t x) {
    x = max(x, dpp_u32<kDppQuadXor1>(x));
    x = max(x, dpp_u32<kDppQuadXor2>(x));
    x = max(x, dpp_u32<kDppRowHalfMirror>(x));
    return x;
}

// Two bf16 values packed in a dword -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |f| as raw bits: for non-NaN values unsigned order equals magnitude order.
__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

// Group scale of the e4m3 per-token cast: sf = max(amax, 1e-4) / 448 and
// inv = 1 / sf, both correctly rounded fp32 divisions.
__device__ __forceinline__ void e4m3_group_scale(uint32_t amax_bits, float& sf, float& inv) {
    const float amax = __uint_as_float(amax_bits);
    const float clamped = amax > 1e-4f ? amax : 1e-4f;
    sf = clamped / 448.0f;
    inv = 1.0f / sf;
}

// Four fp32 values -> four OCP e4m3fn codes (round to nearest even) in one
// dword, value a in the lowest byte.  gfx950's v_cvt_pk_fp8_f32 writes two
// codes into the low or high half of the destination.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return static_cast<uint32_t>(r);
}

// Eight bf16 values (one 16-byte vector) -> fp32.
__device__ __forceinline__ void unpack8_bf16(const uint4& raw, float f[8]) {
    f[0] = bf16_lo(raw.x); f[1] = bf16_hi(raw.x);
    f[2] = bf16_lo(raw.y); f[3] = bf16_hi(raw.y);
    f[4] = bf16_lo(raw.z); f[5] = bf16_hi(raw.z);
    f[6] = bf16_lo(raw.w); f[7] = bf16_hi(raw.w);
}

__device__ __forceinline__ uint32_t absmax8(const float f[8]) {
    uint32_t m = abs_bits(f[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = max(m, abs_bits(f[i]));
    return m;
}

// |v| maximum of eight fp32 values that are results of arithmetic (never a
// signalling NaN, so the compiler folds |.| into v_max3_f32 source
// modifiers without canonicalising), returned as bits.
__device__ __forceinline__ uint32_t absmax8_computed(const float v[8]) {
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
    m = fmaxf(fmaxf(m, fabsf(v[3])), fabsf(v[4]));
    m = fmaxf(fmaxf(m, fabsf(v[5])), fabsf(v[6]));
    m = fmaxf(m, fabsf(v[7]));
    return __float_as_uint(m);
}

// Streaming (non-temporal) 16-byte / 8-byte global accesses: data that is
// touched once should not displace reusable lines from L2 and the MALL.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream16(uint4* p, const uint4& q) {
    const u32x4_t v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_stream8(uint2* p, const uint2& q) {
    const u32x2_t v = {q.x, q.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

// Eight fp32 values scaled by inv -> eight e4m3 codes (8 bytes).
__device__ __forceinline__ uint2 quant8_e4m3(const float f[8], float inv) {
    uint2 q;
    q.x = pack4_e4m3(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
    q.y = pack4_e4m3(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
    return q;
}

// Per-token cast of one 16-channel vector v of a bf16 row: codes for the 16
// channels and the scale of their 128-channel group ("DeepSeek open-sources
// TileKernels", sections 3.1-3.2).  The group amax is reduced over the 8
// lanes that hold the group (aligned groups of 8 lanes, all active).
__device__ __forceinline__ void cast16_e4m3_raw(const uint4& ra, const uint4& rb, uint4& codes, float& sf) {
    float f[8], g[8];
    unpack8_bf16(ra, f);
    unpack8_bf16(rb, g);
    const uint32_t amax = row8_max_u32(max(absmax8(f), absmax8(g)));
    float inv;
    e4m3_group_scale(amax, sf, inv);
    const uint2 lo = quant8_e4m3(f, inv);
    const uint2 hi = quant8_e4m3(g, inv);
    codes = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The same from a row in memory, with streaming (non-temporal) loads or
// ordinary ones.
template <bool STREAM>
__device__ __forceinline__ void cast16_e4m3(const uint4* __restrict__ row, int v, uint4& codes,
                                            float& sf) {
    if constexpr (STREAM)
        cast16_e4m3_raw(load_stream16(row + 2 * v), load_stream16(row + 2 * v + 1), codes, sf);
    else
        cast16_e4m3_raw(row[2 * v], row[2 * v + 1], codes, sf);
}

}  // namespace moe
