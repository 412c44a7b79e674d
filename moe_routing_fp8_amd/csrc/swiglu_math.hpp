// SwiGLU activation arithmetic shared by the SwiGLU + cast kernels
// ("DeepSeek open-sources TileKernels", section 3.3).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// silu(l) = l / (1 + exp(-l)) with the hardware exp2 and reciprocal.
//
// exp(-l) = 2^(l * c) with c = -log2(e).  c is split as c_hi + c_lo where c_hi
// has 16 significant bits, so for a bf16 l (8 significant bits) the product
// l * c_hi is exact in fp32; the factor 2^(l * c_lo) is replaced by its
// linear term 1 + l * c_lo * ln2.  The dropped second-order term is
// (l * c_lo * ln2)^2 / 2: under 3.5e-9 relative (0.03 ulp of 1) for
// |l| < 17, where silu(l) differs from l, and at most 9.5e-8 (0.8 ulp) at
// |l| = 89.  Hence exp(-l) is the hardware exp2 of an exact argument times
// one correction factor.
// l >= 17: 1 + exp(-l) rounds to 1 and silu(l) == l exactly.
// l <= -89: exp2 overflows to +inf (the correction factor is positive) and
// the result is -0, as in the IEEE expression.
// Finite l only: l = +inf gives 0 * (-inf) = NaN where the IEEE expression
// gives +inf (the SwiGLU entry points require finite gate values).
__device__ __forceinline__ float silu_bf16_arg(float l) {
    constexpr float kCHi = -1.44268798828125f;  // -log2(e) rounded to 16 bits
    constexpr float kCLoLn2 = -4.8884954e-06f;  // (-log2(e) - kCHi) * ln 2
    const float ex = __builtin_amdgcn_exp2f(l * kCHi) * __builtin_fmaf(l, kCLoLn2, 1.0f);
    return l * __builtin_amdgcn_rcpf(1.0f + ex);
}

// Same for an arbitrary fp32 argument (a clamped gate need not be a bf16
// value): the product l * c is carried as head + tail with two FMAs.
__device__ __forceinline__ float silu_any_arg(float l) {
    constexpr float kNegLog2eHi = -1.44269502162933349609375f;  // fp32(-log2 e)
    constexpr float kNegLog2eLo = -1.9259629889e-8f;            // -log2 e - hi
    constexpr float kLn2 = 0.693147180559945309417232f;
    const float p = l * kNegLog2eHi;
    float e = __builtin_fmaf(l, kNegLog2eHi, -p);
    e = __builtin_fmaf(l, kNegLog2eLo, e);
    const float ex = __builtin_amdgcn_exp2f(p) * __builtin_fmaf(e, kLn2, 1.0f);
    return l * __builtin_amdgcn_rcpf(1.0f + ex);
}

}  // namespace moe
