// Host-side helpers shared by the C-ABI entry points (moe_fp8_api.hip and
// the entry points in files of their own): argument limits, alignment
// checks and the HIP-error-to-status mapping behind moe_last_hip_error().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_fp8.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 16;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// MOE_OK for hipSuccess; otherwise records err as the calling thread's last
// HIP error (moe_last_hip_error) and returns MOE_ERR_HIP.
moe_status hip_status(hipError_t err);

}  // namespace moe
