// moe_token_map_noalloc: moe_token_map for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Same kernels, same results; the count
// table that moe_token_map keeps in the caller's workspace lives here in a
// fixed device array instead.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_common.hpp"
#include "kernels.hpp"
#include "moe_fp8.h"

namespace {

// The token map's per-chunk count table: at most 256 chunks x 1024 experts
// x 4 bytes = 1 MiB, the largest table plan_token_map asks for.  One copy
// per device, held from the library's load until the process ends.  On the
// host the array's name only names the symbol, never an address: host code
// uses the device address hipGetSymbolAddress gives, looked up once per
// device.
constexpr size_t kScratchBytes = size_t{1} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with it current); nullptr, with *err set, on failure.
void* scratch_device_ptr(hipError_t* err) {
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        if (p == nullptr) {
            *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

}  // namespace

extern "C" moe_status moe_token_map_noalloc(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                                            int32_t num_experts, int32_t* expert_counts,
                                            int32_t* expert_offsets, int32_t* pos, int32_t* row_token,
                                            hipStream_t stream) {
    using moe::aligned;
    // the checks of moe_token_map, without the workspace
    if (num_tokens < 0 || num_topk < 1 || num_topk > moe::kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (num_experts < 1 || num_experts > moe::kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens * num_topk > INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (expert_counts == nullptr || expert_offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(expert_counts, 4) || !aligned(expert_offsets, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0) {
        if (topk_idx == nullptr || pos == nullptr) return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned(topk_idx, 8) || !aligned(pos, 4) || !aligned(row_token, 4)) return MOE_ERR_INVALID_ARGUMENT;
    }
    const moe::TokenMapPlan plan = moe::plan_token_map(num_tokens, num_topk, num_experts);
    // always true for the shapes admitted above; kept so no plan can overrun the array
    if (plan.workspace_bytes > kScratchBytes) return MOE_ERR_UNSUPPORTED;
    hipError_t err = hipSuccess;
    void* ws = scratch_device_ptr(&err);
    if (ws == nullptr) return moe::hip_status(err);
    // every count the map reads is written by the same call first: nothing to clear
    return moe::hip_status(moe::launch_token_map(topk_idx, num_tokens, num_topk, 0, num_experts, 1, expert_counts,
                                                 expert_offsets, pos, row_token, num_tokens * num_topk,
                                                 static_cast<int32_t*>(ws), plan, stream));
}
