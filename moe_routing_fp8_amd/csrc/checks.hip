// Device-side checks of the inputs the dispatch kernels assume but do not
// test on their fast path:
//   scores      finite ("DeepSeek open-sources TileKernels", section 2.1:
//               the iterative maximum compares scores, so a NaN has no place
//               in the order) and, for renormalised weights, positive
//               (section 2, "Weight Normalization": each selected score is
//               divided by the sum of the selected scores);
//   topk_idx    every id in [0, E) and no id twice in one token's row
//               (section 2.1: each round masks its winner, so a row's K ids
//               are K distinct experts);
//   pos         every entry in [-1, num_rows) and no row reached by two
//               copies (section 2.2: -1 marks a copy that is skipped; every
//               other copy owns its destination row);
//   bf16 values finite (sections 3.2-3.3: the group scale is the amax of the
//               group's magnitudes divided by the format maximum, defined for
//               finite values only);
//   dispatch    the time-out word of a single-launch dispatch's workspace
//               ("CuTeDSL at Perplexity", grid synchronisation: the grid
//               barrier assumes every workgroup is resident).
// Each check ORs MOE_CHECK_* bits into a caller-zeroed device word.  Checks
// are debugging aids: plain grid-stride loops, no tuning.
#include "device_utils.hpp"
#include "kernels.hpp"
#include "moe_fp8.h"

namespace moe {
namespace {

constexpr int kCheckThreads = 256;
constexpr int64_t kCheckMaxBlocks = 2048;

// One atomic per wave that found something.
__device__ __forceinline__ void report(uint32_t bits, uint32_t* flags) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) bits |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(bits), m));
    if ((threadIdx.x & (kWave - 1)) == 0 && bits != 0) atomicOr(flags, bits);
}

__global__ __launch_bounds__(kCheckThreads) void check_scores_kernel(const float* __restrict__ scores, int64_t n,
                                                                     int require_positive,
                                                                     uint32_t* __restrict__ flags) {
    uint32_t bits = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n; i += stride) {
        const float s = scores[i];
        if (!__builtin_isfinite(s)) bits |= MOE_CHECK_NONFINITE_SCORE;
        else if (require_positive && !(s > 0.0f)) bits |= MOE_CHECK_NONPOSITIVE_SCORE;
    }
    report(bits, flags);
}

// One thread per token row: K <= 16 ids, pairwise compared.
__global__ __launch_bounds__(kCheckThreads) void check_topk_idx_kernel(const int64_t* __restrict__ idx,
                                                                       int64_t num_tokens, int num_topk,
                                                                       int num_experts,
                                                                       uint32_t* __restrict__ flags) {
    uint32_t bits = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckThreads;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; t < num_tokens; t += stride) {
        const int64_t* row = idx + t * num_topk;
        for (int k = 0; k < num_topk; ++k) {
            const int64_t e = row[k];
            if (e < 0 || e >= num_experts) bits |= MOE_CHECK_ID_RANGE;
            for (int j = 0; j < k; ++j)
                if (row[j] == e) bits |= MOE_CHECK_ID_DUPLICATE;
        }
    }
    report(bits, flags);
}

__global__ __launch_bounds__(kCheckThreads) void zero_words_kernel(uint32_t* __restrict__ words, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n; i += stride)
        words[i] = 0u;
}

// A bitmap of the rows already reached: the copy whose atomicOr finds its
// row's bit set is a second copy to that row.  Only entries in [0, num_rows)
// index the bitmap.
__global__ __launch_bounds__(kCheckThreads) void check_pos_kernel(const int32_t* __restrict__ pos, int64_t n,
                                                                  int64_t num_rows, uint32_t* __restrict__ seen,
                                                                  uint32_t* __restrict__ flags) {
    uint32_t bits = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n; i += stride) {
        const int64_t r = pos[i];
        if (r < -1 || r >= num_rows) {
            bits |= MOE_CHECK_POS_RANGE;
        } else if (r >= 0) {
            const uint32_t bit = 1u << (r & 31);
            if (atomicOr(seen + (r >> 5), bit) & bit) bits |= MOE_CHECK_POS_DUPLICATE;
        }
    }
    report(bits, flags);
}

// bf16 bit patterns with an all-ones exponent field are infinities or NaN.
__global__ __launch_bounds__(kCheckThreads) void check_bf16_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                   uint32_t* __restrict__ flags) {
    uint32_t bits = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCheckThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n; i += stride)
        if ((x[i] & 0x7F80u) == 0x7F80u) bits |= MOE_CHECK_NONFINITE_ACTIVATION;
    report(bits, flags);
}

// One wave reads the barrier's time-out word of a dispatch workspace header.
__global__ __launch_bounds__(kWave) void check_dispatch_kernel(const uint32_t* __restrict__ header, int word,
                                                               uint32_t* __restrict__ flags) {
    const uint32_t bits = (threadIdx.x == 0 && header[word] != 0u) ? MOE_CHECK_DISPATCH_TIMEOUT : 0u;
    report(bits, flags);
}

unsigned check_blocks(int64_t items) {
    const int64_t b = (items + kCheckThreads - 1) / kCheckThreads;
    return static_cast<unsigned>(b < 1 ? 1 : (b > kCheckMaxBlocks ? kCheckMaxBlocks : b));
}

}  // namespace

hipError_t launch_check_scores(const float* scores, int64_t num_tokens, int num_experts, bool require_positive,
                               uint32_t* flags, hipStream_t stream) {
    const int64_t n = num_tokens * num_experts;
    hipLaunchKernelGGL(check_scores_kernel, dim3(check_blocks(n)), dim3(kCheckThreads), 0, stream, scores, n,
                       require_positive ? 1 : 0, flags);
    return hipGetLastError();
}

hipError_t launch_check_topk_idx(const int64_t* idx, int64_t num_tokens, int num_topk, int num_experts,
                                 uint32_t* flags, hipStream_t stream) {
    hipLaunchKernelGGL(check_topk_idx_kernel, dim3(check_blocks(num_tokens)), dim3(kCheckThreads), 0, stream, idx,
                       num_tokens, num_topk, num_experts, flags);
    return hipGetLastError();
}

hipError_t launch_check_pos(const int32_t* pos, int64_t num_entries, int64_t num_rows, uint32_t* seen,
                            uint32_t* flags, hipStream_t stream) {
    const int64_t words = (num_rows + 31) / 32;
    if (words > 0) {
        hipLaunchKernelGGL(zero_words_kernel, dim3(check_blocks(words)), dim3(kCheckThreads), 0, stream, seen,
                           words);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(check_pos_kernel, dim3(check_blocks(num_entries)), dim3(kCheckThreads), 0, stream, pos,
                       num_entries, num_rows, seen, flags);
    return hipGetLastError();
}

hipError_t launch_check_bf16(const uint16_t* x, int64_t n, uint32_t* flags, hipStream_t stream) {
    hipLaunchKernelGGL(check_bf16_kernel, dim3(check_blocks(n)), dim3(kCheckThreads), 0, stream, x, n, flags);
    return hipGetLastError();
}

hipError_t launch_check_dispatch(const uint32_t* header, int word, uint32_t* flags, hipStream_t stream) {
    hipLaunchKernelGGL(check_dispatch_kernel, dim3(1), dim3(kWave), 0, stream, header, word, flags);
    return hipGetLastError();
}

}  // namespace moe
