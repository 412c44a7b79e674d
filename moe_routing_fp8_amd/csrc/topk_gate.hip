// Top-k gating on gfx950: one wave64 per token row ("DeepSeek open-sources
// TileKernels", section 2.1 Top-K gating; the per-row selection lives in
// topk_device.hpp).  One token per wave, four per 256-thread workgroup; no
// LDS, no barriers.
#include "device_utils.hpp"
#include "kernels.hpp"
#include "topk_device.hpp"

namespace moe {
namespace {

// Each wave handles one token; four tokens per 256-thread workgroup.
template <int P, bool VEC>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ scores,
                                                        int64_t num_tokens, int num_experts,
                                                        int num_topk, int renormalize,
                                                        int64_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_weights) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= num_tokens) return;  // whole wave leaves together
    topk::topk_row<P, VEC>(scores, t, num_experts, num_topk, renormalize, topk_idx, topk_weights, lane);
}

template <int P>
hipError_t launch_p(bool vec, const float* scores, int64_t T, int E, int K, bool renorm,
                    int64_t* idx, float* w, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((T + 3) / 4));
    if (vec)
        hipLaunchKernelGGL((topk_gate_kernel<P, true>), grid, dim3(256), 0, stream, scores, T, E, K,
                           renorm ? 1 : 0, idx, w);
    else
        hipLaunchKernelGGL((topk_gate_kernel<P, false>), grid, dim3(256), 0, stream, scores, T, E, K,
                           renorm ? 1 : 0, idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_gate(const float* scores, int64_t T, int E, int K, bool renormalize,
                            int64_t* topk_idx, float* topk_weights, hipStream_t stream) {
    const bool aligned16 = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
    const bool vec4 = aligned16 && (E % 4 == 0);
    if (E <= 64) return launch_p<1>(false, scores, T, E, K, renormalize, topk_idx, topk_weights, stream);
    if (E <= 128) return launch_p<2>(false, scores, T, E, K, renormalize, topk_idx, topk_weights, stream);
    if (E <= 256) return launch_p<4>(vec4, scores, T, E, K, renormalize, topk_idx, topk_weights, stream);
    if (E <= 512) return launch_p<8>(vec4, scores, T, E, K, renormalize, topk_idx, topk_weights, stream);
    return launch_p<16>(vec4, scores, T, E, K, renormalize, topk_idx, topk_weights, stream);
}

}  // namespace moe
