// Top-k gating on gfx950: one wave64 per token row.
//
// Operation ("DeepSeek open-sources TileKernels", section 2.1 Top-K gating):
// K rounds of "row maximum -> lowest expert index holding it -> mask that
// expert to -inf"; round k's winner is topk_idx[t, k].  Optional weights are
// the selected scores, renormalised to sum to one (section 2, "Weight
// Normalization"): sum in k order in fp32, then one IEEE division each.
//
// MI355X mapping:
//   * lane l holds the P = E/64 (rounded up to a power of two) contiguous
//     scores [l*P, l*P + P) in registers, loaded with 16-byte loads;
//   * each score becomes an order-preserving 32-bit key (-0 folded onto +0,
//     NaN onto -inf), so a round is an unsigned max: P-1 lane-local maxes,
//     four DPP row steps, four readlanes and a scalar max;
//   * the winner is the lowest lane whose local best equals the maximum (a
//     ballot and find-first-set): lanes own ascending index ranges, so that
//     is the lowest index, the tie rule of the pages;
//   * four tokens per 256-thread workgroup; no LDS, no barriers.
#include "device_utils.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // key(-inf)

// Order-preserving key: unsigned order of keys == IEEE order of scores, with
// -0 and +0 given one key (IEEE equality) and NaN read as -inf.
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f != f) return kKeyNegInf;
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float canon_score(float f) { return (f != f) ? -INFINITY : f; }

template <int P, bool VEC>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ scores,
                                                        int64_t num_tokens, int num_experts,
                                                        int num_topk, int renormalize,
                                                        int64_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_weights) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= num_tokens) return;  // whole wave leaves together
    const float* row = scores + t * num_experts;
    const int base = lane * P;

    uint32_t key[P];
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < P; j += 4) {
            if (base + j < num_experts) {  // num_experts % 4 == 0
                const float4 v = *reinterpret_cast<const float4*>(row + base + j);
                key[j + 0] = score_key(v.x);
                key[j + 1] = score_key(v.y);
                key[j + 2] = score_key(v.z);
                key[j + 3] = score_key(v.w);
            } else {
                key[j + 0] = key[j + 1] = key[j + 2] = key[j + 3] = kKeyNegInf;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < P; ++j)
            key[j] = (base + j < num_experts) ? score_key(row[base + j]) : kKeyNegInf;
    }

    int my_idx = 0;  // lane k ends up holding round k's winner
    for (int k = 0; k < num_topk; ++k) {
        uint32_t best = key[0];
#pragma unroll
        for (int j = 1; j < P; ++j) best = max(best, key[j]);
        const uint32_t m = wave_max_u32(best);
        const uint64_t holders = __ballot(best == m);
        const int win_lane = __builtin_ctzll(holders);
        int first = P - 1;
#pragma unroll
        for (int j = P - 1; j >= 0; --j)
            if (key[j] == m) first = j;
        const int win_j = __builtin_amdgcn_readlane(first, win_lane);
        const int idx = win_lane * P + win_j;
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (lane == win_lane && j == win_j) key[j] = kKeyNegInf;
        if (lane == k) my_idx = idx;
    }

    if (lane < num_topk) topk_idx[t * num_topk + lane] = my_idx;
    if (topk_weights != nullptr) {
        const float g = (lane < num_topk) ? canon_score(row[my_idx]) : 0.0f;
        float w = g;
        if (renormalize) {
            float sum = 0.0f;
            for (int k = 0; k < num_topk; ++k)
                sum = sum + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), k));
            w = g / sum;
        }
        if (lane < num_topk) topk_weights[t * num_topk + lane] = w;
    }
}

template <int P>
hipError_t launch_p(bool vec, const float* scores, int64_t T, int E, int K, bool renorm,
                    int64_t* idx, float* w, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((T + 3) / 4));
    if (vec)
        hipLaunchKernelGGL((topk_gate_kernel<P, true>), grid, dim3(256), 0, stream, scores, T, E, K,
                           renorm ? 1 : 0, idx, w);
    else
        hipLaunchKernelGGL((topk_gate_kernel<P, false>), grid, dim3(256), 0, stream, scores, T, E,
                           K, renorm ? 1 : 0, idx, w);
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
