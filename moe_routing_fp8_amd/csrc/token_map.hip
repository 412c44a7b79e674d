// Token -> expert map on gfx950: group counting, exclusive offsets and the
// slot of every routed copy ("DeepSeek open-sources TileKernels", section 2:
// Group Counting and Token-Expert Mapping; "CuTeDSL at Perplexity", MoE
// dispatch, local kernel: count each expert's tokens, then give each token a
// unique index in its expert's list).
//
// The result is the stable counting sort of the routed copies (t, k) by
// expert: inside an expert's segment, rows follow row-major (t, k) order.
// The pages assign slots with shared-memory atomics (arrival order); here
// the order is fixed so the map is deterministic, with no global atomics:
//
//   1. count   one workgroup per chunk of copies: wave-aggregated LDS
//              histogram -> workspace[e * B + b]   (expert-major, block-minor)
//   2. scan    one workgroup: exclusive scan of the E*B counts in that order.
//              Entry (e, b) becomes the first slot of expert e's copies from
//              chunk b, and entry (e, 0) is offsets[e].
//   3. rank    one workgroup per chunk again: in 1024-copy tiles, each wave
//              matches equal expert ids with ballots (a multisplit over the
//              id bits); the rank among equal ids below a lane is a popcount,
//              a per-(wave, expert) scan in LDS orders the waves, and a
//              running per-expert cursor orders the tiles.
#include "device_utils.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// Lanes of this wave that hold the same (valid) expert id as this lane.
__device__ __forceinline__ uint64_t match_peers(int e, bool valid, int nbits) {
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t m = __ballot(b);
        peers &= b ? m : ~m;
    }
    return valid ? peers : 0ull;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

template <int NT>
__global__ __launch_bounds__(NT) void map_count_kernel(const int64_t* __restrict__ topk_idx,
                                                       int64_t num_items, int chunk,
                                                       int num_blocks, int num_experts, int nbits,
                                                       int32_t* __restrict__ ws) {
    extern __shared__ int32_t hist[];  // [num_experts]
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < num_experts; e += NT) hist[e] = 0;
    __syncthreads();
    const int64_t start = static_cast<int64_t>(b) * chunk;
    const int64_t end = min(start + chunk, num_items);
    const int lane = threadIdx.x & (kWave - 1);
    for (int64_t base = start; base < end; base += NT) {
        const int64_t i = base + threadIdx.x;
        int e = -1;
        if (i < end) {
            const int64_t v = topk_idx[i];
            e = (v >= 0 && v < num_experts) ? static_cast<int>(v) : -1;
        }
        const uint64_t peers = match_peers(e, e >= 0, nbits);
        if (peers != 0ull && lane == __builtin_ctzll(peers))
            atomicAdd(&hist[e], __popcll(peers));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < num_experts; e += NT)
        ws[static_cast<int64_t>(e) * num_blocks + b] = hist[e];
}

// Exclusive scan of ws[0 .. E*B) in place (one workgroup), then
// offsets[e] = ws[e*B], offsets[E] = total, counts[e] = offsets[e+1] - offsets[e].
__global__ __launch_bounds__(kScanThreads) void map_scan_kernel(int32_t* __restrict__ ws,
                                                                int num_blocks, int num_experts,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets) {
    __shared__ int32_t wave_sums[kScanThreads / kWave];
    __shared__ int32_t total_s;
    const int64_t m = static_cast<int64_t>(num_experts) * num_blocks;
    const int64_t span = (m + kScanThreads - 1) / kScanThreads;
    const int64_t lo = min(m, span * threadIdx.x);
    const int64_t hi = min(m, lo + span);
    int32_t local = 0;
    for (int64_t i = lo; i < hi; ++i) local += ws[i];

    // inclusive scan of `local` across the workgroup
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) wave_sums[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t acc = 0;
        for (int w = 0; w < kScanThreads / kWave; ++w) {
            const int32_t s = wave_sums[w];
            wave_sums[w] = acc;
            acc += s;
        }
        total_s = acc;
    }
    __syncthreads();
    int32_t run = wave_sums[wave] + incl - local;  // exclusive prefix of this span
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t c = ws[i];
        ws[i] = run;
        run += c;
    }
    __syncthreads();
    const int32_t total = total_s;
    // offsets[e] = first slot of expert e = scanned entry (e, 0)
    auto offset_of = [&](int e) -> int32_t {
        return e == num_experts ? total : ws[static_cast<int64_t>(e) * num_blocks];
    };
    for (int e = threadIdx.x; e <= num_experts; e += kScanThreads) {
        const int32_t here = num_blocks == 0 ? 0 : offset_of(e);
        offsets[e] = here;
        if (e < num_experts) counts[e] = (num_blocks == 0 ? 0 : offset_of(e + 1)) - here;
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void map_rank_kernel(const int64_t* __restrict__ topk_idx,
                                                      int64_t num_items, int num_topk, int chunk,
                                                      int num_blocks, int num_experts, int nbits,
                                                      const int32_t* __restrict__ ws,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ pos,
                                                      int32_t* __restrict__ row_token) {
    constexpr int W = NT / kWave;
    extern __shared__ int32_t lds[];
    int32_t* wcnt = lds;                    // [W][num_experts]
    int32_t* run = lds + W * num_experts;   // [num_experts]
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < num_experts; e += NT)
        run[e] = ws[static_cast<int64_t>(e) * num_blocks + b];

    const int64_t start = static_cast<int64_t>(b) * chunk;
    const int64_t end = min(start + chunk, num_items);
    for (int64_t base = start; base < end; base += NT) {
        for (int j = threadIdx.x; j < W * num_experts; j += NT) wcnt[j] = 0;
        __syncthreads();
        const int64_t i = base + threadIdx.x;
        const bool in_range = i < end;
        int e = -1;
        if (in_range) {
            const int64_t v = topk_idx[i];
            e = (v >= 0 && v < num_experts) ? static_cast<int>(v) : -1;
        }
        const bool valid = e >= 0;
        const uint64_t peers = match_peers(e, valid, nbits);
        const int rank = __popcll(peers & lanes_below(lane));
        if (valid && lane == __builtin_ctzll(peers)) wcnt[wave * num_experts + e] = __popcll(peers);
        __syncthreads();
        for (int ex = threadIdx.x; ex < num_experts; ex += NT) {
            int32_t acc = run[ex];
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const int32_t c = wcnt[w * num_experts + ex];
                wcnt[w * num_experts + ex] = acc;
                acc += c;
            }
            run[ex] = acc;
        }
        __syncthreads();
        if (in_range) {
            if (valid) {
                const int32_t p = wcnt[wave * num_experts + e] + rank;
                pos[i] = p;
                if (row_token != nullptr && p >= 0 && p < num_items)
                    row_token[p] = static_cast<int32_t>(i / num_topk);
            } else {
                pos[i] = -1;
            }
        }
        __syncthreads();
    }

    // rows past the last routed copy (ids outside [0, E)) have no token
    if (row_token != nullptr) {
        const int64_t total = offsets[num_experts];
        for (int64_t r = total + static_cast<int64_t>(b) * NT + threadIdx.x; r < num_items;
             r += static_cast<int64_t>(num_blocks) * NT)
            row_token[r] = -1;
    }
}

int id_bits(int num_experts) {
    int n = 0;
    while ((1 << n) < num_experts) ++n;
    return n;
}

}  // namespace

TokenMapPlan plan_token_map(int64_t num_tokens, int num_topk, int num_experts) {
    TokenMapPlan p{};
    p.num_items = num_tokens * num_topk;
    if (p.num_items <= 0) {
        p.chunk = 0;
        p.num_blocks = 0;
        p.workspace_bytes = 0;
        return p;
    }
    // At most 256 chunks (bounds the serial scan), at least 2048 copies each.
    int64_t chunk = 2048;
    if ((p.num_items + chunk - 1) / chunk > 256) {
        chunk = (p.num_items + 255) / 256;
        chunk = (chunk + 1023) / 1024 * 1024;
    }
    p.chunk = static_cast<int32_t>(chunk);
    p.num_blocks = static_cast<int32_t>((p.num_items + chunk - 1) / chunk);
    const size_t bytes = static_cast<size_t>(num_experts) * p.num_blocks * sizeof(int32_t);
    p.workspace_bytes = (bytes + 255) / 256 * 256;
    return p;
}

hipError_t launch_token_map(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                            int num_experts, int32_t* counts, int32_t* offsets, int32_t* pos,
                            int32_t* row_token, int32_t* ws, const TokenMapPlan& plan,
                            hipStream_t stream) {
    (void)num_tokens;
    const int nbits = id_bits(num_experts);
    if (plan.num_blocks > 0) {
        hipLaunchKernelGGL((map_count_kernel<1024>), dim3(plan.num_blocks), dim3(1024),
                           num_experts * sizeof(int32_t), stream, topk_idx, plan.num_items,
                           plan.chunk, plan.num_blocks, num_experts, nbits, ws);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(map_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, ws, plan.num_blocks,
                       num_experts, counts, offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || plan.num_blocks == 0) return err;
    if (num_experts <= 512) {
        constexpr int NT = 1024;
        const size_t lds = (NT / kWave + 1) * num_experts * sizeof(int32_t);
        hipLaunchKernelGGL((map_rank_kernel<NT>), dim3(plan.num_blocks), dim3(NT), lds, stream,
                           topk_idx, plan.num_items, num_topk, plan.chunk, plan.num_blocks,
                           num_experts, nbits, ws, offsets, pos, row_token);
    } else {
        constexpr int NT = 512;
        const size_t lds = (NT / kWave + 1) * num_experts * sizeof(int32_t);
        hipLaunchKernelGGL((map_rank_kernel<NT>), dim3(plan.num_blocks), dim3(NT), lds, stream,
                           topk_idx, plan.num_items, num_topk, plan.chunk, plan.num_blocks,
                           num_experts, nbits, ws, offsets, pos, row_token);
    }
    return hipGetLastError();
}

}  // namespace moe
