// Token -> expert map on gfx950: group counting, exclusive offsets and the
// slot of every routed copy ("DeepSeek open-sources TileKernels", section 2:
// Group Counting and Token-Expert Mapping; "CuTeDSL at Perplexity", MoE
// dispatch, local kernel: count each expert's tokens, then give each token a
// unique index in its expert's list).
//
// The result is the stable counting sort of the routed copies (t, k) by
// expert: inside an expert's segment, rows follow row-major (t, k) order.
// The pages assign slots with shared-memory atomics (arrival order); here
// the order is fixed so the map is deterministic, with no global atomics.
// Up to one chunk of copies (2048), one workgroup does everything
// (map_single_kernel: LDS histogram, offsets, ranks).  Beyond, two launches
// over chunks of 1024 copies (up to 64 chunks) or 2048 and more (at most
// 256 chunks):
//
//   1. count  one workgroup per chunk of copies: a wave-aggregated LDS
//             histogram -> workspace[b * E + e] (this chunk's count of e).
//   2. rank   one workgroup per chunk again.  Prologue: from the E x B
//             counts (L2-resident) each workgroup sums, per expert, the
//             counts of the chunks before its own and of all chunks; an
//             exclusive scan of the totals over experts gives offsets[]
//             (workgroup 0 writes offsets and counts).  Then, in tiles of
//             one copy per thread, each wave matches equal expert ids with
//             ballots (a multisplit over the id bits): the rank among equal
//             ids below a lane is a popcount, a per-(wave, expert) scan in
//             LDS orders the waves, and a running per-expert cursor orders
//             the tiles.
#include "device_utils.hpp"
#include "kernels.hpp"
#include "map_device.hpp"

namespace moe {
namespace {

using namespace mapdev;

#ifndef MOE_MAP_CHUNK
#define MOE_MAP_CHUNK 2048
#endif
// Routed copies per chunk (workgroup) of the count and rank passes.
constexpr int kMapChunk = MOE_MAP_CHUNK;
// Mid-sized batches (more than one chunk, at most kMidMapChunks chunks of
// kMidMapChunk copies) take smaller chunks: twice the workgroups for the
// same prologue.  Measured (E = 256, K = 8, back-to-back calls): 4096 tokens
// 12.6 -> 10.6 us, 1024 tokens 11.4 -> 10.5 us; at 32768 tokens 1024-copy
// chunks are slower (14.0 -> 14.9 us), so large batches keep kMapChunk.
constexpr int kMidMapChunk = 1024;
constexpr int64_t kMidMapChunks = 64;
#ifndef MOE_SMALL_MAP_ITEMS
#define MOE_SMALL_MAP_ITEMS 512
#endif
// Up to this many copies the single-workgroup map runs with 256 threads.
constexpr int64_t kSmallMapItems = MOE_SMALL_MAP_ITEMS;

template <int NT>
__global__ __launch_bounds__(NT) void map_count_kernel(const int64_t* __restrict__ topk_idx,
                                                       int64_t num_items, int chunk,
                                                       int64_t expert_begin, int num_experts,
                                                       int nbits, int32_t* __restrict__ ws) {
    extern __shared__ int32_t hist[];  // [num_experts]
    count_chunk<NT>(blockIdx.x, topk_idx, num_items, chunk, expert_begin, num_experts, nbits, hist, ws);
}

template <int NT>
__global__ __launch_bounds__(NT) void map_rank_kernel(const int64_t* __restrict__ topk_idx,
                                                      int64_t num_items, int num_topk, int chunk,
                                                      int num_blocks, int64_t expert_begin,
                                                      int num_experts, int align, int nbits,
                                                      int wcnt_ints, const int32_t* __restrict__ ws,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ pos,
                                                      int32_t* __restrict__ row_token,
                                                      int64_t num_rows) {
    extern __shared__ int32_t lds[];
    rank_chunk<NT>(blockIdx.x, topk_idx, num_items, num_topk, chunk, num_blocks, expert_begin, num_experts, align,
                   nbits, wcnt_ints, ws, lds, counts, offsets, pos, row_token, num_rows);
}

// The whole map in one workgroup (all copies in one chunk): the histogram
// goes straight to LDS, then offsets and ranks as in map_rank_kernel -- no
// count table, no second launch.
template <int NT>
__global__ __launch_bounds__(NT) void map_single_kernel(const int64_t* __restrict__ topk_idx, int64_t num_items,
                                                        int num_topk, int64_t expert_begin, int num_experts,
                                                        int align, int nbits, int wcnt_ints,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ pos,
                                                        int32_t* __restrict__ row_token, int64_t num_rows) {
    const int E = num_experts;
    extern __shared__ int32_t lds[];
    int32_t* wcnt = lds;
    int32_t* run = lds + wcnt_ints;
    int32_t* tot = run + E;
    int32_t* scan = tot + E;
    const int lane = threadIdx.x & (kWave - 1);
    for (int e = threadIdx.x; e < E; e += NT) {
        tot[e] = 0;
        run[e] = 0;
    }
    __syncthreads();
    // all copies in one pass of kTilesInFlight tiles: the ranking reuses the
    // ids held here instead of loading them again
    const bool one_pass = num_items <= static_cast<int64_t>(kTilesInFlight) * NT;
    int first[kTilesInFlight];
    for (int64_t base = 0; base < num_items; base += kTilesInFlight * NT) {
        int ids[kTilesInFlight];
#pragma unroll
        for (int u = 0; u < kTilesInFlight; ++u)
            ids[u] = load_expert(topk_idx, base + u * NT + threadIdx.x, num_items, expert_begin, E);
#pragma unroll
        for (int u = 0; u < kTilesInFlight; ++u) {
            if (base == 0) first[u] = ids[u];
            const uint64_t peers = match_peers(ids[u], ids[u] >= 0, nbits);
            if (peers != 0ull && lane == __builtin_ctzll(peers)) atomicAdd(&tot[ids[u]], __popcll(peers));
        }
    }
    __syncthreads();
    const int32_t routed_total =
        offsets_from_totals<NT>(tot, run, scan, E, align, 0, 1, true, counts, offsets, row_token, num_rows);
    if (one_pass)
        rank_tiles<NT, true>(topk_idx, 0, num_items, num_topk, expert_begin, E, nbits, wcnt, run, pos, row_token,
                             num_rows, first);
    else
        rank_tiles<NT>(topk_idx, 0, num_items, num_topk, expert_begin, E, nbits, wcnt, run, pos, row_token,
                       num_rows, first);
    fill_tail<NT>(row_token, routed_total, num_rows, 0, 1);
}

// No routed copies: zero counts and offsets, and mark every row empty.
__global__ void map_zero_kernel(int num_experts, int32_t* __restrict__ counts,
                                int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                                int64_t num_rows) {
    for (int e = threadIdx.x; e <= num_experts; e += blockDim.x) {
        offsets[e] = 0;
        if (e < num_experts) counts[e] = 0;
    }
    if (row_token != nullptr)
        for (int64_t r = threadIdx.x; r < num_rows; r += blockDim.x) row_token[r] = -1;
}

int id_bits(int num_experts) {
    int n = 0;
    while ((1 << n) < num_experts) ++n;
    return n;
}

template <int NT>
hipError_t launch_rank(const int64_t* topk_idx, int num_topk, int64_t expert_begin, int num_experts,
                       int align, int nbits, int32_t* counts, int32_t* offsets, int32_t* pos,
                       int32_t* row_token, int64_t num_rows, const int32_t* ws,
                       const TokenMapPlan& plan, hipStream_t stream) {
    const int wcnt_ints = rank_wcnt_ints<NT>(num_experts);
    const size_t lds = (wcnt_ints + 2 * num_experts + NT / kWave + 1) * sizeof(int32_t);
    hipLaunchKernelGGL((map_rank_kernel<NT>), dim3(plan.num_blocks), dim3(NT), lds, stream, topk_idx,
                       plan.num_items, num_topk, plan.chunk, plan.num_blocks, expert_begin, num_experts,
                       align, nbits, wcnt_ints, ws, counts, offsets, pos, row_token, num_rows);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_single(const int64_t* topk_idx, int64_t num_items, int num_topk, int64_t expert_begin,
                         int num_experts, int align, int nbits, int32_t* counts, int32_t* offsets, int32_t* pos,
                         int32_t* row_token, int64_t num_rows, hipStream_t stream) {
    const int wcnt_ints = rank_wcnt_ints<NT>(num_experts);
    const size_t lds = (wcnt_ints + 2 * num_experts + NT / kWave + 1) * sizeof(int32_t);
    hipLaunchKernelGGL((map_single_kernel<NT>), dim3(1), dim3(NT), lds, stream, topk_idx, num_items, num_topk,
                       expert_begin, num_experts, align, nbits, wcnt_ints, counts, offsets, pos, row_token,
                       num_rows);
    return hipGetLastError();
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
    // Up to kMapChunk copies: one chunk (the single-workgroup map).  Up to
    // kMidMapChunks chunks of kMidMapChunk copies: more workgroups for
    // mid-sized batches.  Above that, chunks of at least kMapChunk copies and
    // at most 256 chunks: the prologue of every rank workgroup reads all
    // E x B chunk counts.
    int64_t chunk = kMapChunk;
    if (p.num_items > kMapChunk && p.num_items <= static_cast<int64_t>(kMidMapChunk) * kMidMapChunks)
        chunk = kMidMapChunk;
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
                            int64_t expert_begin, int num_experts, int align, int32_t* counts,
                            int32_t* offsets, int32_t* pos, int32_t* row_token, int64_t num_rows,
                            int32_t* ws, const TokenMapPlan& plan, hipStream_t stream) {
    (void)num_tokens;
    if (plan.num_blocks == 0) {
        hipLaunchKernelGGL(map_zero_kernel, dim3(1), dim3(1024), 0, stream, num_experts, counts, offsets,
                           row_token, num_rows);
        return hipGetLastError();
    }
    const int nbits = id_bits(num_experts);
    if (plan.num_blocks == 1) {  // one chunk: the single-workgroup map
        // few copies: four waves (cheaper barriers and per-expert wave scans)
        if (plan.num_items <= kSmallMapItems)
            return launch_single<256>(topk_idx, plan.num_items, num_topk, expert_begin, num_experts, align, nbits,
                                      counts, offsets, pos, row_token, num_rows, stream);
        if (num_experts <= 512)
            return launch_single<1024>(topk_idx, plan.num_items, num_topk, expert_begin, num_experts, align,
                                       nbits, counts, offsets, pos, row_token, num_rows, stream);
        return launch_single<512>(topk_idx, plan.num_items, num_topk, expert_begin, num_experts, align, nbits,
                                  counts, offsets, pos, row_token, num_rows, stream);
    }
    hipLaunchKernelGGL((map_count_kernel<1024>), dim3(plan.num_blocks), dim3(1024),
                       num_experts * sizeof(int32_t), stream, topk_idx, plan.num_items, plan.chunk,
                       expert_begin, num_experts, nbits, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (num_experts <= 512)
        return launch_rank<1024>(topk_idx, num_topk, expert_begin, num_experts, align, nbits, counts,
                                 offsets, pos, row_token, num_rows, ws, plan, stream);
    return launch_rank<512>(topk_idx, num_topk, expert_begin, num_experts, align, nbits, counts, offsets,
                            pos, row_token, num_rows, ws, plan, stream);
}

}  // namespace moe
