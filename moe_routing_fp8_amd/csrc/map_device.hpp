// Device pieces of the token map ("DeepSeek open-sources TileKernels",
// section 2: Group Counting and Token-Expert Mapping): the per-chunk
// histogram, the exclusive offsets and the stable rank of every routed copy.
// Shared by the map's own kernels (token_map.hip) and the one-launch routing
// kernel (route_fused.hip), which runs the same chunk functions from inside
// its top-k workgroups.
#pragma once

#include "device_utils.hpp"

namespace moe {
namespace mapdev {

// Tiles (one routed copy per thread) whose ids are loaded before any is processed.
constexpr int kTilesInFlight = 4;

// DPP controls (gfx9): shift right within a 16-lane row, and broadcast the
// last lane of a row to the next row (15) or to rows 2 and 3 (31).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// DPP read of x; lanes whose source lies outside their row read 0.
template <int CTRL>
__device__ __forceinline__ int32_t dpp_shift_i32(int32_t x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}

// DPP read of x in the rows of ROW_MASK; the other rows read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int32_t dpp_rows_i32(int32_t x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive sum over the wave: a Hillis-Steele scan inside each 16-lane row
// (shifts 1, 2, 4, 8), then the row totals carried across rows: lane 15 of
// rows 0 and 2 into rows 1 and 3, then lane 31 (rows 0-1) into rows 2 and 3.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t x) {
    x += dpp_shift_i32<kDppRowShr1>(x);
    x += dpp_shift_i32<kDppRowShr2>(x);
    x += dpp_shift_i32<kDppRowShr4>(x);
    x += dpp_shift_i32<kDppRowShr8>(x);
    x += dpp_rows_i32<kDppRowBcast15, 0xA>(x);
    x += dpp_rows_i32<kDppRowBcast31, 0xC>(x);
    return x;
}

// Exclusive scan of one value per thread over the workgroup; also returns
// the total.  `scratch` holds NT/64 + 1 ints of LDS.  Each wave scans its
// lanes with DPP; wave 0 then scans the wave totals the same way.
template <int NT>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* scratch, int32_t& total) {
    constexpr int W = NT / kWave;
    static_assert(W <= kWave, "one wave scans the wave totals");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int32_t incl = wave_inclusive_sum(v);
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int32_t t = lane < W ? scratch[lane] : 0;
        const int32_t ti = wave_inclusive_sum(t);
        if (lane < W) scratch[lane] = ti - t;
        if (lane == W - 1) scratch[W] = ti;
    }
    __syncthreads();
    total = scratch[W];
    const int32_t excl = scratch[wave] + incl - v;
    __syncthreads();  // scratch may be reused by the caller
    return excl;
}

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

// Local expert index of copy i (ids in [expert_begin, expert_begin + E)),
// or -1 for a copy past `end` or routed to another expert.
__device__ __forceinline__ int load_expert(const int64_t* __restrict__ topk_idx, int64_t i,
                                           int64_t end, int64_t expert_begin, int num_experts) {
    if (i >= end) return -1;
    const int64_t v = topk_idx[i] - expert_begin;
    return (v >= 0 && v < num_experts) ? static_cast<int>(v) : -1;
}


// Histogram of chunk b (copies [b * chunk, min((b + 1) * chunk, num_items)))
// into ws[b * E + e]: a wave-aggregated LDS histogram (hist: E ints of LDS).
template <int NT>
__device__ void count_chunk(int b, const int64_t* __restrict__ topk_idx, int64_t num_items, int chunk,
                            int64_t expert_begin, int num_experts, int nbits, int32_t* hist,
                            int32_t* __restrict__ ws) {
    for (int e = threadIdx.x; e < num_experts; e += NT) hist[e] = 0;
    __syncthreads();
    const int64_t start = static_cast<int64_t>(b) * chunk;
    const int64_t end = min(start + chunk, num_items);
    const int lane = threadIdx.x & (kWave - 1);
    for (int64_t base = start; base < end; base += kTilesInFlight * NT) {
        int ids[kTilesInFlight];  // loads of several tiles in flight at once
#pragma unroll
        for (int u = 0; u < kTilesInFlight; ++u)
            ids[u] = load_expert(topk_idx, base + u * NT + threadIdx.x, end, expert_begin, num_experts);
#pragma unroll
        for (int u = 0; u < kTilesInFlight; ++u) {
            const uint64_t peers = match_peers(ids[u], ids[u] >= 0, nbits);
            if (peers != 0ull && lane == __builtin_ctzll(peers)) atomicAdd(&hist[ids[u]], __popcll(peers));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < num_experts; e += NT)
        ws[static_cast<int64_t>(b) * num_experts + e] = hist[e];
}
// LDS layout of the rank kernel (ints):
//   wcnt  [max(W*E, 2*max(NT,E))] per-(wave, expert) counts of a tile; in the
//                               prologue, per-group partial sums
//   run   [E]                   running slot cursor of each expert
//   tot   [E]                   per-expert totals (prologue)
//   scan  [W + 1]               block scan scratch
template <int NT>
int rank_wcnt_ints(int num_experts) {
    const int w = NT / kWave * num_experts;
    const int parts = 2 * (num_experts > NT ? num_experts : NT);
    return w > parts ? w : parts;
}

// Offsets from the per-expert totals tot[] (LDS): segment sizes are the
// totals rounded up to a multiple of align, scanned over experts.  On entry
// run[e] holds the copies of expert e in earlier chunks; on exit the first
// slot of this workgroup's copies of e.  Workgroup `writer` writes offsets
// and counts; padding rows of expert e are marked -1 by workgroup
// e % num_blocks.  Returns the end of the last segment.
template <int NT>
__device__ int32_t offsets_from_totals(const int32_t* tot, int32_t* run, int32_t* scan, int E, int align, int b,
                                       int num_blocks, bool writer, int32_t* __restrict__ counts,
                                       int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                                       int64_t num_rows) {
    constexpr int W = NT / kWave;
    // a thread owns `per` = ceil(E / NT) consecutive experts
    const int per = (E + NT - 1) / NT;
    const int e0 = threadIdx.x * per;
    int32_t mine = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) mine += (tot[e0 + i] + align - 1) / align * align;
    int32_t all = 0;
    int32_t acc = block_exclusive_scan<NT>(mine, scan, all);
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int32_t c = tot[e];
            if (writer) {
                offsets[e] = acc;
                counts[e] = c;
            }
            // padding rows of this segment: [acc + c, acc + size)
            if (row_token != nullptr && e % num_blocks == b) {
                const int32_t size = (c + align - 1) / align * align;
                for (int32_t r = acc + c; r < acc + size && r < num_rows; ++r) row_token[r] = -1;
            }
            run[e] += acc;
            acc += (c + align - 1) / align * align;
        }
    }
    if (writer && threadIdx.x == 0) offsets[E] = all;
    if (threadIdx.x == 0) scan[W] = all;
    __syncthreads();
    return scan[W];
}

// Stable ranks of copies [start, end), one tile of NT copies at a time: a
// wave-level multisplit gives the rank among equal ids below a lane, a
// per-(wave, expert) scan in LDS orders the waves, and run[] (the next slot
// of each expert) orders the tiles.  PRELOADED: [start, end) is one pass of
// kTilesInFlight tiles whose ids the caller already holds in `pre`.
template <int NT, bool PRELOADED = false>
__device__ void rank_tiles(const int64_t* __restrict__ topk_idx, int64_t start, int64_t end, int num_topk,
                           int64_t expert_begin, int E, int nbits, int32_t* wcnt, int32_t* run,
                           int32_t* __restrict__ pos, int32_t* __restrict__ row_token, int64_t num_rows,
                           const int (&pre)[kTilesInFlight]) {
    constexpr int W = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    for (int64_t base4 = start; base4 < end; base4 += kTilesInFlight * NT) {
        int ids[kTilesInFlight];  // loads of several tiles in flight at once
#pragma unroll
        for (int u = 0; u < kTilesInFlight; ++u)
            ids[u] = PRELOADED ? pre[u] : load_expert(topk_idx, base4 + u * NT + threadIdx.x, end, expert_begin, E);
#pragma unroll
        for (int u = 0; u < kTilesInFlight; ++u) {
            const int64_t base = base4 + u * NT;
            if (base >= end) break;  // uniform
            for (int j = threadIdx.x; j < W * E; j += NT) wcnt[j] = 0;
            __syncthreads();
            const int64_t i = base + threadIdx.x;
            const int e = ids[u];
            const bool valid = e >= 0;
            const uint64_t peers = match_peers(e, valid, nbits);
            const int rank = __popcll(peers & lanes_below(lane));
            if (valid && lane == __builtin_ctzll(peers)) wcnt[wave * E + e] = __popcll(peers);
            __syncthreads();
            for (int ex = threadIdx.x; ex < E; ex += NT) {
                int32_t acc = run[ex];
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const int32_t c = wcnt[w * E + ex];
                    wcnt[w * E + ex] = acc;
                    acc += c;
                }
                run[ex] = acc;
            }
            __syncthreads();
            if (i < end) {
                if (valid) {
                    const int32_t p = wcnt[wave * E + e] + rank;
                    pos[i] = p;
                    if (row_token != nullptr && p >= 0 && p < num_rows)
                        row_token[p] = static_cast<int32_t>(i / num_topk);
                } else {
                    pos[i] = -1;
                }
            }
            __syncthreads();
        }
    }
}

// Rows past the last segment have no token (rows [routed_total, num_rows),
// strided over the workgroups).
template <int NT>
__device__ void fill_tail(int32_t* __restrict__ row_token, int32_t routed_total, int64_t num_rows, int b,
                          int num_blocks) {
    if (row_token == nullptr) return;
    for (int64_t r = routed_total + static_cast<int64_t>(b) * NT + threadIdx.x; r < num_rows;
         r += static_cast<int64_t>(num_blocks) * NT)
        row_token[r] = -1;
}

// Offsets and the stable ranks of chunk b's copies from the E x B count table
// ws (prologue: per expert, the counts of earlier chunks and of all chunks),
// as one workgroup of NT threads.  lds: rank_wcnt_ints<NT>(E) + 2 E + NT / 64
// + 1 ints.  The workgroup of chunk 0 writes counts and offsets.
template <int NT>
__device__ void rank_chunk(int b, const int64_t* __restrict__ topk_idx, int64_t num_items, int num_topk,
                           int chunk, int num_blocks, int64_t expert_begin, int num_experts, int align,
                           int nbits, int wcnt_ints, const int32_t* __restrict__ ws, int32_t* lds,
                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ pos, int32_t* __restrict__ row_token, int64_t num_rows) {
    const int E = num_experts;
    int32_t* wcnt = lds;
    int32_t* run = lds + wcnt_ints;
    int32_t* tot = run + E;
    int32_t* scan = tot + E;

    // ---- per expert, the counts of earlier chunks (run) and of all chunks (tot)
    {
        const int groups = E <= NT ? NT / E : 1;  // threads that share one expert
        int32_t* part_below = wcnt;                     // [groups * E] <= max(NT, E)
        int32_t* part_total = wcnt + (E <= NT ? NT : E);  // same size, after it
        if (E <= NT) {
            const int g = threadIdx.x / E;
            const int e = threadIdx.x - g * E;
            if (g < groups) {
                int32_t below = 0, total = 0;
#pragma unroll 8
                for (int bb = g; bb < num_blocks; bb += groups) {
                    const int32_t c = ws[static_cast<int64_t>(bb) * E + e];
                    total += c;
                    below += (bb < b) ? c : 0;
                }
                part_below[g * E + e] = below;
                part_total[g * E + e] = total;
            }
        } else {
            for (int e = threadIdx.x; e < E; e += NT) {
                int32_t below = 0, total = 0;
#pragma unroll 8
                for (int bb = 0; bb < num_blocks; ++bb) {
                    const int32_t c = ws[static_cast<int64_t>(bb) * E + e];
                    total += c;
                    below += (bb < b) ? c : 0;
                }
                part_below[e] = below;
                part_total[e] = total;
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += NT) {
            int32_t below = 0, total = 0;
            for (int g = 0; g < groups; ++g) {
                below += part_below[g * E + e];
                total += part_total[g * E + e];
            }
            run[e] = below;
            tot[e] = total;
        }
        __syncthreads();
    }
    const int32_t routed_total = offsets_from_totals<NT>(tot, run, scan, E, align, b, num_blocks, b == 0, counts,
                                                         offsets, row_token, num_rows);
    const int64_t start = static_cast<int64_t>(b) * chunk;
    const int64_t end = min(start + chunk, num_items);
    const int none[kTilesInFlight] = {};
    rank_tiles<NT>(topk_idx, start, end, num_topk, expert_begin, E, nbits, wcnt, run, pos, row_token, num_rows,
                   none);
    fill_tail<NT>(row_token, routed_total, num_rows, b, num_blocks);
}

}  // namespace mapdev
}  // namespace moe
