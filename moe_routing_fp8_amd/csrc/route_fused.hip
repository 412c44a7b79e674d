// Top-k gating, group counting and the token map in two launches on gfx950
// ("DeepSeek open-sources TileKernels", section 2: the routing chain Top-K
// Gating -> Group Counting -> Token-Expert Mapping, and section 2.1; "CuTeDSL
// at Perplexity", MoE dispatch: count each expert's tokens, then give each
// token its index in its expert's list).
//
// The results are those of topk_gate_kernel followed by the token map, bit
// for bit: the same top-k (topk_device.hpp) and the same stable counting sort
// of the routed copies by expert (slots follow row-major (t, k) order inside
// each expert's segment).
//
// Workgroup b of either kernel owns W = NT / 64 consecutive tokens, one wave
// per token, so its copies are the run [b W K, (b + 1) W K) of the row-major
// order.  The slot of a copy of expert e is
//   offset[e] + (copies of e in earlier workgroups) + (its rank among the
//   workgroup's copies of e),
// and the workgroups are grouped into `rows` super-chunks of `group`
// consecutive workgroups (group about the square root of the grid), so the
// middle term is (copies of e in earlier super-chunks) + (copies of e in
// earlier workgroups of the same super-chunk).
//
//   count  top-k; each wave counts its token's copies per expert in an LDS
//          table of (wave, expert) counts (a token's ids are distinct except
//          when fewer than K scores exceed -inf: then expert 0 repeats, so
//          equal ids within the wave are matched with ballots and ranked by
//          lane).  Per expert, an exclusive scan over the waves gives every
//          copy its rank inside the workgroup (written to pos) and the
//          workgroup's count (written to the workgroup's row of a
//          per-workgroup table and added, device-scope atomics, to its
//          super-chunk's row of a super-chunk table).
//   slot   per expert: the super-chunk rows give the copies in earlier
//          super-chunks and the totals (offsets: exclusive scan over experts;
//          workgroup 0 writes counts and offsets); the rows of the earlier
//          workgroups of the super-chunk give the rest; pos += that, and
//          row_token.
//
// The launch boundary is the only hand-off (an in-launch one through device
// counters measured slower here: about 1.5 us per atomic round trip).  The
// super-chunk table must be zero before the count kernel adds into it.  There
// are two: the count kernel adds into the one a parity word names, records
// which in a second word, records how much of it it uses, and zeroes the part
// of the other that the previous call used; the slot kernel reads the
// recorded table and flips the parity.  Each word is written in one kernel
// and read only in the other (or, for the extents, only by the next call), so
// no workgroup can see a word change under it.
#include "device_utils.hpp"
#include "kernels.hpp"
#include "map_device.hpp"
#include "topk_device.hpp"

namespace moe {
namespace {

using namespace mapdev;

constexpr int kWordParity = 288;   // header: the table the next count kernel adds into
constexpr int kWordUsed = 296;     // header: the table the last count kernel added into
constexpr int kWordExtent0 = 304;  // header: entries of table p the last call adding into it used, at 304 + p

template <int NT, int P, bool VEC>
__global__ __launch_bounds__(NT) void route_count_kernel(const float* __restrict__ scores, int64_t num_tokens,
                                                         int num_experts, int num_topk, int renormalize,
                                                         int64_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_weights, int group, int nbits,
                                                         int32_t* __restrict__ pos, int32_t* __restrict__ super_rows,
                                                         int32_t* __restrict__ block_rows,
                                                         uint32_t* __restrict__ hdr) {
    constexpr int W = NT / kWave;  // tokens per workgroup
    const int E = num_experts;
    extern __shared__ int32_t wcnt[];  // [W][E] presence, then exclusive ranks
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.x;
    const int64_t t = static_cast<int64_t>(b) * W + wave;
    const bool live = t < num_tokens && lane < num_topk;  // this lane holds copy (t, lane)
    const uint32_t parity = hdr[kWordParity] & 1u;         // not written during this kernel

    int e = 0;
    if (t < num_tokens) e = topk::topk_row<P, VEC>(scores, t, E, num_topk, renormalize, topk_idx, topk_weights, lane);
    for (int j = threadIdx.x; j < W * E; j += NT) wcnt[j] = 0;
    {
        // this workgroup's slice of the part of the other table the previous call added into, zeroed for the
        // next call (the extent word of that table is written only by a call adding into it)
        int32_t* other = super_rows + (parity ^ 1u) * kRouteSuperStride;
        const int extent =
            static_cast<int>(min(hdr[kWordExtent0 + (parity ^ 1u)], static_cast<uint32_t>(kRouteSuperStride)));
        const int per = (extent + gridDim.x - 1) / gridDim.x;
        const int lo = b * per;
        const int hi = min(lo + per, extent);
        for (int j = lo + threadIdx.x; j < hi; j += NT) other[j] = 0;
    }
    if (b == 0 && threadIdx.x == 0) {
        hdr[kWordUsed] = parity;
        hdr[kWordExtent0 + parity] = static_cast<uint32_t>((gridDim.x + group - 1) / group * E);
    }
    // lanes of this wave holding the same expert: the rank among them below this lane, and the count (written
    // by the lowest of them)
    const uint64_t peers = match_peers(e, live, nbits);
    const int32_t rank_in_wave = __popcll(peers & lanes_below(lane));
    __syncthreads();
    if (live && lane == __builtin_ctzll(peers)) wcnt[wave * E + e] = __popcll(peers);
    __syncthreads();
    int32_t* table = super_rows + parity * kRouteSuperStride;
    const int s = b / group;  // super-chunk
    for (int ex = threadIdx.x; ex < E; ex += NT) {
        int32_t acc = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int32_t c = wcnt[w * E + ex];
            wcnt[w * E + ex] = acc;
            acc += c;
        }
        block_rows[static_cast<int64_t>(b) * E + ex] = acc;
        if (acc != 0) atomicAdd(table + s * E + ex, acc);
    }
    __syncthreads();
    if (live) pos[t * num_topk + lane] = wcnt[wave * E + e] + rank_in_wave;  // rank inside the workgroup
}

template <int NT>
__global__ __launch_bounds__(NT) void route_slot_kernel(const int64_t* __restrict__ topk_idx, int64_t num_tokens,
                                                        int num_experts, int num_topk, int group, int table_ints,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ pos, int32_t* __restrict__ row_token,
                                                        const int32_t* __restrict__ super_rows,
                                                        const int32_t* __restrict__ block_rows,
                                                        uint32_t* __restrict__ hdr) {
    constexpr int W = NT / kWave;
    const int E = num_experts;
    extern __shared__ int32_t lds[];
    int32_t* part = lds;              // [3][share * E] partial sums
    int32_t* run = lds + table_ints;  // [E] first slot of this workgroup's copies of e
    int32_t* tot = run + E;           // [E] copies of e in the batch
    int32_t* scan = tot + E;          // [W + 1] block scan scratch
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.x;
    const int nblocks = gridDim.x;
    const int64_t t = static_cast<int64_t>(b) * W + wave;
    const bool live = t < num_tokens && lane < num_topk;
    const uint32_t used = hdr[kWordUsed] & 1u;  // not written during this kernel
    const int32_t* table = super_rows + used * kRouteSuperStride;
    // this copy's expert and rank inside its workgroup, loaded before the table rows
    int e = 0;
    int32_t local = 0;
    if (live) {
        e = static_cast<int>(topk_idx[t * num_topk + lane]);
        local = pos[t * num_topk + lane];
    }

    // per expert: copies in earlier super-chunks (below), in the batch (total) and in the earlier workgroups of
    // this super-chunk (mates); `share` threads split one expert's rows.  Indices are clamped to rows that
    // exist (the last super-chunk row, this workgroup's own row) and the values masked after, so that a batch
    // of loads is in flight at once.
    const int s = b / group;
    const int rows = (nblocks + group - 1) / group;
    const int first = s * group;
    const int share = E <= NT ? NT / E : 1;
    const int per_thread = (max(rows, group) + share - 1) / share;
    for (int j = threadIdx.x; j < share * E; j += NT) {
        const int g = j / E;
        const int ex = j - g * E;
        int32_t below = 0, total = 0, mates = 0;
        for (int i0 = 0; i0 < per_thread; i0 += 8) {
            int32_t c[8], m[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = g + (i0 + u) * share;
                c[u] = table[min(r, rows - 1) * E + ex];
                const int bb = first + g + (i0 + u) * share;
                m[u] = block_rows[static_cast<int64_t>(min(bb, b)) * E + ex];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = g + (i0 + u) * share;
                const int bb = first + g + (i0 + u) * share;
                total += r < rows ? c[u] : 0;
                below += r < s ? c[u] : 0;
                mates += bb < b ? m[u] : 0;
            }
        }
        part[j] = below + mates;
        part[share * E + j] = total;
    }
    if (b == 0 && threadIdx.x == 0) hdr[kWordParity] = used ^ 1u;  // the next call adds into the other table
    __syncthreads();
    for (int ex = threadIdx.x; ex < E; ex += NT) {
        int32_t below = 0, total = 0;
        for (int g = 0; g < share; ++g) {
            below += part[g * E + ex];
            total += part[share * E + g * E + ex];
        }
        run[ex] = below;
        tot[ex] = total;
    }
    __syncthreads();
    // offsets (workgroup 0 writes counts and offsets); run[e] += offset[e]
    offsets_from_totals<NT>(tot, run, scan, E, 1, b, nblocks, b == 0, counts, offsets, nullptr, 0);
    if (live) {
        const int32_t p = run[e] + local;
        pos[t * num_topk + lane] = p;
        if (row_token != nullptr && p >= 0 && p < num_tokens * num_topk) row_token[p] = static_cast<int32_t>(t);
    }
}

int isqrt_ceil(int n) {
    int r = 1;
    while (r * r < n) ++r;
    return r;
}

template <int NT, int P, bool VEC>
hipError_t launch_route_t(const float* scores, int64_t T, int E, int K, bool renorm, int64_t* idx, float* w,
                          int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_token, int32_t* super_rows,
                          int32_t* block_rows, uint32_t* hdr, hipStream_t stream) {
    constexpr int W = NT / kWave;
    const int blocks = static_cast<int>((T + W - 1) / W);
    const int group = isqrt_ceil(blocks);  // rows = ceil(blocks / group) <= group <= kRouteSuperRows
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipLaunchKernelGGL((route_count_kernel<NT, P, VEC>), dim3(static_cast<unsigned>(blocks)), dim3(NT),
                       W * E * sizeof(int32_t), stream, scores, T, E, K, renorm ? 1 : 0, idx, w, group, nbits, pos,
                       super_rows, block_rows, hdr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int share_ints = 2 * (E > NT ? E : NT);
    const size_t lds = (share_ints + 2 * E + W + 1) * sizeof(int32_t);
    hipLaunchKernelGGL((route_slot_kernel<NT>), dim3(static_cast<unsigned>(blocks)), dim3(NT), lds, stream, idx, T,
                       E, K, group, share_ints, counts, offsets, pos, row_token, super_rows, block_rows, hdr);
    return hipGetLastError();
}

}  // namespace

int64_t route_fused_tokens_per_block(int num_experts) { return num_experts <= 512 ? 1024 / kWave : 512 / kWave; }

size_t route_fused_block_rows_bytes(int64_t num_tokens, int num_experts) {
    const int64_t w = route_fused_tokens_per_block(num_experts);
    const int64_t blocks = (num_tokens + w - 1) / w;
    if (blocks > kRouteMaxBlocks) return 0;  // never takes the fused form
    return (static_cast<size_t>(blocks) * num_experts * sizeof(int32_t) + 255) / 256 * 256;
}

bool route_fused_fits(int64_t num_tokens, int num_experts) {
    const int64_t w = route_fused_tokens_per_block(num_experts);
    return num_tokens > 0 && (num_tokens + w - 1) / w <= kRouteMaxBlocks;
}

hipError_t launch_route_fused(const float* scores, int64_t T, int E, int K, bool renormalize, int64_t* topk_idx,
                              float* topk_weights, int32_t* counts, int32_t* offsets, int32_t* pos,
                              int32_t* row_token, int32_t* super_rows, int32_t* block_rows, uint32_t* header,
                              hipStream_t stream) {
    const bool aligned16 = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
    const bool vec4 = aligned16 && (E % 4 == 0);
#define MOE_ROUTE_ARGS scores, T, E, K, renormalize, topk_idx, topk_weights, counts, offsets, pos, row_token, \
                       super_rows, block_rows, header, stream
    if (E <= 64) return launch_route_t<1024, 1, false>(MOE_ROUTE_ARGS);
    if (E <= 128) return launch_route_t<1024, 2, false>(MOE_ROUTE_ARGS);
    if (E <= 256)
        return vec4 ? launch_route_t<1024, 4, true>(MOE_ROUTE_ARGS) : launch_route_t<1024, 4, false>(MOE_ROUTE_ARGS);
    if (E <= 512)
        return vec4 ? launch_route_t<1024, 8, true>(MOE_ROUTE_ARGS) : launch_route_t<1024, 8, false>(MOE_ROUTE_ARGS);
    return vec4 ? launch_route_t<512, 16, true>(MOE_ROUTE_ARGS) : launch_route_t<512, 16, false>(MOE_ROUTE_ARGS);
#undef MOE_ROUTE_ARGS
}

}  // namespace moe
