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
// Workgroup b of the count kernel owns W = NT / 64 consecutive tokens, one
// wave per token, so its copies are the run [b W K, (b + 1) W K) of the
// row-major order.  The slot of a copy of expert e is
//   offset[e] + (copies of e in earlier workgroups) + (its rank among the
//   workgroup's copies of e),
// and the workgroups are grouped into `rows` super-chunks of `group`
// consecutive workgroups (group about the square root of the grid), so the
// middle term is (copies of e in earlier super-chunks) + (copies of e in
// earlier workgroups of the same super-chunk).
//
//   count  top-k; each wave counts its token's copies per expert in an LDS
//          table of 16-bit (expert, wave) counts (a token's ids are distinct except
//          when fewer than K scores exceed -inf: then expert 0 repeats, so
//          the lanes holding expert 0 are matched with a ballot and ranked by
//          lane).  Per expert, an exclusive scan over the waves gives every
//          copy its rank inside the workgroup (written to pos) and the
//          workgroup's count (written to the workgroup's row of a
//          per-workgroup table and added, device-scope atomics, to its
//          super-chunk's row of a super-chunk table).
//   slot   per expert: the super-chunk rows give the copies in earlier
//          super-chunks and the totals (offsets: exclusive scan over experts;
//          the first workgroup writes counts and offsets); the rows of the
//          earlier workgroups of the super-chunk give the rest; pos += that,
//          and row_token.  Up to kSlotBlockMax count workgroups, one slot
//          workgroup per count workgroup; above, one per super-chunk.
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
                                                         float* __restrict__ topk_weights, int group,
                                                         int32_t* __restrict__ pos, int32_t* __restrict__ super_rows,
                                                         int32_t* __restrict__ block_rows,
                                                         uint32_t* __restrict__ hdr) {
    constexpr int W = NT / kWave;  // tokens per workgroup
    static_assert(W % 8 == 0, "a column of W 16-bit counts is whole 16-byte words");
    constexpr int V = W / 8;       // 16-byte words per expert column
    const int E = num_experts;
    // [E][W] 16-bit counts of copies per (expert, wave), then their exclusive prefix over the waves: an expert's
    // column is V 16-byte words, so one thread scans it with V loads and V stores (counts <= K <= 16 per
    // cell, prefixes <= 16 W)
    extern __shared__ uint4 cnt_v[];
    uint16_t* cnt = reinterpret_cast<uint16_t*>(cnt_v);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.x;
    const int64_t t = static_cast<int64_t>(b) * W + wave;
    const bool live = t < num_tokens && lane < num_topk;  // this lane holds copy (t, lane)
    const uint32_t parity = hdr[kWordParity] & 1u;         // not written during this kernel

    int e = 0;
    if (t < num_tokens) e = topk::topk_row<P, VEC>(scores, t, E, num_topk, renormalize, topk_idx, topk_weights, lane);
    for (int j = threadIdx.x; j < V * E; j += NT) cnt_v[j] = make_uint4(0u, 0u, 0u, 0u);
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
    // a token's ids are distinct except expert 0: once fewer than K scores exceed -inf, every further round of
    // the top-k picks index 0 again.  So only the lanes holding expert 0 are matched (one ballot): their rank
    // below this lane, and their count, written by the lowest of them
    const uint64_t zeros = __ballot(live && e == 0);
    const int32_t rank_in_wave = e == 0 ? __popcll(zeros & lanes_below(lane)) : 0;
    __syncthreads();
    if (live && (e != 0 || lane == __builtin_ctzll(zeros)))
        cnt[e * W + wave] = static_cast<uint16_t>(e == 0 ? __popcll(zeros) : 1);
    __syncthreads();
    int32_t* table = super_rows + parity * kRouteSuperStride;
    const int s = b / group;  // super-chunk
    for (int ex = threadIdx.x; ex < E; ex += NT) {
        uint32_t words[4 * V];  // the column as 32-bit words: two waves per word
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint4 q = cnt_v[ex * V + i];
            words[4 * i + 0] = q.x;
            words[4 * i + 1] = q.y;
            words[4 * i + 2] = q.z;
            words[4 * i + 3] = q.w;
        }
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < 4 * V; ++i) {
            const uint32_t lo = words[i] & 0xFFFFu, hi = words[i] >> 16;
            words[i] = acc | ((acc + lo) << 16);
            acc += lo + hi;
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            cnt_v[ex * V + i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
        const int32_t total = static_cast<int32_t>(acc);
        block_rows[static_cast<int64_t>(b) * E + ex] = total;
        if (total != 0) atomicAdd(table + s * E + ex, total);
    }
    __syncthreads();
    if (live) pos[t * num_topk + lane] = cnt[e * W + wave] + rank_in_wave;  // rank inside the workgroup
}

// Slot kernel for grids of at most kSlotBlockMax workgroups: one workgroup
// per count-kernel workgroup, which reads the super-chunk table and the rows
// of the earlier workgroups of its super-chunk itself (a few loads per
// thread, all in flight at once) and writes the slots of its own copies.
// Measured faster here than one workgroup per super-chunk (4096 tokens, E =
// 256: 10.9 against 12.1 us for the routing), whose running prefix over the
// super-chunk's rows is serial per expert; above kSlotBlockMax the
// per-workgroup reads (every workgroup reads the whole table) dominate.
constexpr int kSlotBlockMax = 256;

template <int NT>
__global__ __launch_bounds__(NT) void route_slot_block_kernel(
    const int64_t* __restrict__ topk_idx, int64_t num_tokens, int num_experts, int num_topk, int group,
    int table_ints, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ pos,
    int32_t* __restrict__ row_token, const int32_t* __restrict__ super_rows, const int32_t* __restrict__ block_rows,
    uint32_t* __restrict__ hdr) {
    constexpr int W = NT / kWave;
    const int E = num_experts;
    extern __shared__ int32_t lds[];
    int32_t* part = lds;              // [2][share * E] partial sums (below + mates, totals)
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
                // unsigned 32-bit offsets from uniform bases: the scalar-base load form, all loads in flight
                c[u] = table[static_cast<uint32_t>(min(r, rows - 1) * E + ex)];
                const int bb = first + g + (i0 + u) * share;
                m[u] = block_rows[static_cast<uint32_t>(min(bb, b) * E + ex)];
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

// One workgroup per super-chunk s: this super-chunk's workgroup rows become
// running prefixes in LDS (pre[b - first][e] = copies of e in the earlier
// workgroups of the super-chunk), the super-chunk table gives the copies in
// earlier super-chunks and the totals, and every copy of the super-chunk
// gets its slot.  Each row is read by one workgroup only.
constexpr int kSlotThreads = 1024;
constexpr int kSlotPreload = 4;       // copies per thread whose id and rank are loaded before the tables
constexpr int kSlotPreInts = 8192;    // LDS ints of the super-chunk's workgroup rows (group x E)

__global__ __launch_bounds__(kSlotThreads) void route_slot_group_kernel(
    const int64_t* __restrict__ topk_idx, int64_t num_tokens, int num_experts, int num_topk, int tokens_per_block,
    int count_blocks, int group, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token, const int32_t* __restrict__ super_rows,
    const int32_t* __restrict__ block_rows, uint32_t* __restrict__ hdr) {
    constexpr int NT = kSlotThreads;
    const int E = num_experts;
    const int s = blockIdx.x;
    const int rows = gridDim.x;
    const int first = s * group;
    const int nb = min(group, count_blocks - first);  // workgroups of the count kernel in this super-chunk
    const int share = E <= NT ? NT / E : 1;            // threads splitting one expert's table rows
    extern __shared__ int32_t lds[];
    int32_t* pre = lds;                                // [group][E]
    int32_t* part = pre + group * E;                   // [2][share * E]
    int32_t* run = part + 2 * (E > NT ? E : NT);       // [E]
    int32_t* tot = run + E;                            // [E]
    int32_t* scan = tot + E;                           // [NT / 64 + 1]
    const uint32_t used = hdr[kWordUsed] & 1u;         // not written during this kernel
    const int32_t* table = super_rows + used * kRouteSuperStride;

    // this super-chunk's copies: ids and in-workgroup ranks of the first kSlotPreload per thread, loaded first
    const int64_t c_lo = static_cast<int64_t>(first) * tokens_per_block * num_topk;
    const int64_t c_hi = min(static_cast<int64_t>(first + nb) * tokens_per_block, num_tokens) * num_topk;
    int pe[kSlotPreload];
    int32_t pl[kSlotPreload];
#pragma unroll
    for (int u = 0; u < kSlotPreload; ++u) {  // clamped, not predicated: all loads in flight at once
        const int64_t c = min(c_lo + u * NT + threadIdx.x, c_hi - 1);
        pe[u] = static_cast<int>(topk_idx[c]);
        pl[u] = pos[c];
    }
    // per expert: copies in earlier super-chunks (below) and in the batch (total); thread j < share * E takes
    // rows g, g + share, ... of expert ex (share * E <= NT: one slot per thread).  The first eight of its table
    // rows and this super-chunk's workgroup rows (contiguous, at most kSlotPreInts = 8 per thread) are loaded
    // in one straight block, indices clamped and values masked after, so all are in flight at once.
    static_assert(kSlotPreInts == 8 * NT, "eight row values per thread");
    const int jj = threadIdx.x;
    const bool has_slot = jj < share * E;
    const int g = has_slot ? jj / E : 0;
    const int ex = has_slot ? jj - g * E : 0;
    const int n_pre = nb * E;
    const int32_t* my_rows = block_rows + static_cast<int64_t>(first) * E;
    int32_t c[8], rv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        // an unsigned 32-bit offset from the uniform table base: the scalar-base load form, no 64-bit address
        // arithmetic (whose scratch high half the compiler had tied to a load's destination, stalling the batch)
        c[u] = table[static_cast<uint32_t>(min(g + u * share, rows - 1) * E + ex)];
        const int j = u * NT + threadIdx.x;
        rv[u] = my_rows[j < n_pre ? j : 0];
    }
    int32_t below = 0, total = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int r = g + u * share;
        total += r < rows ? c[u] : 0;
        below += r < s ? c[u] : 0;
    }
    for (int r = g + 8 * share; r < rows; r += share) {  // more than eight rows per thread (E > 512)
        const int32_t v = table[r * E + ex];
        total += v;
        below += r < s ? v : 0;
    }
    if (has_slot) {
        part[jj] = below;
        part[share * E + jj] = total;
    }
    if (s == 0 && threadIdx.x == 0) hdr[kWordParity] = used ^ 1u;  // the next call adds into the other table
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int j = u * NT + threadIdx.x;
        if (j < n_pre) pre[j] = rv[u];
    }
    __syncthreads();
    for (int ex = threadIdx.x; ex < E; ex += NT) {
        int32_t below = 0, total = 0;
        for (int g = 0; g < share; ++g) {
            below += part[g * E + ex];
            total += part[share * E + g * E + ex];
        }
        run[ex] = below;
        tot[ex] = total;
        int32_t acc = 0;  // exclusive prefix over the super-chunk's workgroups
        for (int r = 0; r < nb; ++r) {
            const int32_t v = pre[r * E + ex];
            pre[r * E + ex] = acc;
            acc += v;
        }
    }
    __syncthreads();
    // offsets (super-chunk 0 writes counts and offsets); run[e] += offset[e]
    offsets_from_totals<NT>(tot, run, scan, E, 1, s, rows, s == 0, counts, offsets, nullptr, 0);
    const int64_t routed = num_tokens * num_topk;
    for (int64_t c0 = c_lo; c0 < c_hi; c0 += static_cast<int64_t>(kSlotPreload) * NT) {
#pragma unroll
        for (int u = 0; u < kSlotPreload; ++u) {
            const int64_t c = c0 + u * NT + threadIdx.x;
            if (c >= c_hi) break;
            int e = pe[u];
            int32_t local = pl[u];
            if (c0 != c_lo) {  // beyond the preloaded copies
                e = static_cast<int>(topk_idx[c]);
                local = pos[c];
            }
            const int64_t t = c / num_topk;
            const int bl = static_cast<int>(t / tokens_per_block) - first;
            const int32_t p = run[e] + pre[bl * E + e] + local;
            pos[c] = p;
            if (row_token != nullptr && p >= 0 && p < routed) row_token[p] = static_cast<int32_t>(t);
        }
    }
}

int isqrt_ceil(int n) {
    int r = 1;
    while (r * r < n) ++r;
    return r;
}

// Workgroups per super-chunk: about the square root of the grid (so both the table rows and a super-chunk's
// workgroups stay near it), at most what the slot kernel's LDS holds (group x E <= kSlotPreInts).
int route_group(int64_t blocks, int num_experts) {
    const int g = isqrt_ceil(static_cast<int>(blocks));
    if (blocks <= kSlotBlockMax) return g;  // the per-workgroup slot kernel: no LDS cap
    const int cap = kSlotPreInts / num_experts;
    return g < cap ? g : cap;
}

template <int NT, int P, bool VEC>
hipError_t launch_route_t(const float* scores, int64_t T, int E, int K, bool renorm, int64_t* idx, float* w,
                          int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_token, int32_t* super_rows,
                          int32_t* block_rows, uint32_t* hdr, hipStream_t stream) {
    constexpr int W = NT / kWave;
    const int blocks = static_cast<int>((T + W - 1) / W);
    const int group = route_group(blocks, E);
    const int rows = (blocks + group - 1) / group;  // <= kRouteSuperRows (route_fused_fits)
    hipLaunchKernelGGL((route_count_kernel<NT, P, VEC>), dim3(static_cast<unsigned>(blocks)), dim3(NT),
                       W * E * sizeof(uint16_t), stream, scores, T, E, K, renorm ? 1 : 0, idx, w, group, pos,
                       super_rows, block_rows, hdr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (blocks <= kSlotBlockMax) {
        const int share_ints = 2 * (E > NT ? E : NT);
        const size_t lds = (share_ints + 2 * E + W + 1) * sizeof(int32_t);
        hipLaunchKernelGGL((route_slot_block_kernel<NT>), dim3(static_cast<unsigned>(blocks)), dim3(NT), lds, stream,
                           idx, T, E, K, group, share_ints, counts, offsets, pos, row_token, super_rows, block_rows,
                           hdr);
        return hipGetLastError();
    }
    const int part_ints = 2 * (E > kSlotThreads ? E : kSlotThreads);
    const size_t lds = (static_cast<size_t>(group) * E + part_ints + 2 * E + kSlotThreads / kWave + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(route_slot_group_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSlotThreads), lds, stream,
                       idx, T, E, K, W, blocks, group, counts, offsets, pos, row_token, super_rows, block_rows, hdr);
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
    const int64_t blocks = (num_tokens + w - 1) / w;
    if (num_tokens <= 0 || blocks > kRouteMaxBlocks) return false;
    const int group = route_group(blocks, num_experts);
    return (blocks + group - 1) / group <= kRouteSuperRows;
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
