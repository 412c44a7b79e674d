// Single-launch dispatch for decode-sized batches on gfx950: top-k gating,
// the token map and the expand + e4m3 cast in one launch, with one grid
// barrier between routing and copying ("CuTeDSL at Perplexity", grid
// synchronisation: when the work fits in one wave of blocks, route, barrier
// and copy in a single launch instead of two; MoE dispatch: the decode path
// handles little routing data and then signals the rest of the grid).
//
// Results are those of moe_topk_gate -> moe_token_map -> moe_expand_cast_fp8
// bit for bit ("DeepSeek open-sources TileKernels", sections 2.1, 2, 2.2,
// 3.1, 3.2):
//
//   route   one wave per token, the top-k of topk_device.hpp; topk_idx and
//           the weights go to global memory.  The loads of each wave's first
//           bf16 chunk are issued before it, its cast after it.  Up to 32
//           tokens every workgroup routes every token itself instead (into
//           LDS, one or two tokens per wave, with routing-only waves added
//           from 5 tokens; workgroup 0 writes topk_idx and the weights), and
//           the barrier and the reload below are skipped (DeepSeek-V3 shape,
//           per call: 1 token 7.5 against 9.4 us, 16 tokens 9.3 against 11.7,
//           32 tokens 11.9 against 12.5).  Or the top-k kernel has run just
//           before on the stream (moe_dispatch's top-k-then-copy form): no
//           routing here and no barrier, the ids and weights are read from
//           memory as after the barrier.  With no channels (hidden 0) the
//           launch is the routing alone (moe_route's local form).
//   barrier every workgroup arrives (agent-scope release) at a weighted
//           counter (through one of eight group counters when there are more
//           than eight workgroups) and polls until the arrivals of this call
//           are complete, then acquires.  At most one workgroup per compute
//           unit, so all are resident on an idle device; every wait is
//           bounded and reports a time-out instead of hanging.
//   map     every workgroup copies the T*K expert ids into LDS.  One wave
//           per expert counts the ids below it and equal to it: offsets and
//           counts.  The slot of a copy is its stable counting-sort
//           position, computed directly: pos(t, k) = (copies routed to a
//           lower expert) + (copies to the same expert that come before
//           (t, k) in row-major order).  The wave of a (token, chunk) unit
//           counts both over the ids in LDS for the token's K copies, so no
//           second barrier is needed.
//   copy    one (token, 1024-channel chunk) unit per wave: the wave counts
//           the slots of the token's K copies, casts its chunk and writes the
//           K copies; no workgroup barrier, so the latencies of a
//           workgroup's four units overlap.
#include "device_utils.hpp"
#include "grid_sync.hpp"
#include "kernels.hpp"
#include "topk_device.hpp"

namespace moe {
namespace {

constexpr int kFusedWaves = 4;          // copying waves per workgroup (all of its waves with the grid barrier)
constexpr int kLocalWaves = 16;         // waves per workgroup when 5 or more tokens route locally
constexpr int kLocalMaxTokens = static_cast<int>(kDispatchLocalMaxTokens);  // two tokens per wave above 16
constexpr int kFusedMaxTopk = kKernelMaxTopk;
constexpr int kRouteBarrier = 0;  // top-k spread over the grid, then the grid barrier
constexpr int kRouteLocal = 1;    // every workgroup routes every token itself
constexpr int kRoutePrior = 2;    // routed by the top-k kernel launched just before
constexpr uint16_t kNoExpert = 0xFFFF;  // an id outside [0, E) in the LDS copy of the ids

// Grid barrier on the epoch counters of grid_sync.hpp (header zero before the
// first call).  With more than kBarGroups workgroups the arrivals go first to
// one of kBarGroups group counters on their own 128-byte lines (at most
// ceil(G / kBarGroups) same-address atomics each) and the completing arrival
// of each group goes on to the top counter.  The first member of a group
// adds kEpoch - (members - 1), every other member 1.
constexpr int kBarGroups = 8;

// Adds this member's weight to a counter; returns true if that completed the epoch.
__device__ __forceinline__ bool bar_arrive(uint32_t* ctr, bool first_member, uint32_t members) {
    const uint32_t w = first_member ? gsync::kEpoch - (members - 1u) : 1u;
    return gsync::completes(gsync::arrive(ctr, w), w);
}

// Grid-wide barrier; returns false (for the whole workgroup) if the wait
// timed out, after setting the error word.
__device__ bool grid_barrier(uint32_t* __restrict__ bar, uint32_t num_blocks, int* ok_lds) {
    gsync::wave_stores_done();  // every wave's global writes are in the L2
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        uint32_t* top = bar + gsync::kWordBarrierTop;
        // the top counter is below the next epoch until this workgroup arrives
        const uint32_t base =
            gsync::epoch_base(__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        __threadfence();  // release the workgroup's writes device-wide
        const uint32_t groups = num_blocks < kBarGroups ? num_blocks : kBarGroups;
        const uint32_t g = blockIdx.x % groups;
        const uint32_t members = num_blocks / groups + (g < num_blocks % groups ? 1u : 0u);
        bool go_up = true;
        if (members > 1) go_up = bar_arrive(bar + gsync::kWordBarrierGroup0 * (g + 1), blockIdx.x < groups, members);
        bool done = false;
        if (go_up) done = bar_arrive(top, g == 0, groups);
        if (!done && !gsync::wait_epoch(top, base, bar + gsync::kWordError)) ok = 0;
        __threadfence();  // acquire the other workgroups' writes
        *ok_lds = ok;
    }
    __syncthreads();
    return *ok_lds != 0;
}

// Sum over the wave, wave-uniform: row sums by DPP, then the four row totals.
__device__ __forceinline__ int32_t wave_sum_i32(int32_t x) {
    uint32_t v = static_cast<uint32_t>(x);
    v += dpp_u32<kDppQuadXor1>(v);
    v += dpp_u32<kDppQuadXor2>(v);
    v += dpp_u32<kDppRowHalfMirror>(v);
    v += dpp_u32<kDppRowMirror>(v);
    const int32_t s = __builtin_amdgcn_readlane(static_cast<int>(v), 0) +
                      __builtin_amdgcn_readlane(static_cast<int>(v), 16) +
                      __builtin_amdgcn_readlane(static_cast<int>(v), 32) +
                      __builtin_amdgcn_readlane(static_cast<int>(v), 48);
    return s;
}

template <int P, bool VEC, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void dispatch_fused_kernel(
    const float* __restrict__ scores, const uint16_t* __restrict__ x, int64_t num_tokens,
    int num_experts, int num_topk, int hidden, int renormalize, int64_t* topk_idx,
    float* topk_weights, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token, uint8_t* __restrict__ out,
    float* __restrict__ out_sf, float* __restrict__ out_weights, uint32_t* __restrict__ bar, int route_mode) {
    // route_mode: kRouteBarrier, kRouteLocal, or kRoutePrior (topk_idx and the weights written by an earlier
    // launch on the stream: no routing here, no barrier)
    const bool local_route = route_mode == kRouteLocal;
    // [T*K padded to 8] expert ids; with local routing, then [T*K] weights
    extern __shared__ __attribute__((aligned(16))) uint16_t ids[];
    __shared__ int ok;
    constexpr int NT = WAVES * kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int E = num_experts;
    const int K = num_topk;
    const int V = hidden >> 4;               // 16-channel vectors per row
    const int G = hidden >> 7;               // 128-channel groups per row
    // 1024-channel chunks per row; with no channels (hidden 0: the routing
    // alone) one unit per token still writes its copies' slots
    const int CH = V > 0 ? (V + kWave - 1) / kWave : 1;
    const int64_t units = num_tokens * CH;
    // waves 0 .. kFusedWaves - 1 of a workgroup copy (and, through the grid
    // barrier, route); further waves (WAVES = 16) only route locally
    const int64_t num_waves = static_cast<int64_t>(gridDim.x) * kFusedWaves;
    const int64_t u0 = static_cast<int64_t>(blockIdx.x) * kFusedWaves + wave;

    // ---- the cast of this wave's first unit does not depend on routing:
    // its loads are issued before the top-k's, its arithmetic after
    uint4 ra = make_uint4(0u, 0u, 0u, 0u), rb = ra;
    int v0 = V;  // no first unit
    if (wave < kFusedWaves && u0 < units) {
        const int64_t t = u0 / CH;
        v0 = static_cast<int>(u0 - t * CH) * kWave + lane;
        if (v0 < V) {
            const uint4* xr = reinterpret_cast<const uint4*>(x + t * hidden);
            ra = load_stream16(xr + 2 * v0);
            rb = load_stream16(xr + 2 * v0 + 1);
        }
    }

    const int32_t N = static_cast<int32_t>(num_tokens * K);  // <= 16384
    const int32_t n_pad = (N + 7) & ~7;
    float* wts = reinterpret_cast<float*>(ids + n_pad);  // local routing only
    uint4 q0 = make_uint4(0u, 0u, 0u, 0u);
    float sf0 = 0.0f;

    if (local_route) {
        // ---- route locally: every workgroup computes the top-k of every
        // token (T <= WAVES: wave t takes token t) into LDS, the same
        // values in every workgroup; workgroup 0 alone writes topk_idx and the
        // weights.  No workgroup reads another's results: no grid barrier.
        for (int t = wave; t < num_tokens; t += WAVES) {
            float w = 0.0f;
            const int my =
                topk::topk_row_values<P, VEC>(scores, t, E, K, renormalize, topk_weights != nullptr, lane, &w);
            if (lane < K) {
                ids[t * K + lane] = static_cast<uint16_t>(my);  // in [0, E)
                wts[t * K + lane] = w;
                if (blockIdx.x == 0) {
                    topk_idx[t * K + lane] = my;
                    if (topk_weights != nullptr) topk_weights[t * K + lane] = w;
                }
            }
        }
        for (int32_t j = N + static_cast<int32_t>(threadIdx.x); j < n_pad; j += NT) ids[j] = kNoExpert;
        if (v0 < V) cast16_e4m3_raw(ra, rb, q0, sf0);  // whole 8-lane groups (V % 8 == 0)
        __syncthreads();
        if (wave >= kFusedWaves) return;  // a routing-only wave: no barrier follows
    } else {
        // ---- route: one wave per token, then the grid barrier (with
        // kRoutePrior the ids are already in memory: neither)
        if (route_mode == kRouteBarrier)
            for (int64_t t = u0; t < num_tokens; t += num_waves)
                topk::topk_row<P, VEC>(scores, t, E, K, renormalize, topk_idx, topk_weights, lane);

        if (v0 < V) cast16_e4m3_raw(ra, rb, q0, sf0);  // whole 8-lane groups (V % 8 == 0)

        if (route_mode == kRouteBarrier && !grid_barrier(bar, gridDim.x, &ok)) return;

        // ---- all T*K ids into LDS, loads of four per thread in flight; the
        // padding up to a multiple of 8 entries reads as no expert
        for (int32_t j0 = 0; j0 < n_pad; j0 += 4 * NT) {
            int64_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t j = j0 + i * NT + threadIdx.x;
                e[i] = j < N ? topk_idx[j] : -1;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t j = j0 + i * NT + threadIdx.x;
                if (j < n_pad) ids[j] = (e[i] >= 0 && e[i] < E) ? static_cast<uint16_t>(e[i]) : kNoExpert;
            }
        }
        __syncthreads();
    }

    // ---- counts and offsets: offsets[e] = valid ids below e, counts[e] =
    // ids equal to e (e = E gives the total).  Few ids: one expert per lane,
    // every lane reading all ids (LDS broadcasts, 8 per read); else one
    // expert per wave, its lanes splitting the ids.
    const int64_t experts = static_cast<int64_t>(E) + 1;
    const int64_t lane_cost = 5 * static_cast<int64_t>(N) * ((experts + kWave * num_waves - 1) / (kWave * num_waves));
    const int64_t wave_cost = ((experts + num_waves - 1) / num_waves) * (6 * ((N + kWave - 1) / kWave) + 40);
    if (lane_cost <= wave_cost) {
        const uint4* ids8 = reinterpret_cast<const uint4*>(ids);
        for (int64_t e0 = u0 * kWave; e0 < experts; e0 += num_waves * kWave) {
            const int e = static_cast<int>(e0) + lane;
            int32_t below = 0, equal = 0;
            for (int32_t j8 = 0; j8 < n_pad / 8; ++j8) {
                const uint4 w = ids8[j8];
                const uint32_t pair[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int a = static_cast<int>(pair[i] & 0xFFFFu), b = static_cast<int>(pair[i] >> 16);
                    below += (a < e ? 1 : 0) + (b < e ? 1 : 0);  // kNoExpert > E: never below
                    equal += (a == e ? 1 : 0) + (b == e ? 1 : 0);
                }
            }
            if (e < experts) {
                offsets[e] = below;
                if (e < E) counts[e] = equal;
            }
        }
    } else {
        for (int64_t e = u0; e < experts; e += num_waves) {
            int32_t below = 0, equal = 0;
#pragma unroll 4
            for (int32_t j = lane; j < N; j += kWave) {
                const int id = ids[j];
                below += id < e ? 1 : 0;
                equal += id == e ? 1 : 0;
            }
            below = wave_sum_i32(below);
            equal = wave_sum_i32(equal);
            if (lane == 0) {
                offsets[e] = below;
                if (e < E) counts[e] = equal;
            }
        }
    }

    // ---- slots and copies: one (token, 1024-channel chunk) unit per wave
    for (int64_t u = u0; u < units; u += num_waves) {
        const int64_t t = u / CH;
        const int chunk = static_cast<int>(u - t * CH);
        const int32_t first = static_cast<int32_t>(t * K);
        // Copies are ordered by key = expert * N + (row-major copy index), a
        // total order (N * E < 2^31); the slot of copy k is the number of
        // valid keys below its own.
        int32_t key[kFusedMaxTopk];
        int32_t c[kFusedMaxTopk];
#pragma unroll
        for (int k = 0; k < kFusedMaxTopk; ++k) {
            const int e = k < K ? ids[first + k] : kNoExpert;
            key[k] = e != kNoExpert ? e * N + first + k : -1;
            c[k] = 0;
        }
#pragma unroll 4
        for (int32_t j = lane; j < N; j += kWave) {
            // an invalid id (kNoExpert) keys above every valid key: never counted
            const int32_t kj = static_cast<int32_t>(ids[j]) * N + j;  // < 2^16 * 2^14
#pragma unroll
            for (int k = 0; k < kFusedMaxTopk; ++k)
                if (k < K) c[k] += kj < key[k] ? 1 : 0;
        }
        const int v = chunk * kWave + lane;
        uint4 q = q0;
        float sf = sf0;
        if (u != u0 && v < V)  // later units: cast now
            cast16_e4m3<true>(reinterpret_cast<const uint4*>(x + t * hidden), v, q, sf);
#pragma unroll
        for (int k = 0; k < kFusedMaxTopk; ++k) {
            if (k >= K) continue;  // uniform
            const int32_t slot = wave_sum_i32(c[k]);
            if (key[k] < 0) {
                if (chunk == 0 && lane == 0) pos[first + k] = -1;
            } else {
                const int64_t r = slot;
                if (v < V) {
                    store_stream16(reinterpret_cast<uint4*>(out + r * hidden + static_cast<int64_t>(v) * 16), q);
                    if ((v & 7) == 0) out_sf[r * G + (v >> 3)] = sf;
                }
                if (chunk == 0 && lane == 0) {
                    pos[first + k] = slot;
                    if (row_token != nullptr) row_token[r] = static_cast<int32_t>(t);
                    if (out_weights != nullptr) out_weights[r] = local_route ? wts[first + k] : topk_weights[first + k];
                }
            }
        }
    }
}

template <int P, bool VEC>
hipError_t launch_fused_p(const float* scores, const uint16_t* x, int64_t T, int E, int K, int H,
                          bool renorm, int64_t* idx, float* w, int32_t* counts, int32_t* offsets,
                          int32_t* pos, int32_t* row_token, uint8_t* out, float* out_sf, float* out_w,
                          uint32_t* bar, bool prior, hipStream_t stream) {
    if (prior) {  // the ids and weights come from the top-k launch before this one
        const unsigned grid = static_cast<unsigned>(fused_dispatch_grid(T, H, E));
        const size_t lds = (static_cast<size_t>(T) * K + 7) / 8 * 16;
        hipLaunchKernelGGL((dispatch_fused_kernel<P, VEC, kFusedWaves>), dim3(grid), dim3(kFusedWaves * kWave), lds,
                           stream, scores, x, T, E, K, H, renorm ? 1 : 0, idx, w, counts, offsets, pos, row_token,
                           out, out_sf, out_w, bar, kRoutePrior);
        return hipGetLastError();
    }
    // up to kLocalMaxTokens tokens every workgroup routes all of them itself, one token per wave: four-wave
    // workgroups up to four tokens, sixteen-wave ones above (whose first four waves copy, so the copy units
    // spread over as many workgroups as with four)
    const bool local = T <= kLocalMaxTokens;
    const int waves = (local && T > kFusedWaves) ? kLocalWaves : kFusedWaves;
    const unsigned grid = static_cast<unsigned>(fused_dispatch_grid(T, H, E));
    const size_t n = static_cast<size_t>(T) * K;
    const size_t lds = (n + 7) / 8 * 16 + (local ? n * sizeof(float) : 0);  // ids padded to 8 entries, weights
    if (waves == kLocalWaves) {
        hipLaunchKernelGGL((dispatch_fused_kernel<P, VEC, kLocalWaves>), dim3(grid), dim3(kLocalWaves * kWave),
                           lds, stream, scores, x, T, E, K, H, renorm ? 1 : 0, idx, w, counts, offsets, pos,
                           row_token, out, out_sf, out_w, bar, kRouteLocal);
    } else {
        hipLaunchKernelGGL((dispatch_fused_kernel<P, VEC, kFusedWaves>), dim3(grid), dim3(kFusedWaves * kWave), lds,
                           stream, scores, x, T, E, K, H, renorm ? 1 : 0, idx, w, counts, offsets, pos, row_token,
                           out, out_sf, out_w, bar, local ? kRouteLocal : kRouteBarrier);
    }
    return hipGetLastError();
}

template <int P>
hipError_t launch_fused_v(bool vec, const float* scores, const uint16_t* x, int64_t T, int E, int K, int H,
                          bool renorm, int64_t* idx, float* w, int32_t* counts, int32_t* offsets,
                          int32_t* pos, int32_t* row_token, uint8_t* out, float* out_sf, float* out_w,
                          uint32_t* bar, bool prior, hipStream_t stream) {
    if (vec)
        return launch_fused_p<P, true>(scores, x, T, E, K, H, renorm, idx, w, counts, offsets, pos, row_token,
                                       out, out_sf, out_w, bar, prior, stream);
    return launch_fused_p<P, false>(scores, x, T, E, K, H, renorm, idx, w, counts, offsets, pos, row_token,
                                    out, out_sf, out_w, bar, prior, stream);
}

}  // namespace

int64_t fused_dispatch_grid(int64_t num_tokens, int hidden, int num_experts) {
    const int64_t chunks = (hidden / 16 + kWave - 1) / kWave;
    const int64_t route_blocks = (num_tokens + kFusedWaves - 1) / kFusedWaves;
    const int64_t copy_blocks = (num_tokens * chunks + kFusedWaves - 1) / kFusedWaves;
    // the routing alone (no channels): a copying wave per expert for the counts and offsets (with a few
    // waves, each scanning many experts in turn, 24 tokens took 12.3 against 10.5 us with the copies)
    const int64_t count_blocks = hidden == 0 ? (num_experts + 1 + kFusedWaves - 1) / kFusedWaves : 0;
    int64_t want = route_blocks > copy_blocks ? route_blocks : copy_blocks;
    want = want > count_blocks ? want : count_blocks;
    const int64_t cus = device_cu_count();  // the hardware count: residency depends on it
    return want < cus ? (want > 0 ? want : 1) : cus;
}

hipError_t launch_dispatch_fused(const float* scores, const uint16_t* x, int64_t T, int E, int K, int H,
                                 bool renormalize, int64_t* topk_idx, float* topk_weights,
                                 int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_token,
                                 uint8_t* out, float* out_sf, float* out_weights, uint32_t* barrier,
                                 bool after_topk, hipStream_t stream) {
    if (after_topk) {  // the split top-k first, then the map and the copies in one launch without a barrier
        const hipError_t err = launch_topk_gate(scores, T, E, K, renormalize, topk_idx, topk_weights, stream);
        if (err != hipSuccess) return err;
    }
    const bool aligned16 = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
    const bool vec4 = aligned16 && (E % 4 == 0);
#define MOE_FUSED_ARGS scores, x, T, E, K, H, renormalize, topk_idx, topk_weights, counts, offsets, pos, \
                       row_token, out, out_sf, out_weights, barrier, after_topk, stream
    if (E <= 64) return launch_fused_v<1>(false, MOE_FUSED_ARGS);
    if (E <= 128) return launch_fused_v<2>(false, MOE_FUSED_ARGS);
    if (E <= 256) return launch_fused_v<4>(vec4, MOE_FUSED_ARGS);
    if (E <= 512) return launch_fused_v<8>(vec4, MOE_FUSED_ARGS);
    return launch_fused_v<16>(vec4, MOE_FUSED_ARGS);
#undef MOE_FUSED_ARGS
}

}  // namespace moe
