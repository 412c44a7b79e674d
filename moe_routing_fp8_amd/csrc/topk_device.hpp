// Top-k gating of one token row by one wave64 ("DeepSeek open-sources
// TileKernels", section 2.1 Top-K gating; section 2, "Weight
// Normalization"), shared by the top-k kernel and the single-launch
// dispatch.
//
// K rounds of "row maximum -> lowest expert index holding it -> mask that
// expert to -inf"; round k's winner is topk_idx[t, k].  Lane l holds the
// P = E/64 (rounded up to a power of two) contiguous scores [l*P, l*P + P)
// as order-preserving 32-bit keys (-0 folded onto +0, NaN onto -inf), sorted
// once per lane (key descending, index ascending); a round is the maximum of
// the lane heads (DPP), the lowest lane holding it (ballot, find-first-set:
// lanes own ascending index ranges, so that is the lowest index) and a pop in
// that lane.  Optional weights are the selected scores, renormalised by a
// k-order fp32 sum and one IEEE division each.
#pragma once

#include <type_traits>

#include "device_utils.hpp"

// v_writelane_b32: `src` (wave-uniform) into lane `lane` of `old`, the other
// lanes unchanged.  The LLVM intrinsic has no clang builtin here; declaring
// it by name keeps it a compiler-visible instruction (scheduling, hazards).
extern "C" __device__ int moe_amdgcn_writelane(int src, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

namespace moe {
namespace topk {

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // key(-inf)

constexpr int kDppRowBcast15 = 0x142;  // lane 15 of a row -> every lane of the next row (gfx9 DPP)
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> every lane of rows 2 and 3
constexpr int kDppRowShr1 = 0x111;     // lane i - 1 of the same row (lane 0 of a row reads 0)

// Maximum over the whole wave, returned as a wave-uniform value: row maxima,
// then the two row broadcasts carry rows 0-2 into row 3, whose last lane
// holds the wave maximum.  The broadcasts run on every row: a row with no
// source row reads its own value (the lane layout measured on gfx950: row 0
// under row_bcast:15, rows 0-1 under row_bcast:31), which the maximum leaves
// unchanged, and each step then compiles to one v_max_u32_dpp instead of a
// move, a masked DPP move and a maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = row16_max_u32(x);
    x = max(x, dpp_u32<kDppRowBcast15>(x));
    x = max(x, dpp_u32<kDppRowBcast31>(x));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), kWave - 1));
}

// Order-preserving key: unsigned order of keys == IEEE order of scores, with
// -0 and +0 given one key (IEEE equality) and NaN read as -inf.  Adding +0
// turns -0 into +0 (a sum of opposite zeros rounds to +0) and leaves every
// other value, subnormals included (fp32 denormals are kept), unchanged; the
// sign mask then flips all bits of a negative value and only the sign bit of
// a positive one.
__device__ __forceinline__ uint32_t score_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    const uint32_t flip = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u;
    return (f != f) ? kKeyNegInf : (u ^ flip);
}

__device__ __forceinline__ float canon_score(float f) { return (f != f) ? -INFINITY : f; }

// Loads one score row into the lane's P keys (lane l holds [l*P, l*P + P)).
template <int P, bool VEC>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int num_experts, int lane,
                                          uint32_t (&key)[P]) {
    const int base = lane * P;
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
}

// Compare-exchange on (key, slot) pairs ordered by key descending, then slot
// ascending: a total order, so any sorting network yields the one sorted list.
__device__ __forceinline__ void cas_desc(uint32_t& ka, uint32_t& sa, uint32_t& kb, uint32_t& sb) {
    const bool swap = (kb > ka) || (kb == ka && sb < sa);
    const uint32_t k0 = swap ? kb : ka, s0 = swap ? sb : sa;
    const uint32_t k1 = swap ? ka : kb, s1 = swap ? sa : sb;
    ka = k0; sa = s0; kb = k1; sb = s1;
}

// Slot order of a lane's P keys, 4 bits per entry: 32 bits hold up to 8.
template <int P>
using perm_t = typename std::conditional<(P <= 8), uint32_t, uint64_t>::type;

// Sorts the lane's P keys; returns the slot order packed 4 bits per entry
// (entry j in bits [4j, 4j + 4)), so the head's slot is `perm & 15`.
template <int P>
__device__ __forceinline__ perm_t<P> sort_lane(uint32_t (&key)[P]) {
    uint32_t slot[P];
#pragma unroll
    for (int j = 0; j < P; ++j) slot[j] = j;
    if constexpr (P == 2) {
        cas_desc(key[0], slot[0], key[1], slot[1]);
    } else if constexpr (P == 4) {  // optimal 5-comparator network
        cas_desc(key[0], slot[0], key[1], slot[1]);
        cas_desc(key[2], slot[2], key[3], slot[3]);
        cas_desc(key[0], slot[0], key[2], slot[2]);
        cas_desc(key[1], slot[1], key[3], slot[3]);
        cas_desc(key[1], slot[1], key[2], slot[2]);
    } else if constexpr (P > 4) {  // bitonic network
#pragma unroll
        for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const int j = i ^ stride;
                    if (j > i) {
                        if ((i & size) == 0)
                            cas_desc(key[i], slot[i], key[j], slot[j]);
                        else
                            cas_desc(key[j], slot[j], key[i], slot[i]);
                    }
                }
            }
        }
    }
    perm_t<P> perm = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) perm |= static_cast<perm_t<P>>(slot[j]) << (4 * j);
    return perm;
}

// K rounds of "row maximum -> lowest index holding it -> mask to -inf" on
// lane-sorted keys.  A lane's head is its best (key, lowest index); the
// maximum over heads is the row maximum and the lowest lane holding it owns
// the lowest such index (lanes own ascending index ranges).  Masking the
// winner to -inf = popping the head.  Once the maximum is -inf every entry
// of the row is -inf (popped or not), so the lowest index holding it is 0:
// the pages' rule, reproduced exactly.  Returns, in lane k, round k's winner
// (the winner is wave-uniform, so one lane write records it).
template <int P>
__device__ __forceinline__ int select_topk(uint32_t (&key)[P], int num_topk, int lane) {
    perm_t<P> perm = sort_lane<P>(key);
    int my_idx = 0;
    for (int k = 0; k < num_topk; ++k) {
        const uint32_t m = wave_max_u32(key[0]);
        int idx = 0;
        if (m != kKeyNegInf) {
            const int win_lane = __builtin_ctzll(__ballot(key[0] == m));
            const int head_slot =
                __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(perm) & 15u), win_lane);
            idx = win_lane * P + head_slot;
            if (lane == win_lane) {
#pragma unroll
                for (int j = 0; j + 1 < P; ++j) key[j] = key[j + 1];
                key[P - 1] = kKeyNegInf;
                perm >>= 4;
            }
        }
        my_idx = moe_amdgcn_writelane(idx, k, my_idx);
    }
    return my_idx;
}

// Top-k of token t (row `scores + t * num_experts`) by the calling wave,
// without writing it: lane k < num_topk returns topk_idx[t, k] and, if
// `weights`, sets *w to that copy's weight (other lanes return unspecified
// values).
template <int P, bool VEC>
__device__ __forceinline__ int topk_row_values(const float* __restrict__ scores, int64_t t, int num_experts,
                                                int num_topk, int renormalize, bool weights, int lane, float* w) {
    const float* row = scores + t * num_experts;
    uint32_t key[P];
    load_keys<P, VEC>(row, num_experts, lane, key);
    const int my_idx = select_topk<P>(key, num_topk, lane);
    if (weights) {
        const float g = (lane < num_topk) ? canon_score(row[my_idx]) : 0.0f;
        float v = g;
        if (renormalize) {
            // k-order sum ((0 + g_0) + g_1) + ... by a lane-serial scan in row 0
            // (num_topk <= 16 lanes): step j gives lane i the value g_i + (lane
            // i - 1's value after step j - 1), lane 0 adding the shifted-in 0,
            // so after num_topk steps lane K - 1 holds the sequential sum
            // exactly (an fp32 sum of two values does not depend on their order).
            float s = 0.0f;
            for (int k = 0; k < num_topk; ++k)
                s = g + __uint_as_float(dpp_u32<kDppRowShr1>(__float_as_uint(s)));
            const float sum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), num_topk - 1));
            v = g / sum;
        }
        *w = v;
    }
    return my_idx;
}

// The same, written out: lane k < num_topk writes topk_idx[t, k] and, if
// requested, the weight, and returns that expert id.
template <int P, bool VEC>
__device__ __forceinline__ int topk_row(const float* __restrict__ scores, int64_t t, int num_experts,
                                         int num_topk, int renormalize, int64_t* __restrict__ topk_idx,
                                         float* __restrict__ topk_weights, int lane) {
    float w = 0.0f;
    const int my_idx =
        topk_row_values<P, VEC>(scores, t, num_experts, num_topk, renormalize, topk_weights != nullptr, lane, &w);
    if (lane < num_topk) {  // row bases from the wave-uniform token; 32-bit lane offsets
        (topk_idx + t * num_topk)[lane] = my_idx;
        if (topk_weights != nullptr) (topk_weights + t * num_topk)[lane] = w;
    }
    return my_idx;
}

}  // namespace topk
}  // namespace moe
