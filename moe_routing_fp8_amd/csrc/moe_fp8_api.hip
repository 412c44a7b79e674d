// C-ABI entry points of libmoe_fp8.so (declared in include/moe_fp8.h).
//
// Every entry point validates its arguments on the host before any HIP call
// and returns a status code; no exception crosses the ABI.  Kernels are
// enqueued on the caller's stream; the library allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_common.hpp"
#include "kernels.hpp"
#include "moe_fp8.h"

static_assert(moe::kMaxTopk <= moe::kKernelMaxTopk, "the top-k kernels keep a token's K in one 16-lane row");

namespace {

thread_local int g_last_hip_error = 0;

using moe::aligned;
using moe::hip_status;
using moe::kMaxExperts;
using moe::kMaxTopk;
constexpr int kGroup = 128;
constexpr int kMaxAlign = 4096;  // segment alignment (rows) of the aligned map
// moe_dispatch and moe_route workspace: the 2048-byte header of counters,
// then the one-launch routing's super-chunk table (zero between calls), then
// the token map's count table or the one-launch routing's per-workgroup
// counts (both rewritten by every call that uses them).
constexpr size_t kDispatchHeaderBytes = 2048;
constexpr size_t kRouteTablesOffset = kDispatchHeaderBytes + moe::kRouteSuperBytes;
// moe_route AUTO takes the fused form above this many routed copies (graph replay, DeepSeek-V3 shape, whole
// dispatch: 64 tokens 14.1 against 13.4 us split, 128 tokens 14.8 against 14.6, 256 tokens 16.1 against 17.8)
constexpr int64_t kRouteAutoMinCopies = 1024;
// ... and while its grid is at most this many workgroups per compute unit (16384 tokens on 256 compute units
// at E <= 512): past that its 1024-thread count workgroups run the top-k in more rounds than the split top-k.
constexpr int64_t kRouteAutoBlocksPerCu = 4;
// moe_dispatch AUTO takes the single launch (local routing) up to this many tokens (at most
// moe::kDispatchLocalMaxTokens); the crossover with the top-k-then-copy form measured between 24 and 32.
constexpr int64_t kDispatchAutoLocalTokens = 24;
// moe_route AUTO takes its one-launch local form up to this many tokens (at most
// moe::kDispatchLocalMaxTokens): graph replay, DeepSeek-V3 scores, 1 token 6.6 against 7.4 us split, 8 tokens
// 6.8 against 7.7, 16 tokens 7.7 against 7.9; above, where a wave routes two tokens, the split form is faster
// (24: 9.1 against 8.0, 32: 10.3 against 8.2).
constexpr int64_t kRouteAutoLocalTokens = 16;
static_assert(kDispatchAutoLocalTokens <= moe::kDispatchLocalMaxTokens, "local routing only");
// uint32 index, in that header, of the word a timed-out barrier wait sets.
constexpr int kDispatchTimeoutWord = 2;
// Single-launch form: every workgroup holds all T*K expert ids in LDS
// (2 bytes each) and every copy unit counts over them.
constexpr int64_t kFusedMaxCopies = 16384;
// One workgroup per token / row: the grid x-dimension times the workgroup
// size must stay below 2^32 work-items.
constexpr int64_t kMaxRowsPerLaunch = (int64_t{1} << 32) / 256 - 1;
constexpr int64_t kMaxFlatThreads = (int64_t{1} << 32) - 256;

// Group sizes of the e4m3 / fp32-scale entry points: 128 on the dedicated
// kernels, 16 and 32 on the block-scaled ones in the same format (the same
// scale formula: sf = max(amax, 1e-4) / 448, inv = 1 / sf).
bool e4m3_group_supported(int32_t g) { return g == 16 || g == 32 || g == kGroup; }
moe::MxFormat e4m3_format(int32_t g) { return moe::MxFormat{0, g, false, false, 0.0f}; }

}  // namespace

namespace moe {

moe_status hip_status(hipError_t err) {
    if (err == hipSuccess) return MOE_OK;
    g_last_hip_error = static_cast<int>(err);
    return MOE_ERR_HIP;
}

// The single-launch dispatch sizes its grid by this count (all its
// workgroups must be resident at once), so an unknown count reads as 1:
// slow but safe.
int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 1;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {  // an int: any value a caller passes is well defined here
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "unknown status";
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_fp8_version(void) { return 300; /* 0.3.0 */ }

moe_status moe_topk_gate(const float* scores, int64_t num_tokens, int32_t num_experts,
                         int32_t num_topk, int32_t renormalize, int64_t* topk_idx,
                         float* topk_weights, hipStream_t stream) {
    if (num_tokens < 0 || num_experts < 1 || num_experts > kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (num_topk < 1 || num_topk > num_experts || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (renormalize && topk_weights == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return MOE_OK;
    if (scores == nullptr || topk_idx == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(scores, 4) || !aligned(topk_idx, 8) || !aligned(topk_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens > kMaxRowsPerLaunch * 4) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_topk_gate(scores, num_tokens, num_experts, num_topk,
                                            renormalize != 0, topk_idx, topk_weights, stream));
}

size_t moe_token_map_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk || num_experts < 1 ||
        num_experts > kMaxExperts || num_tokens * num_topk > INT32_MAX)
        return 0;
    return moe::plan_token_map(num_tokens, num_topk, num_experts).workspace_bytes;
}

moe_status moe_token_map(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                         int32_t num_experts, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* pos, int32_t* row_token, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (num_experts < 1 || num_experts > kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens * num_topk > INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (expert_counts == nullptr || expert_offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(expert_counts, 4) || !aligned(expert_offsets, 4)) return MOE_ERR_INVALID_ARGUMENT;
    const moe::TokenMapPlan plan = moe::plan_token_map(num_tokens, num_topk, num_experts);
    if (num_tokens > 0) {
        if (topk_idx == nullptr || pos == nullptr) return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned(topk_idx, 8) || !aligned(pos, 4) || !aligned(row_token, 4))
            return MOE_ERR_INVALID_ARGUMENT;
        if (workspace == nullptr || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < plan.workspace_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    }
    return hip_status(moe::launch_token_map(topk_idx, num_tokens, num_topk, 0, num_experts, 1,
                                            expert_counts, expert_offsets, pos, row_token,
                                            num_tokens * num_topk, static_cast<int32_t*>(workspace),
                                            plan, stream));
}

moe_status moe_expand_cast_fp8(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                               int32_t num_topk, const int32_t* pos, const float* topk_weights,
                               int64_t num_rows, int32_t group_size, uint8_t* out_fp8,
                               float* out_sf, float* out_weights, hipStream_t stream) {
    if (num_tokens < 0 || hidden < 1 || num_topk < 1 || num_topk > kMaxTopk || group_size < 1)
        return MOE_ERR_INVALID_ARGUMENT;
    if (hidden % group_size != 0) return MOE_ERR_INVALID_ARGUMENT;
    if ((topk_weights == nullptr) != (out_weights == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (pos == nullptr && (num_topk != 1 || num_rows != num_tokens)) return MOE_ERR_INVALID_ARGUMENT;
    if (pos != nullptr && num_rows != num_tokens * num_topk) return MOE_ERR_INVALID_ARGUMENT;
    if (!e4m3_group_supported(group_size)) return MOE_ERR_UNSUPPORTED;
    if (num_tokens == 0) return MOE_OK;
    if (x_bf16 == nullptr || out_fp8 == nullptr || out_sf == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(x_bf16, 16) || !aligned(out_fp8, 16) || !aligned(out_sf, 4) || !aligned(pos, 4) ||
        !aligned(topk_weights, 4) || !aligned(out_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    // the grid must hold fewer than 2^32 threads: at most 128 threads per
    // 64-vector (1024-channel) chunk of a row
    const int64_t chunks_per_row = (hidden / 16 + 63) / 64;
    if (num_tokens > kMaxFlatThreads / 128 || num_tokens * chunks_per_row * 128 > kMaxFlatThreads)
        return MOE_ERR_UNSUPPORTED;
    if (group_size != kGroup)  // groups of 16 or 32: the block-scaled kernels in the same e4m3 format
        return hip_status(moe::launch_expand_cast_mx(x_bf16, num_tokens, hidden, num_topk, pos, topk_weights,
                                                     num_rows, e4m3_format(group_size), out_fp8, out_sf,
                                                     out_weights, stream));
    return hip_status(moe::launch_expand_cast_fp8(x_bf16, num_tokens, hidden, num_topk, pos,
                                                  topk_weights, num_rows, out_fp8, out_sf,
                                                  out_weights, nullptr, stream));
}

moe_status swiglu_cast_fp8(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                           const float* row_weights, float clamp_value, int32_t group_size,
                           uint8_t* out_fp8, float* out_sf, hipStream_t stream) {
    if (num_rows < 0 || inter < 1 || group_size < 1 || inter % group_size != 0)
        return MOE_ERR_INVALID_ARGUMENT;
    if (clamp_value != clamp_value) return MOE_ERR_INVALID_ARGUMENT;  // NaN clamp
    if (!e4m3_group_supported(group_size)) return MOE_ERR_UNSUPPORTED;
    if (num_rows == 0) return MOE_OK;
    if (gate_up_bf16 == nullptr || out_fp8 == nullptr || out_sf == nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(gate_up_bf16, 16) || !aligned(out_fp8, 16) || !aligned(out_sf, 4) ||
        !aligned(row_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    if (num_rows > kMaxRowsPerLaunch) return MOE_ERR_UNSUPPORTED;
    if (group_size != kGroup)
        return hip_status(moe::launch_swiglu_cast_mx(gate_up_bf16, num_rows, inter, row_weights, clamp_value,
                                                     e4m3_format(group_size), out_fp8, out_sf, stream));
    return hip_status(moe::launch_swiglu_cast_fp8(gate_up_bf16, num_rows, inter, row_weights,
                                                  clamp_value, out_fp8, out_sf, stream));
}

size_t moe_token_map_aligned_rows(int64_t num_tokens, int32_t num_topk, int32_t num_local_experts,
                                  int32_t align) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk || num_local_experts < 1 ||
        num_local_experts > kMaxExperts || align < 1 || align > kMaxAlign)
        return 0;
    const int64_t rows = num_tokens * num_topk + static_cast<int64_t>(num_local_experts) * (align - 1);
    return rows > INT32_MAX ? 0 : static_cast<size_t>(rows);
}

moe_status moe_token_map_aligned(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                                 int32_t expert_begin, int32_t expert_end, int32_t align,
                                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                                 int32_t* row_token, int64_t num_rows, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (expert_begin < 0 || expert_end <= expert_begin || expert_end - expert_begin > kMaxExperts)
        return MOE_ERR_INVALID_ARGUMENT;
    if (align < 1 || align > kMaxAlign) return MOE_ERR_INVALID_ARGUMENT;
    const int32_t num_local = expert_end - expert_begin;
    const size_t bound = moe_token_map_aligned_rows(num_tokens, num_topk, num_local, align);
    if (bound == 0 && num_tokens > 0) return MOE_ERR_INVALID_ARGUMENT;  // > 2^31 - 1 rows
    if (num_rows < static_cast<int64_t>(bound) || num_rows > INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (expert_counts == nullptr || expert_offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(expert_counts, 4) || !aligned(expert_offsets, 4) || !aligned(row_token, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    const moe::TokenMapPlan plan = moe::plan_token_map(num_tokens, num_topk, num_local);
    if (num_tokens > 0) {
        if (topk_idx == nullptr || pos == nullptr) return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned(topk_idx, 8) || !aligned(pos, 4)) return MOE_ERR_INVALID_ARGUMENT;
        if (workspace == nullptr || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < plan.workspace_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    }
    return hip_status(moe::launch_token_map(topk_idx, num_tokens, num_topk, expert_begin, num_local,
                                            align, expert_counts, expert_offsets, pos, row_token,
                                            num_rows, static_cast<int32_t*>(workspace), plan, stream));
}

moe_status moe_expand_cast_fp8_padded(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                                      int32_t num_topk, const int32_t* pos, const float* topk_weights,
                                      const int32_t* row_token, int64_t num_rows, int32_t group_size,
                                      uint8_t* out_fp8, float* out_sf, float* out_weights,
                                      hipStream_t stream) {
    if (num_tokens < 0 || hidden < 1 || num_topk < 1 || num_topk > kMaxTopk || group_size < 1)
        return MOE_ERR_INVALID_ARGUMENT;
    if (hidden % group_size != 0 || num_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
    // weights in iff weights out (with no tokens the weights may be absent)
    if (topk_weights != nullptr && out_weights == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && topk_weights == nullptr && out_weights != nullptr)
        return MOE_ERR_INVALID_ARGUMENT;
    if (group_size != kGroup) return MOE_ERR_UNSUPPORTED;
    if (num_tokens == 0 && num_rows == 0) return MOE_OK;
    if (num_tokens > 0 && (x_bf16 == nullptr || pos == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_rows > 0 && (row_token == nullptr || out_fp8 == nullptr || out_sf == nullptr))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(x_bf16, 16) || !aligned(out_fp8, 16) || !aligned(out_sf, 4) || !aligned(pos, 4) ||
        !aligned(topk_weights, 4) || !aligned(out_weights, 4) || !aligned(row_token, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    const int64_t chunks_per_row = (hidden / 16 + 63) / 64;
    if (num_tokens > kMaxFlatThreads / 128 || num_rows > kMaxFlatThreads / 128 ||
        (num_tokens + num_rows) * chunks_per_row * 128 > kMaxFlatThreads)
        return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_expand_cast_fp8(x_bf16, num_tokens, hidden, num_topk, pos,
                                                  topk_weights, num_rows, out_fp8, out_sf,
                                                  out_weights, row_token, stream));
}

size_t moe_dispatch_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk || num_experts < 1 ||
        num_experts > kMaxExperts || num_tokens * num_topk > INT32_MAX)
        return 0;
    const size_t map_bytes = moe::plan_token_map(num_tokens, num_topk, num_experts).workspace_bytes;
    const size_t rows_bytes = moe::route_fused_block_rows_bytes(num_tokens, num_experts);
    return kRouteTablesOffset + (map_bytes > rows_bytes ? map_bytes : rows_bytes);
}

size_t moe_route_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts) {
    return moe_dispatch_workspace_bytes(num_tokens, num_topk, num_experts);
}

moe_status moe_route(const float* scores, int64_t num_tokens, int32_t num_experts, int32_t num_topk,
                     int32_t renormalize, int64_t* topk_idx, float* topk_weights, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* pos, int32_t* row_token, void* workspace,
                     size_t workspace_bytes, int32_t mode, hipStream_t stream) {
    if (mode != MOE_ROUTE_AUTO && mode != MOE_ROUTE_FUSED && mode != MOE_ROUTE_SPLIT && mode != MOE_ROUTE_LOCAL)
        return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens < 0 || num_experts < 1 || num_experts > kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (num_topk < 1 || num_topk > num_experts || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (renormalize && topk_weights == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens * num_topk > INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (expert_counts == nullptr || expert_offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(expert_counts, 4) || !aligned(expert_offsets, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace == nullptr || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < moe_route_workspace_bytes(num_tokens, num_topk, num_experts))
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (num_tokens > 0) {
        if (scores == nullptr || topk_idx == nullptr || pos == nullptr) return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned(scores, 4) || !aligned(topk_idx, 8) || !aligned(topk_weights, 4) || !aligned(pos, 4) ||
            !aligned(row_token, 4))
            return MOE_ERR_INVALID_ARGUMENT;
        if (num_tokens > kMaxRowsPerLaunch * 4) return MOE_ERR_UNSUPPORTED;
    }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    // one launch in which every workgroup routes the whole batch (the single-launch dispatch's kernel with no
    // channels to copy): up to kDispatchLocalMaxTokens tokens
    const bool local_fits = num_tokens > 0 && num_tokens <= moe::kDispatchLocalMaxTokens;
    if (mode == MOE_ROUTE_LOCAL && num_tokens > 0 && !local_fits) return MOE_ERR_UNSUPPORTED;
    if (local_fits && (mode == MOE_ROUTE_LOCAL || (mode == MOE_ROUTE_AUTO && num_tokens <= kRouteAutoLocalTokens)))
        return hip_status(moe::launch_dispatch_fused(scores, nullptr, num_tokens, num_experts, num_topk, 0,
                                                     renormalize != 0, topk_idx, topk_weights, expert_counts,
                                                     expert_offsets, pos, row_token, nullptr, nullptr, nullptr,
                                                     reinterpret_cast<uint32_t*>(ws), false, stream));
    const bool one = moe::route_fused_fits(num_tokens, num_experts);
    if (mode == MOE_ROUTE_FUSED && num_tokens > 0 && !one) return MOE_ERR_UNSUPPORTED;
    // AUTO: the fused form above kRouteAutoMinCopies routed copies (up to there the split form is two short
    // launches, the map in one workgroup, and measured as fast or faster) while its grid is at most
    // kRouteAutoBlocksPerCu workgroups per compute unit (E = 256, K = 8, graph replay: 16384 tokens 19.6
    // against 21.3 us split, 24576 tokens 24.9 against 24.6, 32768 tokens 30.4 against 28.9)
    const int64_t tpb = moe::route_fused_tokens_per_block(num_experts);
    const bool auto_fused =
        num_tokens * num_topk > kRouteAutoMinCopies &&
        (num_tokens + tpb - 1) / tpb <= kRouteAutoBlocksPerCu * static_cast<int64_t>(moe::device_cu_count());
    const bool take_one = mode == MOE_ROUTE_FUSED || (mode == MOE_ROUTE_AUTO && auto_fused);
    if (one && take_one)
        return hip_status(moe::launch_route_fused(
            scores, num_tokens, num_experts, num_topk, renormalize != 0, topk_idx, topk_weights, expert_counts,
            expert_offsets, pos, row_token, reinterpret_cast<int32_t*>(ws + kDispatchHeaderBytes),
            reinterpret_cast<int32_t*>(ws + kRouteTablesOffset), reinterpret_cast<uint32_t*>(ws), stream));
    const moe_status st = moe_topk_gate(scores, num_tokens, num_experts, num_topk, renormalize, topk_idx,
                                        topk_weights, stream);
    if (st != MOE_OK) return st;
    return moe_token_map(topk_idx, num_tokens, num_topk, num_experts, expert_counts, expert_offsets, pos,
                         row_token, ws + kRouteTablesOffset, workspace_bytes - kRouteTablesOffset, stream);
}

moe_status moe_dispatch(const float* scores, const uint16_t* x_bf16, int64_t num_tokens,
                        int32_t num_experts, int32_t num_topk, int32_t hidden, int32_t renormalize,
                        int32_t group_size, int64_t* topk_idx, float* topk_weights,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                        int32_t* row_token, uint8_t* out_fp8, float* out_sf, float* out_weights,
                        void* workspace, size_t workspace_bytes, int32_t mode, hipStream_t stream) {
    if (mode != MOE_DISPATCH_AUTO && mode != MOE_DISPATCH_SINGLE_LAUNCH && mode != MOE_DISPATCH_SPLIT &&
        mode != MOE_DISPATCH_ROUTE_FUSED && mode != MOE_DISPATCH_TOPK_THEN_COPY)
        return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens < 0 || num_experts < 1 || num_experts > kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (num_topk < 1 || num_topk > num_experts || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (renormalize && topk_weights == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if ((topk_weights == nullptr) != (out_weights == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (hidden < 1 || group_size < 1 || hidden % group_size != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (group_size != kGroup) return MOE_ERR_UNSUPPORTED;
    if (num_tokens * num_topk > INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (expert_counts == nullptr || expert_offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(expert_counts, 4) || !aligned(expert_offsets, 4)) return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = moe_dispatch_workspace_bytes(num_tokens, num_topk, num_experts);
    if (workspace == nullptr || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (num_tokens > 0) {
        if (scores == nullptr || x_bf16 == nullptr || topk_idx == nullptr || pos == nullptr ||
            out_fp8 == nullptr || out_sf == nullptr)
            return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned(scores, 4) || !aligned(x_bf16, 16) || !aligned(topk_idx, 8) ||
            !aligned(topk_weights, 4) || !aligned(pos, 4) || !aligned(row_token, 4) ||
            !aligned(out_fp8, 16) || !aligned(out_sf, 4) || !aligned(out_weights, 4))
            return MOE_ERR_INVALID_ARGUMENT;
    }
    const int64_t copies = num_tokens * num_topk;
    const bool fits_one_launch = num_tokens > 0 && copies <= kFusedMaxCopies;
    bool single = false, after_topk = false;
    if (mode == MOE_DISPATCH_SINGLE_LAUNCH || mode == MOE_DISPATCH_TOPK_THEN_COPY) {
        if (num_tokens > 0 && !fits_one_launch) return MOE_ERR_UNSUPPORTED;
        single = num_tokens > 0;  // no tokens: the routed path below zeroes counts and offsets, as in every mode
        after_topk = mode == MOE_DISPATCH_TOPK_THEN_COPY;
    } else if (mode == MOE_DISPATCH_AUTO) {
        // measured against each other under graph replay, DeepSeek-V3 shape
        // (us per call at 16 / 32 / 64 / 128 tokens): the single launch
        // routing locally 9.3 / 11.9 / - / -, the top-k kernel then the map
        // and copies 10.6 / 10.7 / 11.7 / 13.9, split 11.7 / 11.8 / 13.5 /
        // 14.8, fused routing 13.1 / 13.7 / 14.0 / 14.7 (and from 192 tokens
        // the fastest): the first up to kDispatchAutoLocalTokens tokens, the
        // second up to kRouteAutoMinCopies routed copies, then moe_route AUTO
        single = fits_one_launch &&
                 (num_tokens <= kDispatchAutoLocalTokens || copies <= kRouteAutoMinCopies);
        after_topk = single && num_tokens > kDispatchAutoLocalTokens;
    }
    if (single)
        return hip_status(moe::launch_dispatch_fused(
            scores, x_bf16, num_tokens, num_experts, num_topk, hidden, renormalize != 0, topk_idx,
            topk_weights, expert_counts, expert_offsets, pos, row_token, out_fp8, out_sf, out_weights,
            static_cast<uint32_t*>(workspace), after_topk, stream));
    const int32_t route_mode = mode == MOE_DISPATCH_SPLIT          ? MOE_ROUTE_SPLIT
                               : mode == MOE_DISPATCH_ROUTE_FUSED ? MOE_ROUTE_FUSED
                                                                   : MOE_ROUTE_AUTO;
    const moe_status st = moe_route(scores, num_tokens, num_experts, num_topk, renormalize, topk_idx,
                                    topk_weights, expert_counts, expert_offsets, pos, row_token, workspace,
                                    workspace_bytes, route_mode, stream);
    if (st != MOE_OK || num_tokens == 0) return st;
    return moe_expand_cast_fp8(x_bf16, num_tokens, hidden, num_topk, pos, topk_weights, copies, group_size,
                               out_fp8, out_sf, out_weights, stream);
}

// Checks a block-scaled format and converts it; false if invalid.
static bool check_format(const moe_cast_format* f, moe::MxFormat& out) {
    if (f == nullptr) return false;
    if (f->dtype != MOE_FMT_E4M3 && f->dtype != MOE_FMT_E2M1) return false;
    if (f->group_size != 16 && f->group_size != 32 && f->group_size != 128) return false;
    if ((f->round_sf != 0 && f->round_sf != 1) || (f->sf_ue8m0 != 0 && f->sf_ue8m0 != 1)) return false;
    if (f->sf_ue8m0 && !f->round_sf) return false;  // UE8M0 holds powers of two only
    const float maxv = f->dtype == MOE_FMT_E2M1 ? 6.0f : 448.0f;
    if (f->clamp_min != f->clamp_min) return false;  // NaN
    // a custom clamp keeps the scale a normal fp32 number, at most 2^126
    if (f->clamp_min > 0.0f && (f->clamp_min < maxv * 0x1p-126f || f->clamp_min > 0x1p126f))
        return false;
    out.dtype = f->dtype;
    out.group_size = f->group_size;
    out.round_sf = f->round_sf != 0;
    out.sf_ue8m0 = f->sf_ue8m0 != 0;
    out.clamp_min = f->clamp_min > 0.0f ? f->clamp_min : 0.0f;
    return true;
}

moe_status moe_expand_cast(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden, int32_t num_topk,
                           const int32_t* pos, const float* topk_weights, int64_t num_rows,
                           const moe_cast_format* format, uint8_t* out, void* out_sf, float* out_weights,
                           hipStream_t stream) {
    moe::MxFormat f;
    if (!check_format(format, f)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens < 0 || hidden < 1 || num_topk < 1 || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (hidden % f.group_size != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (f.dtype == MOE_FMT_E2M1 && hidden % 32 != 0) return MOE_ERR_UNSUPPORTED;  // 32 channels per lane
    if ((topk_weights == nullptr) != (out_weights == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (pos == nullptr && (num_topk != 1 || num_rows != num_tokens)) return MOE_ERR_INVALID_ARGUMENT;
    if (pos != nullptr && num_rows != num_tokens * num_topk) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return MOE_OK;
    if (x_bf16 == nullptr || out == nullptr || out_sf == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(x_bf16, 16) || !aligned(out, 16) || !aligned(out_sf, f.sf_ue8m0 ? 1 : 4) ||
        !aligned(pos, 4) || !aligned(topk_weights, 4) || !aligned(out_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    const int64_t chunks_per_row = (hidden / 16 + 63) / 64;
    if (num_tokens > kMaxFlatThreads / 128 || num_tokens * chunks_per_row * 128 > kMaxFlatThreads)
        return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_expand_cast_mx(x_bf16, num_tokens, hidden, num_topk, pos, topk_weights,
                                                 num_rows, f, out, out_sf, out_weights, stream));
}

moe_status swiglu_cast(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                       const float* row_weights, float clamp_value, const moe_cast_format* format,
                       uint8_t* out, void* out_sf, hipStream_t stream) {
    moe::MxFormat f;
    if (!check_format(format, f)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_rows < 0 || inter < 1 || inter % f.group_size != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (clamp_value != clamp_value) return MOE_ERR_INVALID_ARGUMENT;  // NaN clamp
    if (num_rows == 0) return MOE_OK;
    if (gate_up_bf16 == nullptr || out == nullptr || out_sf == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    const uintptr_t out_align = f.dtype == MOE_FMT_E2M1 ? 4 : 8;
    if (!aligned(gate_up_bf16, 16) || !aligned(out, out_align) || !aligned(out_sf, f.sf_ue8m0 ? 1 : 4) ||
        !aligned(row_weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    if (num_rows > kMaxRowsPerLaunch) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_swiglu_cast_mx(gate_up_bf16, num_rows, inter, row_weights, clamp_value, f, out,
                                                 out_sf, stream));
}

moe_status moe_combine(const uint16_t* y_rows_bf16, int64_t num_rows, int32_t hidden,
                       const int32_t* pos, const float* weights, int64_t num_tokens, int32_t num_topk,
                       uint16_t* out_bf16, hipStream_t stream) {
    if (num_rows < 0 || num_tokens < 0 || hidden < 8 || hidden % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (num_topk < 1 || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return MOE_OK;
    if (pos == nullptr || out_bf16 == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (num_rows > 0 && y_rows_bf16 == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(y_rows_bf16, 16) || !aligned(out_bf16, 16) || !aligned(pos, 4) || !aligned(weights, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    // one thread per 8 channels: the grid must hold fewer than 2^32 threads
    if (num_tokens > kMaxFlatThreads || num_tokens * (hidden / 8) > kMaxFlatThreads)
        return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_combine(y_rows_bf16, num_rows, hidden, pos, weights, num_tokens,
                                          num_topk, out_bf16, stream));
}

moe_status moe_check_scores(const float* scores, int64_t num_tokens, int32_t num_experts,
                            int32_t require_positive, uint32_t* flags, hipStream_t stream) {
    if (num_tokens < 0 || num_experts < 1 || num_experts > kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (require_positive != 0 && require_positive != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens > INT64_MAX / kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (flags == nullptr || !aligned(flags, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return MOE_OK;
    if (scores == nullptr || !aligned(scores, 4)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_check_scores(scores, num_tokens, num_experts, require_positive != 0, flags,
                                               stream));
}

moe_status moe_check_topk_idx(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                              int32_t num_experts, uint32_t* flags, hipStream_t stream) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (num_experts < 1 || num_experts > kMaxExperts) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens > INT64_MAX / kMaxTopk) return MOE_ERR_INVALID_ARGUMENT;
    if (flags == nullptr || !aligned(flags, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return MOE_OK;
    if (topk_idx == nullptr || !aligned(topk_idx, 8)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_check_topk_idx(topk_idx, num_tokens, num_topk, num_experts, flags, stream));
}

size_t moe_check_pos_workspace_bytes(int64_t num_rows) {
    if (num_rows <= 0 || num_rows > INT64_MAX - 31) return 0;
    return static_cast<size_t>((num_rows + 31) / 32) * 4;
}

moe_status moe_check_pos(const int32_t* pos, int64_t num_tokens, int32_t num_topk, int64_t num_rows,
                         void* workspace, size_t workspace_bytes, uint32_t* flags, hipStream_t stream) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk || num_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens > INT64_MAX / kMaxTopk || num_rows > INT64_MAX - 31) return MOE_ERR_INVALID_ARGUMENT;
    if (flags == nullptr || !aligned(flags, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return MOE_OK;
    if (pos == nullptr || !aligned(pos, 4)) return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = moe_check_pos_workspace_bytes(num_rows);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 4))) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(moe::launch_check_pos(pos, num_tokens * num_topk, num_rows,
                                            static_cast<uint32_t*>(workspace), flags, stream));
}

moe_status moe_check_activations(const uint16_t* x_bf16, int64_t num_values, uint32_t* flags,
                                 hipStream_t stream) {
    if (num_values < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (flags == nullptr || !aligned(flags, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (num_values == 0) return MOE_OK;
    if (x_bf16 == nullptr || !aligned(x_bf16, 2)) return MOE_ERR_INVALID_ARGUMENT;
    return hip_status(moe::launch_check_bf16(x_bf16, num_values, flags, stream));
}

moe_status moe_check_dispatch(const void* workspace, size_t workspace_bytes, uint32_t* flags,
                              hipStream_t stream) {
    if (flags == nullptr || !aligned(flags, 4)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace == nullptr || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kDispatchHeaderBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(moe::launch_check_dispatch(static_cast<const uint32_t*>(workspace), kDispatchTimeoutWord,
                                                 flags, stream));
}

}  // extern "C"
