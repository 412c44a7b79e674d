// Internal launchers of the gfx950 kernels.  The C-ABI entry points
// (moe_fp8_api.hip) validate every argument before calling these; the
// launchers only choose launch shapes and enqueue work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// The compute-unit count of the current device (cached per device).
int device_cu_count();

hipError_t launch_topk_gate(const float* scores, int64_t num_tokens, int num_experts, int num_topk,
                            bool renormalize, int64_t* topk_idx, float* topk_weights,
                            hipStream_t stream);

// Token map launch plan: routed copies are split into blocks of `chunk`
// copies; the workspace holds one count per (expert, block).
struct TokenMapPlan {
    int64_t num_items;   // T * K
    int32_t chunk;       // copies per block
    int32_t num_blocks;  // ceil(num_items / chunk)
    size_t workspace_bytes;
};
TokenMapPlan plan_token_map(int64_t num_tokens, int num_topk, int num_experts);

// Copies routed to experts [expert_begin, expert_begin + num_experts) are
// mapped (local index = id - expert_begin), the rest get pos = -1; segments
// are padded to a multiple of `align` rows; row_token has num_rows entries.
hipError_t launch_token_map(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                            int64_t expert_begin, int num_experts, int align, int32_t* counts,
                            int32_t* offsets, int32_t* pos, int32_t* row_token, int64_t num_rows,
                            int32_t* workspace, const TokenMapPlan& plan, hipStream_t stream);

// row_token != nullptr: a padded expand; rows r < num_rows with
// row_token[r] < 0 are zero-filled by the same launch.
hipError_t launch_expand_cast_fp8(const uint16_t* x, int64_t num_tokens, int hidden, int num_topk,
                                  const int32_t* pos, const float* topk_weights, int64_t num_rows,
                                  uint8_t* out, float* out_sf, float* out_weights,
                                  const int32_t* row_token, hipStream_t stream);

hipError_t launch_swiglu_cast_fp8(const uint16_t* gate_up, int64_t num_rows, int inter,
                                  const float* row_weights, float clamp_value, uint8_t* out,
                                  float* out_sf, hipStream_t stream);

// Block-scaled cast formats: dtype 0 = e4m3, 1 = e2m1; group 16, 32 or 128;
// power-of-two scales; UE8M0 scale bytes; clamp_min <= 0 = the format default.
struct MxFormat {
    int dtype;
    int group_size;
    bool round_sf;
    bool sf_ue8m0;
    float clamp_min;
};
// pos == nullptr: the identity cast (num_rows == num_tokens).
hipError_t launch_expand_cast_mx(const uint16_t* x, int64_t num_tokens, int hidden, int num_topk,
                                 const int32_t* pos, const float* topk_weights, int64_t num_rows,
                                 const MxFormat& fmt, uint8_t* out, void* out_sf, float* out_weights,
                                 hipStream_t stream);
hipError_t launch_swiglu_cast_mx(const uint16_t* gate_up, int64_t num_rows, int inter,
                                 const float* row_weights, float clamp_value, const MxFormat& fmt,
                                 uint8_t* out, void* out_sf, hipStream_t stream);

hipError_t launch_combine(const uint16_t* y_rows, int64_t num_rows, int hidden, const int32_t* pos,
                          const float* weights, int64_t num_tokens, int num_topk, uint16_t* out,
                          hipStream_t stream);

// Top-k and the token map in two launches (route_fused.hip): a count kernel
// (top-k, in-workgroup ranks, per-workgroup and per-super-chunk counts) and a
// slot kernel.  Workgroups of route_fused_tokens_per_block(E) tokens, at most
// kRouteMaxBlocks of them (route_fused_fits).  `header` is the 2048-byte
// header of the workspace (zero before the first call); `super_rows` two
// tables of kRouteSuperRows x 1024 super-chunk counts (zero before the first
// call; a call adds into one and zeroes what the previous call used of the
// other); `block_rows` route_fused_block_rows_bytes of per-workgroup counts
// (rewritten by every call).
constexpr int kRouteSuperRows = 64;
constexpr int kRouteSuperStride = kRouteSuperRows * 1024;  // ints per table (E <= 1024)
constexpr int64_t kRouteMaxBlocks = kRouteSuperRows * kRouteSuperRows;
constexpr size_t kRouteSuperBytes = 2 * static_cast<size_t>(kRouteSuperStride) * sizeof(int32_t);
int64_t route_fused_tokens_per_block(int num_experts);
size_t route_fused_block_rows_bytes(int64_t num_tokens, int num_experts);
bool route_fused_fits(int64_t num_tokens, int num_experts);
hipError_t launch_route_fused(const float* scores, int64_t num_tokens, int num_experts, int num_topk,
                              bool renormalize, int64_t* topk_idx, float* topk_weights, int32_t* counts,
                              int32_t* offsets, int32_t* pos, int32_t* row_token, int32_t* super_rows,
                              int32_t* block_rows, uint32_t* header, hipStream_t stream);

// Single-launch dispatch (top-k -> map -> expand + cast with one grid
// barrier, or none up to 16 tokens: there every workgroup routes every token
// itself).  Grid: one copying wave per (token, 1024-channel chunk) unit or
// per token, whichever is more (four per workgroup; workgroups of 5 to 32
// tokens add routing-only waves up to sixteen; with no channels, at least
// one per expert), capped at one workgroup per compute unit.
// `barrier` points at the 2048-byte barrier header of the workspace (zero
// before the first call; every completed call adds whole epochs of 2^16 to
// its counters; the uint32 at byte 8 becomes nonzero if a wait timed out).
int64_t fused_dispatch_grid(int64_t num_tokens, int hidden, int num_experts);
// Largest top-k the kernels take: a token's K winners and the renormalising
// weight sum live in the first 16-lane DPP row of its wave.
constexpr int kKernelMaxTopk = 16;
// Batches of at most this many tokens route inside every workgroup of the
// single launch (no grid barrier).  With hidden == 0 (x, out, out_sf and
// out_weights null) the launch is the routing alone: top-k and the map.
constexpr int64_t kDispatchLocalMaxTokens = 32;
hipError_t launch_dispatch_fused(const float* scores, const uint16_t* x, int64_t num_tokens,
                                 int num_experts, int num_topk, int hidden, bool renormalize,
                                 int64_t* topk_idx, float* topk_weights, int32_t* counts,
                                 int32_t* offsets, int32_t* pos, int32_t* row_token, uint8_t* out,
                                 float* out_sf, float* out_weights, uint32_t* barrier, bool after_topk,
                                 hipStream_t stream);

// Input checks: OR MOE_CHECK_* bits into *flags.  check_pos zeroes `seen`
// ((num_rows + 31) / 32 words) first.
hipError_t launch_check_scores(const float* scores, int64_t num_tokens, int num_experts, bool require_positive,
                               uint32_t* flags, hipStream_t stream);
hipError_t launch_check_topk_idx(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                                 uint32_t* flags, hipStream_t stream);
hipError_t launch_check_pos(const int32_t* pos, int64_t num_entries, int64_t num_rows, uint32_t* seen,
                            uint32_t* flags, hipStream_t stream);
hipError_t launch_check_bf16(const uint16_t* x, int64_t n, uint32_t* flags, hipStream_t stream);
// ORs MOE_CHECK_DISPATCH_TIMEOUT if header[word] != 0.
hipError_t launch_check_dispatch(const uint32_t* header, int word, uint32_t* flags, hipStream_t stream);

}  // namespace moe
