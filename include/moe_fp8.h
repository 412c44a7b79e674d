/*
 * moe_fp8.h -- C ABI of the MI355X (gfx950) MoE dispatch library
 * (libmoe_fp8.so).
 *
 * The dispatch path, in pipeline order:
 *   moe_topk_gate        top-k expert ids (+ optional renormalised weights)
 *   moe_token_map        per-expert counts, exclusive offsets, slot positions
 *   moe_expand_cast_fp8  per-token, per-128-channel e4m3 cast, scattered into
 *                        the expert-grouped layout with the routing weights
 *   swiglu_cast_fp8      SwiGLU (x routing weight) fused with the e4m3 cast,
 *                        feeding the expert down-projection GEMM
 *   moe_combine          after the expert GEMMs: the weighted reduce of each
 *                        token's expert outputs back to token order
 *
 * The whole dispatch in one call (moe_dispatch): top-k -> map -> expand,
 * as one launch with a grid barrier for decode-sized batches, else as the
 * separate launches above.
 *
 * Other block-scaled output formats (moe_expand_cast, swiglu_cast): e4m3 or
 * FP4 e2m1 codes, groups of 16, 32 or 128 channels, scales rounded to powers
 * of two and stored as fp32 or UE8M0 bytes.
 *
 * Padded, expert-local variant of the map and the expand (segments aligned
 * to the grouped GEMM's row tile; only a contiguous range of experts mapped):
 *   moe_token_map_aligned_rows, moe_token_map_aligned,
 *   moe_expand_cast_fp8_padded
 *
 * Device-side checks of the inputs' preconditions, for debugging:
 *   moe_check_scores, moe_check_topk_idx, moe_check_pos,
 *   moe_check_activations, and of a single-launch dispatch's barrier:
 *   moe_check_dispatch
 *
 * Sources (page title, section):
 *   [TK]  "DeepSeek open-sources TileKernels: GPU operators written in Python
 *         approach the hardware limit" (itsolotime.com): section 2 (the
 *         routing chain), 2.1 (Top-K gating), 2.2 (Fused expand), 3.1 (cast
 *         configuration), 3.2 (per-token cast), 3.3 (SwiGLU fusion).
 *   [PPX] "CuTeDSL at Perplexity" (perplexity.ai blog): "MoE dispatch and
 *         combine" (the local TP=1 kernel, padded buffers, tensor-parallel
 *         routing of the rank's experts), "Grid synchronisation" (decode in
 *         one launch), the Blackwell section (MXFP8 / MXFP4 / NVFP4 group
 *         sizes).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *     The library never allocates, frees, synchronises the host or keeps a
 *     pointer after the call returns.
 *   - Work is enqueued on `stream` (NULL = the null stream) and runs
 *     asynchronously; outputs are valid once the stream reaches that point.
 *   - Arguments are validated on the host before any HIP call.  An invalid
 *     argument returns MOE_ERR_INVALID_ARGUMENT (or MOE_ERR_UNSUPPORTED for a
 *     valid but unimplemented variant) and enqueues nothing.  num_tokens == 0
 *     (or num_rows == 0) returns MOE_OK and enqueues nothing, except that
 *     moe_token_map still zeroes its counts and offsets.
 *   - A failed kernel launch returns MOE_ERR_HIP; moe_last_hip_error() then
 *     gives the hipError_t (per host thread).
 *   - Calls that overlap on the same output buffers race; calls on
 *     independent buffers may run concurrently on different streams.
 *   - bf16 tensors are passed as uint16_t bit patterns; e4m3 outputs are OCP
 *     FP8 E4M3FN bytes (no infinities, max 448, NaN 0x7F/0xFF).
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4
} moe_status;

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* moe_status_string(int status);

/* hipError_t of the last MOE_ERR_HIP returned on the calling host thread
 * (0 if none). */
int moe_last_hip_error(void);

/* ABI version, MAJOR * 10000 + MINOR * 100 + PATCH. */
int moe_fp8_version(void);

/*
 * moe_topk_gate -- [TK] 2.1 Top-K gating; weights: [TK] 2 "Weight
 * Normalization".
 *
 * For each token t, K rounds of: take the maximum score of the row, pick the
 * LOWEST expert index whose score equals it (IEEE equality, so -0 == +0),
 * then mask that expert to -inf.  topk_idx[t, k] is round k's winner, so the
 * ids come out in descending score order.  A NaN score reads as -inf.
 *
 * scores        fp32 [num_tokens, num_experts], 4-byte aligned.
 * num_tokens    T >= 0.
 * num_experts   E, 1 <= E <= 1024.
 * num_topk      K, 1 <= K <= min(E, 16).
 * renormalize   0: topk_weights (if given) receives the selected scores.
 *               1: topk_weights[t,k] = s_k / (((s_0 + s_1) + ...) + s_{K-1}),
 *                  fp32, summed in k order (requires topk_weights).
 * topk_idx      int64 [T, K] output.
 * topk_weights  fp32 [T, K] output, or NULL.
 */
moe_status moe_topk_gate(const float* scores, int64_t num_tokens, int32_t num_experts,
                         int32_t num_topk, int32_t renormalize, int64_t* topk_idx,
                         float* topk_weights, hipStream_t stream);

/*
 * Bytes of device workspace moe_token_map needs for this shape (a multiple
 * of 256; 0 when num_tokens == 0).  Returns 0 for an invalid shape.
 */
size_t moe_token_map_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts);

/*
 * moe_token_map -- [TK] 2 group counting + token-expert mapping;
 * [PPX] local kernel (count each expert's tokens, then give every token copy
 * a unique index in its expert's list).
 *
 * With N = num_tokens * num_topk routed copies (t, k) in row-major order:
 *   expert_counts[e]   = number of copies routed to e
 *   expert_offsets[0]  = 0, expert_offsets[e+1] = expert_offsets[e] + counts[e]
 *   pos[t, k]          = expert_offsets[e] + number of copies routed to e that
 *                        come before (t, k) in row-major order
 *   row_token[r]       = the token whose copy lands in row r
 * Rows inside an expert's segment are therefore in ascending token order (a
 * stable counting sort; deterministic, no global atomics).  An id outside
 * [0, E) is not counted and gets pos = -1; row_token entries past
 * expert_offsets[E] are set to -1.
 *
 * topk_idx        int64 [T, K] (from moe_topk_gate or any source).
 * num_tokens      T >= 0; T * K <= 2^31 - 1.
 * num_topk        K, 1 <= K <= 16.
 * num_experts     E, 1 <= E <= 1024.
 * expert_counts   int32 [E] output.
 * expert_offsets  int32 [E + 1] output.
 * pos             int32 [T, K] output.
 * row_token       int32 [T * K] output, or NULL.
 * workspace       device scratch of at least moe_token_map_workspace_bytes()
 *                 bytes, 256-byte aligned; contents need not be initialised
 *                 and are garbage afterwards.
 * With T == 0 the counts and offsets are still zeroed (one small launch).
 */
moe_status moe_token_map(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                         int32_t num_experts, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* pos, int32_t* row_token, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * moe_token_map_noalloc -- moe_token_map with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments
 * (minus workspace), results and errors as moe_token_map, from the same
 * kernels.
 *
 * The count table lives in a fixed 1 MiB device array inside the library
 * (the largest table any admitted shape needs: 256 chunks x 1024 experts x
 * 4 bytes), one per device, held from the library's load until the process
 * ends; its device address is looked up on the first call on each device.
 * The call allocates nothing, and needs nothing cleared: every count it
 * reads it has written first.  Every call on a device shares that device's
 * array, so calls that overlap on one device (on several streams, or from
 * several host threads without ordering) race; calls in one stream's order
 * do not.  A shape whose table would exceed the array returns
 * MOE_ERR_UNSUPPORTED (none does within the limits of moe_token_map).
 */
moe_status moe_token_map_noalloc(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                                 int32_t num_experts, int32_t* expert_counts, int32_t* expert_offsets,
                                 int32_t* pos, int32_t* row_token, hipStream_t stream);

/*
 * moe_expand_cast_fp8 -- [TK] 2.2 Fused expand with the [TK] 3.2 per-token
 * cast ([TK] 3.1 e4m3 configuration).
 *
 * For each token row and each group of group_size channels:
 *   amax = max |x|;  sf = max(amax, 1e-4) / 448;  inv = 1 / sf;
 *   code = e4m3(x * inv)   (round to nearest even)
 * then for each k with r = pos[t, k] in [0, num_rows): row r of out_fp8
 * receives the codes, row r of out_sf the group scales and, if given,
 * out_weights[r] = topk_weights[t, k].  Rows that no copy lands in are not
 * written.  pos == NULL is the identity map (requires num_topk == 1 and
 * num_rows == num_tokens): the plain per-token cast.
 *
 * Precondition: every x value is finite (the scale of a group is defined
 * by its largest magnitude; a NaN or infinity gives unspecified codes and
 * scales for its group).  Not tested on the fast path; moe_check_activations
 * tests it.
 *
 * x_bf16        bf16 [T, hidden], 16-byte aligned.
 * num_tokens    T >= 0.
 * hidden        H, a multiple of group_size.
 * num_topk      K, 1 <= K <= 16.
 * pos           int32 [T, K] (from moe_token_map), or NULL.  The non-negative
 *               entries must be distinct (two copies to one row race).
 * topk_weights  fp32 [T, K], or NULL; given iff out_weights is given.
 * num_rows      R == T * K (pos given) or T (identity).
 * group_size    16, 32 or 128 (anything else: MOE_ERR_UNSUPPORTED); 16 and 32
 *               run on the block-scaled kernels of moe_expand_cast in this
 *               same format.
 * out_fp8       e4m3 [R, H] output, 16-byte aligned.
 * out_sf        fp32 [R, H / group_size] output (row-major), 4-byte aligned.
 * out_weights   fp32 [R] output, or NULL.
 */
moe_status moe_expand_cast_fp8(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                               int32_t num_topk, const int32_t* pos, const float* topk_weights,
                               int64_t num_rows, int32_t group_size, uint8_t* out_fp8,
                               float* out_sf, float* out_weights, hipStream_t stream);

/*
 * swiglu_cast_fp8 -- [TK] 3.3 SwiGLU fused with the per-token cast.
 *
 * For row r and column j < inter, with gate l = x[r, j] and up u =
 * x[r, inter + j] (bf16 -> fp32):
 *   if clamp_value > 0:  l = min(l, c);  u = max(min(u, c), -c)
 *   v = l / (1 + exp(-l)) * u  [* row_weights[r]]      (fp32)
 * then each group of group_size columns of v is cast as in
 * moe_expand_cast_fp8.  The fp32 arithmetic uses hardware exp2 and
 * reciprocal: results agree with an IEEE evaluation to a few ulp (scales
 * within 1e-6 relative, codes within one e4m3 step).
 * Precondition: every gate and up value is finite (a gate of +inf, for one,
 * gives NaN here where the IEEE expression gives +inf).  Not tested on the
 * fast path; moe_check_activations tests it.
 *
 * gate_up_bf16  bf16 [num_rows, 2 * inter] = [gate | up], 16-byte aligned.
 * num_rows      R >= 0.
 * inter         I, a multiple of group_size.
 * row_weights   fp32 [R] (routing weight of each row), or NULL.
 * clamp_value   <= 0: no clamp.
 * group_size    16, 32 or 128 (anything else: MOE_ERR_UNSUPPORTED).
 * out_fp8       e4m3 [R, I] output, 16-byte aligned.
 * out_sf        fp32 [R, I / group_size] output, 4-byte aligned.
 */
moe_status swiglu_cast_fp8(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                           const float* row_weights, float clamp_value, int32_t group_size,
                           uint8_t* out_fp8, float* out_sf, hipStream_t stream);

/*
 * moe_combine -- [PPX] "MoE dispatch and combine" (the combine accumulates,
 * in registers, each token's expert outputs found through the positions the
 * dispatch computed); [TK] 2, the Fused Expand/Reduce step.
 *
 *   out[t, :] = bf16( sum over k = 0..K-1 of w[t,k] * y_rows[pos[t,k], :] )
 *
 * fp32 products and fp32 sums, one rounding each, in k order; rows with
 * pos[t,k] outside [0, num_rows) are skipped (a token with none gets +0);
 * the bf16 result is rounded to nearest even.  Inputs must be finite
 * (moe_check_activations tests y_rows).
 *
 * y_rows_bf16  bf16 [num_rows, hidden], expert outputs in the expert-grouped
 *              row order of the dispatch, 16-byte aligned.
 * num_rows     R >= 0.
 * hidden       H, a multiple of 8.
 * pos          int32 [num_tokens, K] (from moe_token_map).
 * weights      fp32 [num_tokens, K] (routing weights), or NULL for weight 1.
 * num_tokens   T >= 0.
 * num_topk     K, 1 <= K <= 16.
 * out_bf16     bf16 [T, H] output, 16-byte aligned.
 */
moe_status moe_combine(const uint16_t* y_rows_bf16, int64_t num_rows, int32_t hidden,
                       const int32_t* pos, const float* weights, int64_t num_tokens, int32_t num_topk,
                       uint16_t* out_bf16, hipStream_t stream);

/*
 * Rows an aligned map may fill: num_tokens * num_topk + num_local_experts *
 * (align - 1), the size of row_token / the padded expand's outputs.  Returns
 * 0 for an invalid shape or a bound above 2^31 - 1.
 */
size_t moe_token_map_aligned_rows(int64_t num_tokens, int32_t num_topk, int32_t num_local_experts,
                                  int32_t align);

/*
 * moe_token_map_aligned -- moe_token_map restricted to the local experts
 * [expert_begin, expert_end) and with every expert's segment padded to a
 * multiple of `align` rows.  [TK] 2.2 (copies with a negative position are
 * skipped; the expand zero-fills the invalid rows in the same grid); [PPX]
 * local kernel (optional padded buffers for the grouped GEMM) and the
 * tensor-parallel dispatch (a rank routes only the tokens of its experts).
 *
 * With EL = expert_end - expert_begin and local index j = id - expert_begin:
 *   expert_counts[j]   = copies routed to expert expert_begin + j
 *   expert_offsets[0]  = 0, expert_offsets[j+1] = expert_offsets[j] +
 *                        ceil(counts[j] / align) * align
 *   pos[t, k]          = expert_offsets[j] + number of copies routed to the
 *                        same expert that come before (t, k) in row-major
 *                        order; -1 for a copy routed outside the range
 *   row_token[r]       = token of the copy in row r; -1 for the padding rows
 *                        of each segment and for every r >= expert_offsets[EL]
 * align == 1 over [0, E) is exactly moe_token_map.
 *
 * topk_idx        int64 [T, K].
 * num_tokens      T >= 0.
 * num_topk        K, 1 <= K <= 16.
 * expert_begin,   0 <= expert_begin < expert_end, EL <= 1024.
 * expert_end
 * align           1 <= align <= 4096.
 * expert_counts   int32 [EL] output.
 * expert_offsets  int32 [EL + 1] output.
 * pos             int32 [T, K] output.
 * row_token       int32 [num_rows] output, or NULL.
 * num_rows        >= moe_token_map_aligned_rows(T, K, EL, align) (the most
 *                 rows any routing can fill), <= 2^31 - 1.
 * workspace       at least moe_token_map_workspace_bytes(T, K, EL) bytes,
 *                 256-byte aligned, as for moe_token_map.
 * With T == 0 the counts and offsets are zeroed and row_token set to -1.
 */
moe_status moe_token_map_aligned(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                                 int32_t expert_begin, int32_t expert_end, int32_t align,
                                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                                 int32_t* row_token, int64_t num_rows, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expand_cast_fp8_padded -- moe_expand_cast_fp8 into the rows of an
 * aligned map: [TK] 2.2 (one grid both copies the routed rows and
 * zero-fills the invalid ones).
 *
 * Every copy with r = pos[t, k] in [0, num_rows) is cast and written as in
 * moe_expand_cast_fp8; every row r < num_rows with row_token[r] < 0 gets
 * zero codes, zero scales and (if out_weights) a zero weight, in the same
 * launch.  All num_rows rows are therefore written.  pos and row_token must
 * agree (row_token[pos[t,k]] == t, as moe_token_map_aligned leaves them):
 * a row that is both routed and marked empty is written twice and races.
 *
 * x_bf16        bf16 [T, hidden], 16-byte aligned.
 * num_tokens    T >= 0.
 * hidden        H, a multiple of group_size.
 * num_topk      K, 1 <= K <= 16.
 * pos           int32 [T, K] (required when T > 0).
 * topk_weights  fp32 [T, K], or NULL; given iff out_weights is given (may
 *               be NULL with out_weights when T == 0).
 * row_token     int32 [num_rows] (required when num_rows > 0).
 * num_rows      R >= 0.
 * group_size    must be 128.
 * out_fp8       e4m3 [R, H] output, 16-byte aligned.
 * out_sf        fp32 [R, H / group_size] output, 4-byte aligned.
 * out_weights   fp32 [R] output, or NULL.
 */
moe_status moe_expand_cast_fp8_padded(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                                      int32_t num_topk, const int32_t* pos, const float* topk_weights,
                                      const int32_t* row_token, int64_t num_rows, int32_t group_size,
                                      uint8_t* out_fp8, float* out_sf, float* out_weights,
                                      hipStream_t stream);

/*
 * Block-scaled output format.  [TK] 3.1 (the cast output configuration:
 * dtype, scaling block size, round_sf, clamp_min_value, packed UE8M0);
 * [PPX] Blackwell section (MXFP8 / MXFP4 absmax over 32 elements, NVFP4 over
 * 16).  For each group of group_size channels:
 *   c    = max(amax, clamp)   clamp = clamp_min if > 0, else 1e-4 (e4m3) or
 *                             6 * 2^-126 (e2m1)
 *   sf   = c / max_value      (448 for e4m3, 6 for e2m1; fp32, correctly
 *                             rounded); round_sf = 1: the smallest power of
 *                             two with sf * max_value >= c (no code saturates)
 *   code = format(x * (1 / sf)), round to nearest, ties to even, saturating.
 * Codes: e4m3 one byte per channel (OCP E4M3FN); e2m1 half a byte (OCP
 * E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), element 2i in the low
 * nibble of byte i, so a row holds hidden / 2 bytes.
 * Scales: fp32 [rows, hidden / group_size], or with sf_ue8m0 = 1 (requires
 * round_sf) one byte per group holding the biased exponent of sf (2^(b-127));
 * four consecutive groups form one little-endian 32-bit word (packed UE8M0).
 */
#define MOE_FMT_E4M3 0
#define MOE_FMT_E2M1 1

typedef struct moe_cast_format {
    int32_t dtype;      /* MOE_FMT_E4M3 or MOE_FMT_E2M1 */
    int32_t group_size; /* 16, 32 or 128 */
    int32_t round_sf;   /* 0 or 1 */
    int32_t sf_ue8m0;   /* 0: fp32 scales; 1: UE8M0 bytes (requires round_sf) */
    float clamp_min;    /* <= 0: the format default; else in [max_value * 2^-126, 2^126] */
} moe_cast_format;

/*
 * moe_expand_cast -- moe_expand_cast_fp8 in any block-scaled format (same
 * rows, positions, weights and identity mode), [TK] 2.2, 3.1, 3.2.
 *
 * x_bf16        bf16 [T, hidden], 16-byte aligned.
 * hidden        a multiple of format->group_size; for e2m1 also of 32
 *               (else MOE_ERR_UNSUPPORTED).
 * pos, topk_weights, num_rows, out_weights: as for moe_expand_cast_fp8.
 * format        host pointer, read during the call only.
 * out           codes [num_rows, hidden] (e4m3) or [num_rows, hidden / 2]
 *               bytes (e2m1), 16-byte aligned.
 * out_sf        fp32 (4-byte aligned) or UE8M0 bytes, [num_rows, hidden /
 *               group_size].
 */
moe_status moe_expand_cast(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden, int32_t num_topk,
                           const int32_t* pos, const float* topk_weights, int64_t num_rows,
                           const moe_cast_format* format, uint8_t* out, void* out_sf, float* out_weights,
                           hipStream_t stream);

/*
 * swiglu_cast -- swiglu_cast_fp8 in any block-scaled format, [TK] 3.3, 3.1.
 * The SwiGLU value (clamp, row weight) is as for swiglu_cast_fp8; each group
 * of group_size columns is then cast as above.
 *
 * gate_up_bf16  bf16 [num_rows, 2 * inter], 16-byte aligned.
 * inter         a multiple of format->group_size.
 * out           codes [num_rows, inter] (e4m3, 8-byte aligned) or
 *               [num_rows, inter / 2] bytes (e2m1, 4-byte aligned).
 * out_sf        fp32 (4-byte aligned) or UE8M0 bytes, [num_rows, inter /
 *               group_size].
 */
moe_status swiglu_cast(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                       const float* row_weights, float clamp_value, const moe_cast_format* format,
                       uint8_t* out, void* out_sf, hipStream_t stream);

/* moe_route modes */
#define MOE_ROUTE_AUTO 0  /* the local form up to 16 tokens; the fused form when the batch has more than
                             1024 routed copies and its grid is at most four workgroups per compute
                             unit (16384 tokens on 256 compute units; 8192 when E > 512); else the
                             split form -- each where it measured fastest */
#define MOE_ROUTE_FUSED 1 /* always the fused form (MOE_ERR_UNSUPPORTED if the batch does not fit it) */
#define MOE_ROUTE_SPLIT 2 /* moe_topk_gate, then moe_token_map */
#define MOE_ROUTE_LOCAL 3 /* one launch in which every workgroup routes the whole batch (the single-launch
                             dispatch's kernel with no channels): up to 32 tokens (MOE_ERR_UNSUPPORTED above) */

/*
 * Bytes of device workspace moe_route needs: a 2048-byte header, two
 * 262144-byte tables of the fused form, then the larger of moe_token_map's
 * workspace and the fused form's per-workgroup counts -- the same layout and
 * size as moe_dispatch's, so one workspace serves both.  Returns 0 for an
 * invalid shape.
 */
size_t moe_route_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts);

/*
 * moe_route -- moe_topk_gate followed by moe_token_map, with the same
 * outputs bit for bit, with the top-k and the counting fused.  [TK] 2: the
 * routing chain Top-K Gating -> Group Counting -> Token-Expert Mapping; [PPX]
 * "MoE dispatch and combine": count each expert's tokens, then give each
 * token its index in its expert's list.
 *
 * Fused form, two launches.  The first runs the top-k, one wave per token
 * and 16 tokens per workgroup (8 when E > 512); each workgroup ranks its own
 * copies among themselves (written to pos) and counts them per expert, into
 * its row of the workspace and, summed over groups of consecutive
 * workgroups (about the square root of their number), into a table.  The
 * second turns those counts into the offsets and adds to each copy's rank
 * the copies of its expert in earlier workgroups (one workgroup per group of
 * consecutive workgroups).  The split form needs three launches for batches
 * of more than 2048 routed copies.  The fused form takes at most 64 groups
 * of at most 8192 / E workgroups each: 65536 tokens at E <= 128, 32768 at
 * E = 256, 16384 at E = 512, 4096 at E = 1024; larger batches run the split
 * form, and MOE_ROUTE_FUSED on them returns MOE_ERR_UNSUPPORTED.  No
 * workgroup waits for another: the launch boundary is the only hand-off.
 *
 * Local form (up to 32 tokens), one launch: the single-launch dispatch's
 * kernel with no channels to copy; every workgroup computes the top-k of
 * every token itself and workgroup 0 writes topk_idx and the weights.  It
 * does not touch the workspace.
 *
 * Arguments as for moe_topk_gate and moe_token_map (scores fp32 [T, E], any
 * 4-byte alignment; topk_idx int64 [T, K]; topk_weights fp32 [T, K] or NULL,
 * required with renormalize = 1; expert_counts int32 [E]; expert_offsets
 * int32 [E + 1]; pos int32 [T, K]; row_token int32 [T * K] or NULL), and:
 * workspace     >= moe_route_workspace_bytes(T, K, E) bytes, 256-byte aligned.
 *               Its first 2048 + 524288 bytes must be zero before the first
 *               call on it (zero the whole workspace once when allocating
 *               it); every call leaves them ready for the next (it zeroes
 *               what the previous call used of the table it does not use), so
 *               it can be reused without clearing.  Calls sharing a workspace
 *               must not overlap.  The same workspace may serve moe_dispatch.
 * mode          MOE_ROUTE_AUTO, MOE_ROUTE_FUSED, MOE_ROUTE_SPLIT or
 *               MOE_ROUTE_LOCAL.
 * T == 0 zeroes counts and offsets in every mode.
 */
moe_status moe_route(const float* scores, int64_t num_tokens, int32_t num_experts, int32_t num_topk,
                     int32_t renormalize, int64_t* topk_idx, float* topk_weights, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* pos, int32_t* row_token, void* workspace,
                     size_t workspace_bytes, int32_t mode, hipStream_t stream);

/* moe_dispatch modes */
#define MOE_DISPATCH_AUTO 0          /* single launch for the smallest batches, else as below */
#define MOE_DISPATCH_SINGLE_LAUNCH 1 /* always one launch (MOE_ERR_UNSUPPORTED if too big) */
#define MOE_DISPATCH_SPLIT 2         /* moe_topk_gate, moe_token_map, moe_expand_cast_fp8 */
#define MOE_DISPATCH_ROUTE_FUSED 3   /* moe_route's fused form, then moe_expand_cast_fp8
                                        (MOE_ERR_UNSUPPORTED where the fused form does not fit) */
#define MOE_DISPATCH_TOPK_THEN_COPY 4 /* moe_topk_gate's kernel, then the single launch's map and
                                        copies reading its ids (no grid barrier; the same limit) */

/*
 * Bytes of device workspace moe_dispatch needs: moe_route_workspace_bytes
 * (its 2048-byte header also holds the single-launch form's barrier).
 * Returns 0 for an invalid shape.
 */
size_t moe_dispatch_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts);

/*
 * moe_dispatch -- the dispatch path in one call: moe_topk_gate, then
 * moe_token_map, then moe_expand_cast_fp8 of every routed copy, with the
 * same outputs bit for bit.  [PPX] "Grid synchronisation" and "MoE dispatch
 * and combine": for few tokens, routing, a grid barrier and the copy run in
 * one launch; for many, as separate launches (the launch boundary is the
 * barrier).
 *
 * Single-launch form: one copying wave per (token, 1024-channel chunk) unit
 * or per token, whichever is more, four per workgroup, at most one
 * workgroup per compute unit (so all are resident at once on an otherwise
 * idle device).  Above 32 tokens it has a grid barrier, and there residency
 * is assumed, not guaranteed: the launch is an ordinary one, so work on
 * other streams (or other processes) that holds compute units can keep some
 * workgroups from starting until it ends.  Each barrier
 * wait is bounded (about a second); a wait that gives up sets the time-out
 * word (below) and the call's outputs are invalid, yet the call still
 * returns MOE_OK (the failure happens on the device after the call
 * returned).  moe_check_dispatch reports the word stream-ordered; the
 * Python binding runs it after every moe_dispatch in debug mode.  Top-k runs one wave per token; after the grid barrier every
 * workgroup holds the T*K ids in LDS, one wave per expert writes its count
 * and offset, and the wave of each unit computes the slots of its token's
 * copies directly as (copies to lower experts) + (earlier copies to the same
 * expert) and writes the cast rows.  Up to 32 tokens there is no barrier and
 * no residency assumption: every workgroup computes the top-k of every token
 * itself (routing-only waves join the four copying waves of a workgroup from
 * 5 tokens, each routing one token, two above 16) and workgroup 0 writes
 * topk_idx and the weights.  Limits: T * K <= 16384 (the ids of the
 * batch are held in LDS).  MOE_DISPATCH_TOPK_THEN_COPY runs moe_topk_gate's
 * kernel first and then this form's map and copies, which read the ids
 * from memory: no grid barrier, no residency assumption, the same limit.
 * MOE_DISPATCH_AUTO takes the single launch up to 24 tokens, the
 * top-k-then-copy form up to 1024 routed copies, and above that moe_route
 * (MOE_ROUTE_AUTO, see there) and then moe_expand_cast_fp8 -- each where it
 * measured fastest (DeepSeek-V3 shape, graph replay: 16 tokens 9.3 us, 64
 * tokens 11.7 against 13.5 split, 128 tokens 13.9 against 14.7).
 *
 * scores        fp32 [T, E], any 4-byte alignment.
 * x_bf16        bf16 [T, hidden], 16-byte aligned.
 * num_tokens    T >= 0 (T == 0: counts and offsets zeroed, nothing else).
 * num_experts   E, 1 <= E <= 1024.
 * num_topk      K, 1 <= K <= min(E, 16).
 * hidden        a multiple of group_size.
 * renormalize   0 or 1, as for moe_topk_gate (1 requires topk_weights).
 * group_size    must be 128.
 * topk_idx      int64 [T, K] output.
 * topk_weights  fp32 [T, K] output, or NULL; given iff out_weights is given.
 * expert_counts int32 [E] output;  expert_offsets int32 [E + 1] output.
 * pos           int32 [T, K] output;  row_token int32 [T * K] output or NULL.
 * out_fp8       e4m3 [T * K, hidden] output, 16-byte aligned.
 * out_sf        fp32 [T * K, hidden / group_size] output.
 * out_weights   fp32 [T * K] output, or NULL.
 * workspace     >= moe_dispatch_workspace_bytes(T, K, E) bytes, 256-byte
 *               aligned.  Its first 2048 + 524288 bytes (the barrier
 *               counters, and moe_route's words and tables) must be zero
 *               before the first call on it (zero the whole workspace once
 *               when allocating it); every completed call leaves them ready
 *               (each barrier counter a whole number of epochs of 2^16), so
 *               it can be reused without clearing.  The uint32 at byte 8 is
 *               set nonzero if a barrier wait of the single-launch form ever
 *               timed out (about a second; only if some workgroup could not
 *               become resident): that call's outputs are then invalid.  Calls sharing a
 *               workspace must not overlap.  Single-launch calls on several
 *               streams at once need all their workgroups resident together
 *               (each uses at most one per compute unit; a few such calls fit
 *               side by side); more concurrent calls than fit can time out.
 * mode          MOE_DISPATCH_AUTO, MOE_DISPATCH_SINGLE_LAUNCH,
 *               MOE_DISPATCH_SPLIT, MOE_DISPATCH_ROUTE_FUSED or
 *               MOE_DISPATCH_TOPK_THEN_COPY.
 */
moe_status moe_dispatch(const float* scores, const uint16_t* x_bf16, int64_t num_tokens,
                        int32_t num_experts, int32_t num_topk, int32_t hidden, int32_t renormalize,
                        int32_t group_size, int64_t* topk_idx, float* topk_weights,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                        int32_t* row_token, uint8_t* out_fp8, float* out_sf, float* out_weights,
                        void* workspace, size_t workspace_bytes, int32_t mode, hipStream_t stream);

/*
 * Input checks.  The calls above assume their inputs meet these conditions
 * and do not test them on their fast path; these calls test them on the
 * device, for debugging.  Each ORs the bits of the conditions it finds
 * violated into *flags, a device uint32 the caller zeroes before the first
 * check, and is stream-ordered and asynchronous like every other call (read
 * *flags after the stream reaches it).  Arguments are validated as for the
 * calls above; T == 0 (no entries) enqueues nothing.
 *
 * moe_check_scores   scores fp32 [T, E] (4-byte aligned): every score
 *   finite ([TK] 2.1: the iterative maximum orders the scores; a NaN has no
 *   place in that order) and, with require_positive = 1, every score > 0
 *   ([TK] 2 "Weight Normalization": renormalised weights divide each
 *   selected score by the sum of the selected scores).  E <= 1024.
 * moe_check_topk_idx topk_idx int64 [T, K] (8-byte aligned): every id in
 *   [0, E) and no id twice in a row ([TK] 2.1: each round masks its
 *   winner, so a token's K ids are distinct experts).  K <= 16, E <= 1024.
 * moe_check_pos      pos int32 [T, K] (4-byte aligned): every entry in
 *   [-1, num_rows) and no row reached by two copies ([TK] 2.2: -1 marks a
 *   skipped copy; every other copy owns its destination row).  workspace:
 *   at least moe_check_pos_workspace_bytes(num_rows) bytes, 4-byte aligned,
 *   a bitmap of the rows reached (zeroed by the call, garbage afterwards).
 */
#define MOE_CHECK_NONFINITE_SCORE 0x01u   /* a score is NaN or infinite */
#define MOE_CHECK_NONPOSITIVE_SCORE 0x02u /* require_positive and a finite score <= 0 */
#define MOE_CHECK_ID_RANGE 0x04u          /* an id outside [0, E) */
#define MOE_CHECK_ID_DUPLICATE 0x08u      /* an id repeated within a token's row */
#define MOE_CHECK_POS_RANGE 0x10u         /* an entry outside [-1, num_rows) */
#define MOE_CHECK_POS_DUPLICATE 0x20u     /* two copies with the same destination row */
#define MOE_CHECK_NONFINITE_ACTIVATION 0x40u /* a bf16 activation is NaN or infinite */
#define MOE_CHECK_DISPATCH_TIMEOUT 0x80u  /* a single-launch dispatch's barrier wait timed out */

moe_status moe_check_scores(const float* scores, int64_t num_tokens, int32_t num_experts,
                            int32_t require_positive, uint32_t* flags, hipStream_t stream);
moe_status moe_check_topk_idx(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                              int32_t num_experts, uint32_t* flags, hipStream_t stream);
/* Bytes of workspace moe_check_pos needs: 4 * ceil(num_rows / 32) (0 for
 * num_rows <= 0). */
size_t moe_check_pos_workspace_bytes(int64_t num_rows);
moe_status moe_check_pos(const int32_t* pos, int64_t num_tokens, int32_t num_topk, int64_t num_rows,
                         void* workspace, size_t workspace_bytes, uint32_t* flags, hipStream_t stream);

/*
 * moe_check_activations -- every one of num_values contiguous bf16 values
 * x_bf16[0..num_values) (2-byte aligned) is finite: the precondition of the
 * casts ([TK] 3.2, 3.3: a group's scale is its largest magnitude over the
 * format maximum) and of the combine.  Sets MOE_CHECK_NONFINITE_ACTIVATION.
 * num_values == 0 enqueues nothing.
 */
moe_status moe_check_activations(const uint16_t* x_bf16, int64_t num_values, uint32_t* flags,
                                 hipStream_t stream);

/*
 * moe_check_dispatch -- the time-out word of a moe_dispatch workspace
 * ([PPX] "Grid synchronisation": the single-launch form's grid barrier needs
 * every workgroup resident).  Sets MOE_CHECK_DISPATCH_TIMEOUT if any
 * single-launch call on this workspace, up to this point of the stream, gave
 * up a barrier wait (the word is sticky: zero the workspace to clear it).
 * workspace_bytes must be at least 2048 (the header).
 */
moe_status moe_check_dispatch(const void* workspace, size_t workspace_bytes, uint32_t* flags,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
