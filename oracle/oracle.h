/*
 * CPU oracle for the MoE dispatch path: top-k gating, token->expert map,
 * expand with per-token per-128-channel FP8 e4m3 cast, and SwiGLU + FP8 cast.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded
 * statement of what the GPU library computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant generator with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [TK]   "DeepSeek open-sources TileKernels: GPU operators written in Python
 *          approach the hardware limit" (itsolotime.com article on
 *          deepseek-ai/TileKernels).  Sections 2 (MoE routing chain),
 *          2.1 (Top-K gating), 2.2 (Fused expand), 3.1 (cast configuration),
 *          3.2 (per-token cast kernel), 3.3 (SwiGLU + quantisation fusion).
 *   [PPX]  "CuTeDSL at Perplexity" (perplexity.ai blog), section
 *          "MoE dispatch and combine", sub-section on the local (TP=1) kernel.
 *
 * Floating point: the pages fix fp32 for the scores, the scale factors and
 * the SwiGLU arithmetic, so the oracle computes in IEEE fp32 with
 * round-to-nearest-even (built with -ffp-contract=off, no fast-math).
 *
 * All functions return 0 on success and a negative value on an invalid
 * argument.  All pointers are host pointers owned by the caller.
 */
#ifndef MOE_FP8_ORACLE_H
#define MOE_FP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OCP FP8 E4M3FN encode (round to nearest, ties to even; finite overflow
 * saturates to +-448; NaN -> 0x7F with the sign bit of x) and decode. */
uint8_t oracle_e4m3_encode(float x);
float   oracle_e4m3_decode(uint8_t code);
/* Encode n floats (convenience for tests). */
void    oracle_e4m3_encode_n(const float* x, int64_t n, uint8_t* out);

/* One scale group: amax, clamped amax, sf = amax_c / 448, inv = 1 / sf,
 * q[i] = e4m3(v[i] * inv).  [TK] 3.1, 3.2. */
void oracle_cast_group(const float* v, int32_t n, uint8_t* q, float* sf);

/* Top-k gating.  [TK] 2.1 (iterative max, lowest index among equal maxima,
 * winner masked to -inf); weight normalisation named in [TK] 2. */
int oracle_topk_gate(const float* scores, int64_t num_tokens, int32_t num_experts,
                     int32_t num_topk, int32_t renormalize,
                     int64_t* topk_idx, float* topk_weights);

/* Group counting + token-expert mapping.  [TK] 2; [PPX] local kernel. */
int oracle_token_map(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                     int32_t num_experts, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* pos, int32_t* row_token);

/* Per-token cast then expand.  [TK] 2.2, 3.2.  pos == NULL: identity (K == 1). */
int oracle_expand_cast_fp8(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                           int32_t num_topk, const int32_t* pos,
                           const float* topk_weights, int64_t num_rows,
                           int32_t group_size, uint8_t* out_fp8, float* out_sf,
                           float* out_weights);

/* SwiGLU (+ optional clamp, + optional row weight) then per-group cast.  [TK] 3.3. */
int oracle_swiglu_cast_fp8(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                           const float* row_weights, float clamp_value,
                           int32_t group_size, uint8_t* out_fp8, float* out_sf);

/* Token map over the local experts [expert_begin, expert_end) with every
 * segment padded to a multiple of `align` rows.  [TK] 2.2 (pos < 0 skips;
 * invalid rows zero-filled by the expand); [PPX] local kernel (optional
 * padded buffers for the grouped GEMM; tensor-parallel dispatch selects the
 * tokens of the rank's experts).  counts/offsets index local experts
 * j = e - expert_begin; row_token has num_rows entries (-1 for padding and
 * for rows past offsets[E_local]); num_rows must be >= offsets[E_local]. */
int oracle_token_map_aligned(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                             int32_t expert_begin, int32_t expert_end, int32_t align,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                             int32_t* row_token, int64_t num_rows);

/* Expand into padded segments: expand_cast_fp8 for the routed copies, then
 * every row r < num_rows with row_token[r] < 0 is zero-filled (codes 0,
 * scales 0, weight 0).  [TK] 2.2. */
int oracle_expand_cast_fp8_padded(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                                  int32_t num_topk, const int32_t* pos, const float* topk_weights,
                                  const int32_t* row_token, int64_t num_rows, int32_t group_size,
                                  uint8_t* out_fp8, float* out_sf, float* out_weights);

/* Combine (weighted reduce back to token order).  [PPX] combine kernel;
 * [TK] 2 "Fused Expand/Reduce".  out[t,:] = bf16(sum over k, in k order, of
 * w[t,k] * y_rows[pos[t,k],:]) with fp32 products and sums; pos outside
 * [0, num_rows) is skipped; w == NULL means weight 1. */
int oracle_combine(const uint16_t* y_rows_bf16, int64_t num_rows, int32_t hidden,
                   const int32_t* pos, const float* weights, int64_t num_tokens,
                   int32_t num_topk, uint16_t* out_bf16);

/* fp32 -> bf16, round to nearest even (NaN -> quiet NaN with its sign). */
uint16_t oracle_f32_to_bf16(float x);


/* Cast formats ([TK] 3.1 CastOutputConfig; [PPX] Blackwell section, MXFP8 /
 * MXFP4 / NVFP4 group sizes). */
#define ORACLE_FMT_E4M3 0
#define ORACLE_FMT_E2M1 1

/* OCP FP4 E2M1 (code in the low 4 bits): round to nearest, ties to the even
 * code, saturating at +-6. */
uint8_t oracle_e2m1_encode(float x);
float   oracle_e2m1_decode(uint8_t code);
/* The format's default clamp: 1e-4 (e4m3), 6 * 2^-126 (e2m1). */
float   oracle_default_clamp(int32_t dtype);
/* One group in any format; round_sf: the smallest power-of-two scale with
 * sf * max_value >= max(amax, clamp); clamp_min <= 0: the format default. */
void    oracle_cast_group_fmt(const float* v, int32_t n, int32_t dtype, int32_t round_sf,
                              float clamp_min, uint8_t* q, float* sf);
/* UE8M0 byte of a power of two (biased exponent), and back. */
uint8_t oracle_ue8m0_encode(float pow2);
float   oracle_ue8m0_decode(uint8_t b);
/* Expand + cast / SwiGLU + cast in any format: e4m3 rows of H bytes or e2m1
 * rows of H / 2 bytes (element 2i in the low nibble); scales fp32 or, with
 * sf_ue8m0 (requires round_sf), one UE8M0 byte per group. */
int oracle_expand_cast(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                       int32_t num_topk, const int32_t* pos, const float* topk_weights,
                       int64_t num_rows, int32_t dtype, int32_t group_size, int32_t round_sf,
                       float clamp_min, int32_t sf_ue8m0, uint8_t* out, void* out_sf,
                       float* out_weights);
int oracle_swiglu_cast(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                       const float* row_weights, float clamp_value, int32_t dtype,
                       int32_t group_size, int32_t round_sf, float clamp_min, int32_t sf_ue8m0,
                       uint8_t* out, void* out_sf);

#ifdef __cplusplus
}
#endif

#endif
