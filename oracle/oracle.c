/*
 * CPU oracle for the MoE dispatch path.  TEST INFRASTRUCTURE ONLY: loaded by
 * the tests, the smoke check and the CPU-baseline leg of the benchmark; never
 * by the library.  Plain single-threaded C, IEEE fp32, round-to-nearest-even,
 * no contraction (see oracle/build.py for the flags).
 *
 * Each function states the definition it follows.  Pages cited:
 *   [TK]  "DeepSeek open-sources TileKernels: GPU operators written in Python
 *         approach the hardware limit" (itsolotime.com), sections 2, 2.1, 2.2,
 *         3.1, 3.2, 3.3.
 *   [PPX] "CuTeDSL at Perplexity" (perplexity.ai blog), "MoE dispatch and
 *         combine", local (TP=1) kernel.
 * Readings where the pages are silent are marked READING.
 */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* --------------------------------------------------------------------------
 * OCP FP8 E4M3FN.  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
 * Exponent field 0 holds subnormals m * 2^-9.  Field 15 with mantissa 7 is
 * NaN; there are no infinities, so the largest finite magnitude is
 * 1.75 * 2^8 = 448 (code 0x7E).  The pages name the format as float8_e4m3fn
 * ([TK] 3.1) without stating a rounding rule.
 * READING: round to nearest, ties to even mantissa; a finite magnitude that
 * rounds past 448 saturates to 448.
 * ------------------------------------------------------------------------ */

float oracle_e4m3_decode(uint8_t code) {
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    float v;
    if (e == 15 && m == 7) return s ? -NAN : NAN;
    if (e == 0)
        v = (float)m * ldexpf(1.0f, -9);
    else
        v = (1.0f + (float)m / 8.0f) * ldexpf(1.0f, e - 7);
    return s ? -v : v;
}

/* Round r >= 0 to an integer, ties to even. */
static float round_half_even(float r) {
    float n = floorf(r);
    float frac = r - n; /* exact for the magnitudes used here (r < 2^5) */
    if (frac > 0.5f) return n + 1.0f;
    if (frac < 0.5f) return n;
    return (fmodf(n, 2.0f) == 0.0f) ? n : n + 1.0f;
}

uint8_t oracle_e4m3_encode(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return sign | 0x7F;
    float a = fabsf(x);
    /* 464 is the midpoint between 448 and the first magnitude past the
     * format (480); ties go to the even mantissa of 448, and everything above
     * saturates. */
    if (a >= 464.0f) return sign | 0x7E;

    /* Spacing of representable values around a: 2^(e-3) in binade
     * [2^e, 2^(e+1)) for e >= -6, and 2^-9 below 2^-6 (subnormals). */
    float quantum;
    if (a < ldexpf(1.0f, -6)) {
        quantum = ldexpf(1.0f, -9);
    } else {
        int fe;
        (void)frexpf(a, &fe); /* a = f * 2^fe, f in [0.5, 1) -> binade 2^(fe-1) */
        quantum = ldexpf(1.0f, fe - 1 - 3);
    }
    float n = round_half_even(a / quantum); /* division by a power of two: exact */
    float y = n * quantum;                   /* the rounded magnitude, exact */

    /* Encode the representable magnitude y. */
    if (y == 0.0f) return sign;
    if (y < ldexpf(1.0f, -6)) return sign | (uint8_t)(y / ldexpf(1.0f, -9));
    int fe;
    (void)frexpf(y, &fe);
    int e = fe - 1;                                   /* y in [2^e, 2^(e+1)) */
    int m = (int)((y / ldexpf(1.0f, e) - 1.0f) * 8.0f); /* exact */
    return sign | (uint8_t)(((e + 7) << 3) | m);
}

void oracle_e4m3_encode_n(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

/* --------------------------------------------------------------------------
 * One scale group ([TK] 3.2 steps 2-4; clamp from [TK] 3.1).
 *   amax  = max |v_i|                      (exact)
 *   amax' = max(amax, 1e-4)                READING: the e4m3 clamp_min_value
 *                                          bounds amax (so sf stays normal)
 *   sf    = amax' / 448                    (fp32, RN)
 *   inv   = 1 / sf                         ("multiply by the inverse of SF")
 *   q_i   = e4m3(v_i * inv)                (one fp32 multiply, RN)
 * ------------------------------------------------------------------------ */
void oracle_cast_group(const float* v, int32_t n, uint8_t* q, float* sf_out) {
    float amax = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    const float clamp_min = 1e-4f;
    float amax_c = (amax > clamp_min) ? amax : clamp_min;
    float sf = amax_c / 448.0f;
    float inv = 1.0f / sf;
    for (int32_t i = 0; i < n; ++i) q[i] = oracle_e4m3_encode(v[i] * inv);
    *sf_out = sf;
}

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* --------------------------------------------------------------------------
 * Top-k gating ([TK] 2.1).  For each token: K rounds of
 *   (1) amax = max over the row,
 *   (2) idx  = the lowest index i with row[i] == amax (IEEE ==, so -0 == +0),
 *   (3) row[idx] = -inf.
 * topk_idx[t, k] is the round-k winner, so the K ids come out in descending
 * score order.
 * READING: a NaN score is treated as -inf (the pages assume finite scores).
 * Weights ([TK] 2, "Weight Normalization", no formula given).
 * READING: w_k is the selected (NaN-canonicalised) score; with renormalize,
 *   sum = ((g_0 + g_1) + ...) + g_{K-1} in fp32, then w_k = g_k / sum.
 * ------------------------------------------------------------------------ */
int oracle_topk_gate(const float* scores, int64_t num_tokens, int32_t num_experts,
                     int32_t num_topk, int32_t renormalize,
                     int64_t* topk_idx, float* topk_weights) {
    if (num_tokens < 0 || num_experts < 1 || num_topk < 1 || num_topk > num_experts)
        return ORACLE_EINVAL;
    if (num_tokens > 0 && (!scores || !topk_idx)) return ORACLE_EINVAL;
    if (renormalize && !topk_weights) return ORACLE_EINVAL;
    const int32_t E = num_experts, K = num_topk;
    float* s = (float*)malloc((size_t)E * sizeof(float));
    float* g = (float*)malloc((size_t)K * sizeof(float));
    if (!s || !g) { free(s); free(g); return ORACLE_ENOMEM; }

    for (int64_t t = 0; t < num_tokens; ++t) {
        const float* row = scores + t * E;
        for (int32_t i = 0; i < E; ++i) s[i] = isnan(row[i]) ? -INFINITY : row[i];
        for (int32_t k = 0; k < K; ++k) {
            float amax = s[0];
            for (int32_t i = 1; i < E; ++i)
                if (s[i] > amax) amax = s[i];
            int32_t best = INT32_MAX;
            for (int32_t i = 0; i < E; ++i)
                if (s[i] == amax && i < best) best = i;
            topk_idx[t * K + k] = best;
            g[k] = isnan(row[best]) ? -INFINITY : row[best];
            s[best] = -INFINITY;
        }
        if (topk_weights) {
            if (renormalize) {
                float sum = 0.0f;
                for (int32_t k = 0; k < K; ++k) sum = sum + g[k];
                for (int32_t k = 0; k < K; ++k) topk_weights[t * K + k] = g[k] / sum;
            } else {
                for (int32_t k = 0; k < K; ++k) topk_weights[t * K + k] = g[k];
            }
        }
    }
    free(s);
    free(g);
    return 0;
}

/* --------------------------------------------------------------------------
 * Group counting + token-expert mapping ([TK] 2; [PPX] local kernel: count
 * the tokens of each expert, then give each token a unique index in its
 * expert's list).
 *   counts[e]    = #{(t,k) : idx[t,k] == e}
 *   offsets[0]   = 0, offsets[e+1] = offsets[e] + counts[e]
 *   pos[t,k]     = offsets[e] + #{(t',k') before (t,k) in row-major order
 *                                 with idx[t',k'] == e}
 *   row_token[r] = the token whose copy lands in row r
 * READING: rows inside an expert's segment are in ascending (t,k) order (a
 * stable counting sort); the pages' shared-memory atomics give arrival order,
 * which is one of the valid groupings.
 * READING: an id outside [0, E) is not counted and gets pos = -1 (the pages'
 * "pos < 0: skip" convention); row_token rows past offsets[E] hold -1.
 * ------------------------------------------------------------------------ */
int oracle_token_map(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                     int32_t num_experts, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* pos, int32_t* row_token) {
    if (num_tokens < 0 || num_topk < 1 || num_experts < 1) return ORACLE_EINVAL;
    if (num_tokens * (int64_t)num_topk > INT32_MAX) return ORACLE_EINVAL;
    if (!expert_counts || !expert_offsets) return ORACLE_EINVAL;
    if (num_tokens > 0 && (!topk_idx || !pos)) return ORACLE_EINVAL;
    const int32_t E = num_experts, K = num_topk;
    const int64_t R = num_tokens * K;

    for (int32_t e = 0; e < E; ++e) expert_counts[e] = 0;
    for (int64_t i = 0; i < R; ++i) {
        int64_t e = topk_idx[i];
        if (e >= 0 && e < E) expert_counts[e] += 1;
    }
    expert_offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];

    int32_t* cursor = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    if (!cursor) return ORACLE_ENOMEM;
    for (int32_t e = 0; e < E; ++e) cursor[e] = expert_offsets[e];
    if (row_token)
        for (int64_t r = 0; r < R; ++r) row_token[r] = -1;
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0 || e >= E) {
                pos[t * K + k] = -1;
                continue;
            }
            int32_t p = cursor[e];
            cursor[e] = p + 1;
            pos[t * K + k] = p;
            if (row_token) row_token[p] = (int32_t)t;
        }
    }
    free(cursor);
    return 0;
}

/* --------------------------------------------------------------------------
 * Expand + cast ([TK] 2.2 fused expand, [TK] 3.2 per-token cast).
 * Plain definition: cast token row t group by group (oracle_cast_group), then
 * for each k with r = pos[t,k] in [0, num_rows) copy the codes, the scale row
 * and (if given) the routing weight w[t,k] to row r.  Rows no copy lands in
 * are left untouched.  pos == NULL is the identity map (K == 1, r = t): the
 * plain per-token cast.
 * ------------------------------------------------------------------------ */
int oracle_expand_cast_fp8(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                           int32_t num_topk, const int32_t* pos,
                           const float* topk_weights, int64_t num_rows,
                           int32_t group_size, uint8_t* out_fp8, float* out_sf,
                           float* out_weights) {
    if (num_tokens < 0 || hidden < 1 || num_topk < 1 || group_size < 1) return ORACLE_EINVAL;
    if (hidden % group_size != 0) return ORACLE_EINVAL;
    if ((topk_weights == NULL) != (out_weights == NULL)) return ORACLE_EINVAL;
    if (pos == NULL && (num_topk != 1 || num_rows != num_tokens)) return ORACLE_EINVAL;
    if (pos != NULL && num_rows != num_tokens * num_topk) return ORACLE_EINVAL;
    if (num_tokens > 0 && (!x_bf16 || !out_fp8 || !out_sf)) return ORACLE_EINVAL;
    const int32_t H = hidden, K = num_topk, G = hidden / group_size;

    float* v = (float*)malloc((size_t)group_size * sizeof(float));
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sf = (float*)malloc((size_t)G * sizeof(float));
    if (!v || !q || !sf) { free(v); free(q); free(sf); return ORACLE_ENOMEM; }

    for (int64_t t = 0; t < num_tokens; ++t) {
        const uint16_t* xr = x_bf16 + t * H;
        for (int32_t g = 0; g < G; ++g) {
            for (int32_t i = 0; i < group_size; ++i) v[i] = bf16_to_f32(xr[g * group_size + i]);
            oracle_cast_group(v, group_size, q + g * group_size, &sf[g]);
        }
        for (int32_t k = 0; k < K; ++k) {
            int64_t r = pos ? (int64_t)pos[t * K + k] : t;
            if (r < 0 || r >= num_rows) continue;
            memcpy(out_fp8 + r * H, q, (size_t)H);
            memcpy(out_sf + r * G, sf, (size_t)G * sizeof(float));
            if (out_weights) out_weights[r] = topk_weights[t * K + k];
        }
    }
    free(v);
    free(q);
    free(sf);
    return 0;
}

/* --------------------------------------------------------------------------
 * SwiGLU + cast ([TK] 3.3).  For row r and column j < I:
 *   l = gate = x[r, j],  u = up = x[r, I + j]          (bf16 -> fp32, exact)
 *   if clamp c > 0:  l = min(l, c);  u = max(min(u, c), -c)
 *   v = l / (1 + exp(-l)) * u [* w[r]]                 (fp32, left to right)
 * then each 128-column group of v is cast (oracle_cast_group).
 * READING: gate is the left half of the last dimension, up the right half;
 * v stays fp32 (no bf16 rounding) before the amax.
 * ------------------------------------------------------------------------ */
int oracle_swiglu_cast_fp8(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                           const float* row_weights, float clamp_value,
                           int32_t group_size, uint8_t* out_fp8, float* out_sf) {
    if (num_rows < 0 || inter < 1 || group_size < 1 || inter % group_size != 0)
        return ORACLE_EINVAL;
    if (num_rows > 0 && (!gate_up_bf16 || !out_fp8 || !out_sf)) return ORACLE_EINVAL;
    const int32_t I = inter, G = inter / group_size;
    float* v = (float*)malloc((size_t)group_size * sizeof(float));
    if (!v) return ORACLE_ENOMEM;
    for (int64_t r = 0; r < num_rows; ++r) {
        const uint16_t* xr = gate_up_bf16 + r * 2 * (int64_t)I;
        for (int32_t g = 0; g < G; ++g) {
            for (int32_t i = 0; i < group_size; ++i) {
                int32_t j = g * group_size + i;
                float l = bf16_to_f32(xr[j]);
                float u = bf16_to_f32(xr[I + j]);
                if (clamp_value > 0.0f) {
                    l = fminf(l, clamp_value);
                    u = fmaxf(fminf(u, clamp_value), -clamp_value);
                }
                float val = l / (1.0f + expf(-l));
                val = val * u;
                if (row_weights) val = val * row_weights[r];
                v[i] = val;
            }
            oracle_cast_group(v, group_size, out_fp8 + r * I + g * group_size, &out_sf[r * G + g]);
        }
    }
    free(v);
    return 0;
}

/* --------------------------------------------------------------------------
 * Combine ([PPX] "MoE dispatch and combine": the combine accumulates, in
 * registers, each token's expert outputs found through the positions the
 * dispatch computed, and writes the final token; [TK] 2 names the step
 * "Fused Expand/Reduce").
 *   acc = 0; for k = 0..K-1 with r = pos[t,k] in [0, R):
 *       acc = acc + w[t,k] * y_rows[r, h]          (fp32 multiply, fp32 add)
 *   out[t, h] = bf16(acc)                          (round to nearest even)
 * READING: the sum runs in k order (the routing order), one rounding per
 * product and per add (no fused multiply-add); a missing weight is 1.
 * ------------------------------------------------------------------------ */
uint16_t oracle_f32_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
    /* round to nearest, ties to even, on the 16 dropped bits */
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

int oracle_combine(const uint16_t* y_rows_bf16, int64_t num_rows, int32_t hidden,
                   const int32_t* pos, const float* weights, int64_t num_tokens,
                   int32_t num_topk, uint16_t* out_bf16) {
    if (num_rows < 0 || hidden < 1 || num_tokens < 0 || num_topk < 1) return ORACLE_EINVAL;
    if (num_tokens > 0 && (!pos || !out_bf16)) return ORACLE_EINVAL;
    if (num_rows > 0 && num_tokens > 0 && !y_rows_bf16) return ORACLE_EINVAL;
    const int32_t H = hidden, K = num_topk;
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int64_t r = pos[t * K + k];
                if (r < 0 || r >= num_rows) continue;
                float wk = weights ? weights[t * K + k] : 1.0f;
                float prod = wk * bf16_to_f32(y_rows_bf16[r * H + h]);
                acc = acc + prod;
            }
            out_bf16[t * H + h] = oracle_f32_to_bf16(acc);
        }
    }
    return 0;
}

/* --------------------------------------------------------------------------
 * Aligned, expert-local token map.  [TK] 2.2: positions < 0 are skipped and
 * the expand's grid also zero-fills the invalid rows; [PPX] local kernel:
 * tokens are optionally copied into padded buffers for the MoE GEMM, and the
 * tensor-parallel variant routes only the tokens of the rank's experts.
 * READING: local experts are the contiguous id range [expert_begin,
 * expert_end); segment j (expert expert_begin + j) starts at
 *   offsets[j] = sum over j' < j of ceil(counts[j'] / align) * align
 * and holds its copies in ascending (t, k) order, then padding rows up to
 * the next multiple of align.  Copies of other experts get pos = -1.
 * ------------------------------------------------------------------------ */
int oracle_token_map_aligned(const int64_t* topk_idx, int64_t num_tokens, int32_t num_topk,
                             int32_t expert_begin, int32_t expert_end, int32_t align,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* pos,
                             int32_t* row_token, int64_t num_rows) {
    if (num_tokens < 0 || num_topk < 1 || align < 1 || expert_begin < 0 ||
        expert_end <= expert_begin)
        return ORACLE_EINVAL;
    if (!expert_counts || !expert_offsets) return ORACLE_EINVAL;
    if (num_tokens > 0 && (!topk_idx || !pos)) return ORACLE_EINVAL;
    const int32_t EL = expert_end - expert_begin, K = num_topk;
    const int64_t N = num_tokens * K;
    for (int32_t j = 0; j < EL; ++j) expert_counts[j] = 0;
    for (int64_t i = 0; i < N; ++i) {
        int64_t e = topk_idx[i];
        if (e >= expert_begin && e < expert_end) expert_counts[e - expert_begin] += 1;
    }
    int64_t acc = 0;
    for (int32_t j = 0; j < EL; ++j) {
        expert_offsets[j] = (int32_t)acc;
        acc += (expert_counts[j] + (int64_t)align - 1) / align * align;
    }
    expert_offsets[EL] = (int32_t)acc;
    if (acc > num_rows) return ORACLE_EINVAL;
    int32_t* cursor = (int32_t*)malloc((size_t)EL * sizeof(int32_t));
    if (!cursor) return ORACLE_ENOMEM;
    for (int32_t j = 0; j < EL; ++j) cursor[j] = expert_offsets[j];
    if (row_token)
        for (int64_t r = 0; r < num_rows; ++r) row_token[r] = -1;
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < expert_begin || e >= expert_end) {
                pos[t * K + k] = -1;
                continue;
            }
            int32_t p = cursor[e - expert_begin]++;
            pos[t * K + k] = p;
            if (row_token) row_token[p] = (int32_t)t;
        }
    }
    free(cursor);
    return 0;
}

/* --------------------------------------------------------------------------
 * Expand into padded segments ([TK] 2.2: one grid covers both the routed
 * copies and the invalid rows, which it zero-fills).  The plain definition:
 * expand the routed copies (oracle_expand_cast_fp8 semantics, rows past
 * T*K allowed), then every row r with row_token[r] < 0 gets codes 0,
 * scales 0 and weight 0.
 * ------------------------------------------------------------------------ */
int oracle_expand_cast_fp8_padded(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                                  int32_t num_topk, const int32_t* pos, const float* topk_weights,
                                  const int32_t* row_token, int64_t num_rows, int32_t group_size,
                                  uint8_t* out_fp8, float* out_sf, float* out_weights) {
    if (num_tokens < 0 || hidden < 1 || num_topk < 1 || group_size < 1 || hidden % group_size != 0)
        return ORACLE_EINVAL;
    if ((topk_weights == NULL) != (out_weights == NULL)) return ORACLE_EINVAL;
    if (num_rows < 0 || (num_rows > 0 && (!row_token || !out_fp8 || !out_sf))) return ORACLE_EINVAL;
    if (num_tokens > 0 && (!x_bf16 || !pos)) return ORACLE_EINVAL;
    const int32_t H = hidden, K = num_topk, G = hidden / group_size;
    float* v = (float*)malloc((size_t)group_size * sizeof(float));
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sf = (float*)malloc((size_t)G * sizeof(float));
    if (!v || !q || !sf) { free(v); free(q); free(sf); return ORACLE_ENOMEM; }
    for (int64_t t = 0; t < num_tokens; ++t) {
        const uint16_t* xr = x_bf16 + t * H;
        for (int32_t g = 0; g < G; ++g) {
            for (int32_t i = 0; i < group_size; ++i) v[i] = bf16_to_f32(xr[g * group_size + i]);
            oracle_cast_group(v, group_size, q + g * group_size, &sf[g]);
        }
        for (int32_t k = 0; k < K; ++k) {
            int64_t r = pos[t * K + k];
            if (r < 0 || r >= num_rows) continue;
            memcpy(out_fp8 + r * H, q, (size_t)H);
            memcpy(out_sf + r * G, sf, (size_t)G * sizeof(float));
            if (out_weights) out_weights[r] = topk_weights[t * K + k];
        }
    }
    for (int64_t r = 0; r < num_rows; ++r) {
        if (row_token[r] >= 0) continue;
        memset(out_fp8 + r * H, 0, (size_t)H);
        for (int32_t g = 0; g < G; ++g) out_sf[r * G + g] = 0.0f;
        if (out_weights) out_weights[r] = 0.0f;
    }
    free(v);
    free(q);
    free(sf);
    return 0;
}

/* --------------------------------------------------------------------------
 * Cast formats beyond e4m3 / 128 ([TK] 3.1: CastOutputConfig carries the
 * output dtype, the scaling block size, round_sf and the clamp; the clamp of
 * float4_e2m1fn is max_value * 2^-126; [PPX] Blackwell section: MXFP8 and
 * MXFP4 take the absmax over 32 elements, NVFP4 over 16).
 *
 * OCP FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; codes
 * 0..7 are the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (no inf, no NaN).
 * READING: round to nearest, ties to the even code, magnitudes past 6
 * saturate to 6; a NaN input (never produced by a finite cast) encodes as the
 * saturated magnitude.
 * ------------------------------------------------------------------------ */

static const float kE2m1Mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float oracle_e2m1_decode(uint8_t code) {
    float m = kE2m1Mag[code & 7];
    return (code & 8) ? -m : m;
}

uint8_t oracle_e2m1_encode(float x) {
    uint8_t sign = signbit(x) ? 8 : 0;
    if (isnan(x)) return sign | 7;
    float a = fabsf(x);
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        float d = fabsf(a - kE2m1Mag[c]), db = fabsf(a - kE2m1Mag[best]);
        /* strictly nearer wins; on a tie the even code wins */
        if (d < db || (d == db && (c & 1) == 0)) best = c;
    }
    return sign | (uint8_t)best;
}

/* Largest finite magnitude of the output format. */
static float fmt_max(int32_t dtype) { return dtype == ORACLE_FMT_E2M1 ? 6.0f : 448.0f; }

/* The clamp of [TK] 3.1: 1e-4 for e4m3, max_value * 2^-126 for e2m1, unless
 * the caller gives one (custom_clamp_min_value). */
float oracle_default_clamp(int32_t dtype) {
    return dtype == ORACLE_FMT_E2M1 ? 6.0f * ldexpf(1.0f, -126) : 1e-4f;
}

/* One group in any format:
 *   amax = max |v_i|,  c = max(amax, clamp)
 *   round_sf == 0:  sf = c / max_value (fp32, RN)
 *   round_sf == 1:  sf = the smallest power of two with sf * max_value >= c
 *                   READING of round_sf ("round the scale to a power of
 *                   two"): rounding up keeps |v_i / sf| <= max_value, so no
 *                   code saturates.
 *   inv = 1 / sf;  q_i = encode(v_i * inv)  (one byte per value; an e2m1
 *   code sits in the low 4 bits). */
void oracle_cast_group_fmt(const float* v, int32_t n, int32_t dtype, int32_t round_sf,
                           float clamp_min, uint8_t* q, float* sf_out) {
    float amax = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    const float clamp = clamp_min > 0.0f ? clamp_min : oracle_default_clamp(dtype);
    const float c = amax > clamp ? amax : clamp;
    const float maxv = fmt_max(dtype);
    float sf;
    if (round_sf) {
        /* powers of two times 448 or 6 are exact in double */
        double s = ldexp(1.0, -149);
        while (s * (double)maxv < (double)c) s *= 2.0;
        sf = (float)s;
    } else {
        sf = c / maxv;
    }
    const float inv = 1.0f / sf;
    for (int32_t i = 0; i < n; ++i) {
        float y = v[i] * inv;
        q[i] = dtype == ORACLE_FMT_E2M1 ? oracle_e2m1_encode(y) : oracle_e4m3_encode(y);
    }
    *sf_out = sf;
}

/* UE8M0 scale byte: the biased exponent e + 127 of a power of two 2^e,
 * e in [-127, 127] (255 would be NaN).  READING of "packed UE8M0": one byte
 * per group, four consecutive groups in one little-endian 32-bit word, which
 * is the same memory as a byte per group in row-major order. */
uint8_t oracle_ue8m0_encode(float pow2) {
    int e;
    float f = frexpf(pow2, &e); /* pow2 = 0.5 * 2^e */
    (void)f;
    return (uint8_t)(e - 1 + 127);
}

float oracle_ue8m0_decode(uint8_t b) { return ldexpf(1.0f, (int)b - 127); }

/* Stores one cast row: codes (e4m3: a byte each; e2m1: element 2i in the low
 * nibble of byte i, 2i+1 in the high nibble) and scales (fp32 or UE8M0). */
static void store_row_fmt(const uint8_t* q, const float* sf, int32_t H, int32_t G, int32_t dtype,
                          int32_t sf_ue8m0, uint8_t* out_row, void* sf_row) {
    if (dtype == ORACLE_FMT_E2M1) {
        for (int32_t i = 0; i < H / 2; ++i)
            out_row[i] = (uint8_t)((q[2 * i] & 0xF) | ((q[2 * i + 1] & 0xF) << 4));
    } else {
        memcpy(out_row, q, (size_t)H);
    }
    for (int32_t g = 0; g < G; ++g) {
        if (sf_ue8m0)
            ((uint8_t*)sf_row)[g] = oracle_ue8m0_encode(sf[g]);
        else
            ((float*)sf_row)[g] = sf[g];
    }
}

static int fmt_ok(int32_t dtype, int32_t group_size, int32_t round_sf, int32_t sf_ue8m0) {
    if (dtype != ORACLE_FMT_E4M3 && dtype != ORACLE_FMT_E2M1) return 0;
    if (group_size < 2 || group_size % 2) return 0;
    if (sf_ue8m0 && !round_sf) return 0; /* UE8M0 holds powers of two only */
    return 1;
}

/* Expand + cast in any format ([TK] 2.2, 3.1, 3.2): as oracle_expand_cast_fp8
 * with the group cast oracle_cast_group_fmt.  Row bytes: H (e4m3) or H / 2
 * (e2m1); scale rows: H / group_size fp32 or UE8M0 bytes. */
int oracle_expand_cast(const uint16_t* x_bf16, int64_t num_tokens, int32_t hidden,
                       int32_t num_topk, const int32_t* pos, const float* topk_weights,
                       int64_t num_rows, int32_t dtype, int32_t group_size, int32_t round_sf,
                       float clamp_min, int32_t sf_ue8m0, uint8_t* out, void* out_sf,
                       float* out_weights) {
    if (!fmt_ok(dtype, group_size, round_sf, sf_ue8m0)) return ORACLE_EINVAL;
    if (num_tokens < 0 || hidden < 1 || num_topk < 1 || hidden % group_size != 0) return ORACLE_EINVAL;
    if ((topk_weights == NULL) != (out_weights == NULL)) return ORACLE_EINVAL;
    if (pos == NULL && (num_topk != 1 || num_rows != num_tokens)) return ORACLE_EINVAL;
    if (pos != NULL && num_rows != num_tokens * num_topk) return ORACLE_EINVAL;
    if (num_tokens > 0 && (!x_bf16 || !out || !out_sf)) return ORACLE_EINVAL;
    const int32_t H = hidden, K = num_topk, G = hidden / group_size;
    const int64_t row_bytes = dtype == ORACLE_FMT_E2M1 ? H / 2 : H;
    const size_t sf_bytes = sf_ue8m0 ? 1 : sizeof(float);
    float* v = (float*)malloc((size_t)H * sizeof(float));
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sf = (float*)malloc((size_t)G * sizeof(float));
    uint8_t* row = (uint8_t*)malloc((size_t)row_bytes);
    uint8_t* srow = (uint8_t*)malloc((size_t)G * sf_bytes);
    if (!v || !q || !sf || !row || !srow) {
        free(v); free(q); free(sf); free(row); free(srow);
        return ORACLE_ENOMEM;
    }
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int32_t j = 0; j < H; ++j) v[j] = bf16_to_f32(x_bf16[t * H + j]);
        for (int32_t g = 0; g < G; ++g)
            oracle_cast_group_fmt(v + g * group_size, group_size, dtype, round_sf, clamp_min,
                                  q + g * group_size, &sf[g]);
        store_row_fmt(q, sf, H, G, dtype, sf_ue8m0, row, srow);
        for (int32_t k = 0; k < K; ++k) {
            int64_t r = pos ? (int64_t)pos[t * K + k] : t;
            if (r < 0 || r >= num_rows) continue;
            memcpy(out + r * row_bytes, row, (size_t)row_bytes);
            memcpy((uint8_t*)out_sf + r * G * (int64_t)sf_bytes, srow, (size_t)G * sf_bytes);
            if (out_weights) out_weights[r] = topk_weights[t * K + k];
        }
    }
    free(v); free(q); free(sf); free(row); free(srow);
    return 0;
}

/* SwiGLU + cast in any format ([TK] 3.3 with [TK] 3.1's configurations): v
 * as in oracle_swiglu_cast_fp8, then oracle_cast_group_fmt per group. */
int oracle_swiglu_cast(const uint16_t* gate_up_bf16, int64_t num_rows, int32_t inter,
                       const float* row_weights, float clamp_value, int32_t dtype,
                       int32_t group_size, int32_t round_sf, float clamp_min, int32_t sf_ue8m0,
                       uint8_t* out, void* out_sf) {
    if (!fmt_ok(dtype, group_size, round_sf, sf_ue8m0)) return ORACLE_EINVAL;
    if (num_rows < 0 || inter < 1 || inter % group_size != 0) return ORACLE_EINVAL;
    if (num_rows > 0 && (!gate_up_bf16 || !out || !out_sf)) return ORACLE_EINVAL;
    const int32_t I = inter, G = inter / group_size;
    const int64_t row_bytes = dtype == ORACLE_FMT_E2M1 ? I / 2 : I;
    const size_t sf_bytes = sf_ue8m0 ? 1 : sizeof(float);
    float* v = (float*)malloc((size_t)I * sizeof(float));
    uint8_t* q = (uint8_t*)malloc((size_t)I);
    float* sf = (float*)malloc((size_t)G * sizeof(float));
    if (!v || !q || !sf) { free(v); free(q); free(sf); return ORACLE_ENOMEM; }
    for (int64_t r = 0; r < num_rows; ++r) {
        const uint16_t* xr = gate_up_bf16 + r * 2 * (int64_t)I;
        for (int32_t j = 0; j < I; ++j) {
            float l = bf16_to_f32(xr[j]);
            float u = bf16_to_f32(xr[I + j]);
            if (clamp_value > 0.0f) {
                l = fminf(l, clamp_value);
                u = fmaxf(fminf(u, clamp_value), -clamp_value);
            }
            float val = l / (1.0f + expf(-l));
            val = val * u;
            if (row_weights) val = val * row_weights[r];
            v[j] = val;
        }
        for (int32_t g = 0; g < G; ++g)
            oracle_cast_group_fmt(v + g * group_size, group_size, dtype, round_sf, clamp_min,
                                  q + g * group_size, &sf[g]);
        store_row_fmt(q, sf, I, G, dtype, sf_ue8m0, out + r * row_bytes,
                      (uint8_t*)out_sf + r * G * (int64_t)sf_bytes);
    }
    free(v); free(q); free(sf);
    return 0;
}
