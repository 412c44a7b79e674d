/* Drives every oracle function on small inputs (with edge cases) so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer can check the
 * oracle's memory accesses and arithmetic.  Prints "ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint32_t rng_state = 12345u;
static float frand(void) {
    rng_state = rng_state * 1664525u + 1013904223u;
    return ((float)(rng_state >> 8) / 16777216.0f - 0.5f) * 8.0f;
}
static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void) {
    const int64_t T = 37;
    const int32_t E = 24, K = 5, H = 256, I = 256;
    float* scores = malloc(sizeof(float) * T * E);
    for (int64_t i = 0; i < T * E; ++i) scores[i] = frand();
    scores[3] = NAN;
    scores[E + 1] = -INFINITY;
    int64_t* idx = malloc(sizeof(int64_t) * T * K);
    float* w = malloc(sizeof(float) * T * K);
    if (oracle_topk_gate(scores, T, E, K, 1, idx, w)) return 1;
    int32_t *counts = malloc(4 * E), *offsets = malloc(4 * (E + 1)), *pos = malloc(4 * T * K),
            *row_token = malloc(4 * T * K);
    if (oracle_token_map(idx, T, K, E, counts, offsets, pos, row_token)) return 2;
    uint16_t* x = malloc(2 * T * H);
    for (int64_t i = 0; i < T * H; ++i) x[i] = bf16(frand() * (i % 7 ? 1.0f : 100.0f));
    uint8_t* q = calloc(T * K * H, 1);
    float* sf = calloc(T * K * (H / 128), sizeof(float));
    float* ow = calloc(T * K, sizeof(float));
    if (oracle_expand_cast_fp8(x, T, H, K, pos, w, T * K, 128, q, sf, ow)) return 3;
    uint16_t* gu = malloc(2 * T * 2 * I);
    for (int64_t i = 0; i < T * 2 * I; ++i) gu[i] = bf16(frand() * 4.0f);
    uint8_t* sq = malloc(T * I);
    float* ssf = malloc(sizeof(float) * T * (I / 128));
    if (oracle_swiglu_cast_fp8(gu, T, I, w, 2.5f, 128, sq, ssf)) return 4;
    uint16_t* y = malloc(2 * T * K * H);
    for (int64_t i = 0; i < T * K * H; ++i) y[i] = bf16(frand());
    uint16_t* comb = malloc(2 * T * H);
    if (oracle_combine(y, T * K, H, pos, w, T, K, comb)) return 5;
    const int32_t align = 8, EL = 10, rows = (int32_t)(T * K + EL * (align - 1));
    int32_t* rt = malloc(4 * rows);
    if (oracle_token_map_aligned(idx, T, K, 4, 14, align, counts, offsets, pos, rt, rows)) return 6;
    uint8_t* pq = malloc((size_t)rows * H);
    float* psf = malloc(sizeof(float) * rows * (H / 128));
    float* pw = malloc(sizeof(float) * rows);
    if (oracle_expand_cast_fp8_padded(x, T, H, K, pos, w, rt, rows, 128, pq, psf, pw)) return 7;
    for (int dt = 0; dt < 2; ++dt)
        for (int g = 16; g <= 128; g *= 2) {
            if (g == 64) continue;
            for (int r = 0; r < 2; ++r) {
                uint8_t* mq = malloc(T * K * H);
                uint8_t* msf = malloc(sizeof(float) * T * K * (H / g));
                if (oracle_expand_cast(x, T, H, K, pos, w, T * K, dt, g, r, 0.0f, r, mq, msf, ow)) return 8;
                if (oracle_swiglu_cast(gu, T, I, NULL, 0.0f, dt, g, r, 0.5f, 0, mq, msf)) return 9;
                free(mq);
                free(msf);
            }
        }
    for (uint32_t b = 0; b < 65536; ++b) {
        uint32_t u = b << 16;
        float f;
        memcpy(&f, &u, 4);
        (void)oracle_e4m3_encode(f);
        (void)oracle_e2m1_encode(f);
    }
    for (int c = 0; c < 256; ++c) (void)oracle_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 16; ++c) (void)oracle_e2m1_decode((uint8_t)c);
    (void)oracle_ue8m0_decode(oracle_ue8m0_encode(0.5f));
    /* empty batch and invalid arguments */
    if (oracle_token_map(idx, 0, K, E, counts, offsets, pos, row_token)) return 10;
    if (oracle_topk_gate(scores, 4, E, E + 1, 0, idx, NULL) == 0) return 11;
    free(scores); free(idx); free(w); free(counts); free(offsets); free(pos); free(row_token);
    free(x); free(q); free(sf); free(ow); free(gu); free(sq); free(ssf); free(y); free(comb);
    free(rt); free(pq); free(psf); free(pw);
    puts("ok");
    return 0;
}
