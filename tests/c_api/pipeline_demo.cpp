// Standalone use of the C ABI (include/moe_fp8.h) from C++ with the HIP
// runtime only -- no Python, no torch: device buffers from hipMalloc, one
// stream, the four calls of the dispatch path (top-k gating, token map,
// expand + e4m3 cast, SwiGLU + e4m3 cast), then host checks of what the
// definitions fix without a reference implementation:
//   top-k   ids distinct and in range, scores non-increasing in k, weights
//           the renormalised scores;
//   map     counts = histogram of the ids, offsets = their exclusive scan,
//           pos a permutation with row_token its inverse, stable order
//           inside each expert's segment;
//   expand  every copy of a token identical, scales = max(amax, 1e-4) / 448
//           of the token's 128-channel groups, weights carried;
//   SwiGLU  scales positive and finite;
//   route   moe_route's fused form equals the top-k and map calls bit for
//           bit, three calls on one workspace;
//   errors  an invalid argument returns MOE_ERR_INVALID_ARGUMENT.
// Prints "c-api pipeline ok" and exits 0 when every check holds.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "moe_fp8.h"

#define HIP_OK(x)                                                                        \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
            std::exit(2);                                                                \
        }                                                                                \
    } while (0)
#define MOE_OK_(x)                                                                       \
    do {                                                                                 \
        int s_ = (x);                                                                    \
        if (s_ != MOE_OK) {                                                              \
            std::fprintf(stderr, "%s: %s\n", #x, moe_status_string(s_));                 \
            std::exit(3);                                                                \
        }                                                                                \
    } while (0)

static int failures = 0;
static void check(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "check failed: %s\n", what);
        ++failures;
    }
}

static uint32_t next(uint32_t& s) { return s = s * 1664525u + 1013904223u; }
static float uniform(uint32_t& s, float lo, float hi) { return lo + (hi - lo) * (next(s) >> 8) * 0x1p-24f; }
static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint16_t to_bf16(float f) {  // round to nearest even
    const uint32_t u = bits(f);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <typename T>
static T* upload(const std::vector<T>& h) {
    T* d = nullptr;
    HIP_OK(hipMalloc(&d, h.size() * sizeof(T)));
    HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}
template <typename T>
static T* alloc(size_t n) {
    T* d = nullptr;
    HIP_OK(hipMalloc(&d, (n ? n : 1) * sizeof(T)));
    return d;
}
template <typename T>
static std::vector<T> download(const T* d, size_t n) {
    std::vector<T> h(n);
    HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

int main() {
    const int64_t T = 300;
    const int E = 64, K = 6, H = 1024, I = 512, G = H / 128;
    const int64_t R = T * K;
    std::printf("c-api pipeline: T=%lld E=%d K=%d H=%d I=%d (library version %d)\n", static_cast<long long>(T), E, K,
                H, I, moe_fp8_version());

    uint32_t seed = 12345u;
    std::vector<float> scores(T * E);
    for (auto& v : scores) v = uniform(seed, 0.0f, 1.0f);
    std::vector<uint16_t> x(T * H), gate_up(R * 2 * I);
    for (auto& v : x) v = to_bf16(uniform(seed, -4.0f, 4.0f));
    for (auto& v : gate_up) v = to_bf16(uniform(seed, -3.0f, 3.0f));

    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    float* d_scores = upload(scores);
    uint16_t* d_x = upload(x);
    uint16_t* d_gu = upload(gate_up);
    int64_t* d_idx = alloc<int64_t>(T * K);
    float* d_w = alloc<float>(T * K);
    int32_t* d_counts = alloc<int32_t>(E);
    int32_t* d_offsets = alloc<int32_t>(E + 1);
    int32_t* d_pos = alloc<int32_t>(T * K);
    int32_t* d_rt = alloc<int32_t>(R);
    const size_t ws_bytes = moe_token_map_workspace_bytes(T, K, E);
    uint8_t* d_ws = alloc<uint8_t>(ws_bytes > 256 ? ws_bytes : 256);
    uint8_t* d_q = alloc<uint8_t>(R * H);
    float* d_sf = alloc<float>(R * G);
    float* d_ow = alloc<float>(R);
    uint8_t* d_sq = alloc<uint8_t>(R * I);
    float* d_ssf = alloc<float>(R * (I / 128));

    MOE_OK_(moe_topk_gate(d_scores, T, E, K, 1, d_idx, d_w, st));
    MOE_OK_(moe_token_map(d_idx, T, K, E, d_counts, d_offsets, d_pos, d_rt, d_ws, ws_bytes > 256 ? ws_bytes : 256,
                          st));
    MOE_OK_(moe_expand_cast_fp8(d_x, T, H, K, d_pos, d_w, R, 128, d_q, d_sf, d_ow, st));
    MOE_OK_(swiglu_cast_fp8(d_gu, R, I, d_ow, 0.0f, 128, d_sq, d_ssf, st));
    HIP_OK(hipStreamSynchronize(st));

    const auto idx = download(d_idx, T * K);
    const auto w = download(d_w, T * K);
    const auto counts = download(d_counts, E);
    const auto offsets = download(d_offsets, E + 1);
    const auto pos = download(d_pos, T * K);
    const auto rt = download(d_rt, R);
    const auto q = download(d_q, R * H);
    const auto sf = download(d_sf, R * G);
    const auto ow = download(d_ow, R);
    const auto ssf = download(d_ssf, R * (I / 128));

    // top-k
    for (int64_t t = 0; t < T; ++t) {
        float sum = 0.0f;
        for (int k = 0; k < K; ++k) sum = sum + scores[t * E + idx[t * K + k]];
        for (int k = 0; k < K; ++k) {
            const int64_t e = idx[t * K + k];
            check(e >= 0 && e < E, "top-k id in range");
            for (int j = 0; j < k; ++j) check(idx[t * K + j] != e, "top-k ids distinct");
            if (k > 0) check(scores[t * E + idx[t * K + k - 1]] >= scores[t * E + e], "top-k scores non-increasing");
            check(bits(w[t * K + k]) == bits(scores[t * E + e] / sum), "renormalised weight");
        }
    }
    // map
    std::vector<int32_t> hist(E, 0);
    for (int64_t i = 0; i < T * K; ++i) ++hist[idx[i]];
    int32_t acc = 0;
    for (int e = 0; e < E; ++e) {
        check(counts[e] == hist[e], "count");
        check(offsets[e] == acc, "offset");
        acc += hist[e];
    }
    check(offsets[E] == T * K, "offsets[E]");
    std::vector<int> seen(R, 0);
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            const int32_t p = pos[t * K + k];
            const int64_t e = idx[t * K + k];
            check(p >= offsets[e] && p < offsets[e + 1], "pos inside its expert's segment");
            if (p >= 0 && p < R) {
                ++seen[p];
                check(rt[p] == t, "row_token inverts pos");
            }
        }
    for (int64_t r = 0; r < R; ++r) check(seen[r] == 1, "pos is a permutation");
    for (int e = 0; e < E; ++e)
        for (int32_t r = offsets[e] + 1; r < offsets[e + 1]; ++r) check(rt[r - 1] <= rt[r], "stable segment order");
    // expand
    for (int64_t t = 0; t < T; ++t) {
        const int32_t p0 = pos[t * K];
        bool in_range = true;
        for (int k = 0; k < K; ++k) in_range = in_range && pos[t * K + k] >= 0 && pos[t * K + k] < R;
        if (!in_range) {
            check(false, "pos in range");
            continue;
        }
        for (int g = 0; g < G; ++g) {
            uint32_t amax = 0;
            for (int c = 0; c < 128; ++c) {
                const uint32_t a = (static_cast<uint32_t>(x[t * H + g * 128 + c]) << 16) & 0x7FFFFFFFu;
                amax = a > amax ? a : amax;
            }
            const float m = from_bits(amax);
            check(bits(sf[p0 * G + g]) == bits((m > 1e-4f ? m : 1e-4f) / 448.0f), "group scale");
        }
        for (int k = 0; k < K; ++k) {
            const int32_t p = pos[t * K + k];
            check(std::memcmp(&q[p * H], &q[p0 * H], H) == 0, "copies identical (codes)");
            check(std::memcmp(&sf[p * G], &sf[p0 * G], G * 4) == 0, "copies identical (scales)");
            check(bits(ow[p]) == bits(w[t * K + k]), "weight carried");
        }
    }
    // SwiGLU
    for (float s : ssf) check(std::isfinite(s) && s > 0.0f, "SwiGLU scale positive and finite");
    // moe_route's fused form (top-k with the counting, then the slots): the same outputs bit for bit, three calls
    // on one workspace zeroed once (the form alternates its tables from call to call)
    {
        const size_t rws = moe_route_workspace_bytes(T, K, E);
        uint8_t* d_rws = alloc<uint8_t>(rws);
        HIP_OK(hipMemset(d_rws, 0, rws));
        int64_t* f_idx = alloc<int64_t>(T * K);
        float* f_w = alloc<float>(T * K);
        int32_t* f_counts = alloc<int32_t>(E);
        int32_t* f_offsets = alloc<int32_t>(E + 1);
        int32_t* f_pos = alloc<int32_t>(T * K);
        int32_t* f_rt = alloc<int32_t>(R);
        for (int call = 0; call < 3; ++call) {
            MOE_OK_(moe_route(d_scores, T, E, K, 1, f_idx, f_w, f_counts, f_offsets, f_pos, f_rt, d_rws, rws,
                              MOE_ROUTE_FUSED, st));
            HIP_OK(hipStreamSynchronize(st));
            check(download(f_idx, T * K) == idx, "fused routing: ids");
            const auto fw = download(f_w, T * K);
            check(std::memcmp(fw.data(), w.data(), w.size() * 4) == 0, "fused routing: weights");
            check(download(f_counts, E) == counts, "fused routing: counts");
            check(download(f_offsets, E + 1) == offsets, "fused routing: offsets");
            check(download(f_pos, T * K) == pos, "fused routing: pos");
            check(download(f_rt, R) == rt, "fused routing: row_token");
        }
        for (void* p : {static_cast<void*>(d_rws), static_cast<void*>(f_idx), static_cast<void*>(f_w),
                        static_cast<void*>(f_counts), static_cast<void*>(f_offsets), static_cast<void*>(f_pos),
                        static_cast<void*>(f_rt)})
            HIP_OK(hipFree(p));
    }
    // moe_dispatch in every form (one workspace, zeroed once): the composed calls' outputs bit for bit; at this
    // batch AUTO runs moe_route and the expand, SINGLE_LAUNCH the grid-barrier form (more than 32 tokens)
    {
        const size_t dws = moe_dispatch_workspace_bytes(T, K, E);
        uint8_t* d_dws = alloc<uint8_t>(dws);
        HIP_OK(hipMemset(d_dws, 0, dws));
        int64_t* g_idx = alloc<int64_t>(T * K);
        float* g_w = alloc<float>(T * K);
        int32_t* g_counts = alloc<int32_t>(E);
        int32_t* g_offsets = alloc<int32_t>(E + 1);
        int32_t* g_pos = alloc<int32_t>(T * K);
        int32_t* g_rt = alloc<int32_t>(R);
        uint8_t* g_q = alloc<uint8_t>(R * H);
        float* g_sf = alloc<float>(R * G);
        float* g_ow = alloc<float>(R);
        const auto ow = download(d_ow, R);
        const int modes[] = {MOE_DISPATCH_AUTO, MOE_DISPATCH_SINGLE_LAUNCH, MOE_DISPATCH_SPLIT,
                             MOE_DISPATCH_ROUTE_FUSED, MOE_DISPATCH_TOPK_THEN_COPY};
        for (int mode : modes) {
            HIP_OK(hipMemset(g_q, 0xA5, R * H));  // garbage: every row must be written
            MOE_OK_(moe_dispatch(d_scores, d_x, T, E, K, H, 1, 128, g_idx, g_w, g_counts, g_offsets, g_pos, g_rt,
                                 g_q, g_sf, g_ow, d_dws, dws, mode, st));
            HIP_OK(hipStreamSynchronize(st));
            check(download(g_idx, T * K) == idx, "dispatch: ids");
            const auto gw = download(g_w, T * K);
            check(std::memcmp(gw.data(), w.data(), w.size() * 4) == 0, "dispatch: weights");
            check(download(g_counts, E) == counts && download(g_offsets, E + 1) == offsets, "dispatch: counts");
            check(download(g_pos, T * K) == pos && download(g_rt, R) == rt, "dispatch: map");
            check(download(g_q, R * H) == q, "dispatch: e4m3 rows");
            const auto gsf = download(g_sf, R * G);
            check(std::memcmp(gsf.data(), sf.data(), sf.size() * 4) == 0, "dispatch: scales");
            const auto gow = download(g_ow, R);
            check(std::memcmp(gow.data(), ow.data(), ow.size() * 4) == 0, "dispatch: row weights");
        }
        const auto hdr = download(reinterpret_cast<uint32_t*>(d_dws), 512);
        check(hdr[2] == 0, "dispatch: no barrier wait timed out");
        for (void* p : {static_cast<void*>(d_dws), static_cast<void*>(g_idx), static_cast<void*>(g_w),
                        static_cast<void*>(g_counts), static_cast<void*>(g_offsets), static_cast<void*>(g_pos),
                        static_cast<void*>(g_rt), static_cast<void*>(g_q), static_cast<void*>(g_sf),
                        static_cast<void*>(g_ow)})
            HIP_OK(hipFree(p));
    }
    // moe_route's local form on the first 16 tokens (one launch; no workspace use) against the composed calls on
    // those tokens
    {
        const int64_t Ts = 16, Rs = Ts * K;
        const size_t mws = moe_token_map_workspace_bytes(Ts, K, E);
        uint8_t* d_mws = alloc<uint8_t>(mws > 256 ? mws : 256);
        int64_t* s_idx = alloc<int64_t>(Rs);
        float* s_w = alloc<float>(Rs);
        int32_t *s_counts = alloc<int32_t>(E), *s_offsets = alloc<int32_t>(E + 1), *s_pos = alloc<int32_t>(Rs),
                *s_rt = alloc<int32_t>(Rs);
        MOE_OK_(moe_topk_gate(d_scores, Ts, E, K, 1, s_idx, s_w, st));
        MOE_OK_(moe_token_map(s_idx, Ts, K, E, s_counts, s_offsets, s_pos, s_rt, d_mws, mws > 256 ? mws : 256, st));
        HIP_OK(hipStreamSynchronize(st));
        const auto e_idx = download(s_idx, Rs);
        const auto e_w = download(s_w, Rs);
        const auto e_counts = download(s_counts, E);
        const auto e_offsets = download(s_offsets, E + 1);
        const auto e_pos = download(s_pos, Rs);
        const auto e_rt = download(s_rt, Rs);
        const size_t rws16 = moe_route_workspace_bytes(Ts, K, E), rws33 = moe_route_workspace_bytes(33, K, E);
        const size_t rws = rws16 > rws33 ? rws16 : rws33;  // large enough for the refused 33-token call too
        uint8_t* d_rws = alloc<uint8_t>(rws);
        HIP_OK(hipMemset(d_rws, 0, rws));
        MOE_OK_(moe_route(d_scores, Ts, E, K, 1, s_idx, s_w, s_counts, s_offsets, s_pos, s_rt, d_rws, rws,
                          MOE_ROUTE_LOCAL, st));
        HIP_OK(hipStreamSynchronize(st));
        check(download(s_idx, Rs) == e_idx, "local routing: ids");
        const auto lw = download(s_w, Rs);
        check(std::memcmp(lw.data(), e_w.data(), e_w.size() * 4) == 0, "local routing: weights");
        check(download(s_counts, E) == e_counts && download(s_offsets, E + 1) == e_offsets, "local routing: counts");
        check(download(s_pos, Rs) == e_pos && download(s_rt, Rs) == e_rt, "local routing: map");
        check(moe_route(d_scores, 33, E, K, 1, s_idx, s_w, s_counts, s_offsets, s_pos, s_rt, d_rws, rws,
                        MOE_ROUTE_LOCAL, st) == MOE_ERR_UNSUPPORTED, "local routing: at most 32 tokens");
        for (void* p : {static_cast<void*>(d_mws), static_cast<void*>(s_idx), static_cast<void*>(s_w),
                        static_cast<void*>(s_counts), static_cast<void*>(s_offsets), static_cast<void*>(s_pos),
                        static_cast<void*>(s_rt), static_cast<void*>(d_rws)})
            HIP_OK(hipFree(p));
    }
    // an error path: K = 0 is rejected before any launch
    check(moe_topk_gate(d_scores, T, E, 0, 0, d_idx, nullptr, st) == MOE_ERR_INVALID_ARGUMENT, "invalid K rejected");

    for (void* p : {static_cast<void*>(d_scores), static_cast<void*>(d_x), static_cast<void*>(d_gu),
                    static_cast<void*>(d_idx), static_cast<void*>(d_w), static_cast<void*>(d_counts),
                    static_cast<void*>(d_offsets), static_cast<void*>(d_pos), static_cast<void*>(d_rt),
                    static_cast<void*>(d_ws), static_cast<void*>(d_q), static_cast<void*>(d_sf),
                    static_cast<void*>(d_ow), static_cast<void*>(d_sq), static_cast<void*>(d_ssf)})
        HIP_OK(hipFree(p));
    HIP_OK(hipStreamDestroy(st));
    if (failures) {
        std::printf("c-api pipeline: %d checks failed\n", failures);
        return 1;
    }
    std::printf("c-api pipeline ok\n");
    return 0;
}
