// Fused expand + per-token e4m3 cast on gfx950 (the SwiGLU + e4m3 cast runs
// on the block-scaled SwiGLU kernel of cast_mx.hip in its e4m3 / 128 / fp32
// format).
//
// Operations ("DeepSeek open-sources TileKernels"):
//   section 3.2 per-token cast: per 128-channel group, amax -> scale factor
//     -> codes = e4m3(x * (1 / sf)), all in registers;
//   section 3.1: the e4m3 clamp_min_value 1e-4 bounds the amax;
//   section 2.2 fused expand: the token's codes and scale row are written to
//     every expert slot pos[t, k] >= 0 (one launch instead of cast + copy).
//
// MI355X mapping (HBM-bound streams):
//   * expand: a flat grid over (token, 16-channel vector); a thread does two
//     16-byte bf16 loads and one 16-byte e4m3 store per destination row, so a
//     128-channel group is an 8-lane half row and its amax is three DPP max
//     steps -- no LDS, no barrier.  Stores are streaming (non-temporal):
//     every byte is written once, K x more than is read.  The bf16 loads
//     are ordinary for inputs up to half the 256 MB Infinity Cache and
//     streaming above: cold, ordinary loads measured faster (4096 tokens,
//     hidden 7168: 2-3%), but an input larger than the cache read that way
//     evicts everything else in it (on 32768 tokens the next top-k, whose
//     scores had stayed cached, lost 1 us).
#include "device_utils.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Zero-fill part of a padded expand ("DeepSeek open-sources TileKernels",
// section 2.2: one grid both copies the routed rows and zero-fills the
// invalid ones).  The first kFillRows-row blocks of the grid are the fill
// part: each wave checks 64 rows with one row_token load per lane and a
// ballot, then writes every row it found with row_token < 0 whole (zero
// codes, zero scales, zero weight).  Padding rows sit in runs at the ends of
// the segments, so most waves find none; the fill workgroups come first in
// the grid, so their writes overlap the copies.  (One wave per 1024-channel
// chunk of every row, as before, launched ~2 million mostly idle waves on
// 32768 tokens and took the padded expand from ~440 to 536 us.)
constexpr int kFillRows = 256;  // rows per fill workgroup: 4 waves x 64
__device__ __forceinline__ void zero_fill_rows(int64_t fill_block, int hidden, int64_t num_rows,
                                               const int32_t* __restrict__ row_token,
                                               uint8_t* __restrict__ out, float* __restrict__ out_sf,
                                               float* __restrict__ out_weights) {
    const int V = hidden >> 4;
    const int G = hidden >> 7;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row0 = fill_block * kFillRows + (threadIdx.x >> 6) * kWave;
    const int64_t rl = row0 + lane;
    const bool pad = rl < num_rows && row_token[rl] < 0;
    if (pad && out_weights != nullptr) out_weights[rl] = 0.0f;
    uint64_t m = __ballot(pad);
    while (m != 0ull) {  // wave-uniform
        const int64_t r = row0 + __builtin_ctzll(m);
        m &= m - 1ull;
        for (int v = lane; v < V; v += kWave)
            store_stream16(reinterpret_cast<uint4*>(out + r * hidden + static_cast<int64_t>(v) * 16),
                           make_uint4(0u, 0u, 0u, 0u));
        for (int g = lane; g < G; g += kWave) out_sf[r * G + g] = 0.0f;
    }
}

// Flat layout: thread i of the grid owns the 16 channels [16v, 16v + 16) of
// token t, where i = t * V + v and V = hidden / 16.  It issues two 16-byte
// bf16 loads and, per destination row, one streaming 16-byte e4m3 store;
// the 8 lanes of a 128-channel group sit in one DPP half row (three max
// steps for the amax).  One vector per thread keeps register use small,
// so many waves stay resident and the memory pipes full.
template <bool STREAM_LOADS>
__global__ __launch_bounds__(256) void expand_cast_kernel(const uint16_t* __restrict__ x,
                                                          int64_t num_tokens, int hidden,
                                                          int num_topk,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ topk_weights,
                                                          int64_t num_rows,
                                                          uint8_t* __restrict__ out,
                                                          float* __restrict__ out_sf,
                                                          float* __restrict__ out_weights,
                                                          const int32_t* __restrict__ row_token,
                                                          uint32_t fill_blocks) {
    if (blockIdx.x < fill_blocks) {
        zero_fill_rows(blockIdx.x, hidden, num_rows, row_token, out, out_sf, out_weights);
        return;
    }
    const uint32_t bid = blockIdx.x - fill_blocks;  // this workgroup in the token part
    const int V = hidden >> 4;  // 16-channel vectors per row
    const int G = hidden >> 7;  // 128-channel groups per row
    // token of this thread: one division per workgroup, then at most
    // 256 / V + 1 steps (a workgroup spans few tokens)
    const uint32_t i0 = bid * 256u;  // the token part has fewer than 2^32 threads
    int64_t t = i0 / static_cast<uint32_t>(V);
    int64_t off = static_cast<int64_t>(i0) - t * V + threadIdx.x;
    while (off >= V) {
        off -= V;
        ++t;
    }
    if (t >= num_tokens) return;  // whole 8-lane groups leave together (V % 8 == 0)
    const int v = static_cast<int>(off);

    uint4 q;
    float sf;
    cast16_e4m3<STREAM_LOADS>(reinterpret_cast<const uint4*>(x + t * hidden), v, q, sf);

    for (int k = 0; k < num_topk; ++k) {
        const int64_t r = pos ? static_cast<int64_t>(pos[t * num_topk + k]) : t;
        if (r < 0 || r >= num_rows) continue;
        store_stream16(reinterpret_cast<uint4*>(out + r * hidden + static_cast<int64_t>(v) * 16), q);
        if ((v & 7) == 0) out_sf[r * G + (v >> 3)] = sf;
        if (out_weights != nullptr && v == 0) out_weights[r] = topk_weights[t * num_topk + k];
    }
}

// Split-copy layout, for K >= 4.  HBM write throughput drops when each
// thread drives many write streams (one per destination row): a plain fill
// reaches ~6.4 TB/s with 1-2 stores per thread but ~5.8 TB/s with 4-8.  So a
// workgroup of 4 waves first casts two 64-vector chunks (2 x 1024 channels)
// of token rows into LDS -- waves 0 and 1, one chunk each, same lane layout as
// the flat kernel -- and then every wave writes the copies k = wave,
// wave + 4, ... of both chunks: 2 destination rows per thread at K = 8.
constexpr int kSplitWaves = 4;
constexpr int kSplitChunks = 2;
#ifndef MOE_EXPAND_SPLIT_MIN_K
#define MOE_EXPAND_SPLIT_MIN_K 4
#endif
// Smallest K that takes the split-copy kernel (fewer copies: the flat one).
constexpr int kSplitMinTopk = MOE_EXPAND_SPLIT_MIN_K;

template <bool STREAM_LOADS>
__global__ __launch_bounds__(kSplitWaves * kWave) void expand_cast_split_kernel(
    const uint16_t* __restrict__ x, int64_t num_tokens, int hidden, int num_topk,
    const int32_t* __restrict__ pos, const float* __restrict__ topk_weights, int64_t num_rows,
    uint8_t* __restrict__ out, float* __restrict__ out_sf, float* __restrict__ out_weights,
    const int32_t* __restrict__ row_token, uint32_t fill_blocks) {
    if (blockIdx.x < fill_blocks) {  // whole workgroup: no barrier is skipped by part of it
        zero_fill_rows(blockIdx.x, hidden, num_rows, row_token, out, out_sf, out_weights);
        return;
    }
    __shared__ uint4 codes[kSplitChunks][kWave];
    __shared__ float scales[kSplitChunks][kWave / 8];
    const int V = hidden >> 4;           // 16-channel vectors per row
    const int G = hidden >> 7;           // 128-channel groups per row
    const int CH = (V + kWave - 1) / kWave;  // 64-vector chunks per row
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk0 = static_cast<int64_t>(blockIdx.x - fill_blocks) * kSplitChunks;

    if (wave < kSplitChunks) {
        const int64_t tc = chunk0 + wave;
        const int64_t t = tc / CH;
        const int v = static_cast<int>(tc - t * CH) * kWave + lane;
        if (t < num_tokens && v < V) {  // whole 8-lane groups (V % 8 == 0)
            uint4 q;
            float sf;
            cast16_e4m3<STREAM_LOADS>(reinterpret_cast<const uint4*>(x + t * hidden), v, q, sf);
            codes[wave][lane] = q;
            if ((lane & 7) == 0) scales[wave][lane >> 3] = sf;
        }
    }
    __syncthreads();

    for (int c = 0; c < kSplitChunks; ++c) {
        const int64_t tc = chunk0 + c;
        const int64_t t = tc / CH;
        if (t >= num_tokens) break;
        const int chunk = static_cast<int>(tc - t * CH);
        const int v = chunk * kWave + lane;
        const int g0 = chunk * (kWave / 8);
        const uint4 q = codes[c][lane];
        const float sf = scales[c][lane & 7];
        for (int k = wave; k < num_topk; k += kSplitWaves) {
            const int64_t r = pos[t * num_topk + k];
            if (r < 0 || r >= num_rows) continue;
            if (v < V)
                store_stream16(reinterpret_cast<uint4*>(out + r * hidden + static_cast<int64_t>(v) * 16), q);
            if (lane < 8 && g0 + lane < G) out_sf[r * G + g0 + lane] = sf;
            if (out_weights != nullptr && chunk == 0 && lane == 0)
                out_weights[r] = topk_weights[t * num_topk + k];
        }
    }
}

// Inputs above this many bytes are read with streaming loads (see the header).
constexpr int64_t kStreamLoadBytes = int64_t{128} << 20;

template <bool STREAM_LOADS>
hipError_t launch_expand_cast_loads(const uint16_t* x, int64_t T, int H, int K, const int32_t* pos,
                                    const float* w, int64_t R, uint8_t* out, float* out_sf,
                                    float* out_w, const int32_t* row_token, hipStream_t stream) {
    // workgroups of the zero-fill part, first in the grid: kFillRows rows each
    const int64_t fill_blocks = row_token != nullptr ? (R + kFillRows - 1) / kFillRows : 0;
    if (pos != nullptr && K >= kSplitMinTopk) {
        const int64_t chunks = T * ((H / 16 + kWave - 1) / kWave);
        const int64_t token_blocks = (chunks + kSplitChunks - 1) / kSplitChunks;
        hipLaunchKernelGGL(expand_cast_split_kernel<STREAM_LOADS>,
                           dim3(static_cast<unsigned>(token_blocks + fill_blocks)), dim3(kSplitWaves * kWave), 0,
                           stream, x, T, H, K, pos, w, R, out, out_sf, out_w, row_token,
                           static_cast<uint32_t>(fill_blocks));
        return hipGetLastError();
    }
    const int64_t token_blocks = (T * (H / 16) + 255) / 256;
    hipLaunchKernelGGL(expand_cast_kernel<STREAM_LOADS>, dim3(static_cast<unsigned>(token_blocks + fill_blocks)),
                       dim3(256), 0, stream, x, T, H, K, pos, w, R, out, out_sf, out_w, row_token,
                       static_cast<uint32_t>(fill_blocks));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand_cast_fp8(const uint16_t* x, int64_t T, int H, int K, const int32_t* pos,
                                  const float* w, int64_t R, uint8_t* out, float* out_sf,
                                  float* out_w, const int32_t* row_token, hipStream_t stream) {
    if (T * H * 2 > kStreamLoadBytes)
        return launch_expand_cast_loads<true>(x, T, H, K, pos, w, R, out, out_sf, out_w, row_token, stream);
    return launch_expand_cast_loads<false>(x, T, H, K, pos, w, R, out, out_sf, out_w, row_token, stream);
}

hipError_t launch_swiglu_cast_fp8(const uint16_t* gu, int64_t R, int I, const float* w, float c,
                                  uint8_t* out, float* out_sf, hipStream_t stream) {
    // the block-scaled SwiGLU kernel in the e4m3 / 128 / fp32-scale format
    // computes the same values (same scale formula and operation order) and
    // measured faster than a dedicated kernel
    const MxFormat f{0, 128, false, false, 0.0f};
    return launch_swiglu_cast_mx(gu, R, I, w, c, f, out, out_sf, stream);
}

}  // namespace moe
