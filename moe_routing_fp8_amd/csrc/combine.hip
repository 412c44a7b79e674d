// Combine on gfx950: the weighted reduce of expert outputs back to token
// order ("CuTeDSL at Perplexity", MoE dispatch and combine: the combine
// accumulates each token's expert outputs in registers, using the positions
// the dispatch computed, and writes the final token; "DeepSeek open-sources
// TileKernels", section 2, the Fused Expand/Reduce step of the routing chain).
//
//   out[t, :] = bf16( sum over k in k order of w[t,k] * y_rows[pos[t,k], :] )
//
// fp32 products and sums, one rounding each (built without contraction), in
// k order; rows with pos outside [0, num_rows) are skipped; bf16 output is
// rounded to nearest even by gfx950's v_cvt_pk_bf16_f32.
//
// MI355X mapping: a flat grid with one 8-channel vector per thread, K
// 16-byte row loads (K compile time for the usual top-k sizes), then one
// 16-byte store.  HBM-bound: K * 16 bytes read per 16 bytes written.  When
// a row holds a whole number of waves (hidden % 512 == 0) a wave lies in
// one token: its positions and weights are then uniform and come in through
// scalar loads, which leaves the vector memory pipe to the rows (7% faster
// on the large batch than one vector load per position and weight).
#include "device_utils.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ void accumulate8(float acc[8], const uint4& raw, float w) {
    float y[8];
    unpack8_bf16(raw, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + w * y[i];
}

// KT > 0: K == KT, unrolled.  KT == 0: any K, one row at a time.  UNIFORM:
// hidden / 8 is a multiple of 64, so every wave lies in one token.
template <int KT, bool UNIFORM>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_rows,
                                                      int64_t num_rows, int hidden,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ weights,
                                                      int64_t num_tokens, int num_topk,
                                                      uint16_t* __restrict__ out) {
    const int V = hidden >> 3;  // 8-channel vectors per row
    int64_t t;
    int v;
    if constexpr (UNIFORM) {
        // flat index of the wave's lane 0 (a multiple of 64, as is V): the
        // token index is wave-uniform and v stays below V
        const uint32_t w0 = blockIdx.x * 256u +  // the grid has fewer than 2^32 threads
                            64u * static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
        t = w0 / static_cast<uint32_t>(V);
        v = static_cast<int>(w0 - static_cast<uint32_t>(t) * static_cast<uint32_t>(V)) + (threadIdx.x & 63);
    } else {
        const uint32_t i0 = blockIdx.x * 256u;  // the grid has fewer than 2^32 threads
        t = i0 / static_cast<uint32_t>(V);
        int64_t off = static_cast<int64_t>(i0) - t * V + threadIdx.x;
        while (off >= V) {
            off -= V;
            ++t;
        }
        v = static_cast<int>(off);
    }
    if (t >= num_tokens) return;
    const int K = KT > 0 ? KT : num_topk;
    const int32_t* prow = pos + t * K;
    const float* wrow = weights ? weights + t * K : nullptr;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if constexpr (KT > 0) {
        // All positions and weights first.  The row loads then need no branch
        // on their position: an out-of-range one reads row 0 (which exists --
        // the launcher sends an empty row set to the generic kernel) and only
        // the add is skipped.  Loading the position before each row's load
        // instead made every row load wait for the previous one.
        int32_t rr[KT];
        float ww[KT];
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            rr[k] = prow[k];
            ww[k] = wrow ? wrow[k] : 1.0f;
        }
        uint4 raw[KT];
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int64_t r = rr[k] >= 0 && rr[k] < num_rows ? rr[k] : 0;
            raw[k] = load_stream16(reinterpret_cast<const uint4*>(y_rows + r * hidden) + v);
        }
#pragma unroll
        for (int k = 0; k < KT; ++k)
            if (rr[k] >= 0 && rr[k] < num_rows) accumulate8(acc, raw[k], ww[k]);
    } else {
        for (int k = 0; k < K; ++k) {
            const int64_t r = prow[k];
            if (r < 0 || r >= num_rows) continue;
            accumulate8(acc, load_stream16(reinterpret_cast<const uint4*>(y_rows + r * hidden) + v),
                        wrow ? wrow[k] : 1.0f);
        }
    }
    uint4 o;
    o.x = pack2_bf16(acc[0], acc[1]);
    o.y = pack2_bf16(acc[2], acc[3]);
    o.z = pack2_bf16(acc[4], acc[5]);
    o.w = pack2_bf16(acc[6], acc[7]);
    store_stream16(reinterpret_cast<uint4*>(out + t * hidden) + v, o);
}

template <int KT>
hipError_t launch_k(const uint16_t* y, int64_t R, int H, const int32_t* pos, const float* w, int64_t T,
                    int K, uint16_t* out, hipStream_t stream) {
    const int64_t threads = T * (H / 8);
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if ((H / 8) % kWave == 0)
        hipLaunchKernelGGL((combine_kernel<KT, true>), grid, dim3(256), 0, stream, y, R, H, pos, w, T, K, out);
    else
        hipLaunchKernelGGL((combine_kernel<KT, false>), grid, dim3(256), 0, stream, y, R, H, pos, w, T, K, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* y_rows, int64_t num_rows, int hidden, const int32_t* pos,
                          const float* weights, int64_t num_tokens, int num_topk, uint16_t* out,
                          hipStream_t stream) {
    if (num_rows == 0)  // no row to read: every position is skipped
        return launch_k<0>(y_rows, num_rows, hidden, pos, weights, num_tokens, num_topk, out, stream);
    switch (num_topk) {
        case 1: return launch_k<1>(y_rows, num_rows, hidden, pos, weights, num_tokens, 1, out, stream);
        case 2: return launch_k<2>(y_rows, num_rows, hidden, pos, weights, num_tokens, 2, out, stream);
        case 4: return launch_k<4>(y_rows, num_rows, hidden, pos, weights, num_tokens, 4, out, stream);
        case 6: return launch_k<6>(y_rows, num_rows, hidden, pos, weights, num_tokens, 6, out, stream);
        case 8: return launch_k<8>(y_rows, num_rows, hidden, pos, weights, num_tokens, 8, out, stream);
        default:
            return launch_k<0>(y_rows, num_rows, hidden, pos, weights, num_tokens, num_topk, out, stream);
    }
}

}  // namespace moe
