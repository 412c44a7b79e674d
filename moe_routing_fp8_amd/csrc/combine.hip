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
// MI355X mapping: a flat grid with one 8-channel vector per thread; all K
// 16-byte row loads of a thread are issued before the first add (K compile
// time for the usual top-k sizes), then one 16-byte store.  HBM-bound:
// K * 16 bytes read per 16 bytes written.
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

// KT > 0: K == KT, all row loads in flight at once.  KT == 0: any K, one row
// at a time.
template <int KT>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_rows,
                                                      int64_t num_rows, int hidden,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ weights,
                                                      int64_t num_tokens, int num_topk,
                                                      uint16_t* __restrict__ out) {
    const int V = hidden >> 3;  // 8-channel vectors per row
    const uint32_t i0 = blockIdx.x * 256u;  // the grid has fewer than 2^32 threads
    int64_t t = i0 / static_cast<uint32_t>(V);
    int64_t off = static_cast<int64_t>(i0) - t * V + threadIdx.x;
    while (off >= V) {
        off -= V;
        ++t;
    }
    if (t >= num_tokens) return;
    const int v = static_cast<int>(off);
    const int K = KT > 0 ? KT : num_topk;
    const int32_t* prow = pos + t * K;
    const float* wrow = weights ? weights + t * K : nullptr;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if constexpr (KT > 0) {
        uint4 raw[KT];
        bool ok[KT];
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int64_t r = prow[k];
            ok[k] = r >= 0 && r < num_rows;
            if (ok[k]) raw[k] = load_stream16(reinterpret_cast<const uint4*>(y_rows + r * hidden) + v);
        }
#pragma unroll
        for (int k = 0; k < KT; ++k)
            if (ok[k]) accumulate8(acc, raw[k], wrow ? wrow[k] : 1.0f);
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
    hipLaunchKernelGGL((combine_kernel<KT>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256),
                       0, stream, y, R, H, pos, w, T, K, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* y_rows, int64_t num_rows, int hidden, const int32_t* pos,
                          const float* weights, int64_t num_tokens, int num_topk, uint16_t* out,
                          hipStream_t stream) {
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
