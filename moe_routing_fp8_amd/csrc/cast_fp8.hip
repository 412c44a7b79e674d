// Fused expand + per-token e4m3 cast, and SwiGLU + e4m3 cast, on gfx950.
//
// Operations ("DeepSeek open-sources TileKernels"):
//   section 3.2 per-token cast: per 128-channel group, amax -> scale factor
//     -> codes = e4m3(x * (1 / sf)), all in registers;
//   section 3.1: the e4m3 clamp_min_value 1e-4 bounds the amax;
//   section 2.2 fused expand: the token's codes and scale row are written to
//     every expert slot pos[t, k] >= 0 (one launch instead of cast + copy);
//   section 3.3: SwiGLU l / (1 + exp(-l)) * u (* routing weight) fused with
//     the same group cast (one launch instead of three).
//
// MI355X mapping (both kernels are HBM-bound streams):
//   * a lane owns 8 consecutive channels: one 16-byte bf16 load, one 8-byte
//     store of e4m3 codes per destination row, so a wave moves 1 KiB in and
//     512 B out per instruction, fully coalesced;
//   * a 128-channel group is exactly one 16-lane DPP row, so the group amax
//     is four DPP max steps with no LDS and no barrier;
//   * each lane keeps VPT vectors in flight: all loads are issued before any
//     arithmetic, then every code is stored K times (the expand writes
//     K x more than it reads).  One token (or row) per workgroup.
#include "device_utils.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <int NT, int VPT>
__global__ __launch_bounds__(NT) void expand_cast_kernel(const uint16_t* __restrict__ x,
                                                         int hidden, int num_topk,
                                                         const int32_t* __restrict__ pos,
                                                         const float* __restrict__ topk_weights,
                                                         int64_t num_rows,
                                                         uint8_t* __restrict__ out,
                                                         float* __restrict__ out_sf,
                                                         float* __restrict__ out_weights) {
    const int64_t t = blockIdx.x;
    const int V = hidden >> 3;  // 8-channel vectors per row
    const int G = hidden >> 7;  // 128-channel groups per row
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * hidden);

    for (int c0 = 0; c0 < V; c0 += NT * VPT) {
        uint4 raw[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = c0 + j * NT + static_cast<int>(threadIdx.x);
            if (v < V) raw[j] = xr[v];
        }
        uint2 q[VPT];
        float sf[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = c0 + j * NT + static_cast<int>(threadIdx.x);
            if (v < V) {  // uniform over each 16-lane group (V % 16 == 0)
                float f[8];
                unpack8_bf16(raw[j], f);
                const uint32_t amax = row16_max_u32(absmax8(f));
                float inv;
                e4m3_group_scale(amax, sf[j], inv);
                q[j] = quant8_e4m3(f, inv);
            }
        }
        for (int k = 0; k < num_topk; ++k) {
            const int64_t r = pos ? static_cast<int64_t>(pos[t * num_topk + k]) : t;
            if (r < 0 || r >= num_rows) continue;
            uint8_t* orow = out + r * hidden;
            float* srow = out_sf + r * G;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int v = c0 + j * NT + static_cast<int>(threadIdx.x);
                if (v < V) {
                    *reinterpret_cast<uint2*>(orow + static_cast<int64_t>(v) * 8) = q[j];
                    if ((v & 15) == 0) srow[v >> 4] = sf[j];
                }
            }
        }
    }
    if (out_weights != nullptr && static_cast<int>(threadIdx.x) < num_topk) {
        const int k = threadIdx.x;
        const int64_t r = pos ? static_cast<int64_t>(pos[t * num_topk + k]) : t;
        if (r >= 0 && r < num_rows) out_weights[r] = topk_weights[t * num_topk + k];
    }
}

// silu(l) = l / (1 + exp(-l)) with hardware exp2 and reciprocal.  The
// exponent -l*log2(e) is carried as head + tail (two FMAs), so exp(-l) =
// exp2(head) * (1 + tail*ln2) is accurate to about an ulp.  l >= 17 gives
// 1 + exp(-l) == 1 (silu(l) == l exactly); l <= -89 overflows exp2 to +inf
// (the correction factor is positive, so it stays +inf) and gives -0, like
// the IEEE expression.
__device__ __forceinline__ float silu_f32(float l) {
    constexpr float kNegLog2eHi = -1.44269502162933349609375f;      // fp32(-log2 e)
    constexpr float kNegLog2eLo = -1.9259629889e-8f;                 // -log2 e - hi
    constexpr float kLn2 = 0.693147180559945309417232f;
    const float p = l * kNegLog2eHi;
    float e = __builtin_fmaf(l, kNegLog2eHi, -p);
    e = __builtin_fmaf(l, kNegLog2eLo, e);
    const float ex = __builtin_amdgcn_exp2f(p) * __builtin_fmaf(e, kLn2, 1.0f);
    return l * __builtin_amdgcn_rcpf(1.0f + ex);
}

template <int NT, int VPT>
__global__ __launch_bounds__(NT) void swiglu_cast_kernel(const uint16_t* __restrict__ gate_up,
                                                         int inter,
                                                         const float* __restrict__ row_weights,
                                                         float clamp_value,
                                                         uint8_t* __restrict__ out,
                                                         float* __restrict__ out_sf) {
    const int64_t r = blockIdx.x;
    const int V = inter >> 3;
    const int G = inter >> 7;
    const uint4* gate = reinterpret_cast<const uint4*>(gate_up + r * 2 * inter);
    const uint4* up = reinterpret_cast<const uint4*>(gate_up + r * 2 * inter + inter);
    // x * 1.0f == x exactly, so a missing weight is a multiply by one.
    const float wr = row_weights ? row_weights[r] : 1.0f;
    const bool clamp = clamp_value > 0.0f;
    uint8_t* orow = out + r * inter;
    float* srow = out_sf + r * G;

    for (int c0 = 0; c0 < V; c0 += NT * VPT) {
        uint4 rg[VPT], ru[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = c0 + j * NT + static_cast<int>(threadIdx.x);
            if (v < V) {
                rg[j] = gate[v];
                ru[j] = up[v];
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = c0 + j * NT + static_cast<int>(threadIdx.x);
            if (v < V) {
                float l[8], u[8], val[8];
                unpack8_bf16(rg[j], l);
                unpack8_bf16(ru[j], u);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float li = l[i], ui = u[i];
                    if (clamp) {
                        li = fminf(li, clamp_value);
                        ui = fmaxf(fminf(ui, clamp_value), -clamp_value);
                    }
                    val[i] = (silu_f32(li) * ui) * wr;
                }
                const uint32_t amax = row16_max_u32(absmax8(val));
                float sf, inv;
                e4m3_group_scale(amax, sf, inv);
                *reinterpret_cast<uint2*>(orow + static_cast<int64_t>(v) * 8) = quant8_e4m3(val, inv);
                if ((v & 15) == 0) srow[v >> 4] = sf;
            }
        }
    }
}

template <int VPT>
hipError_t launch_expand_vpt(const uint16_t* x, int64_t T, int H, int K, const int32_t* pos,
                             const float* w, int64_t R, uint8_t* out, float* out_sf, float* out_w,
                             hipStream_t stream) {
    hipLaunchKernelGGL((expand_cast_kernel<256, VPT>), dim3(static_cast<unsigned>(T)), dim3(256), 0,
                       stream, x, H, K, pos, w, R, out, out_sf, out_w);
    return hipGetLastError();
}

template <int VPT>
hipError_t launch_swiglu_vpt(const uint16_t* gu, int64_t R, int I, const float* w, float c,
                             uint8_t* out, float* out_sf, hipStream_t stream) {
    hipLaunchKernelGGL((swiglu_cast_kernel<256, VPT>), dim3(static_cast<unsigned>(R)), dim3(256), 0,
                       stream, gu, I, w, c, out, out_sf);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand_cast_fp8(const uint16_t* x, int64_t T, int H, int K, const int32_t* pos,
                                  const float* w, int64_t R, uint8_t* out, float* out_sf,
                                  float* out_w, hipStream_t stream) {
    const int V = H / 8;
    const int per_thread = (V + 255) / 256;
    if (per_thread <= 1) return launch_expand_vpt<1>(x, T, H, K, pos, w, R, out, out_sf, out_w, stream);
    if (per_thread <= 2) return launch_expand_vpt<2>(x, T, H, K, pos, w, R, out, out_sf, out_w, stream);
    if (per_thread <= 4) return launch_expand_vpt<4>(x, T, H, K, pos, w, R, out, out_sf, out_w, stream);
    return launch_expand_vpt<8>(x, T, H, K, pos, w, R, out, out_sf, out_w, stream);
}

hipError_t launch_swiglu_cast_fp8(const uint16_t* gu, int64_t R, int I, const float* w, float c,
                                  uint8_t* out, float* out_sf, hipStream_t stream) {
    const int V = I / 8;
    const int per_thread = (V + 255) / 256;
    if (per_thread <= 1) return launch_swiglu_vpt<1>(gu, R, I, w, c, out, out_sf, stream);
    if (per_thread <= 2) return launch_swiglu_vpt<2>(gu, R, I, w, c, out, out_sf, stream);
    if (per_thread <= 4) return launch_swiglu_vpt<4>(gu, R, I, w, c, out, out_sf, stream);
    return launch_swiglu_vpt<8>(gu, R, I, w, c, out, out_sf, stream);
}

}  // namespace moe
