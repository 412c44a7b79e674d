// Per-token casts in the block-scaled formats beyond e4m3 / 128 on gfx950
// ("DeepSeek open-sources TileKernels", section 3.1: the cast output
// configuration -- dtype, scaling block size, round_sf, clamp_min_value with
// max_value * 2^-126 for float4_e2m1fn, packed UE8M0 scales; section 3.2 the
// per-token cast, 3.3 the SwiGLU fusion; "CuTeDSL at Perplexity", Blackwell
// section: MXFP8 / MXFP4 take the absmax over 32 elements, NVFP4 over 16).
//
// Per group of GROUP channels (16, 32 or 128):
//   c   = max(amax, clamp)                   clamp: 1e-4 (e4m3), 6 * 2^-126 (e2m1)
//   sf  = c / max_value                      (fp32, correctly rounded)
//   round_sf: sf = the smallest power of two >= c / max_value.  The rounded
//         quotient has a zero mantissa only when the exact quotient is that
//         power of two (c has at most 24 significant bits and max_value is
//         7 * 2^6 or 3 * 2, so a quotient above a power of two exceeds it by
//         more than half an ulp), so rounding the fp32 quotient up to the
//         next power of two gives exactly that definition.
//   inv = 1 / sf;  code = format(x * inv)    e4m3 by v_cvt_pk_fp8_f32, e2m1
//         by seven threshold compares (round to nearest, ties to the even
//         code, saturating at 6)
//   scale out: fp32, or the UE8M0 byte (the biased exponent of sf).
// e2m1 rows hold H / 2 bytes: element 2i in the low nibble of byte i.
//
// MI355X mapping, as for the e4m3 / 128 kernels: a lane casts 16 channels
// (two 16-byte streaming loads); a group spans GROUP / 16 lanes, reduced by
// DPP.  Identity casts run a flat grid, one 16-channel vector per thread;
// routed expands run the split-copy shape (waves 0-1 cast a 1024-channel
// chunk each into LDS, all four waves write the copies, k = wave mod 4).
// SwiGLU: one workgroup per row, 8 channels per lane.
#include "device_utils.hpp"
#include "kernels.hpp"
#include "swiglu_math.hpp"

namespace moe {
namespace {

constexpr int kFmtE4m3 = 0;
constexpr int kFmtE2m1 = 1;

// Runtime parts of the format (uniform over the launch).
struct MxParams {
    float clamp;      // resolved clamp_min
    float max_value;  // 448 or 6
    int round_sf;     // power-of-two scales
    int sf_u8;        // UE8M0 scale bytes instead of fp32
};

// Maximum over aligned groups of LANES lanes (1, 2, 4, 8 or 16) by DPP.
template <int LANES>
__device__ __forceinline__ uint32_t lanes_max_u32(uint32_t x) {
    if constexpr (LANES >= 2) x = max(x, dpp_u32<kDppQuadXor1>(x));
    if constexpr (LANES >= 4) x = max(x, dpp_u32<kDppQuadXor2>(x));
    if constexpr (LANES >= 8) x = max(x, dpp_u32<kDppRowHalfMirror>(x));
    if constexpr (LANES >= 16) x = max(x, dpp_u32<kDppRowMirror>(x));
    return x;
}

__device__ __forceinline__ void mx_scale(uint32_t amax_bits, const MxParams& p, float& sf, float& inv) {
    const float amax = __uint_as_float(amax_bits);
    const float c = amax > p.clamp ? amax : p.clamp;
    sf = c / p.max_value;
    if (p.round_sf) {
        uint32_t b = __float_as_uint(sf);
        if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;  // up to the next power of two
        sf = __uint_as_float(b);
    }
    inv = 1.0f / sf;
}

__device__ __forceinline__ uint32_t ue8m0(float pow2) { return (__float_as_uint(pow2) >> 23) & 0xFFu; }

// OCP e2m1 code of y: round to nearest, ties to the even code, |y| > 6
// saturating to 6 (code 7); NaN -> 7 with y's sign.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const float a = fabsf(y);
    uint32_t c = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) +
                 (a >= 1.75f ? 1u : 0u) + (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) +
                 (a > 5.0f ? 1u : 0u);
    if (a != a) c = 7u;
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Eight values -> eight e2m1 codes in one dword, element i in nibble i.
__device__ __forceinline__ uint32_t quant8_e2m1(const float f[8], float inv) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code(f[i] * inv) << (4 * i);
    return w;
}

// Codes of one lane's 16 channels: e4m3 16 bytes (uint4), e2m1 8 bytes (x, y).
template <int FMT>
__device__ __forceinline__ uint4 quant16(const float f[8], const float g[8], float inv) {
    if constexpr (FMT == kFmtE4m3) {
        const uint2 lo = quant8_e4m3(f, inv);
        const uint2 hi = quant8_e4m3(g, inv);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        return make_uint4(quant8_e2m1(f, inv), quant8_e2m1(g, inv), 0u, 0u);
    }
}

// Cast of one lane's 16 channels (v-th vector of the row): codes and the
// scale of its group (all lanes of the group hold it).
template <int FMT, int GROUP>
__device__ __forceinline__ void cast16_mx(const uint4* __restrict__ row, int v, const MxParams& p,
                                          uint4& codes, float& sf) {
    const uint4 ra = load_stream16(row + 2 * v);
    const uint4 rb = load_stream16(row + 2 * v + 1);
    float f[8], g[8];
    unpack8_bf16(ra, f);
    unpack8_bf16(rb, g);
    const uint32_t amax = lanes_max_u32<GROUP / 16>(max(absmax8(f), absmax8(g)));
    float inv;
    mx_scale(amax, p, sf, inv);
    codes = quant16<FMT>(f, g, inv);
}

// Stores one lane's codes (16 channels) at vector v of row r.
template <int FMT>
__device__ __forceinline__ void store_codes16(uint8_t* __restrict__ out, int64_t r, int hidden, int v,
                                              const uint4& q) {
    if constexpr (FMT == kFmtE4m3)
        store_stream16(reinterpret_cast<uint4*>(out + r * hidden + static_cast<int64_t>(v) * 16), q);
    else
        store_stream8(reinterpret_cast<uint2*>(out + r * (hidden / 2) + static_cast<int64_t>(v) * 8),
                      make_uint2(q.x, q.y));
}

__device__ __forceinline__ void store_scale(void* __restrict__ out_sf, int64_t idx, float sf, int sf_u8) {
    if (sf_u8)
        static_cast<uint8_t*>(out_sf)[idx] = static_cast<uint8_t>(ue8m0(sf));
    else
        static_cast<float*>(out_sf)[idx] = sf;
}

// Identity cast: flat grid, thread i owns the 16 channels of vector i % V
// of token i / V.
template <int FMT, int GROUP>
__global__ __launch_bounds__(256) void cast_mx_kernel(const uint16_t* __restrict__ x, int64_t num_tokens,
                                                      int hidden, MxParams p, uint8_t* __restrict__ out,
                                                      void* __restrict__ out_sf) {
    const int V = hidden >> 4;
    const int G = hidden / GROUP;
    const uint32_t i0 = blockIdx.x * 256u;  // the grid has fewer than 2^32 threads
    int64_t t = i0 / static_cast<uint32_t>(V);
    int64_t off = static_cast<int64_t>(i0) - t * V + threadIdx.x;
    while (off >= V) {
        off -= V;
        ++t;
    }
    if (t >= num_tokens) return;  // whole groups of lanes leave together (V % (GROUP / 16) == 0)
    const int v = static_cast<int>(off);
    uint4 q;
    float sf;
    cast16_mx<FMT, GROUP>(reinterpret_cast<const uint4*>(x + t * hidden), v, p, q, sf);
    store_codes16<FMT>(out, t, hidden, v, q);
    if (v % (GROUP / 16) == 0) store_scale(out_sf, t * G + v / (GROUP / 16), sf, p.sf_u8);
}

constexpr int kMxWaves = 4;
constexpr int kMxChunks = 2;

// Routed expand: the split-copy shape of expand_cast_split_kernel.
template <int FMT, int GROUP>
__global__ __launch_bounds__(kMxWaves * kWave) void expand_mx_split_kernel(
    const uint16_t* __restrict__ x, int64_t num_tokens, int hidden, int num_topk,
    const int32_t* __restrict__ pos, const float* __restrict__ topk_weights, int64_t num_rows, MxParams p,
    uint8_t* __restrict__ out, void* __restrict__ out_sf, float* __restrict__ out_weights) {
    constexpr int kScalesPerChunk = 1024 / GROUP;  // 8, 32 or 64
    __shared__ uint4 codes[kMxChunks][kWave];
    __shared__ float scales[kMxChunks][kScalesPerChunk];
    const int V = hidden >> 4;
    const int G = hidden / GROUP;
    const int CH = (V + kWave - 1) / kWave;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk0 = static_cast<int64_t>(blockIdx.x) * kMxChunks;

    if (wave < kMxChunks) {
        const int64_t tc = chunk0 + wave;
        const int64_t t = tc / CH;
        const int v = static_cast<int>(tc - t * CH) * kWave + lane;
        if (t < num_tokens && v < V) {  // whole groups of lanes
            uint4 q;
            float sf;
            cast16_mx<FMT, GROUP>(reinterpret_cast<const uint4*>(x + t * hidden), v, p, q, sf);
            codes[wave][lane] = q;
            if (lane % (GROUP / 16) == 0) scales[wave][lane / (GROUP / 16)] = sf;
        }
    }
    __syncthreads();

    for (int c = 0; c < kMxChunks; ++c) {
        const int64_t tc = chunk0 + c;
        const int64_t t = tc / CH;
        if (t >= num_tokens) break;
        const int chunk = static_cast<int>(tc - t * CH);
        const int v = chunk * kWave + lane;
        const int g0 = chunk * kScalesPerChunk;
        const uint4 q = codes[c][lane];
        const float sf = lane < kScalesPerChunk ? scales[c][lane] : 0.0f;
        for (int k = wave; k < num_topk; k += kMxWaves) {
            const int64_t r = pos[t * num_topk + k];
            if (r < 0 || r >= num_rows) continue;
            if (v < V) store_codes16<FMT>(out, r, hidden, v, q);
            if (lane < kScalesPerChunk && g0 + lane < G) store_scale(out_sf, r * G + g0 + lane, sf, p.sf_u8);
            if (out_weights != nullptr && chunk == 0 && lane == 0) out_weights[r] = topk_weights[t * num_topk + k];
        }
    }
}

// SwiGLU + cast: one workgroup per row, a lane owns 8 channels; a group
// spans GROUP / 8 lanes.
template <int FMT, int GROUP>
__global__ __launch_bounds__(256) void swiglu_mx_kernel(const uint16_t* __restrict__ gate_up, int inter,
                                                        const float* __restrict__ row_weights,
                                                        float clamp_value, MxParams p,
                                                        uint8_t* __restrict__ out, void* __restrict__ out_sf) {
    const int64_t r = blockIdx.x;
    const int V = inter >> 3;
    const int G = inter / GROUP;
    const uint4* gate = reinterpret_cast<const uint4*>(gate_up + r * 2 * inter);
    const uint4* up = reinterpret_cast<const uint4*>(gate_up + r * 2 * inter + inter);
    const bool clamp = clamp_value > 0.0f;
    const float wr = row_weights != nullptr ? row_weights[r] : 1.0f;
    for (int v = threadIdx.x; v - static_cast<int>(threadIdx.x) < V; v += 256) {
        if (v >= V) continue;  // uniform over each group of lanes (V % (GROUP / 8) == 0)
        const uint4 rg = load_stream16(gate + v);
        const uint4 ru = load_stream16(up + v);
        float l[8], u[8], val[8];
        unpack8_bf16(rg, l);
        unpack8_bf16(ru, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float s, ui = u[i];
            if (clamp) {
                s = silu_any_arg(fminf(l[i], clamp_value));
                ui = fmaxf(fminf(ui, clamp_value), -clamp_value);
            } else {
                s = silu_bf16_arg(l[i]);
            }
            val[i] = row_weights != nullptr ? (s * ui) * wr : s * ui;
        }
        const uint32_t amax = lanes_max_u32<GROUP / 8>(absmax8_computed(val));
        float sf, inv;
        mx_scale(amax, p, sf, inv);
        if constexpr (FMT == kFmtE4m3) {
            store_stream8(reinterpret_cast<uint2*>(out + r * inter + static_cast<int64_t>(v) * 8),
                          quant8_e4m3(val, inv));
        } else {
            __builtin_nontemporal_store(quant8_e2m1(val, inv),
                                        reinterpret_cast<uint32_t*>(out + r * (inter / 2) +
                                                                    static_cast<int64_t>(v) * 4));
        }
        if (v % (GROUP / 8) == 0) store_scale(out_sf, r * G + v / (GROUP / 8), sf, p.sf_u8);
    }
}

MxParams make_params(const MxFormat& f) {
    MxParams p;
    p.max_value = f.dtype == kFmtE2m1 ? 6.0f : 448.0f;
    p.clamp = f.clamp_min > 0.0f ? f.clamp_min : (f.dtype == kFmtE2m1 ? 6.0f * 0x1p-126f : 1e-4f);
    p.round_sf = f.round_sf ? 1 : 0;
    p.sf_u8 = f.sf_ue8m0 ? 1 : 0;
    return p;
}

template <int FMT, int GROUP>
hipError_t launch_expand_mx_t(const uint16_t* x, int64_t T, int H, int K, const int32_t* pos, const float* w,
                              int64_t R, const MxParams& p, uint8_t* out, void* out_sf, float* out_w,
                              hipStream_t stream) {
    if (pos == nullptr) {
        const int64_t blocks = (T * (H / 16) + 255) / 256;
        hipLaunchKernelGGL((cast_mx_kernel<FMT, GROUP>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                           stream, x, T, H, p, out, out_sf);
    } else {
        const int64_t chunks = T * ((H / 16 + kWave - 1) / kWave);
        const int64_t blocks = (chunks + kMxChunks - 1) / kMxChunks;
        hipLaunchKernelGGL((expand_mx_split_kernel<FMT, GROUP>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kMxWaves * kWave), 0, stream, x, T, H, K, pos, w, R, p, out, out_sf, out_w);
    }
    return hipGetLastError();
}

template <int FMT, int GROUP>
hipError_t launch_swiglu_mx_t(const uint16_t* gu, int64_t R, int I, const float* w, float c, const MxParams& p,
                              uint8_t* out, void* out_sf, hipStream_t stream) {
    hipLaunchKernelGGL((swiglu_mx_kernel<FMT, GROUP>), dim3(static_cast<unsigned>(R)), dim3(256), 0, stream, gu,
                       I, w, c, p, out, out_sf);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand_cast_mx(const uint16_t* x, int64_t T, int H, int K, const int32_t* pos,
                                 const float* w, int64_t R, const MxFormat& f, uint8_t* out, void* out_sf,
                                 float* out_w, hipStream_t stream) {
    const MxParams p = make_params(f);
#define MOE_MX_EXPAND(FMT, GROUP) \
    return launch_expand_mx_t<FMT, GROUP>(x, T, H, K, pos, w, R, p, out, out_sf, out_w, stream)
    if (f.dtype == kFmtE2m1) {
        if (f.group_size == 16) MOE_MX_EXPAND(kFmtE2m1, 16);
        if (f.group_size == 32) MOE_MX_EXPAND(kFmtE2m1, 32);
        MOE_MX_EXPAND(kFmtE2m1, 128);
    }
    if (f.group_size == 16) MOE_MX_EXPAND(kFmtE4m3, 16);
    if (f.group_size == 32) MOE_MX_EXPAND(kFmtE4m3, 32);
    MOE_MX_EXPAND(kFmtE4m3, 128);
#undef MOE_MX_EXPAND
}

hipError_t launch_swiglu_cast_mx(const uint16_t* gu, int64_t R, int I, const float* w, float c,
                                 const MxFormat& f, uint8_t* out, void* out_sf, hipStream_t stream) {
    const MxParams p = make_params(f);
#define MOE_MX_SWIGLU(FMT, GROUP) return launch_swiglu_mx_t<FMT, GROUP>(gu, R, I, w, c, p, out, out_sf, stream)
    if (f.dtype == kFmtE2m1) {
        if (f.group_size == 16) MOE_MX_SWIGLU(kFmtE2m1, 16);
        if (f.group_size == 32) MOE_MX_SWIGLU(kFmtE2m1, 32);
        MOE_MX_SWIGLU(kFmtE2m1, 128);
    }
    if (f.group_size == 16) MOE_MX_SWIGLU(kFmtE4m3, 16);
    if (f.group_size == 32) MOE_MX_SWIGLU(kFmtE4m3, 32);
    MOE_MX_SWIGLU(kFmtE4m3, 128);
#undef MOE_MX_SWIGLU
}

}  // namespace moe
