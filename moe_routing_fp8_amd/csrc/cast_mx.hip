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
//         by v_cvt_scalef32_pk_fp4_f32 with scale 1 (round to nearest, ties
//         to the even code, saturating at 6)
//   scale out: fp32, or the UE8M0 byte (the biased exponent of sf).
// e2m1 rows hold H / 2 bytes: element 2i in the low nibble of byte i.
//
// MI355X mapping, as for the e4m3 / 128 kernels: every lane produces 16
// bytes of codes -- 16 channels for e4m3, 32 for e2m1 (two streaming or
// four ordinary 16-byte loads) -- so every store is a 16-byte vector store; a group
// spans GROUP / CPL lanes (reduced by DPP) or a lane holds CPL / GROUP
// groups.  Identity casts run a flat grid, one lane vector per thread;
// routed expands run the split-copy shape (waves 0-1 cast a chunk each into
// LDS, all four waves write the copies, k = wave mod 4).  SwiGLU: one
// workgroup per row, 8 channels per lane.
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

// Eight values -> eight OCP e2m1 codes in one dword, element i in nibble i:
// gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1 (round to nearest, ties to
// the even code, saturating at 6; source 0 in the low nibble of the selected
// byte).  Checked equal to the threshold definition on every bf16 value, NaN
// and infinities included, and on fp32 values around every rounding
// threshold.
__device__ __forceinline__ uint32_t quant8_e2m1(const float* f, float inv) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0] * inv, f[1] * inv, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2] * inv, f[3] * inv, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4] * inv, f[5] * inv, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6] * inv, f[7] * inv, 1.0f, 3);
    return w;
}

// Lane layout of a format: a lane casts CPL channels (16 for e4m3, 32 for
// e2m1) into 16 bytes of codes; a group covers LPG lanes, or a lane GPL groups.
template <int FMT, int GROUP>
struct Layout {
    static constexpr int CPL = FMT == kFmtE2m1 ? 32 : 16;
    static constexpr int LPG = GROUP > CPL ? GROUP / CPL : 1;
    static constexpr int GPL = CPL > GROUP ? CPL / GROUP : 1;
    static constexpr int CHUNK = kWave * CPL;  // channels of one wave's chunk
};

// Cast of one lane's CPL channels (vector v of the row): 16 bytes of codes
// and the scales of the lane's GPL groups (all lanes of a group hold it).
template <int FMT, int GROUP>
__device__ __forceinline__ void cast_lane_mx(const uint4* __restrict__ row, int v, const MxParams& p,
                                             uint4& codes, float (&sf)[Layout<FMT, GROUP>::GPL]) {
    using L = Layout<FMT, GROUP>;
    constexpr int NV = L::CPL / 8;  // 16-byte loads
    float f[L::CPL];
    uint4 raw[NV];
    // An e2m1 lane reads 64 contiguous bytes in four loads, so each load
    // instruction touches every 64-byte segment at a lane stride of 64 bytes
    // and the line is read again by the next three.  Streaming loads let L2
    // drop it in between (the expand refetched about 3% of its bytes and ran
    // 4% slower on 262144 rows, 17% on 32768 flushed); ordinary loads keep
    // it.  e4m3 lanes (two loads, 32-byte stride) measured best streaming.
#pragma unroll
    for (int i = 0; i < NV; ++i)
        raw[i] = FMT == kFmtE2m1 ? row[NV * v + i] : load_stream16(row + NV * v + i);
#pragma unroll
    for (int i = 0; i < NV; ++i) unpack8_bf16(raw[i], f + 8 * i);
    float inv[L::GPL];
#pragma unroll
    for (int g = 0; g < L::GPL; ++g) {
        constexpr int PER = L::CPL / L::GPL;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < PER; i += 8) m = max(m, absmax8(f + g * PER + i));
        mx_scale(lanes_max_u32<L::LPG>(m), p, sf[g], inv[g]);
    }
    constexpr int PER = L::CPL / L::GPL;
    if constexpr (FMT == kFmtE4m3) {
        const uint2 lo = quant8_e4m3(f, inv[0]);
        const uint2 hi = quant8_e4m3(f + 8, inv[0]);
        codes = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = quant8_e2m1(f + 8 * i, inv[(8 * i) / PER]);
        codes = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__device__ __forceinline__ void store_scale(void* __restrict__ out_sf, int64_t idx, float sf, int sf_u8) {
    if (sf_u8)
        static_cast<uint8_t*>(out_sf)[idx] = static_cast<uint8_t>(ue8m0(sf));
    else
        static_cast<float*>(out_sf)[idx] = sf;
}

// Bytes of one row of codes.
template <int FMT>
__device__ __forceinline__ int64_t code_row_bytes(int width) {
    return FMT == kFmtE2m1 ? width / 2 : width;
}

// Identity cast: flat grid, thread i owns the CPL channels of vector i % V
// of token i / V.
template <int FMT, int GROUP>
__global__ __launch_bounds__(256) void cast_mx_kernel(const uint16_t* __restrict__ x, int64_t num_tokens,
                                                      int hidden, MxParams p, uint8_t* __restrict__ out,
                                                      void* __restrict__ out_sf) {
    using L = Layout<FMT, GROUP>;
    const int V = hidden / L::CPL;
    const int G = hidden / GROUP;
    const uint32_t i0 = blockIdx.x * 256u;  // the grid has fewer than 2^32 threads
    int64_t t = i0 / static_cast<uint32_t>(V);
    int64_t off = static_cast<int64_t>(i0) - t * V + threadIdx.x;
    while (off >= V) {
        off -= V;
        ++t;
    }
    if (t >= num_tokens) return;  // whole groups of lanes leave together (V % LPG == 0)
    const int v = static_cast<int>(off);
    uint4 q;
    float sf[L::GPL];
    cast_lane_mx<FMT, GROUP>(reinterpret_cast<const uint4*>(x + t * hidden), v, p, q, sf);
    store_stream16(reinterpret_cast<uint4*>(out + t * code_row_bytes<FMT>(hidden) + static_cast<int64_t>(v) * 16), q);
    if (v % L::LPG == 0) {
#pragma unroll
        for (int g = 0; g < L::GPL; ++g) store_scale(out_sf, t * G + (v / L::LPG) * L::GPL + g, sf[g], p.sf_u8);
    }
}

constexpr int kMxWaves = 4;
// Chunks cast per workgroup (one per casting wave, waves 0 and 1).  Both
// formats measured best at two: each wave then writes 2 chunks x K/4 copies,
// and for e2m1 four chunks per workgroup (every wave casting) ran 7% slower
// on 262144 rows.
template <int FMT>
constexpr int mx_chunks() { return 2; }

// Routed expand: the split-copy shape of expand_cast_split_kernel, with
// chunks taken over the flattened (token, lane vector) space, so a wave's 64
// lanes may span two tokens and no lane idles at the end of a row (an e2m1
// row of 7168 channels is 3.5 waves).  Each lane writes the copies of its
// own token: lanes of one token stay contiguous, at most two runs per wave.
template <int FMT, int GROUP>
__global__ __launch_bounds__(kMxWaves * kWave) void expand_mx_split_kernel(
    const uint16_t* __restrict__ x, int64_t num_tokens, int hidden, int num_topk,
    const int32_t* __restrict__ pos, const float* __restrict__ topk_weights, int64_t num_rows, MxParams p,
    uint8_t* __restrict__ out, void* __restrict__ out_sf, float* __restrict__ out_weights) {
    using L = Layout<FMT, GROUP>;
    constexpr int kMxChunks = mx_chunks<FMT>();
    __shared__ uint4 codes[kMxChunks][kWave];
    __shared__ float scales[kMxChunks][kWave][L::GPL];
    const int V = hidden / L::CPL;
    const int G = hidden / GROUP;
    const int64_t total = num_tokens * V;  // lane vectors of the batch
    const int64_t row_bytes = code_row_bytes<FMT>(hidden);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kMxChunks * kWave;

    // token and lane vector of flat index first + c * 64 + lane
    auto locate = [&](int c, int64_t& t, int& v) {
        const int64_t i0 = first + c * kWave;
        t = i0 / V;
        int64_t off = i0 - t * V + lane;
        while (off >= V) {
            off -= V;
            ++t;
        }
        v = static_cast<int>(off);
    };

    if (wave < kMxChunks) {
        int64_t t;
        int v;
        locate(wave, t, v);
        if (first + wave * kWave + lane < total) {  // whole groups of lanes (V % LPG == 0)
            uint4 q;
            float sf[L::GPL];
            cast_lane_mx<FMT, GROUP>(reinterpret_cast<const uint4*>(x + t * hidden), v, p, q, sf);
            codes[wave][lane] = q;
#pragma unroll
            for (int g = 0; g < L::GPL; ++g) scales[wave][lane][g] = sf[g];
        }
    }
    __syncthreads();

    for (int c = 0; c < kMxChunks; ++c) {
        if (first + c * kWave >= total) break;  // uniform
        int64_t t;
        int v;
        locate(c, t, v);
        const bool live = first + c * kWave + lane < total;
        const uint4 q = codes[c][lane];
        for (int k = wave; k < num_topk; k += kMxWaves) {
            const int64_t r = live ? pos[t * num_topk + k] : -1;
            if (r < 0 || r >= num_rows) continue;
            store_stream16(reinterpret_cast<uint4*>(out + r * row_bytes + static_cast<int64_t>(v) * 16), q);
            if (v % L::LPG == 0) {
#pragma unroll
                for (int g = 0; g < L::GPL; ++g)
                    store_scale(out_sf, r * G + (v / L::LPG) * L::GPL + g, scales[c][lane][g], p.sf_u8);
            }
            if (out_weights != nullptr && v == 0) out_weights[r] = topk_weights[t * num_topk + k];
        }
    }
}

// SwiGLU + cast of one lane's 8 channels (vector v of row r) from its gate
// and up vectors; a group spans GROUP / 8 lanes.  PLAIN: the e4m3 format
// with fp32 scales, unrounded, and the default clamp (the scale constants
// are then compile-time: e4m3_group_scale), as swiglu_cast_fp8 asks.
template <int FMT, int GROUP, bool PLAIN = false>
__device__ __forceinline__ void swiglu_vec(const uint4& rg, const uint4& ru, bool weighted, float wr, bool clamp,
                                           float clamp_value, const MxParams& p, int64_t r, int v, int inter,
                                           uint8_t* __restrict__ out, void* __restrict__ out_sf) {
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
        val[i] = weighted ? (s * ui) * wr : s * ui;
    }
    const uint32_t amax = lanes_max_u32<GROUP / 8>(absmax8_computed(val));
    float sf, inv;
    if constexpr (PLAIN)
        e4m3_group_scale(amax, sf, inv);
    else
        mx_scale(amax, p, sf, inv);
    if constexpr (FMT == kFmtE4m3) {
        store_stream8(reinterpret_cast<uint2*>(out + r * inter + static_cast<int64_t>(v) * 8), quant8_e4m3(val, inv));
    } else {
        __builtin_nontemporal_store(quant8_e2m1(val, inv),
                                    reinterpret_cast<uint32_t*>(out + r * (inter / 2) + static_cast<int64_t>(v) * 4));
    }
    if (v % (GROUP / 8) == 0) {
        const int64_t idx = r * (inter / GROUP) + v / (GROUP / 8);
        if constexpr (PLAIN)
            static_cast<float*>(out_sf)[idx] = sf;
        else
            store_scale(out_sf, idx, sf, p.sf_u8);
    }
}

// SwiGLU + cast: one workgroup per row, a lane owns 8 channels per step.
// The row weight is loaded first: for batches many workgroups deep this
// staggers the first loads of the resident workgroups, which measured
// faster (404.8 against 417-426 us on 262144 rows).
template <int FMT, int GROUP>
__global__ __launch_bounds__(256) void swiglu_mx_kernel(const uint16_t* __restrict__ gate_up, int inter,
                                                        const float* __restrict__ row_weights,
                                                        float clamp_value, MxParams p,
                                                        uint8_t* __restrict__ out, void* __restrict__ out_sf) {
    const int64_t r = blockIdx.x;
    const int V = inter >> 3;
    const uint4* gate = reinterpret_cast<const uint4*>(gate_up + r * 2 * inter);
    const uint4* up = reinterpret_cast<const uint4*>(gate_up + r * 2 * inter + inter);
    const bool clamp = clamp_value > 0.0f;
    const bool weighted = row_weights != nullptr;
    const float wr = weighted ? row_weights[r] : 1.0f;
    for (int v = threadIdx.x; v - static_cast<int>(threadIdx.x) < V; v += 256) {
        if (v >= V) continue;  // uniform over each group of lanes (V % (GROUP / 8) == 0)
        const uint4 rg = load_stream16(gate + v);
        const uint4 ru = load_stream16(up + v);
        swiglu_vec<FMT, GROUP>(rg, ru, weighted, wr, clamp, clamp_value, p, r, v, inter, out, out_sf);
    }
}

// The same for rows of at most 256 vectors (inter <= 2048) in a batch a few
// workgroups deep, where each workgroup's latency adds up: above 8 rows per
// compute unit a row is split over one-wave workgroups of 64 vectors each
// (8192 rows of 2048: 15.2 against 15.4 us for one 256-lane workgroup per
// row, back to back; 4096 rows: 9.1 against 9.2 us), the
// gate and up loads go out right after the kernel arguments arrive (a lane
// past the row loads the row's last vector and discards it), before the row
// weight's load and before any branch; the clamp and the plain e4m3 format
// are template flags.
template <int FMT, int GROUP, bool CLAMP, bool PLAIN>
__global__ __launch_bounds__(256) void swiglu_mx_row_kernel(const uint16_t* __restrict__ gate_up, int inter,
                                                              const float* __restrict__ row_weights,
                                                              float clamp_value, MxParams p,
                                                              uint8_t* __restrict__ out, void* __restrict__ out_sf,
                                                              int split_log2, int lanes_log2) {
    // 2^split_log2 workgroups of 2^lanes_log2 lanes per row: shifts, not a
    // division (which goes to the vector unit and delays the loads'
    // addresses: 16.5 against 15.2 us)
    const int64_t r = blockIdx.x >> split_log2;
    const int V = inter >> 3;
    const int v = static_cast<int>((blockIdx.x & ((1u << split_log2) - 1)) << lanes_log2) + threadIdx.x;
    const int vl = v < V ? v : V - 1;  // in bounds for every lane
    const uint4 rg = load_stream16(reinterpret_cast<const uint4*>(gate_up + r * 2 * inter) + vl);
    const uint4 ru = load_stream16(reinterpret_cast<const uint4*>(gate_up + r * 2 * inter + inter) + vl);
    const bool weighted = row_weights != nullptr;
    const float wr = weighted ? row_weights[r] : 1.0f;
    if (v >= V) return;  // whole groups of lanes
    swiglu_vec<FMT, GROUP, PLAIN>(rg, ru, weighted, wr, CLAMP, clamp_value, p, r, v, inter, out, out_sf);
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
    constexpr int CPL = Layout<FMT, GROUP>::CPL;
    if (pos == nullptr) {
        const int64_t blocks = (T * (H / CPL) + 255) / 256;
        hipLaunchKernelGGL((cast_mx_kernel<FMT, GROUP>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                           stream, x, T, H, p, out, out_sf);
    } else {
        const int64_t chunks = (T * (H / CPL) + kWave - 1) / kWave;  // flat 64-vector chunks
        const int64_t blocks = (chunks + mx_chunks<FMT>() - 1) / mx_chunks<FMT>();
        hipLaunchKernelGGL((expand_mx_split_kernel<FMT, GROUP>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kMxWaves * kWave), 0, stream, x, T, H, K, pos, w, R, p, out, out_sf, out_w);
    }
    return hipGetLastError();
}

template <int FMT, int GROUP>
hipError_t launch_swiglu_mx_t(const uint16_t* gu, int64_t R, int I, const float* w, float c, const MxParams& p,
                              uint8_t* out, void* out_sf, hipStream_t stream) {
    // rows <= 32 per compute unit: the whole grid is at most four rounds of
    // resident workgroups (eight per compute unit), where latency dominates
    if (I <= 2048 && R <= 32 * static_cast<int64_t>(device_cu_count())) {
        const bool plain = FMT == kFmtE4m3 && !p.round_sf && !p.sf_u8 && p.clamp == 1e-4f;
        // more than 8 rows per compute unit: one-wave workgroups, enough per
        // row to cover it (2^split_log2 * 64 >= I / 8); else one 256-lane
        // workgroup per row (2048 rows of 2048: 5.5 against 5.7 us)
        const bool split = R > 8 * static_cast<int64_t>(device_cu_count());
        const int split_log2 = split ? (I > 1024 ? 2 : (I > 512 ? 1 : 0)) : 0;
        const int lanes_log2 = split ? 6 : 8;
        const dim3 grid(static_cast<unsigned>(R << split_log2));
        const dim3 block(1u << lanes_log2);
        if (c > 0.0f) {
            if (plain)
                hipLaunchKernelGGL((swiglu_mx_row_kernel<FMT, GROUP, true, true>), grid, block, 0, stream, gu, I,
                                   w, c, p, out, out_sf, split_log2, lanes_log2);
            else
                hipLaunchKernelGGL((swiglu_mx_row_kernel<FMT, GROUP, true, false>), grid, block, 0, stream, gu, I,
                                   w, c, p, out, out_sf, split_log2, lanes_log2);
        } else {
            if (plain)
                hipLaunchKernelGGL((swiglu_mx_row_kernel<FMT, GROUP, false, true>), grid, block, 0, stream, gu, I,
                                   w, c, p, out, out_sf, split_log2, lanes_log2);
            else
                hipLaunchKernelGGL((swiglu_mx_row_kernel<FMT, GROUP, false, false>), grid, block, 0, stream, gu,
                                   I, w, c, p, out, out_sf, split_log2, lanes_log2);
        }
    } else {
        hipLaunchKernelGGL((swiglu_mx_kernel<FMT, GROUP>), dim3(static_cast<unsigned>(R)), dim3(256), 0, stream, gu,
                           I, w, c, p, out, out_sf);
    }
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
