// Weighted combine of the k expert outputs of every token, and the two
// helper kernels that sit beside the forward path (decode export, weight
// quantiser).
//
// Combine: y[t] = sum_j w[t][j] * o[t][j].  The down projection stores the
// output of pair p = t*k + j at row p, so a token's k rows form one
// contiguous block.  The streaming path stores o in float32; the dense path
// stores fp16 codes with one power-of-two scale per 128 columns, decoded here
// exactly.  Each product is rounded to float32 on its own (no fused
// multiply-add), the k products are added in slot order j = 0..k-1 (fixed
// order: deterministic), and the sum is rounded once to the output type.
#include "layer.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// 4 consecutive values of an o row as float32.  OT = float: float32 values;
// OT = uint16_t: fp16 codes times 2^(scale byte - 127) (exact products).
template <typename OT>
__device__ __forceinline__ f32x4_t load_o4(const OT* p, const uint8_t* sc) {
    if constexpr (sizeof(OT) == 4) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    } else {
        const u32x2_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        const int se = (int)*sc - 127;
        auto f = [&](uint32_t h) { return ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)h), se); };
        return f32x4_t{f(b.x & 0xFFFFu), f(b.x >> 16), f(b.y & 0xFFFFu), f(b.y >> 16)};
    }
}

// One thread per 4 consecutive output columns of one token.  KK > 0: k is
// KK and the k row loads are all issued before the sum (the rows are read
// once, so they bypass the caches' retention).  o holds float32 values
// (streaming path) or fp16 codes with a scale byte per 128 columns in os
// (dense path).  layer_st: the state block of the routing expert kernel
// that ran before (nullptr: none), whose queue and chunk counters workgroup
// 0 clears for the stream's next call and whose epoch it advances.
template <int KK, typename OT>
__global__ __launch_bounds__(kThreads) void k_finalize(Dims dm, const OT* __restrict__ o,
                                                       const uint8_t* __restrict__ os,
                                                       const float* __restrict__ topk_w,
                                                       void* __restrict__ out, int out_dtype,
                                                       int32_t* __restrict__ layer_st) {
#pragma clang fp contract(off)
    if (layer_st && blockIdx.x == 0) {
        static_assert(kChunk < kThreads, "one thread per counter");
        if (threadIdx.x == 0) {
            layer_st[kLayerQueue] = 0;
            layer_st[kLayerEpoch] = layer_st[kLayerEpoch] + 1;
        } else if (threadIdx.x <= kChunk) {
            layer_st[kLayerChunkDone + kLayerLine * (threadIdx.x - 1)] = 0;
        }
    }
    const int q = dm.d / 4;
    const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= (size_t)dm.T * q) return;
    const int t = (int)(gid / q), c = (int)(gid % q) * 4;
    const int k = KK > 0 ? KK : dm.k;
    const OT* ot = o + (size_t)t * k * dm.d + c;
    const int ng = dm.d / 128;
    const uint8_t* st = os + (size_t)t * k * ng + c / 128;
    const float* wt = topk_w + (size_t)t * k;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KK > 0) {
        static_assert(KK % 4 == 0, "weights are read 4 at a time");
        f32x4_t v[KK], w4[KK / 4];
#pragma unroll
        for (int j = 0; j < KK; ++j) v[j] = load_o4(ot + (size_t)j * dm.d, st + j * ng);
#pragma unroll
        for (int j = 0; j < KK / 4; ++j) w4[j] = reinterpret_cast<const f32x4_t*>(wt)[j];
#pragma unroll
        for (int j = 0; j < KK; ++j) acc += w4[j / 4][j % 4] * v[j];
    } else {
        for (int j = 0; j < k; ++j) acc += wt[j] * load_o4(ot + (size_t)j * dm.d, st + j * ng);
    }
    if (out_dtype == MOE_OUT_F32) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + (size_t)t * dm.d + c) = acc;
    } else {
        const uint32_t lo = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * dm.d + c) = make_uint2(lo, hi);
    }
}

// Tiled-layout addressing (the byte formulas of the header).
__device__ __forceinline__ int64_t tiled_block_offset(int64_t n, int64_t b, int64_t ns) {
    return 16 * (64 * ((n / 16) * ns + b / 4) + (n % 16) + 16 * (b % 4));
}
__device__ __forceinline__ int64_t tiled_scale_offset(int64_t n, int64_t b, int64_t ng) {
    return 4 * (64 * ((n / 16) * ng + b / 16) + (n % 16) + 16 * (b % 4)) + (b / 4) % 4;
}

// Decode export: one thread per 8 elements (one packed dword) of rows
// [row0, row0 + nrows) of one tiled matrix, with the forward path's
// decode8_bf16, widened to float, written row-major.
__global__ __launch_bounds__(kThreads) void k_debug_dequant(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t K, int32_t row0, int32_t nrows,
                                                            float* __restrict__ out) {
    const int64_t per_row = K / 8;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= per_row * nrows) return;
    const int64_t i = gid / per_row, c8 = gid % per_row;
    const int64_t n = row0 + i, b = c8 / 4;
    const int64_t ns = K / kKStep, ng = (ns + 3) / 4;
    const uint32_t word = *reinterpret_cast<const uint32_t*>(packed + tiled_block_offset(n, b, ns) + (c8 % 4) * 4);
    const uint32_t sb = scales[tiled_scale_offset(n, b, ng)];
    const bf16x8_t v = decode8_bf16(word, e8m0_as_scale(sb));
    float* dst = out + i * K + c8 * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = (float)v[k];
}

// Row-major -> tiled: one thread per 16-byte MX block of packed data.
__global__ __launch_bounds__(kThreads) void k_tile_packed(const uint8_t* __restrict__ src, int64_t rows,
                                                          int64_t K, uint8_t* __restrict__ dst) {
    const int64_t nb = K / kBlock;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= rows * nb) return;
    const int64_t n = gid / nb, b = gid % nb;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + n * (K / 2) + b * 16);
    *reinterpret_cast<u32x4_t*>(dst + tiled_block_offset(n, b, K / kKStep)) = v;
}

// Row-major -> tiled scales: one thread per output dword (16-row tile t,
// group G, lane L): bytes j = 0..3 are the scales of step 4G + j (zero past
// the last step).
__global__ __launch_bounds__(kThreads) void k_tile_scales(const uint8_t* __restrict__ src, int64_t rows,
                                                          int64_t K, uint8_t* __restrict__ dst) {
    const int64_t ns = K / kKStep, ng = (ns + 3) / 4, nb = K / kBlock;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= (rows / 16) * ng * 64) return;
    const int64_t L = gid % 64, G = (gid / 64) % ng, t = gid / (64 * ng);
    const int64_t n = 16 * t + L % 16;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t step = 4 * G + j;
        if (step < ns) word |= (uint32_t)src[n * nb + 4 * step + L / 16] << (8 * j);
    }
    *reinterpret_cast<uint32_t*>(dst + 4 * gid) = word;
}

// E2M1 code of one already-scaled value: nearest of 0, .5, 1, 1.5, 2, 3, 4, 6
// with ties to the even code, saturating; the sign of a zero result kept.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
    const float a = fabsf(q);
    uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                 (a >= 3.5f) + (a > 5.0f);
    return m | ((__float_as_uint(q) >> 28) & 8u);
}

// Weight quantiser: 4 lanes per 32-element block, 8 elements each.
__global__ __launch_bounds__(kThreads) void k_quantize(const float* __restrict__ w, int64_t rows,
                                                       int64_t K, uint8_t* __restrict__ packed,
                                                       uint8_t* __restrict__ scales) {
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nblk = rows * (K / kBlock);
    const int64_t blk = gid / 4;
    const int part = (int)(gid % 4);
    const bool valid = blk < nblk;
    const int64_t r = valid ? blk / (K / kBlock) : 0, b = valid ? blk % (K / kBlock) : 0;
    float v[8];
    float amax = 0.f;
    const float* src = w + r * K + b * kBlock + part * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = valid ? src[i] : 0.f;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    // the 4 lanes of a block are consecutive and 4-aligned within the wave
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    if (!valid) return;
    // floor(log2(amax)) from the exponent field; a subnormal amax is
    // mantissa * 2^-149, so its floor(log2) is 31 - clz(mantissa) - 149
    int fl;
    const uint32_t bits = __float_as_uint(amax);
    const int ef = (int)(bits >> 23);
    if (amax == 0.f) fl = -125;                       // gives the smallest scale, byte 0
    else if (ef > 0) fl = ef - 127;
    else fl = -118 - (int)__clz(bits & 0x7FFFFFu);
    int se = fl - 2;
    se = se < -127 ? -127 : (se > 127 ? 127 : se);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= e2m1_code(ldexpf(v[i], -se)) << (4 * i);
    *reinterpret_cast<uint32_t*>(packed + r * (K / 2) + b * 16 + part * 4) = word;
    if (part == 0) scales[r * (K / kBlock) + b] = (uint8_t)(se + 127);
}

}  // namespace

namespace {

hipError_t finalize(const Dims& dm, const Workspace& ws, void* out, int out_dtype, bool o_f16, hipStream_t s,
                    int32_t* st) {
    const size_t n = (size_t)dm.T * (dm.d / 4);
    const dim3 grid((unsigned)((n + kThreads - 1) / kThreads)), block(kThreads);
    const uint16_t* o16 = reinterpret_cast<const uint16_t*>(ws.o);
    if (dm.k == 8 && o_f16)
        hipLaunchKernelGGL((k_finalize<8, uint16_t>), grid, block, 0, s, dm, o16, ws.os, ws.topk_w, out, out_dtype, st);
    else if (dm.k == 8)
        hipLaunchKernelGGL((k_finalize<8, float>), grid, block, 0, s, dm, ws.o, ws.os, ws.topk_w, out, out_dtype, st);
    else if (o_f16)
        hipLaunchKernelGGL((k_finalize<0, uint16_t>), grid, block, 0, s, dm, o16, ws.os, ws.topk_w, out, out_dtype, st);
    else
        hipLaunchKernelGGL((k_finalize<0, float>), grid, block, 0, s, dm, ws.o, ws.os, ws.topk_w, out, out_dtype, st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_finalize(const Dims& dm, const Workspace& ws, void* out, int out_dtype, bool o_f16,
                           hipStream_t s) {
    return finalize(dm, ws, out, out_dtype, o_f16, s, nullptr);
}

hipError_t launch_finalize_layer(const Dims& dm, const Workspace& ws, void* out, int out_dtype, int32_t* state,
                                 hipStream_t s) {
    return finalize(dm, ws, out, out_dtype, false, s, state);
}

hipError_t launch_debug_dequant(const uint8_t* packed, const uint8_t* scales, int64_t K, int32_t row0,
                                int32_t nrows, float* out, hipStream_t s) {
    const int64_t n = (K / 8) * nrows;
    hipLaunchKernelGGL(k_debug_dequant, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       packed, scales, K, row0, nrows, out);
    return hipGetLastError();
}

hipError_t launch_tile(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                       uint8_t* tpacked, uint8_t* tscales, hipStream_t s) {
    const int64_t nb = rows * (K / kBlock);
    hipLaunchKernelGGL(k_tile_packed, dim3((unsigned)((nb + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       packed, rows, K, tpacked);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ns = K / kKStep, ng = (ns + 3) / 4;
    const int64_t nw = (rows / 16) * ng * 64;
    hipLaunchKernelGGL(k_tile_scales, dim3((unsigned)((nw + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       scales, rows, K, tscales);
    return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales,
                           hipStream_t s) {
    const int64_t n = rows * (K / kBlock) * 4;
    hipLaunchKernelGGL(k_quantize, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       w, rows, K, packed, scales);
    return hipGetLastError();
}

}  // namespace moe
