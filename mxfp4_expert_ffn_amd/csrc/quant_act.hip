// MXFP8 quantisation of the hidden states (the 8192-token chunk's mode):
// per block of 32 along d_model, scale 2^(floor(log2 amax) - 8) (E4M3's
// largest exponent is 8) as an E8M0 byte, elements rounded to E4M3
// nearest-even, saturating.  The pages fix MX block 32 (ai.appwright.xyz
// "投機的デコード", section "第1層：FP4量子化（モデル側）"); the element and
// scale rules are the OCP MX v1.0 ones.  Exact: every decision is taken on
// the bf16 input scaled by a power of two.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

// 4 lanes per block of 32 bf16, 8 each (one 16-byte load, one 8-byte store).
__global__ __launch_bounds__(kThreads) void k_quant_x8(const uint16_t* __restrict__ x, int64_t n_blocks,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t blk = gid / 4;
    const int part = (int)(gid % 4);
    const bool valid = blk < n_blocks;
    const int64_t b = valid ? blk : 0;
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(x + b * kBlock + part * 8);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(raw[i] << 16);
        v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // the 4 lanes of a block are consecutive and 4-aligned within the wave
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    if (!valid) return;
    const int se = mx_scale_exp(amax, 8);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo |= e4m3_code(ldexpf(v[i], -se)) << (8 * i);
        hi |= e4m3_code(ldexpf(v[i + 4], -se)) << (8 * i);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + b * kBlock + part * 8);
    dst[0] = lo;
    dst[1] = hi;
    if (part == 0) scales[b] = (uint8_t)(se + 127);
}

}  // namespace

hipError_t launch_quant_act8(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                             hipStream_t s) {
    const int64_t nb = rows * (K / kBlock);
    const int64_t n = nb * 4;
    hipLaunchKernelGGL(k_quant_x8, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, x,
                       nb, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quant_x8(const uint16_t* x, const Dims& dm, const Workspace& ws, hipStream_t s) {
    return launch_quant_act8(x, dm.T, dm.d, ws.xq, ws.xs, s);
}

}  // namespace moe
