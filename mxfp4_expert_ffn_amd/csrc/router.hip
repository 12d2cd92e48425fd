// Router projection in front of the routing: logits[t][e] = sum_i x[t][i] *
// W[e][i], bf16 inputs, float32 accumulation on the bf16 matrix cores.
//
// The pages keep every module outside the experts in FP8 or its original
// precision (techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 —
// MoE에만 걸린 양자화") and route each token to its experts (same page,
// section "3. TileRT"); they give no router form, so this is the plain
// linear map with bf16 x and W and no bias.
//
// Workgroup = one tile of 16 tokens x 16 experts, KS wavefronts along K
// (contiguous ranges, KS up to 16), so that even a small batch spreads over
// many CUs.  Lane (li, g) of a v_mfma_f32_16x16x32_bf16 step over K [k0,
// k0 + 32) holds x[token li][k0 + 8g ..] and W[expert li][k0 + 8g ..] --
// one 16-byte load each, straight from global memory (a K range is read by
// one wave only, so there is nothing to share through LDS).  The KS partial
// tiles are added through LDS in split order, so the result does not depend
// on timing.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kRouterWaves = 16;
constexpr int kUnroll = 8;                  // MFMA steps (32 K each) per loop turn

struct RouterArgs {
    const uint16_t* x;      // [T][d]
    const uint16_t* w;      // [E][d]
    float* logits;          // [T][E]
    int32_t T, d, E;
    int32_t ks;             // waves along K
};

__global__ __launch_bounds__(kRouterWaves * kWave) void k_router(RouterArgs a) {
    __shared__ f32x4_t part[kRouterWaves][kWave];
    const int lane = threadIdx.x % kWave;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int li = lane % 16, g = lane / 16;
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
    const int kr = a.d / a.ks;                               // K range of one split (multiple of 256)
    const int kbeg = ks * kr;
    // rows past T / experts past E repeat the last one; never stored
    const uint16_t* xrow = a.x + (size_t)min(t0 + li, a.T - 1) * a.d + kbeg + 8 * g;
    const uint16_t* wrow = a.w + (size_t)min(e0 + li, a.E - 1) * a.d + kbeg + 8 * g;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < kr; k += 32 * kUnroll) {
        bf16x8_t xa[kUnroll], wb[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            xa[u] = *reinterpret_cast<const bf16x8_t*>(xrow + k + 32 * u);
            wb[u] = *reinterpret_cast<const bf16x8_t*>(wrow + k + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u], wb[u], acc, 0, 0, 0);
    }
    part[ks][lane] = acc;
    __syncthreads();
    if (ks != 0) return;
    // lane holds D[token 4g + r][expert li]
    for (int q = 1; q < a.ks; ++q) acc += part[q][lane];
    const int e = e0 + li;
    if (e < a.E) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * g + r;
            if (t < a.T) a.logits[(size_t)t * a.E + e] = acc[r];
        }
    }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* w, float* logits, const Dims& dm, hipStream_t s) {
    RouterArgs a{};
    a.x = x; a.w = w; a.logits = logits;
    a.T = dm.T; a.d = dm.d; a.E = dm.E;
    // K splits: a power of two up to 16 whose K range is a multiple of 256
    int ks = kRouterWaves;
    while (ks > 1 && (dm.d % (256 * ks)) != 0) ks /= 2;
    a.ks = ks;
    const dim3 grid((dm.T + 15) / 16, (dm.E + 15) / 16), block(ks * kWave);
    hipLaunchKernelGGL(k_router, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
