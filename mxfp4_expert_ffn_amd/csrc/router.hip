// Router projection in front of the routing: logits[t][e] = sum_i x[t][i] *
// W[e][i], bf16 inputs, float32 accumulation on the bf16 matrix cores.
//
// The pages keep every module outside the experts in FP8 or its original
// precision (techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 —
// MoE에만 걸린 양자화") and route each token to its experts (same page,
// section "3. TileRT"); they give no router form, so this is the plain
// linear map with bf16 x and W and no bias.
//
// Workgroup = one tile of 16 TW tokens x 16 EW experts, KS wavefronts along
// K (contiguous ranges).  Each wave keeps TW x EW accumulator tiles, so a
// loaded x fragment feeds EW MFMAs and a W fragment TW of them: TW = EW = 1
// for small batches (many small workgroups: latency), 4 x 4 for large ones
// (4x less operand traffic per MFMA).  Lane (li, g) of a
// v_mfma_f32_16x16x32_bf16 step over K [k0, k0 + 32) holds x[token li][k0 +
// 8g ..] and W[expert li][k0 + 8g ..] -- 16-byte loads straight from global
// memory (a K range is read by one wave only).  The KS partial tiles are
// added through LDS in split order, so the result does not depend on timing.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kRouterWaves = 16;

struct RouterArgs {
    const uint16_t* x;      // [T][d]
    const uint16_t* w;      // [E][d]
    float* logits;          // [T][E]
    int32_t T, d, E;
    int32_t ks;             // waves along K
};

template <int TW, int EW, int KSMAX, int UNROLL>
__global__ __launch_bounds__(KSMAX * kWave) void k_router(RouterArgs a) {
    __shared__ f32x4_t part[KSMAX][TW * EW][kWave];
    const int lane = threadIdx.x % kWave;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int li = lane % 16, g = lane / 16;
    const int t0 = blockIdx.x * 16 * TW, e0 = blockIdx.y * 16 * EW;
    const int kr = a.d / a.ks;                               // K range of one split (multiple of 256)
    const int kbeg = ks * kr;
    // rows past T / experts past E repeat the last one; never stored
    const uint16_t* xrow[TW];
    const uint16_t* wrow[EW];
#pragma unroll
    for (int i = 0; i < TW; ++i) xrow[i] = a.x + (size_t)min(t0 + 16 * i + li, a.T - 1) * a.d + kbeg + 8 * g;
#pragma unroll
    for (int j = 0; j < EW; ++j) wrow[j] = a.w + (size_t)min(e0 + 16 * j + li, a.E - 1) * a.d + kbeg + 8 * g;
    f32x4_t acc[TW][EW];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < EW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < kr; k += 32 * UNROLL) {
        bf16x8_t xa[UNROLL][TW], wb[UNROLL][EW];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
            for (int i = 0; i < TW; ++i) xa[u][i] = *reinterpret_cast<const bf16x8_t*>(xrow[i] + k + 32 * u);
#pragma unroll
            for (int j = 0; j < EW; ++j) wb[u][j] = *reinterpret_cast<const bf16x8_t*>(wrow[j] + k + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int j = 0; j < EW; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u][i], wb[u][j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < EW; ++j) part[ks][i * EW + j][lane] = acc[i][j];
    __syncthreads();
    if (ks != 0) return;
    // lane holds D[token 16 i + 4g + r][expert 16 j + li] of tile (i, j)
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < EW; ++j) {
            f32x4_t s = acc[i][j];
            for (int q = 1; q < a.ks; ++q) s += part[q][i * EW + j][lane];
            const int e = e0 + 16 * j + li;
            if (e < a.E) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = t0 + 16 * i + 4 * g + r;
                    if (t < a.T) a.logits[(size_t)t * a.E + e] = s[r];
                }
            }
        }
}

template <int TW, int EW, int KSMAX, int UNROLL>
hipError_t launch_tiles(RouterArgs a, hipStream_t s) {
    // K splits: a power of two up to KSMAX whose K range is a multiple of 256
    int ks = KSMAX;
    while (ks > 1 && (a.d % (256 * ks)) != 0) ks /= 2;
    a.ks = ks;
    const dim3 grid((a.T + 16 * TW - 1) / (16 * TW), (a.E + 16 * EW - 1) / (16 * EW)), block(ks * kWave);
    hipLaunchKernelGGL((k_router<TW, EW, KSMAX, UNROLL>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* w, float* logits, const Dims& dm, hipStream_t s) {
    RouterArgs a{};
    a.x = x; a.w = w; a.logits = logits;
    a.T = dm.T; a.d = dm.d; a.E = dm.E;
    // 64 x 64 tiles once they alone fill the GPU, 16 x 16 tiles below that
    const long big_tiles = (long)((dm.T + 63) / 64) * ((dm.E + 63) / 64);
    if (big_tiles >= 128) return launch_tiles<4, 4, 8, 2>(a, s);
    return launch_tiles<1, 1, kRouterWaves, 8>(a, s);
}

}  // namespace moe
