// Measurement probes: the rates this GPU sustains for what the path is bound
// by, so that roofline fractions can be read against the machine as well as
// against its nominal peaks.  Nothing here is part of the forward path.
//
//   kind 0  streaming read: `bytes` (a multiple of 16) read once with 16-byte
//           non-temporal loads, grid-stride over 2048 workgroups of 256
//           threads, four loads in flight per thread.
//   kind 1  v_mfma_f32_16x16x32_bf16 (the verify-batch kernels' instruction)
//   kind 2  v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 x E2M1 operands (the
//           8192-token chunk's)
//   kind 3  the same with E2M1 x E2M1 operands (the MXFP4 peak)
//   kinds 4, 5, 6  kinds 1, 2, 3 with random operands that change from one
//           MFMA to the next (four register sets per operand, drawn from a
//           hash; no NaN or infinite codes).  The chip's clock drops under
//           its power limit when operand bits toggle, so these rates are the
//           ones real data can reach; kinds 1-3 repeat one operand pair.
//
// MFMA kinds: 2048 workgroups of 4 waves, each wave 32 `reps` rounds of 8
// independent accumulator chains (enough to cover the instruction's
// latency), operands in registers.  32 rounds per loop iteration keep the
// loop's own instructions (and the accumulator copies the compiler places
// at its back edge for some kinds: 56 per 256 MFMAs) to a few percent, so
// the rates are slight underestimates.  Results are folded into one value
// that is stored only if it equals a constant it never takes, which keeps
// the work alive without a result buffer.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kProbeGroups = 2048;
constexpr int kProbeThreads = 256;
constexpr int kChains = 8;
constexpr int kUnroll = 32;                 // rounds per loop iteration

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

__global__ __launch_bounds__(kProbeThreads) void k_probe_stream(const u32x4_t* __restrict__ src, size_t n16,
                                                                 uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= (a.x ^ b.y) + (c.z ^ d.w) + (a.y ^ b.x) + (c.w ^ d.z);
    }
    for (; i < n16; i += stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        acc ^= a.x + a.y + a.z + a.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

constexpr int kSets = 4;                    // operand register sets of the random kinds

// 32-bit mix of (thread, index) for the random operands (a murmur3 finaliser)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    return x ^ (x >> 16);
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(int reps, uint32_t* sink) {
    const int lane = threadIdx.x % kWave;
    f32x4_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND >= 4) {
        const uint32_t t = blockIdx.x * kProbeThreads + threadIdx.x;
        if constexpr (KIND == 4) {
            // bf16 values k/16 for k in [-32, 31]: finite, mixed signs and exponents
            bf16x8_t a[kSets], b[kSets];
#pragma unroll
            for (int q = 0; q < kSets; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a[q][i] = (__bf16)((float)((int)(mix32(t * 64u + q * 8u + i) % 64u) - 32) * 0.0625f);
                    b[q][i] = (__bf16)((float)((int)(mix32(t * 64u + q * 8u + i + 32u) % 64u) - 32) * 0.0625f);
                }
            for (int r = 0; r < reps; ++r)
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                    for (int c = 0; c < kChains; ++c)
                        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(u + c) % kSets], b[(u + 3 * c + 1) % kSets],
                                                                         acc[c], 0, 0, 0);
        } else {
            // E4M3 bytes with the low exponent bit clear never encode NaN;
            // every E2M1 code is finite
            constexpr uint32_t amask = KIND == 5 ? 0xF7F7F7F7u : 0xFFFFFFFFu;
            i32x8_t a[kSets], b[kSets];
#pragma unroll
            for (int q = 0; q < kSets; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a[q][i] = (int)(mix32(t * 64u + q * 8u + i) & amask);
                    b[q][i] = (int)mix32(t * 64u + q * 8u + i + 32u);
                }
            constexpr int fmt_a = KIND == 5 ? 0 : 4;
            for (int r = 0; r < reps; ++r)
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                    for (int c = 0; c < kChains; ++c)
                        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a[(u + c) % kSets], b[(u + 3 * c + 1) % kSets], acc[c], fmt_a, 4, 0, 0x7f7f7f7f, 0,
                            0x7f7f7f7f);
        }
    } else if constexpr (KIND == 1) {
        bf16x8_t a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(float)((lane + i) % 7 - 3);
            b[i] = (__bf16)(float)((lane * 3 + i) % 5 - 2);
        }
        for (int r = 0; r < reps; ++r)
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int c = 0; c < kChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    } else {
        i32x8_t a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (int)(0x3a2c1e10u * (uint32_t)(lane + i + 1));
            b[i] = (int)(0x1b2d3f41u * (uint32_t)(lane + 2 * i + 1));
        }
        constexpr int fmt_a = KIND == 2 ? 0 : 4;       // E4M3 or E2M1
        for (int r = 0; r < reps; ++r)
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int c = 0; c < kChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], fmt_a, 4, 0, 0x7f7f7f7f,
                                                                              0, 0x7f7f7f7f);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (s == 1234567.0f) sink[0] = __float_as_uint(s);
}

}  // namespace

hipError_t launch_probe(int kind, const void* src, size_t bytes, int reps, uint32_t* sink, double* work,
                        hipStream_t s) {
    const dim3 grid(kProbeGroups), block(kProbeThreads);
    if (kind == 0) {
        hipLaunchKernelGGL(k_probe_stream, grid, block, 0, s, static_cast<const u32x4_t*>(src), bytes / 16, sink);
        *work = (double)(bytes / 16 * 16);
    } else {
        if (kind == 1) hipLaunchKernelGGL(k_probe_mfma<1>, grid, block, 0, s, reps, sink);
        if (kind == 2) hipLaunchKernelGGL(k_probe_mfma<2>, grid, block, 0, s, reps, sink);
        if (kind == 3) hipLaunchKernelGGL(k_probe_mfma<3>, grid, block, 0, s, reps, sink);
        if (kind == 4) hipLaunchKernelGGL(k_probe_mfma<4>, grid, block, 0, s, reps, sink);
        if (kind == 5) hipLaunchKernelGGL(k_probe_mfma<5>, grid, block, 0, s, reps, sink);
        if (kind == 6) hipLaunchKernelGGL(k_probe_mfma<6>, grid, block, 0, s, reps, sink);
        const double per = kind == 1 || kind == 4 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 128;
        *work = per * kChains * kUnroll * (double)reps * (double)kProbeGroups * (kProbeThreads / kWave);
    }
    return hipGetLastError();
}

}  // namespace moe
