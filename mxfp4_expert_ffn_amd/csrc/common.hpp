// Shared definitions of the HIP path (gfx950 / CDNA4 only).
//
// The expert weights are MXFP4: 4-bit E2M1 elements and one E8M0 scale per
// block of 32 along K (ai.appwright.xyz tag page "投機的デコード", section
// "第1層：FP4量子化（モデル側）"; bit meanings from the OCP MX v1.0 spec).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mxfp4.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront
constexpr int kBlock = 32;         // MX block (elements per E8M0 scale)
constexpr int kKStep = 128;        // K per main-loop step: 4 MX blocks, one per lane group
constexpr int kChunk = 64;         // token pairs per expert work chunk

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// E8M0 byte -> the float32 whose exponent field is that byte.  The gfx950
// scaled converts read only the exponent field of their scale operand, so
// this hands them 2^(byte-127) for every byte 0..254 (byte 0 included).
__device__ __forceinline__ float e8m0_as_scale(uint32_t byte) {
    return __uint_as_float(byte << 23);
}

// Eight E2M1 nibbles (one dword, element 2i in the low nibble of byte i)
// times 2^(scale-127) -> eight bf16, in element order.  Exact: every such
// product is representable in bf16 (overflow aside, which only the two
// largest scale bytes can reach).
__device__ __forceinline__ bf16x8_t decode8_bf16(uint32_t packed, float scale) {
    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 0);
    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 1);
    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 2);
    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 3);
    bf16x8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Workspace carve-up shared by the host code and the kernels' launchers.
struct Workspace {
    int32_t* topk_ids;        // [P]
    float* topk_w;            // [P]
    int32_t* offsets;         // [E+1]
    int32_t* sorted_pairs;    // [P]
    int32_t* inverse;         // [P]   position of pair p in sorted_pairs
    int32_t* active;          // [E+1] active experts (count > 0) by descending count; [E] = how many
    int32_t* chunks;          // [max_chunks][2] (expert, first pair within the expert)
    int32_t* nchunks;         // [1] number of chunks
    uint16_t* h;              // [P][f] bf16, rows in sorted order
    float* o;                 // [P][d] weighted expert outputs, rows in sorted order
};

// Problem description passed by value to kernels.
struct Dims {
    int32_t T, d, f, E, k, P;
};

// Upper bound of the chunk list: one partial chunk per active expert plus
// the full chunks.
inline int max_chunks(const Dims& dm) {
    const int active = dm.E < dm.P ? dm.E : dm.P;
    return active + dm.P / kChunk;
}

// Kernel launchers (each returns hipGetLastError() of its launch).
hipError_t launch_route(const float* logits, const Dims& dm, const Workspace& ws, hipStream_t s);
hipError_t launch_sort(const Dims& dm, const Workspace& ws, hipStream_t s);
hipError_t launch_gateup(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm,
                         const Workspace& ws, hipStream_t s);
hipError_t launch_down(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws,
                       hipStream_t s);
hipError_t launch_finalize(const Dims& dm, const Workspace& ws, void* out, int out_dtype,
                           hipStream_t s);
hipError_t launch_debug_dequant(const uint8_t* packed, const uint8_t* scales, int64_t K, int32_t row0,
                                int32_t nrows, float* out, hipStream_t s);
hipError_t launch_tile(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                       uint8_t* tpacked, uint8_t* tscales, hipStream_t s);

// Bytes of the tiled scale array of one rows x K matrix.
inline int64_t tiled_scale_bytes(int64_t rows, int64_t K) {
    return (rows / 16) * ((K / kKStep + 3) / 4) * 256;
}
hipError_t launch_quantize(const float* w, int64_t rows, int64_t K, uint8_t* packed,
                           uint8_t* scales, hipStream_t s);

}  // namespace moe
