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
constexpr int kChunk = 64;         // token pairs per expert work chunk (bf16 activations)
constexpr int kDenseChunk = 128;   // token pairs per expert work chunk (MXFP8 activations)
constexpr int kChunkRec = 4;       // ints per chunk record
constexpr int kMaxExperts = 512;  // E limit of the library
constexpr int kMaxTopK = 32;      // k limit of the library

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

// Shared scale exponent of an MX block (OCP MX v1.0 scalar-to-MX rule):
// floor(log2(amax)) - emax_elem, clamped to the E8M0 range [-127, 127]; an
// all-zero block gets -127.  floor(log2) comes from the exponent field; a
// subnormal amax is mantissa * 2^-149, so it is 31 - clz(mantissa) - 149.
__device__ __forceinline__ int mx_scale_exp(float amax, int emax_elem) {
    if (amax == 0.f) return -127;
    const uint32_t bits = __float_as_uint(amax);
    const int ef = (int)(bits >> 23);
    const int fl = ef > 0 ? ef - 127 : -118 - (int)__clz(bits & 0x7FFFFFu);
    const int se = fl - emax_elem;
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// E4M3 code (OCP: bias 7, 3 mantissa bits, largest finite 448, no infinity)
// of an already-scaled finite value: nearest, ties to the even code,
// saturating at +-448 (never the NaN code); the sign of a zero result kept.
// The gfx950 convert rounds to nearest-even but turns magnitudes from 464 up
// into the NaN code, so the value is clamped to +-448 first (values in
// (448, 464) round to 448 either way).  Checked against a bitwise
// implementation of the rule on every finite float below 2^10 in magnitude.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    const float c = fminf(fmaxf(q, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
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
    int32_t* active;          // [E+1] active experts (count > 0) by descending count; [E] = how many
    int32_t* chunks;          // [max_chunks][4] (expert, position of the chunk's first pair in
                              //   sorted_pairs, pairs in the chunk, 0)
    int32_t* nchunks;         // [1] number of chunks
    int32_t* xtab;            // per-XCD chunk table: [kXtabHead] chunks per XCD (kXcds used),
                              //   then [kXcds][xcd_slots(dm)] records of kXtabRec ints
    int32_t* sort_part;       // [sort_tiles(P)][E] per-tile expert histograms / first positions
    uint8_t* xq;              // MXFP8 mode: [T][d] E4M3 codes of x
    uint8_t* xs;              // MXFP8 mode: [T][d/32] E8M0 scales of x
    uint8_t* h;               // [P][f] bf16 (or E4M3 codes in MXFP8 mode), rows in sorted order
    uint8_t* hs;              // MXFP8 mode: [P][f/32] E8M0 scales of h
    float* o;                 // [P][d] expert outputs, row p = pair p (token-major); MXFP8
                              // mode: fp16 codes in the first half of that space
    uint8_t* os;              // MXFP8 mode: [P][d/128] scale exponents + 127 of o's fp16
                              // codes, placed after them inside o's space
    int32_t* fctl;            // fused path: work-queue, ticket, error and completion counters
};

// Problem description passed by value to kernels.
struct Dims {
    int32_t T, d, f, E, k, P;
};

// Pair counts up to this are sorted by one workgroup; above, by tiles of
// 2048 pairs (sort_tiles of them).
constexpr int kSortSingleMax = 8192;
inline int sort_tiles(int P) { return P <= kSortSingleMax ? 0 : (P + 2047) / 2048; }

// Upper bound of the chunk list: one partial chunk per active expert plus
// the full chunks.
inline int max_chunks(const Dims& dm) {
    const int active = dm.E < dm.P ? dm.E : dm.P;
    return active + dm.P / kChunk;
}

// Per-XCD chunk table.  The GPU hands workgroups to its kXcds XCDs
// round-robin by workgroup index, and each XCD has its own L2.  The sort
// assigns every active expert to one XCD -- in rank order, each to the XCD
// with the fewest chunks so far (greedy list scheduling) -- and lists each
// XCD's chunks expert by expert; the streaming kernels run XCD x's chunks
// on workgroups x, x + kXcds, ..., so all the units of an expert -- its
// weight tiles, and each chunk's activation rows -- go through one L2.
// Only the speed depends on that dispatch order.  When an XCD receives its
// last expert it holds the fewest chunks, at most floor((nchunks - m) /
// kXcds), so no list exceeds floor(nchunks / kXcds) plus one expert's
// chunks (at most ceil(T / kChunk), every token picking distinct experts),
// which bounds the table's slots.
constexpr int kXcds = 8;
constexpr int kXtabHead = 64;      // ints before the records
// Table record: expert, position of the chunk's first pair in sorted_pairs,
// pairs in the chunk, the chunk's index in the global list, the chunk's
// index among its expert's chunks, the expert's chunk count, 2 unused.
constexpr int kXtabRec = 8;
inline int xcd_slots(const Dims& dm) {
    const int T = dm.T < dm.P ? dm.T : dm.P;
    return (max_chunks(dm) + kXcds - 1) / kXcds + (T + kChunk - 1) / kChunk;
}

// Work unit u of XCD x's list, with nt_per column tiles per chunk
// (u < xstride * nt_per); false for a unit past the list's end.  An
// expert's m chunks fill m consecutive slots, hence units [s * nt_per,
// (s + m) * nt_per) of the list, which run column tile by column tile: the
// m units of one weight tile are neighbours, start together on the XCD and
// share that tile's fetch through its L2 (chunk by chunk instead, a hot
// expert's later chunks fetch its weights again).  The list's length and
// the slot's record are read together, so a single-chunk expert's unit
// waits on one round trip.
struct XcdUnit {
    int e, start, rows, chunk, nt, m;    // m: the expert's chunks
};
__device__ __forceinline__ bool xcd_unit(const int32_t* xtab, int xstride, int x, int u, int nt_per, XcdUnit& w) {
    const int32_t* list = xtab + kXtabHead + (size_t)kXtabRec * x * xstride;
    const int q = u / nt_per;
    const int32_t* r = list + kXtabRec * q;
    const int n = __builtin_amdgcn_readfirstlane(xtab[x]);
    w.e = __builtin_amdgcn_readfirstlane(r[0]);
    w.start = __builtin_amdgcn_readfirstlane(r[1]);
    w.rows = __builtin_amdgcn_readfirstlane(r[2]);
    w.chunk = __builtin_amdgcn_readfirstlane(r[3]);
    const int pos = __builtin_amdgcn_readfirstlane(r[4]);
    const int m = __builtin_amdgcn_readfirstlane(r[5]);
    w.m = m;
    w.nt = u - q * nt_per;
    if (q >= n) return false;                   // (the record is then stale and unused)
    if (m > 1) {
        const int v = u - (q - pos) * nt_per;   // unit within the expert's group
        w.nt = v / m;
        r = list + kXtabRec * (q - pos + (v - w.nt * m));
        w.start = __builtin_amdgcn_readfirstlane(r[1]);
        w.rows = __builtin_amdgcn_readfirstlane(r[2]);
        w.chunk = __builtin_amdgcn_readfirstlane(r[3]);
    }
    return true;
}

// The fused path (bf16 activations): the routing launch clears the
// fused_ctl_ints(dm) counters, the permutation launch writes the chunk list
// and the per-XCD chunk table, then launch_fused runs gate/up and down as
// work units of one launch: ticketed (fused_chain_form) or persistent.  Up
// to kFusedMaxPairs pairs.
constexpr int kFusedMaxPairs = MOE_MXFP4_FUSED_MAX_PAIRS;
bool fused_supported(const Dims& dm);
int fused_ctl_ints(const Dims& dm);
// Index of the error word in the counters: nonzero after a call in which a
// device-side wait gave up.
constexpr int kFusedErrorWord = 64;   // ints from the start of the counters
bool fused_chain_form(const Dims& dm);
hipError_t launch_fused(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws,
                        int spin_limit, hipStream_t s);

// Kernel launchers (each returns hipGetLastError() of its launch).
// Router projection: logits [T][E] = x [T][d] . w [E][d]^T (bf16 in, float32 out).
hipError_t launch_router(const uint16_t* x, const uint16_t* w, float* logits, const Dims& dm, hipStream_t s);
// Measurement probes (not on the forward path): kind 0 streaming read of
// `bytes`, kinds 1-3 MFMA issue loops; *work = bytes read or flops done.
hipError_t launch_probe(int kind, const void* src, size_t bytes, int reps, uint32_t* sink, double* work,
                        hipStream_t s);
// DFlash verify acceptance over B sequences (two launches); the workspace
// holds dflash_workspace_bytes(B, V) bytes.
size_t dflash_workspace_bytes(int32_t B, int32_t V);
hipError_t launch_dflash_accept(int32_t B, int32_t G, int32_t V, const int32_t* draft, const float* p_draft,
                                const float* p_target, const float* u, const float* r, int32_t* n_accepted,
                                int32_t* next_token, void* workspace, hipStream_t s);
// Routing (topk_ids, topk_w); with zero != nullptr the launch also clears
// zero[0 .. nzero).
hipError_t launch_route(const float* logits, const Dims& dm, const Workspace& ws, hipStream_t s,
                        int32_t* zero = nullptr, int nzero = 0);
hipError_t launch_sort(const Dims& dm, const Workspace& ws, int chunk_rows, hipStream_t s);
// Small batches: routing and permutation in one launch (when route_sort_fused).
bool route_sort_fused(const Dims& dm);
hipError_t launch_route_sort(const float* logits, const Dims& dm, const Workspace& ws, int chunk_rows,
                             hipStream_t s, int32_t* zero = nullptr, int nzero = 0);
hipError_t launch_quant_x8(const uint16_t* x, const Dims& dm, const Workspace& ws, hipStream_t s);
hipError_t launch_quant_act8(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                             hipStream_t s);
// bf16 activations (verify batches): weights streamed through registers.
hipError_t launch_gateup(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm,
                         const Workspace& ws, hipStream_t s);
hipError_t launch_down(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s);
// MXFP8 activations (dense regime): 128-pair x 256-weight-row tiles, both
// operands staged in LDS, scaled MFMA.
hipError_t launch_gateup_dense(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws,
                               hipStream_t s);
hipError_t launch_down_dense(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws,
                             hipStream_t s);
// o_f16: the per-pair outputs are fp16 codes in ws.o with scales in ws.os
// (dense path), else float32 in ws.o
hipError_t launch_finalize(const Dims& dm, const Workspace& ws, void* out, int out_dtype, bool o_f16,
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
