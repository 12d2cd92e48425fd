// Expert projections in the dense regime: MXFP8 activations (E4M3 codes,
// one E8M0 scale per 32) times MXFP4 weights on the gfx950 scaled matrix
// cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// With thousands of tokens per call every expert sees hundreds of token
// pairs, so each weight byte feeds hundreds of multiply-adds and the
// projections are bound by matrix-core throughput, not by the weight bytes
// that bound the small verify batches.  The MX formats are the pages' (block
// of 32 sharing a power-of-two scale: ai.appwright.xyz "投機的デコード",
// section "第1層：FP4量子化（モデル側）"; techllm.github.io "Xiaomi MiMo x
// TileRT", section "1. MXFP4 — MoE에만 걸린 양자화"), and the next tile is
// loaded while the current one computes (dothoosh.com article, section
// "TileRT: عصر فشار بر GPU").
//
// Work unit = (chunk of <= 128 pairs of one expert, 256 weight rows).  Both
// operands of a 128-wide K step go through LDS by direct-to-LDS buffer
// loads, double buffered: 16 KB of E4M3 rows (16-byte chunks XOR-swizzled
// by row, so the operand reads are free of bank conflicts) and 16 KB of FP4
// weight tiles in their stored order, which is already the B-operand order
// of the matrix core (lane L: weight row L%16, MX block L/16).  Scales go
// through LDS once per 4 steps: 4 KB of weight scales (the stored dword of a
// lane holds its 4 steps; the MFMA's op_sel picks the step's byte) and 2 KB
// of activation scales.
//
// Four wavefronts in a 2 x 2 grid; each computes 64 pairs x 128 weight rows
// (4 x 8 MFMA tiles, 32 accumulators).  Sharing both operands through LDS
// halves the L2-to-CU bytes per MFMA against streaming the weights into each
// wave's registers, which is what the verify-batch kernels do.
//
// Gate/up: weight rows 0..127 of a unit are W_gate rows (h columns), 128..255
// the W_up rows of the same columns, and a wave's tiles j and j + 4 meet in
// one lane, so SwiGLU and the MXFP8 re-quantisation of h (a wave row's 32
// columns x 2 are two MX blocks) run in the epilogue.  Down: the epilogue
// multiplies by the pair's routing weight and stores float32 per pair.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kW = 4;                       // wavefronts per workgroup
constexpr int kT = kW * kWave;
constexpr int kTM = kDenseChunk;            // pair rows per unit
constexpr int kTiles = 16;                  // 16-row weight tiles per unit
constexpr int kJ = 8;                       // weight tiles per wavefront
constexpr int kMs = 4;                      // 16-row pair sub-tiles per wavefront
constexpr int kASlot = kTM * kKStep;        // E4M3 rows of one step
constexpr int kBSlot = kTiles * 1024;       // FP4 tiles of one step
constexpr int kBsSlot = kTiles * 256;       // weight scales of 4 steps
constexpr int kAsSlot = kTM * 16;           // activation scales of 4 steps
constexpr int kLds = 2 * (kASlot + kBSlot + kBsSlot + kAsSlot);
constexpr int kRsrcWord3 = 0x00020000;      // gfx9 raw buffer descriptor, dword 3

enum { kGateUp = 0, kDown = 1 };

struct DenseArgs {
    const uint8_t* act;          // gate/up: x codes [T][K]; down: h codes [P][K] (sorted rows)
    const uint8_t* act_scale;    // [rows][K/32]
    uint32_t act_rows;
    const uint8_t* w0;           // gate / down, tiled
    const uint8_t* s0;
    const uint8_t* w1;           // up (gate/up only)
    const uint8_t* s1;
    const int32_t* offsets;      // [E+1]
    const int32_t* sorted;       // [P]
    const int32_t* chunks;       // chunk records
    const int32_t* nchunks;
    const float* topk_w;         // [P]
    uint8_t* h_out;              // gate/up: [P][f] E4M3
    uint8_t* h_scale_out;        // gate/up: [P][f/32]
    float* o_out;                // down: [P][d]
    int32_t K, N, n_tiles, k_top, ldo;
};

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Wait for all of this wave's outstanding loads and LDS reads, then a
// workgroup barrier (gfx9 s_waitcnt: vmcnt 0, expcnt 7, lgkmcnt 0).
__device__ __forceinline__ void drain_barrier() {
    __builtin_amdgcn_s_waitcnt(7 << 4);
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

template <int MODE>
struct Dense {
    struct Ctx {
        __amdgpu_buffer_rsrc_t ra, ras, rw, rs;   // activations, their scales, this wave's B matrix + scales
        uint32_t avoff[4];                        // A row loads of this lane
        uint32_t asoff;                           // A scale row of this lane (waves 0, 1)
        uint32_t bvs;                             // lane offset of the B-scale load
        int btile0;                               // first weight tile this wave loads
        int ns, ng, wave;
        uint8_t *lA, *lB, *lBs, *lAs;
    };

    // weight-tile slot of the unit that this wave's tile jj uses
    __device__ static int wslot(int wn, int jj) {
        if constexpr (MODE == kGateUp) return jj < 4 ? wn * 4 + jj : 8 + wn * 4 + (jj - 4);
        else return wn * 8 + jj;
    }

    __device__ static void issue_ab(const Ctx& c, int step, int slot, int lane) {
        uint8_t* dA = c.lA + slot * kASlot;
#pragma unroll
        for (int q = 0; q < 4; ++q) lds_dma16(c.ra, dA + (q * kW + c.wave) * 1024, c.avoff[q], step * kKStep);
        uint8_t* dB = c.lB + slot * kBSlot + c.wave * 4 * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16(c.rw, dB + i * 1024, lane * 16, ((c.btile0 + i) * c.ns + step) * 1024);
    }

    __device__ static void issue_scales(const Ctx& c, int grp, int gs) {
        lds_dma16(c.rs, c.lBs + gs * kBsSlot + c.wave * 4 * 256, c.bvs, (c.btile0 * c.ng + grp) * 256);
        if (c.wave < 2) lds_dma16(c.ras, c.lAs + gs * kAsSlot + c.wave * 1024, c.asoff, grp * 16);
    }

    template <int S4>
    __device__ static void compute(const Ctx& c, f32x4_t (&acc)[kMs][kJ], const uint32_t (&sbw)[kJ], int slot,
                                   int gs, int nms, int wm, int wn, int lane) {
        const int li = lane % 16, g = lane / 16;
        const uint8_t* A = c.lA + slot * kASlot;
        const uint8_t* B = c.lB + slot * kBSlot;
        const uint8_t* As = c.lAs + gs * kAsSlot;
        u32x4_t b[kJ];
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj) b[jj] = *reinterpret_cast<const u32x4_t*>(B + wslot(wn, jj) * 1024 + lane * 16);
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms) {
            if (ms < nms) {
                const int r = wm * 64 + ms * 16 + li;
                const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(A + r * kKStep + swz(r, g) * 16);
                const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(A + r * kKStep + swz(r, 4 + g) * 16);
                const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                const int sa = As[r * 16 + S4 * 4 + g];
#pragma unroll
                for (int jj = 0; jj < kJ; ++jj) {
                    // FP4 B operand: only the low 4 registers are read
                    const i32x8_t bb = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(b[jj], b[jj], 0, 1, 2, 3, 0, 1, 2, 3));
                    acc[ms][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, bb, acc[ms][jj], 0 /* A: E4M3 */, 4 /* B: E2M1 */, 0, sa, S4, (int)sbw[jj]);
                }
            }
        }
    }

    // Step s (s mod 4 == S4): its loads have landed once every wave drains
    // and meets at the barrier; the next step's loads then go to the other
    // buffer, which every wave finished reading before the barrier.
    template <int S4>
    __device__ static void step(const Ctx& c, f32x4_t (&acc)[kMs][kJ], uint32_t (&sbw)[kJ], int s, int nms,
                                int wm, int wn, int lane) {
        drain_barrier();
        if (s + 1 < c.ns) {
            if (S4 == 3) issue_scales(c, (s + 1) / 4, ((s + 1) / 4) & 1);
            issue_ab(c, s + 1, (s + 1) & 1, lane);
        }
        const int gs = (s / 4) & 1;
        if (S4 == 0) {
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj)
                sbw[jj] = *reinterpret_cast<const uint32_t*>(c.lBs + gs * kBsSlot + wslot(wn, jj) * 256 + lane * 4);
        }
        compute<S4>(c, acc, sbw, s & 1, gs, nms, wm, wn, lane);
    }

    __device__ static void run(const DenseArgs& a, uint8_t* smem, int e, int nt, int m0, int c0, int M) {
        const int tid = threadIdx.x, lane = tid % kWave;
        const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
        const int wm = wave & 1, wn = wave >> 1;
        const int li = lane % 16, g = lane / 16;
        const int rows = min(kTM, M - c0);
        const int nms = __builtin_amdgcn_readfirstlane(max(0, min(kMs, (rows - wm * 64 + 15) / 16)));

        Ctx c;
        c.ns = a.K / kKStep;
        c.ng = (c.ns + 3) / 4;
        c.wave = wave;
        c.lA = smem;
        c.lB = c.lA + 2 * kASlot;
        c.lBs = c.lB + 2 * kBSlot;
        c.lAs = c.lBs + 2 * kBsSlot;
        const uint32_t wbytes = (uint32_t)a.N * (uint32_t)(a.K / 2);
        const uint32_t sbytes = (uint32_t)(a.N / 16) * (uint32_t)c.ng * 256u;
        // the 4 weight tiles this wave loads: one matrix, consecutive tiles
        const int jb = wave * 4;
        const bool up = MODE == kGateUp && jb >= 8;
        c.btile0 = MODE == kGateUp ? nt * 8 + (jb & 7) : nt * 16 + jb;
        const uint8_t* wm_ptr = up ? a.w1 : a.w0;
        const uint8_t* sm_ptr = up ? a.s1 : a.s0;
        c.rw = __builtin_amdgcn_make_buffer_rsrc((void*)(wm_ptr + (size_t)e * wbytes), 0, wbytes, kRsrcWord3);
        c.rs = __builtin_amdgcn_make_buffer_rsrc((void*)(sm_ptr + (size_t)e * sbytes), 0, sbytes, kRsrcWord3);
        c.ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.act, 0, a.act_rows * (uint32_t)a.K, kRsrcWord3);
        c.ras = __builtin_amdgcn_make_buffer_rsrc((void*)a.act_scale, 0, a.act_rows * (uint32_t)(a.K / kBlock),
                                                  kRsrcWord3);
        c.bvs = (uint32_t)((lane / 16) * c.ng * 256 + (lane % 16) * 16);

        // Source row of unit row r; rows past the chunk's last pair repeat
        // it (their results are computed and never stored).
        auto src_row = [&](int r) -> uint32_t {
            const int idx = min(c0 + r, M - 1);
            return MODE == kGateUp ? (uint32_t)(a.sorted[m0 + idx] / a.k_top) : (uint32_t)(m0 + idx);
        };
        // A load q of this wave fills LDS bytes (q*4 + wave) KB of the step
        // buffer: 8 rows, lane -> row lane/8, physical chunk lane%8, which
        // holds the logical chunk swz() maps there (swz is an involution).
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 8 * (q * kW + wave) + lane / 8;
            c.avoff[q] = src_row(r) * (uint32_t)a.K + (uint32_t)(swz(r, lane % 8) * 16);
        }
        c.asoff = wave < 2 ? src_row(wave * 64 + lane) * (uint32_t)(a.K / kBlock) : 0u;

        f32x4_t acc[kMs][kJ];
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj) acc[ms][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint32_t sbw[kJ];

        issue_scales(c, 0, 0);
        issue_ab(c, 0, 0, lane);
        for (int s = 0; s < c.ns; s += 4) {
            step<0>(c, acc, sbw, s, nms, wm, wn, lane);
            if (s + 1 < c.ns) step<1>(c, acc, sbw, s + 1, nms, wm, wn, lane);
            if (s + 2 < c.ns) step<2>(c, acc, sbw, s + 2, nms, wm, wn, lane);
            if (s + 3 < c.ns) step<3>(c, acc, sbw, s + 3, nms, wm, wn, lane);
        }

        // Epilogue.  Lane holds D[pair wm*64 + ms*16 + 4g + r][column li] of
        // tile jj.
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms) {
            if (ms >= nms) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = c0 + wm * 64 + ms * 16 + 4 * g + r;
                const size_t orow = (size_t)(m0 + idx);
                if constexpr (MODE == kGateUp) {
                    const int col0 = nt * 128 + wn * 64;          // h columns of this wave
                    float h[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) h[jj] = silu(acc[ms][jj][r]) * acc[ms][jj + 4][r];
                    float am0 = fmaxf(fabsf(h[0]), fabsf(h[1]));
                    float am1 = fmaxf(fabsf(h[2]), fabsf(h[3]));
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) {
                        am0 = fmaxf(am0, __shfl_xor(am0, off));
                        am1 = fmaxf(am1, __shfl_xor(am1, off));
                    }
                    const int se0 = mx_scale_exp(am0, 8), se1 = mx_scale_exp(am1, 8);
                    if (idx < M) {
                        uint8_t* hr = a.h_out + orow * a.ldo + col0 + li;
                        hr[0] = (uint8_t)e4m3_code(ldexpf(h[0], -se0));
                        hr[16] = (uint8_t)e4m3_code(ldexpf(h[1], -se0));
                        hr[32] = (uint8_t)e4m3_code(ldexpf(h[2], -se1));
                        hr[48] = (uint8_t)e4m3_code(ldexpf(h[3], -se1));
                        if (li < 2)
                            a.h_scale_out[orow * (a.ldo / kBlock) + col0 / kBlock + li] =
                                (uint8_t)((li == 0 ? se0 : se1) + 127);
                    }
                } else {
                    if (idx < M) {
                        const float wgt = a.topk_w[a.sorted[m0 + idx]];
                        float* orow_p = a.o_out + orow * a.ldo + nt * 256 + wn * 128 + li;
#pragma unroll
                        for (int jj = 0; jj < kJ; ++jj) orow_p[jj * 16] = wgt * acc[ms][jj][r];
                    }
                }
            }
        }
    }
};

template <int MODE>
__global__ __launch_bounds__(kT, 2) void k_dense(DenseArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
    // Work unit = (chunk, column tile), chunk-major; chunks are listed
    // expert by expert, hottest first.  Uniform values go to scalar
    // registers so that the buffer descriptors built from them are scalar.
    const int unit = blockIdx.x;
    const int chunk = unit / a.n_tiles;
    const int nt = unit % a.n_tiles;
    if (chunk >= __builtin_amdgcn_readfirstlane(*a.nchunks)) return;
    const int* rec = a.chunks + kChunkRec * chunk;
    const int e = __builtin_amdgcn_readfirstlane(rec[0]);
    const int c0 = __builtin_amdgcn_readfirstlane(rec[1]);
    const int m0 = __builtin_amdgcn_readfirstlane(a.offsets[e]);
    const int M = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - m0;
    Dense<MODE>::run(a, smem, e, nt, m0, c0, M);
}

// Upper bound of the chunk list at kDenseChunk pairs per chunk.
int max_dense_chunks(const Dims& dm) {
    const int active = dm.E < dm.P ? dm.E : dm.P;
    return active + dm.P / kDenseChunk;
}

template <int MODE>
hipError_t launch(const DenseArgs& a, int units, hipStream_t s) {
    hipLaunchKernelGGL(k_dense<MODE>, dim3(units), dim3(kT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_dense(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    DenseArgs a{};
    a.act = ws.xq; a.act_scale = ws.xs; a.act_rows = (uint32_t)dm.T;
    a.w0 = w.w_gate; a.s0 = w.w_gate_scale;
    a.w1 = w.w_up;   a.s1 = w.w_up_scale;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.topk_w = ws.topk_w;
    a.h_out = ws.h; a.h_scale_out = ws.hs; a.o_out = nullptr;
    a.K = dm.d; a.N = dm.f; a.n_tiles = dm.f / 128; a.k_top = dm.k; a.ldo = dm.f;
    return launch<kGateUp>(a, max_dense_chunks(dm) * a.n_tiles, s);
}

hipError_t launch_down_dense(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    DenseArgs a{};
    a.act = ws.h; a.act_scale = ws.hs; a.act_rows = (uint32_t)dm.P;
    a.w0 = w.w_down; a.s0 = w.w_down_scale;
    a.w1 = nullptr;  a.s1 = nullptr;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.topk_w = ws.topk_w;
    a.h_out = nullptr; a.h_scale_out = nullptr; a.o_out = ws.o;
    a.K = dm.f; a.N = dm.d; a.n_tiles = dm.d / 256; a.k_top = dm.k; a.ldo = dm.d;
    return launch<kDown>(a, max_dense_chunks(dm) * a.n_tiles, s);
}

}  // namespace moe
