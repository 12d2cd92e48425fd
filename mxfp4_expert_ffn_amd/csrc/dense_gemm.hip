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
// loads into two step buffers (the loads of step s+1 are issued when step s
// starts): 16 KB of E4M3 rows (16-byte chunks XOR-swizzled by row, so the
// operand reads are free of bank conflicts) and 16 KB of FP4 weight tiles in
// their stored order, which is already the B-operand order of the matrix
// core (lane L: weight row L%16, MX block L/16).  Scales go through LDS once
// per 4 steps: 4 KB of weight scales (the stored dword of a lane holds its 4
// steps; the MFMA's op_sel picks the step's byte) and 2 KB of activation
// scales.  76 KB of LDS per workgroup of 4 wavefronts: two workgroups per CU,
// so one's barrier and load waits overlap the other's MFMAs.
//
// The 4 wavefronts form a 2 x 2 grid; each computes 64 pairs x 128 weight
// rows (4 x 8 MFMA tiles, 32 accumulators).  Sharing both operands through
// LDS halves the L2-to-CU bytes per MFMA against streaming the weights into
// each wave's registers, which is what the verify-batch kernels do.  The
// shape and ring depth are template parameters (Shape<WN, STAGES>); the
// other shapes tried were slower on this GPU.
//
// Gate/up: weight rows 0..127 of a unit are W_gate rows (h columns), 128..255
// the W_up rows of the same columns, and a wave's tiles j and j + kJ/2 meet
// in one lane, so SwiGLU and the MXFP8 re-quantisation of h (each run of 32
// h columns is one MX block) run in the epilogue.  Down: the epilogue stores
// each result row at its pair's own row p = t*k + j as fp16 codes with one
// power-of-two scale per 128 columns (the combine applies the routing
// weights).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kTM = kDenseChunk;            // pair rows per unit
constexpr int kTiles = 16;                  // 16-row weight tiles per unit
constexpr int kMs = 4;                      // 16-row pair sub-tiles per wavefront (64 pairs)
constexpr int kASlot = kTM * kKStep;        // E4M3 rows of one step
constexpr int kBSlot = kTiles * 1024;       // FP4 tiles of one step
constexpr int kBsSlot = kTiles * 256;       // weight scales of 4 steps
constexpr int kAsSlot = kTM * 16;           // activation scales of 4 steps
constexpr int kOStride = 256 * 2 + 16;      // bytes per row of down's bf16 output tile (padded: no bank conflicts)
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
    const int32_t* sorted;       // [P]
    const int32_t* chunks;       // chunk records
    const int32_t* nchunks;
    const int32_t* xtab;         // per-XCD chunk table (xcd_unit)
    int32_t xstride;
    uint8_t* h_out;              // gate/up: [P][f] E4M3
    uint8_t* h_scale_out;        // gate/up: [P][f/32]
    uint16_t* o_out;             // down: [P][d] fp16 codes, row = pair index
    uint8_t* o_scale_out;        // down: [P][d/128] scale exponents + 127 of those codes
    int32_t K, N, n_tiles, k_top, ldo;
};

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
// silu(g) = g * sigmoid(g), with the hardware reciprocal (1 ulp)
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Wait until at most N of this wave's loads are outstanding and its LDS
// reads have returned, then a workgroup barrier (gfx9 s_waitcnt encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// Largest value over the 16 lanes of each DPP row (all 16 get it): quad
// swaps, then the half-row and row mirrors.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float row16_max(float v) {
    v = dpp_max<0xB1>(v);       // quad_perm [1, 0, 3, 2]
    v = dpp_max<0x4E>(v);       // quad_perm [2, 3, 0, 1]
    v = dpp_max<0x141>(v);      // row_half_mirror
    return dpp_max<0x140>(v);   // row_mirror
}

// Tile shape: 2 x WN wavefronts, each 64 pairs x (256 / WN) weight rows;
// STAGES step buffers in the LDS ring (loads issued STAGES - 1 steps ahead).
template <int WN, int STAGES>
struct Shape {
    static constexpr int kW = 2 * WN;                  // wavefronts per workgroup
    static constexpr int kT = kW * kWave;
    static constexpr int kJ = kTiles / WN;             // weight tiles per wavefront
    static constexpr int kQ = kTiles / kW;             // 1 KB loads per wave per step, A and B each
    static constexpr int kLds = STAGES * (kASlot + kBSlot) + 2 * (kBsSlot + kAsSlot);
    static constexpr int kPerCu = kLds <= 80 * 1024 ? 2 : 1;
    static_assert(kLds <= 160 * 1024, "LDS of one CU");
    static_assert(STAGES >= 2 && STAGES <= 5, "the 2-slot scale ring needs STAGES <= 5");
    // loads a wave issues for step j: A and B, plus 2 scale loads at the
    // first step of a 4-step group
    static constexpr int loads_of_step(int j) { return 2 * kQ + (j % 4 == 0 ? 2 : 0); }
    static constexpr int pending(int s4, int n) {
        int c = 0;
        for (int i = 1; i <= n; ++i) c += loads_of_step(s4 + i);
        return c;
    }
};

template <int MODE, int WN, int STAGES>
struct Dense {
    using S = Shape<WN, STAGES>;
    static constexpr int kW = S::kW, kJ = S::kJ, kQ = S::kQ;
    static_assert(MODE != kDown || kTM * kOStride + kTM * 4 <= S::kLds, "down's output tile fits the LDS ring");
    static_assert(MODE != kDown || (WN == 2 && kJ * 16 == 128), "down: 256-column units, 128 columns per wave");

    struct Ctx {
        __amdgpu_buffer_rsrc_t ra, ras, rw, rs;   // activations, their scales, this wave's B matrix + scales
        uint32_t avoff[kQ];                       // A row loads of this lane
        uint32_t asoff;                           // A scale row of this lane
        uint32_t bvs;                             // lane offset of the B-scale load
        int btile0;                               // first weight tile this wave loads
        int ns, ng, wave;
        uint8_t *lA, *lB, *lBs, *lAs;
    };

    // weight-tile slot of the unit that this wave's tile jj uses
    __device__ static int wslot(int wn, int jj) {
        constexpr int h = kJ / 2;
        if constexpr (MODE == kGateUp) return jj < h ? wn * h + jj : 8 + wn * h + (jj - h);
        else return wn * kJ + jj;
    }

    __device__ static void issue_ab(const Ctx& c, int step, int lane) {
        const int slot = step % STAGES;
        uint8_t* dA = c.lA + slot * kASlot;
#pragma unroll
        for (int q = 0; q < kQ; ++q) lds_dma16(c.ra, dA + (q * kW + c.wave) * 1024, c.avoff[q], step * kKStep);
        uint8_t* dB = c.lB + slot * kBSlot + c.wave * kQ * 1024;
#pragma unroll
        for (int i = 0; i < kQ; ++i) lds_dma16(c.rw, dB + i * 1024, lane * 16, ((c.btile0 + i) * c.ns + step) * 1024);
    }

    // B scales: this wave's kQ tiles x 256 B; A scales: 128 / kW rows of 16 B.
    __device__ static void issue_scales(const Ctx& c, int grp, int lane) {
        const int gs = grp & 1;
        if (lane < 16 * kQ)
            lds_dma16(c.rs, c.lBs + gs * kBsSlot + c.wave * kQ * 256, c.bvs, (c.btile0 * c.ng + grp) * 256);
        if (lane < kTM / kW) lds_dma16(c.ras, c.lAs + gs * kAsSlot + c.wave * (kTM / kW) * 16, c.asoff, grp * 16);
    }

    // LDS reads of a step: the operands of the first MFMA (A sub-tile 0 and
    // weight tile 0) first, then the other A sub-tiles, each MFMA waiting
    // only for its own operands (LDS reads return in order).  Gate/up also
    // reads all its weight tiles up front, into registers of their own;
    // down lacks the registers and reads each tile one ahead of its MFMAs.
    // FULL: every sub-tile of the wave holds pairs (otherwise only the first
    // nms are multiplied).
    template <int S4, bool FULL>
    __device__ static void compute(const Ctx& c, f32x4_t (&acc)[kMs][kJ], const uint32_t (&sbw)[kJ], int slot,
                                   int gs, int nms, int wm, int wn, int lane) {
        const int li = lane % 16, g = lane / 16;
        const uint8_t* A = c.lA + slot * kASlot;
        const uint8_t* B = c.lB + slot * kBSlot + lane * 16;
        const uint8_t* As = c.lAs + gs * kAsSlot;
        i32x8_t a[kMs];
        int sa[kMs];
        auto load_a = [&](int ms) {
            const int r = wm * 64 + ms * 16 + li;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(A + r * kKStep + swz(r, g) * 16);
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(A + r * kKStep + swz(r, 4 + g) * 16);
            a[ms] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            sa[ms] = As[r * 16 + S4 * 4 + g];
        };
        load_a(0);
        u32x4_t b = *reinterpret_cast<const u32x4_t*>(B + wslot(wn, 0) * 1024);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ms = 1; ms < kMs; ++ms) load_a(ms);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE == kGateUp) {
            u32x4_t bt[kJ];
            bt[0] = b;
#pragma unroll
            for (int jj = 1; jj < kJ; ++jj) bt[jj] = *reinterpret_cast<const u32x4_t*>(B + wslot(wn, jj) * 1024);
            __builtin_amdgcn_sched_barrier(0);             // keeps the reads ahead of the MFMAs
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj) {
                // FP4 B operand: only the low 4 registers are read
                const i32x8_t bb =
                    __builtin_bit_cast(i32x8_t, __builtin_shufflevector(bt[jj], bt[jj], 0, 1, 2, 3, 0, 1, 2, 3));
#pragma unroll
                for (int ms = 0; ms < kMs; ++ms)
                    if (FULL || ms < nms)
                        acc[ms][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a[ms], bb, acc[ms][jj], 0 /* A: E4M3 */, 4 /* B: E2M1 */, 0, sa[ms], S4, (int)sbw[jj]);
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj) {
                u32x4_t bn = b;
                if (jj + 1 < kJ) bn = *reinterpret_cast<const u32x4_t*>(B + wslot(wn, jj + 1) * 1024);
                const i32x8_t bb = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3));
#pragma unroll
                for (int ms = 0; ms < kMs; ++ms)
                    if (FULL || ms < nms)
                        acc[ms][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a[ms], bb, acc[ms][jj], 0 /* A: E4M3 */, 4 /* B: E2M1 */, 0, sa[ms], S4, (int)sbw[jj]);
                b = bn;
            }
        }
    }

    // Step s (s mod 4 == S4).  The loads of step s were issued STAGES - 1
    // steps earlier; those of the (up to STAGES - 2) steps after it may
    // still be in flight and the issue order is fixed, so a vmcnt wait on
    // their number plus the barrier (every wave's direct-to-LDS writes done)
    // makes step s's buffer valid.  The barrier also means every wave has
    // finished step s-1, whose buffer then takes step s + STAGES - 1.
    template <int S4, bool FULL>
    __device__ static void step(const Ctx& c, f32x4_t (&acc)[kMs][kJ], uint32_t (&sbw)[kJ], int s, int nms,
                                int wm, int wn, int lane) {
        const int ahead = min(STAGES - 2, c.ns - 1 - s);
        if (STAGES >= 4 && ahead >= 2)
            wait_barrier<S::pending(S4, STAGES >= 4 ? 2 : 0)>();
        else if (STAGES >= 3 && ahead >= 1)
            wait_barrier<S::pending(S4, STAGES >= 3 ? 1 : 0)>();
        else
            wait_barrier<0>();
        if (s + STAGES - 1 < c.ns) {
            if ((S4 + STAGES - 1) % 4 == 0) issue_scales(c, (s + STAGES - 1) / 4, lane);
            issue_ab(c, s + STAGES - 1, lane);
        }
        const int gs = (s / 4) & 1;
        if (S4 == 0) {
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj)
                sbw[jj] = *reinterpret_cast<const uint32_t*>(c.lBs + gs * kBsSlot + wslot(wn, jj) * 256 + lane * 4);
        }
        compute<S4, FULL>(c, acc, sbw, s % STAGES, gs, nms, wm, wn, lane);
    }

    template <bool FULL>
    __device__ static void main_loop(const Ctx& c, f32x4_t (&acc)[kMs][kJ], uint32_t (&sbw)[kJ], int nms, int wm,
                                     int wn, int lane) {
        for (int s = 0; s < c.ns; s += 4) {
            step<0, FULL>(c, acc, sbw, s, nms, wm, wn, lane);
            if (s + 1 < c.ns) step<1, FULL>(c, acc, sbw, s + 1, nms, wm, wn, lane);
            if (s + 2 < c.ns) step<2, FULL>(c, acc, sbw, s + 2, nms, wm, wn, lane);
            if (s + 3 < c.ns) step<3, FULL>(c, acc, sbw, s + 3, nms, wm, wn, lane);
        }
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
        c.lB = c.lA + STAGES * kASlot;
        c.lBs = c.lB + STAGES * kBSlot;
        c.lAs = c.lBs + 2 * kBsSlot;
        const uint32_t wbytes = (uint32_t)a.N * (uint32_t)(a.K / 2);
        const uint32_t sbytes = (uint32_t)(a.N / 16) * (uint32_t)c.ng * 256u;
        // the kQ weight tiles this wave loads: one matrix, consecutive tiles
        const int jb = wave * kQ;
        const bool up = MODE == kGateUp && jb >= 8;
        c.btile0 = MODE == kGateUp ? nt * 8 + (jb & 7) : nt * 16 + jb;
        const uint8_t* wm_ptr = up ? a.w1 : a.w0;
        const uint8_t* sm_ptr = up ? a.s1 : a.s0;
        c.rw = __builtin_amdgcn_make_buffer_rsrc((void*)(wm_ptr + (size_t)e * wbytes), 0, wbytes, kRsrcWord3);
        c.rs = __builtin_amdgcn_make_buffer_rsrc((void*)(sm_ptr + (size_t)e * sbytes), 0, sbytes, kRsrcWord3);
        c.ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.act, 0, a.act_rows * (uint32_t)a.K, kRsrcWord3);
        c.ras = __builtin_amdgcn_make_buffer_rsrc((void*)a.act_scale, 0, a.act_rows * (uint32_t)(a.K / kBlock),
                                                  kRsrcWord3);
        c.bvs = (uint32_t)(((lane / 16) % kQ) * c.ng * 256 + (lane % 16) * 16);

        // Source row of unit row r; rows past the chunk's last pair repeat
        // it (their results are computed and never stored).
        auto src_row = [&](int r) -> uint32_t {
            const int idx = min(c0 + r, M - 1);
            return MODE == kGateUp ? (uint32_t)(a.sorted[m0 + idx] / a.k_top) : (uint32_t)(m0 + idx);
        };
        // A load q of this wave fills LDS bytes (q*kW + wave) KB of the step
        // buffer: 8 rows, lane -> row lane/8, physical chunk lane%8, which
        // holds the logical chunk swz() maps there (swz is an involution).
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int r = 8 * (q * kW + wave) + lane / 8;
            c.avoff[q] = src_row(r) * (uint32_t)a.K + (uint32_t)(swz(r, lane % 8) * 16);
        }
        c.asoff = src_row(wave * (kTM / kW) + lane % (kTM / kW)) * (uint32_t)(a.K / kBlock);

        f32x4_t acc[kMs][kJ];
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj) acc[ms][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint32_t sbw[kJ];
        // down: pair indices (output rows) of this lane's rows, loaded
        // before the main loop so that the epilogue does not wait on them
        int32_t pr[kMs][4];
        if constexpr (MODE == kDown) {
#pragma unroll
            for (int ms = 0; ms < kMs; ++ms)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    pr[ms][r] = a.sorted[m0 + min(c0 + wm * 64 + ms * 16 + 4 * g + r, M - 1)];
        }

        // prologue: steps 0 .. STAGES-2, the first group's scales first
        // (sched_barrier keeps the issue order that the vmcnt waits count on)
        issue_scales(c, 0, lane);
#pragma unroll
        for (int j = 0; j < STAGES - 1; ++j) {
            if (j < c.ns) issue_ab(c, j, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nms == kMs)
            main_loop<true>(c, acc, sbw, nms, wm, wn, lane);
        else
            main_loop<false>(c, acc, sbw, nms, wm, wn, lane);

        // Epilogue.  Lane holds D[pair wm*64 + ms*16 + 4g + r][column li] of
        // tile jj.  Down scales each row's 128 columns of this wave by a
        // power of two (their largest magnitude lands in [2^14, 2^15)),
        // rounds them to fp16 into an LDS tile (the operand ring is free once
        // every wave is past the main loop) and then stores whole 512-byte
        // row pieces.
        uint8_t* ostage = smem;                      // [kTM rows][kOStride bytes]
        int32_t* orows = reinterpret_cast<int32_t*>(smem + kTM * kOStride);
        if constexpr (MODE == kDown) __syncthreads();
#pragma unroll
        for (int ms = 0; ms < kMs; ++ms) {
            if (ms >= nms) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = c0 + wm * 64 + ms * 16 + 4 * g + r;
                if constexpr (MODE == kGateUp) {
                    const size_t orow = (size_t)(m0 + idx);
                    // the wave's h columns: kJ/2 tiles of 16, MX blocks of 2 tiles
                    constexpr int h = kJ / 2;
                    const int col0 = nt * 128 + wn * h * 16;
#pragma unroll
                    for (int bk = 0; bk < h / 2; ++bk) {
                        const float h0 = silu(acc[ms][2 * bk][r]) * acc[ms][2 * bk + h][r];
                        const float h1 = silu(acc[ms][2 * bk + 1][r]) * acc[ms][2 * bk + 1 + h][r];
                        float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
                        for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
                        const int se = mx_scale_exp(amax, 8);
                        if (idx < M) {
                            uint8_t* hr = a.h_out + orow * a.ldo + col0 + bk * 32 + li;
                            hr[0] = (uint8_t)e4m3_code(ldexpf(h0, -se));
                            hr[16] = (uint8_t)e4m3_code(ldexpf(h1, -se));
                            if (li == 0)
                                a.h_scale_out[orow * (a.ldo / kBlock) + col0 / kBlock + bk] = (uint8_t)(se + 127);
                        }
                    }
                } else {
                    const int lr = wm * 64 + ms * 16 + 4 * g + r;
                    float m = 0.f;
#pragma unroll
                    for (int jj = 0; jj < kJ; ++jj) m = fmaxf(m, fabsf(acc[ms][jj][r]));
                    m = row16_max(m);
                    // m >= 0: its biased exponent field is floor(log2 m) + 127
                    // (0 for zero and subnormals, which the clamp covers)
                    const int se = max((int)(__float_as_uint(m) >> 23) - 127 - 14, -127);
                    const float inv = __uint_as_float((uint32_t)(127 - se) << 23);   // 2^-se, se <= 113
                    uint8_t* srow = ostage + lr * kOStride + (wn * kJ * 16 + li) * 2;
#pragma unroll
                    for (int jj = 0; jj < kJ; ++jj)
                        *reinterpret_cast<_Float16*>(srow + jj * 32) = (_Float16)(acc[ms][jj][r] * inv);
                    if (li == 0) {
                        if (wn == 0) orows[lr] = pr[ms][r];
                        if (idx < M) a.o_scale_out[(size_t)pr[ms][r] * (a.ldo / 128) + nt * 2 + wn] = (uint8_t)(se + 127);
                    }
                }
            }
        }
        if constexpr (MODE == kDown) {
            __syncthreads();
            // 32 lanes x 16 bytes per row; kT / 32 rows per pass
            constexpr int kRowsPerPass = S::kT / 32;
            const int piece = tid % 32;
            for (int row = tid / 32; row < rows; row += kRowsPerPass) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ostage + row * kOStride + piece * 16);
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(a.o_out + (size_t)orows[row] * a.ldo +
                                                                          nt * 256 + piece * 8));
            }
        }
    }
};

template <int MODE, int WN, int STAGES>
__global__ __launch_bounds__((Shape<WN, STAGES>::kT), (Shape<WN, STAGES>::kPerCu)) void k_dense(DenseArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Shape<WN, STAGES>::kLds];
    // Work unit = (chunk, column tile) of the per-XCD chunk table: workgroup
    // g runs on XCD g mod kXcds (the GPU's round-robin) and takes unit
    // g / kXcds of that XCD's list, where each expert's 4-5 chunks run
    // column tile by column tile (xcd_unit), so they share the weight tile,
    // and its chunks their activation rows, through one L2.  Uniform values
    // go to scalar registers so that the buffer descriptors built from them
    // are scalar.
    XcdUnit w;
    if (!xcd_unit(a.xtab, a.xstride, blockIdx.x % kXcds, blockIdx.x / kXcds, a.n_tiles, w)) return;
    const int e = w.e, start = w.start, rows = w.rows, nt = w.nt;
    // run() takes (first sorted position m0, chunk offset c0, pairs M) with
    // the chunk's pairs at m0 + c0 .. m0 + M - 1
    Dense<MODE, WN, STAGES>::run(a, smem, e, nt, start, 0, rows);
}

// Upper bound of the chunk list at kDenseChunk pairs per chunk.
int max_dense_chunks(const Dims& dm) {
    const int active = dm.E < dm.P ? dm.E : dm.P;
    return active + dm.P / kDenseChunk;
}

// 2 x 2 wavefronts, two step buffers: the fastest shape measured (2 x 4
// wavefronts and 3- or 4-deep rings leave one workgroup per CU).
template <int MODE>
hipError_t launch(DenseArgs a, const Dims& dm, hipStream_t s) {
    constexpr int WN = 2, ST = 2;
    a.xstride = xcd_slots(dm);
    // slots an XCD's list can fill at kDenseChunk pairs per chunk (the
    // greedy bound: an eighth of the chunks plus one expert's)
    const int T = dm.T < dm.P ? dm.T : dm.P;
    const int slots = (max_dense_chunks(dm) + kXcds - 1) / kXcds + (T + kDenseChunk - 1) / kDenseChunk;
    hipLaunchKernelGGL((k_dense<MODE, WN, ST>), dim3(kXcds * slots * a.n_tiles), dim3(Shape<WN, ST>::kT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_dense(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    DenseArgs a{};
    a.act = ws.xq; a.act_scale = ws.xs; a.act_rows = (uint32_t)dm.T;
    a.w0 = w.w_gate; a.s0 = w.w_gate_scale;
    a.w1 = w.w_up;   a.s1 = w.w_up_scale;
    a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks; a.xtab = ws.xtab;
    a.h_out = ws.h; a.h_scale_out = ws.hs; a.o_out = nullptr;
    a.K = dm.d; a.N = dm.f; a.n_tiles = dm.f / 128; a.k_top = dm.k; a.ldo = dm.f;
    return launch<kGateUp>(a, dm, s);
}

hipError_t launch_down_dense(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    DenseArgs a{};
    a.act = ws.h; a.act_scale = ws.hs; a.act_rows = (uint32_t)dm.P;
    a.w0 = w.w_down; a.s0 = w.w_down_scale;
    a.w1 = nullptr;  a.s1 = nullptr;
    a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks; a.xtab = ws.xtab;
    a.h_out = nullptr; a.h_scale_out = nullptr;
    a.o_out = reinterpret_cast<uint16_t*>(ws.o); a.o_scale_out = ws.os;
    a.K = dm.f; a.N = dm.d; a.n_tiles = dm.d / 256; a.k_top = dm.k; a.ldo = dm.d;
    return launch<kDown>(a, dm, s);
}

}  // namespace moe
