// Expert projections: packed MXFP4 weights streamed from HBM and multiplied
// on the matrix cores.
//
// The pages' point is that decoding a huge MoE is bound by the bytes of
// expert weights it must stream, which FP4 on the experts cuts
// (ai.appwright.xyz "投機的デコード", section "第1層：FP4量子化（モデル側）";
// techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 — MoE에만 걸린
// 양자화"), and that the next tile should stream in while the current one
// computes (dothoosh.com article, section "TileRT: عصر فشار بر GPU").  So
// every kernel here is one pipelined pass over the weights of the experts a
// batch touches:
//
//   work unit = (chunk of <= 64 token pairs of one expert, tile of output
//   columns).  The permutation kernel lists the chunks; chunks of a hot
//   expert run as separate workgroups at the same time, so they share its
//   weights through the caches instead of one workgroup re-streaming them.
//
//   workgroup = 4 wavefronts, each owning RT tiles of 16 weight rows.  A
//   lane owns one weight row of each tile and, per 128-wide K step, one
//   16-byte MX block of it (lane group g = lane / 16 takes block 4s + g).
//   The weights are stored tiled (see the header), so that is one
//   contiguous 1 KB buffer load per tile and step, plus one contiguous
//   256-byte load of the dword of scales that covers the lane's 4 steps.
//   Weights run D steps ahead in a register ring; activations run D - 1
//   steps ahead in an LDS ring filled by direct-to-LDS loads (no register
//   staging), in a layout whose 16-byte chunks are XOR-swizzled by row so
//   that the matrix-core operand reads are free of bank conflicts.
//
//   bf16 activations: the 32 nibbles of a block feed four
//   v_mfma_f32_16x16x32_bf16 steps; the hardware scaled convert turns 8
//   nibbles and the block's E8M0 scale into the 8 bf16 of the B operand
//   (exact).  The reduction index only has to agree between A and B, so the
//   A operand is read in the same block order.
//
//   MXFP8 activations: one v_mfma_scale_f32_16x16x128_f8f6f4 per step takes
//   the tiled 1 KB of FP4 weights as its B operand unchanged (lane L: row
//   L%16, MX block L/16, low nibble first) with the block scales as E8M0
//   operands, and E4M3 activations as A (lane: row, bytes k 16g..16g+15 and
//   64+16g..64+16g+15 of the step), with their block scales.
//
//   Gate/up: tiles 0..RT/2-1 come from W_gate and RT/2.. from W_up, so the
//   gate and up accumulators of a (token, column) sit in the same lane and
//   SwiGLU h = silu(g) * u runs in the epilogue; h is stored in bf16 (or
//   re-quantised to MXFP8 along d_ff, a wave's 32 columns being exactly one
//   block), rows in expert-sorted order.  Down: A = those h rows; the
//   epilogue multiplies by the pair's routing weight and stores float32 per
//   pair (combined later in a fixed order, so the result is deterministic).
//
// Memory ordering is explicit: the loads of a step are always issued in the
// same order (activations, then weights) and pinned there, so a fixed vmcnt
// wait before each step's barrier guarantees that the step's data has
// landed, and the barrier makes every wave's direct-to-LDS writes visible.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxMs = kChunk / 16;            // token sub-tiles of 16 per chunk
constexpr int kRsrcWord3 = 0x00020000;         // gfx9 raw buffer descriptor, dword 3

enum { kGateUp = 0, kDown = 1 };
enum { kBf16 = 0, kMx8 = 1 };

// Bytes of one activation row per K step, and of one LDS ring slot.
constexpr int row_bytes(int act) { return act == kBf16 ? kKStep * 2 : kKStep; }
constexpr int slot_bytes(int act) { return kMaxMs * 16 * row_bytes(act); }
// Row stride (bytes) of the per-chunk activation-scale table in LDS: one
// byte per MX block, padded to an odd number of dwords against bank conflicts.
constexpr int xs_stride(int K) { return K / kBlock + 4; }

struct GemmArgs {
    const uint8_t* act;         // gate/up: x [T][K]; down: h [P][K] (sorted rows); bf16 or E4M3
    const uint8_t* act_scale;   // MXFP8: [rows][K/32] E8M0 scales of `act`
    const uint8_t* w0;          // gate / down tiled packed
    const uint8_t* s0;
    const uint8_t* w1;          // up tiled packed (gate/up only)
    const uint8_t* s1;
    const int32_t* offsets;     // [E+1]
    const int32_t* sorted;      // [P]
    const int32_t* chunks;      // [n][2]: (expert, first pair of the chunk within the expert)
    const int32_t* nchunks;     // device count of chunks
    const float* topk_w;        // [P]
    uint8_t* h_out;             // gate/up: h [P][f] (bf16 or E4M3 codes)
    uint8_t* h_scale_out;       // gate/up MXFP8: [P][f/32]
    float* o_out;               // down: [P][d]
    int32_t K;                  // reduction length
    int32_t N;                  // rows per weight matrix
    int32_t n_tiles;            // column tiles per expert
    int32_t k_top;
    int32_t ldo;                // output row length (elements)
};

// silu(g) = g * sigmoid(g), with the hardware reciprocal (1 ulp)
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS reads have returned, then a workgroup barrier
// (gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void step_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ void pin() { __builtin_amdgcn_sched_barrier(0); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

template <int MODE, int ACT, int RT, int MS, int D>
struct Pipe {
    static constexpr int kHalf = MODE == kGateUp ? RT / 2 : RT;
    static constexpr int kColsPerWave = kHalf * 16;
    static constexpr int kRow = row_bytes(ACT);           // activation bytes per row and step
    static constexpr int kSlot = slot_bytes(ACT);
    static constexpr int kChunksPerRow = kRow / 16;       // 16 (bf16) or 8 (E4M3)
    static constexpr int kRowsPerKb = 1024 / kRow;        // rows one direct-to-LDS load fills
    // direct-to-LDS loads per wave per step: MS*16 rows over 4 waves
    static constexpr int kNx = MS * 16 / (kRowsPerKb * kWaves);
    static_assert(kNx * kRowsPerKb * kWaves == MS * 16, "MXFP8 chunks use an even number of sub-tiles");

    // weight loads of step j: one 16-byte block and one scale dword per tile
    // (the dword holds the scales of 4 steps; each step reads its own copy so
    // that no register is carried across loop iterations)
    static constexpr int nw(int j) { return (void)j, 2 * RT; }

    // Issue schedule over n steps (X = activations to LDS, W = weights):
    //   prologue: W0, [X0 W1], [X1 W2], ..., [X(D-2) W(D-1)]
    //   step s:   wait + barrier, X(s+D-1) if < n, compute s, W(s+D) if < n
    // Loads that follow X(s) in that order when step s waits, given the
    // steps remaining after it (R = n - 1 - s) and s mod 4 (n is a multiple
    // of 4 or equal to D, so only s mod 4 matters).
    static constexpr int after_x(int R, int s4) {
        int cnt = R >= 1 ? nw(s4 + 1) : 0;                  // W(s+1)
        for (int j = 1; j <= D - 2 && j <= R; ++j)          // groups [X(s+j) W(s+j+1)]
            cnt += kNx + (j + 1 <= R ? nw(s4 + j + 1) : 0);
        return cnt;
    }

    // Physical 16-byte chunk of logical chunk c in LDS row r.
    __device__ static int swz(int r, int c) {
        return ACT == kBf16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
    }

    struct Ctx {
        __amdgpu_buffer_rsrc_t rw[2], rs[2];
        int32_t lane16, lane4;            // lane offsets within a 1 KB tile step / 256 B scale group
        int32_t tile0;                    // first 16-row tile of this wave (per matrix)
        int32_t ns, ng;                   // K steps, scale groups
        const uint8_t* xbase;             // activation rows (bytes)
        uint32_t xoff[kNx > 0 ? kNx : 1]; // this lane's direct-to-LDS source offsets
        uint8_t* lds;                     // activation ring
        const uint8_t* xs;                // MXFP8: per-chunk activation scale table in LDS
        int wave;
    };

    __device__ static void issue_w(const Ctx& c, u32x4_t (&w)[RT], uint32_t (&sg)[RT], int step) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int mat = (MODE == kGateUp && rt >= kHalf) ? 1 : 0;
            const int tile = c.tile0 + rt % kHalf;
            w[rt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    c.rw[mat], c.lane16, (tile * c.ns + step) * 1024, 0));
            sg[rt] = __builtin_amdgcn_raw_buffer_load_b32(c.rs[mat], c.lane4, (tile * c.ng + step / 4) * 256, 0);
        }
    }

    __device__ static void issue_x(const Ctx& c, int slot, int step) {
#pragma unroll
        for (int q = 0; q < kNx; ++q)
            __builtin_amdgcn_global_load_lds(
                c.xbase + c.xoff[q] + step * kRow,
                (lds_void*)(c.lds + slot * kSlot + (q * kWaves + c.wave) * 1024), 16, 0, 0);
    }

    template <int S4>
    __device__ static void compute(f32x4_t (&acc)[MS][RT], const u32x4_t (&w)[RT], const uint32_t (&sg)[RT],
                                   const uint8_t* xs, int li, int g, int step, const Ctx& c) {
        if constexpr (ACT == kBf16) {
            float sc[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sc[rt] = e8m0_as_scale((sg[rt] >> (8 * S4)) & 0xFFu);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x8_t b[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) b[rt] = decode8_bf16(w[rt][i], sc[rt]);
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const int r = ms * 16 + li;
                    const bf16x8_t a =
                        *reinterpret_cast<const bf16x8_t*>(xs + r * kRow + swz(r, 4 * g + i) * 16);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[ms][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[rt], acc[ms][rt], 0, 0, 0);
                }
            }
        } else {
            uint32_t sb[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sb[rt] = (sg[rt] >> (8 * S4)) & 0xFFu;
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const int r = ms * 16 + li;
                const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(xs + r * kRow + swz(r, g) * 16);
                const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(xs + r * kRow + swz(r, 4 + g) * 16);
                const i32x8_t a = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                const int sa = c.xs[r * xs_stride(c.ns * kKStep) + 4 * step + g];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    // FP4 B operand: only the low 4 registers are read
                    const i32x8_t b = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(w[rt], w[rt], 0, 1, 2, 3, 0, 1, 2, 3));
                    acc[ms][rt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, b, acc[ms][rt], 0 /* A: E4M3 */, 4 /* B: E2M1 */, 0, sa, 0, (int)sb[rt]);
                }
            }
        }
    }

    // One step using ring slot SLOT (== s mod D; s mod 4 == S4).  R < 0:
    // steady state (every load of the schedule issued); R >= 0: one of the
    // last D steps, R steps after it.
    template <int SLOT, int S4, int R>
    __device__ static void step(const Ctx& c, f32x4_t (&acc)[MS][RT], u32x4_t (&w)[RT], uint32_t (&sg)[RT],
                                int s, int li, int g) {
        if (R < 0)
            step_barrier<after_x(D, S4)>();
        else
            step_barrier<after_x(R, S4)>();
        pin();
        if (R < 0 || R >= D - 1) issue_x(c, (SLOT + D - 1) % D, s + D - 1);
        pin();
        compute<S4>(acc, w, sg, c.lds + SLOT * kSlot, li, g, s, c);
        pin();
        if (R < 0) issue_w(c, w, sg, s + D);
        pin();
    }

    __device__ static void run(const GemmArgs& a, uint8_t* lds, uint8_t* lds_xs, int e, int nt, int m0,
                               int c0, int M) {
        const int tid = threadIdx.x, lane = tid % kWave;
        const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
        const int li = lane % 16, g = lane / 16;
        const int col0 = nt * (kWaves * kColsPerWave) + wave * kColsPerWave;

        Ctx c;
        c.ns = a.K / kKStep;
        c.ng = (c.ns + 3) / 4;
        const int wbytes = a.N * (a.K / 2);                 // one expert matrix
        const int sbytes = (a.N / 16) * c.ng * 256;         // its tiled scales
        const size_t ew = (size_t)e * wbytes, es = (size_t)e * sbytes;
        c.rw[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.w0 + ew), 0, wbytes, kRsrcWord3);
        c.rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.s0 + es), 0, sbytes, kRsrcWord3);
        if (MODE == kGateUp) {
            c.rw[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.w1 + ew), 0, wbytes, kRsrcWord3);
            c.rs[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.s1 + es), 0, sbytes, kRsrcWord3);
        } else {
            c.rw[1] = c.rw[0];
            c.rs[1] = c.rs[0];
        }
        c.lane16 = lane * 16;
        c.lane4 = lane * 4;
        c.tile0 = col0 / 16;
        c.xbase = a.act;
        c.lds = lds;
        c.xs = lds_xs;
        c.wave = wave;
        // Source row of chunk row r: rows past the chunk's last pair repeat
        // it; their results are computed and never stored.
        auto src_row = [&](int r) {
            const int idx = min(c0 + r, M - 1);
            return MODE == kGateUp ? a.sorted[m0 + idx] / a.k_top : m0 + idx;
        };
        // Direct-to-LDS load q of this wave fills the 1 KB at slot offset
        // (q * 4 + wave) KB: rows kRowsPerKb * (q * 4 + wave) + lane /
        // kChunksPerRow, physical chunk lane % kChunksPerRow, which holds the
        // logical chunk that swz() maps there (swz is an involution).
#pragma unroll
        for (int q = 0; q < kNx; ++q) {
            const int r = kRowsPerKb * (q * kWaves + wave) + lane / kChunksPerRow;
            const int lchunk = swz(r, lane % kChunksPerRow);
            c.xoff[q] = (uint32_t)src_row(r) * (uint32_t)(a.K * (ACT == kBf16 ? 2 : 1)) + (uint32_t)(lchunk * 16);
        }
        if constexpr (ACT == kMx8) {
            // the chunk's activation scales, all of K, into LDS (row stride padded)
            const int nb = a.K / kBlock;
            for (int i = tid; i < MS * 16 * nb; i += kThreads) {
                const int r = i / nb, b = i % nb;
                lds_xs[r * xs_stride(a.K) + b] = a.act_scale[(size_t)src_row(r) * nb + b];
            }
            __syncthreads();
        }

        f32x4_t acc[MS][RT];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[ms][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const int n = c.ns;                    // a multiple of 4, or equal to D
        u32x4_t w[D][RT];
        uint32_t sg[D][RT];
        pin();
        issue_w(c, w[0], sg[0], 0);
        pin();
#pragma unroll
        for (int j = 0; j < D - 1; ++j) {
            issue_x(c, j, j);
            pin();
            issue_w(c, w[j + 1], sg[j + 1], j + 1);
            pin();
        }

        int s = 0;
        for (; s < n - D; s += D) {
            step<0, 0, -1>(c, acc, w[0], sg[0], s + 0, li, g);
            if constexpr (D > 1) step<1 % D, 1, -1>(c, acc, w[1 % D], sg[1 % D], s + 1, li, g);
            if constexpr (D > 2) step<2 % D, 2, -1>(c, acc, w[2 % D], sg[2 % D], s + 2, li, g);
            if constexpr (D > 3) step<3 % D, 3, -1>(c, acc, w[3 % D], sg[3 % D], s + 3, li, g);
        }
        step<0, 0, D - 1>(c, acc, w[0], sg[0], s + 0, li, g);
        if constexpr (D > 1) step<1 % D, 1, D - 2>(c, acc, w[1 % D], sg[1 % D], s + 1, li, g);
        if constexpr (D > 2) step<2 % D, 2, D - 3>(c, acc, w[2 % D], sg[2 % D], s + 2, li, g);
        if constexpr (D > 3) step<3 % D, 3, D - 4>(c, acc, w[3 % D], sg[3 % D], s + 3, li, g);

        // Epilogue.  Lane holds D[token 4g + r][column li] of every (ms, rt).
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = c0 + ms * 16 + 4 * g + r;
                const size_t orow = (size_t)(m0 + idx);
                if constexpr (MODE == kGateUp && ACT == kBf16) {
                    if (idx < M) {
                        uint16_t* h = reinterpret_cast<uint16_t*>(a.h_out);
#pragma unroll
                        for (int rt = 0; rt < RT / 2; ++rt) {
                            const float hv = silu(acc[ms][rt][r]) * acc[ms][rt + RT / 2][r];
                            h[orow * a.ldo + col0 + rt * 16 + li] = f32_to_bf16_rne(hv);
                        }
                    }
                } else if constexpr (MODE == kGateUp) {
                    // the wave's 32 columns of this token row are one MX block
                    static_assert(RT == 4, "one MXFP8 block per wave row");
                    const float h0 = silu(acc[ms][0][r]) * acc[ms][2][r];
                    const float h1 = silu(acc[ms][1][r]) * acc[ms][3][r];
                    float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
                    const int se = mx_scale_exp(amax, 8);
                    if (idx < M) {
                        a.h_out[orow * a.ldo + col0 + li] = (uint8_t)e4m3_code(ldexpf(h0, -se));
                        a.h_out[orow * a.ldo + col0 + 16 + li] = (uint8_t)e4m3_code(ldexpf(h1, -se));
                        if (li == 0) a.h_scale_out[orow * (a.ldo / kBlock) + col0 / kBlock] = (uint8_t)(se + 127);
                    }
                } else {
                    if (idx < M) {
                        const float wgt = a.topk_w[a.sorted[m0 + idx]];
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            a.o_out[orow * a.ldo + col0 + rt * 16 + li] = wgt * acc[ms][rt][r];
                    }
                }
            }
        }
    }
};

template <int MODE, int ACT, int RT, int D>
__global__ __launch_bounds__(kThreads, 2) void k_expert(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[D * slot_bytes(ACT)];
    // MXFP8: the chunk's activation scales (64 rows x (K/32 + 4) bytes, K <= 8192)
    __shared__ __attribute__((aligned(16))) uint8_t lds_xs[ACT == kMx8 ? kMaxMs * 16 * xs_stride(8192) : 16];
    // Work unit = (chunk, column tile), chunk-major: the column tiles of a
    // chunk (same activation rows) are adjacent.  Chunks are listed expert
    // by expert, hottest expert first.  Workgroup-uniform values are kept in
    // scalar registers so that the buffer descriptors built from them are
    // scalar too.
    const int unit = blockIdx.x;
    const int chunk = unit / a.n_tiles;
    const int nt = unit % a.n_tiles;
    if (chunk >= __builtin_amdgcn_readfirstlane(*a.nchunks)) return;     // uniform per workgroup
    const int* rec = a.chunks + kChunkRec * chunk;
    const int e = __builtin_amdgcn_readfirstlane(rec[0]);
    const int c0 = __builtin_amdgcn_readfirstlane(rec[1]);
    const int m0 = __builtin_amdgcn_readfirstlane(a.offsets[e]);
    const int M = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - m0;
    int nsub = min(kMaxMs, (M - c0 + 15) / 16);
    if constexpr (ACT == kMx8) {
        nsub = nsub <= 2 ? 2 : 4;                     // E4M3 rows fill 1 KB loads in pairs of sub-tiles
        switch (nsub) {
            case 2: Pipe<MODE, ACT, RT, 2, D>::run(a, lds, lds_xs, e, nt, m0, c0, M); break;
            default: Pipe<MODE, ACT, RT, 4, D>::run(a, lds, lds_xs, e, nt, m0, c0, M); break;
        }
    } else {
        switch (nsub) {
            case 1: Pipe<MODE, ACT, RT, 1, D>::run(a, lds, lds_xs, e, nt, m0, c0, M); break;
            case 2: Pipe<MODE, ACT, RT, 2, D>::run(a, lds, lds_xs, e, nt, m0, c0, M); break;
            case 3: Pipe<MODE, ACT, RT, 3, D>::run(a, lds, lds_xs, e, nt, m0, c0, M); break;
            default: Pipe<MODE, ACT, RT, 4, D>::run(a, lds, lds_xs, e, nt, m0, c0, M); break;
        }
    }
}

constexpr int kRtGateUp = 4;     // 2 gate + 2 up tiles per wave: 128 h columns per workgroup
constexpr int kRtDown = 4;       // 4 tiles per wave: 256 output columns per workgroup

template <int MODE, int ACT, int RT>
hipError_t launch(const GemmArgs& a, int max_units, hipStream_t s) {
    const int nsteps = a.K / kKStep;          // 2 (K = 256) or a multiple of 4
    const dim3 grid(max_units), block(kThreads);
    if (nsteps % 4 == 0)
        hipLaunchKernelGGL((k_expert<MODE, ACT, RT, 4>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_expert<MODE, ACT, RT, 2>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

int gateup_cols_per_block() { return kWaves * (kRtGateUp / 2) * 16; }
int down_cols_per_block() { return kWaves * kRtDown * 16; }

hipError_t launch_gateup(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm,
                         const Workspace& ws, bool mx8, hipStream_t s) {
    GemmArgs a{};
    a.act = mx8 ? ws.xq : reinterpret_cast<const uint8_t*>(x);
    a.act_scale = mx8 ? ws.xs : nullptr;
    a.w0 = w.w_gate; a.s0 = w.w_gate_scale;
    a.w1 = w.w_up;   a.s1 = w.w_up_scale;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.topk_w = ws.topk_w;
    a.h_out = ws.h; a.h_scale_out = ws.hs; a.o_out = nullptr;
    a.K = dm.d; a.N = dm.f; a.n_tiles = dm.f / gateup_cols_per_block();
    a.k_top = dm.k; a.ldo = dm.f;
    const int units = max_chunks(dm) * a.n_tiles;
    return mx8 ? launch<kGateUp, kMx8, kRtGateUp>(a, units, s) : launch<kGateUp, kBf16, kRtGateUp>(a, units, s);
}

hipError_t launch_down(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, bool mx8,
                       hipStream_t s) {
    GemmArgs a{};
    a.act = ws.h;
    a.act_scale = mx8 ? ws.hs : nullptr;
    a.w0 = w.w_down; a.s0 = w.w_down_scale;
    a.w1 = nullptr;  a.s1 = nullptr;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.topk_w = ws.topk_w;
    a.h_out = nullptr; a.h_scale_out = nullptr; a.o_out = ws.o;
    a.K = dm.f; a.N = dm.d; a.n_tiles = dm.d / down_cols_per_block();
    a.k_top = dm.k; a.ldo = dm.d;
    const int units = max_chunks(dm) * a.n_tiles;
    return mx8 ? launch<kDown, kMx8, kRtDown>(a, units, s) : launch<kDown, kBf16, kRtDown>(a, units, s);
}

}  // namespace moe
