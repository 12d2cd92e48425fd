// Streaming expert pipeline for bf16 activations: packed MXFP4 weights
// streamed from HBM and multiplied on the matrix cores.  Shared by the
// per-phase kernels (expert_gemm.hip) and the persistent fused kernel
// (fused.hip).
//
// The pages' point is that decoding a huge MoE is bound by the bytes of
// expert weights it must stream, which FP4 on the experts cuts
// (ai.appwright.xyz "投機的デコード", section "第1層：FP4量子化（モデル側）";
// techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 — MoE에만 걸린
// 양자화"), and that the next tile should stream in while the current one
// computes (dothoosh.com article, section "TileRT: عصر فشار بر GPU").  So
// every work unit here is one pipelined pass over a slice of the weights of
// one expert:
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
//   Weights run D steps ahead in a register ring (the HBM stream);
//   activations, which the column tiles of a chunk share through L2, run
//   D - 1 steps ahead in a D-slot LDS ring filled by direct-to-LDS loads, in
//   a layout whose 16-byte chunks are XOR-swizzled by row so that the
//   matrix-core operand reads are free of bank conflicts.
//
//   The 32 nibbles of a block feed four v_mfma_f32_16x16x32_bf16 steps; the
//   hardware scaled convert turns 8 nibbles and the block's E8M0 scale into
//   the 8 bf16 of the B operand (exact).  The reduction index only has to
//   agree between A and B, so the A operand is read in the same block order.
//
//   Gate/up: tiles 0..RT/2-1 come from W_gate and RT/2.. from W_up, so the
//   gate and up accumulators of a (token, column) sit in the same lane and
//   SwiGLU h = silu(g) * u runs in the epilogue; h is stored in bf16, rows in
//   expert-sorted order.  Down: A = those h rows; the epilogue stores each
//   float32 result row at its pair's own row p = t*k + j, so that the
//   combine (routing weights, k-slot sum in a fixed order, hence
//   deterministic) reads every token's k rows as one contiguous block.
//
// Memory ordering is explicit.  Vector-memory loads retire in issue order,
// so waiting for one load waits for every older one; the loads are always
// issued in the same interleaved order (W_j = weights of step j, X_j =
// activations of step j: prologue W_0 X_0 W_1 X_1 .. W_{D-2} X_{D-2} W_{D-1};
// step s: X_{s+D-1}, then W_{s+D}) and pinned there, so a fixed vmcnt wait
// before each step's barrier guarantees that the step's data has landed
// while everything issued in the D - 1 steps since stays in flight, and the
// barrier makes every wave's direct-to-LDS writes visible (and frees the
// slot the step's own activation load refills).
#pragma once

#include "common.hpp"

namespace moe {
namespace stream {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxMs = kChunk / 16;            // token sub-tiles of 16 per chunk
constexpr int kRow = kKStep * 2;               // bf16 activation bytes per row and step
constexpr int kSlot = kMaxMs * 16 * kRow;      // one LDS activation slot
constexpr int kRsrcWord3 = 0x00020000;         // gfx9 raw buffer descriptor, dword 3
// Cache policy of the weight loads: nt (non-temporal).  Each weight byte is
// streamed once per chunk, so it should not displace the activation rows
// the column tiles share; measured 3-14% faster than the default policy
// (and setting it on the small scale loads as well was slower).  The
// chunks of an expert with several chunks load with the default policy
// instead (kSharedWeightAux): their units of one weight tile run together
// (xcd_unit), and nt lines leave the L2 before the later units read them.
constexpr int kWeightAux = 2;
constexpr int kSharedWeightAux = 0;

enum { kGateUp = 0, kDown = 1 };

struct GemmArgs {
    const uint8_t* act;         // gate/up: x [T][K]; down: h [P][K] (sorted rows); bf16
    const uint8_t* w0;          // gate / down tiled packed
    const uint8_t* s0;
    const uint8_t* w1;          // up tiled packed (gate/up only)
    const uint8_t* s1;
    const int32_t* sorted;      // [P]
    const int32_t* chunks;      // chunk records
    const int32_t* nchunks;     // device count of chunks
    const int32_t* xtab;        // per-XCD chunk table (per-phase kernels)
    int32_t xstride;            // its slots per XCD
    uint8_t* h_out;             // gate/up: h [P][f] bf16
    float* o_out;               // down: [P][d], row = pair index
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

// 16 bytes per lane from global memory straight into LDS (lane L writes
// lds + 16 L).
__device__ __forceinline__ void lds_dma16(const uint8_t* src, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
}

// H_COHERENT: gate/up stores h with agent-scope (device-coherent) stores,
// which another workgroup may read during the same launch once this one has
// waited for them; otherwise plain stores (read by a later launch).
template <int MODE, int RT, int MS, int D, bool H_COHERENT = false, int WAUX = kWeightAux>
struct Pipe {
    static constexpr int kHalf = MODE == kGateUp ? RT / 2 : RT;
    static constexpr int kColsPerWave = kHalf * 16;
    static constexpr int kChunksPerRow = kRow / 16;       // 16-byte chunks per row and step
    static constexpr int kRowsPerKb = 1024 / kRow;        // rows one direct-to-LDS load fills
    // direct-to-LDS loads per wave per step: MS*16 rows over 4 waves
    static constexpr int kNx = MS * 16 / (kRowsPerKb * kWaves);
    static_assert(kNx * kRowsPerKb * kWaves == MS * 16, "whole 1 KB loads per sub-tile");
    // weight loads per step: one 16-byte block and one scale dword per tile
    // (the dword holds the scales of 4 steps; each step reads its own copy
    // so that no register is carried across loop iterations)
    static constexpr int kNw = 2 * RT;

    // Physical 16-byte chunk of logical chunk c in LDS row r.
    __device__ static int swz(int r, int c) { return c ^ (r & 15); }

    struct Ctx {
        __amdgpu_buffer_rsrc_t rw[2], rs[2];
        int32_t lane16, lane4;            // lane offsets within a 1 KB tile step / 256 B scale group
        int32_t tile0;                    // first 16-row tile of this wave (per matrix)
        int32_t ns, ng;                   // K steps, scale groups
        const uint8_t* xbase;             // activation rows (bytes)
        uint32_t xoff[kNx];               // this lane's direct-to-LDS source offsets
        uint8_t* lds;                     // activation ring (D slots)
        int wave;
    };

    __device__ static void issue_w(const Ctx& c, u32x4_t (&w)[RT], uint32_t (&sg)[RT], int step) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int mat = (MODE == kGateUp && rt >= kHalf) ? 1 : 0;
            const int tile = c.tile0 + rt % kHalf;
            w[rt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    c.rw[mat], c.lane16, (tile * c.ns + step) * 1024, WAUX));
            sg[rt] = __builtin_amdgcn_raw_buffer_load_b32(c.rs[mat], c.lane4, (tile * c.ng + step / 4) * 256, 0);
        }
    }

    // activations of `step` into LDS slot XSLOT (== step mod 2, a constant
    // so that the compiler can tell the slot apart from the one being read)
    template <int XSLOT>
    __device__ static void issue_x(const Ctx& c, int step) {
#pragma unroll
        for (int q = 0; q < kNx; ++q)
            lds_dma16(c.xbase + c.xoff[q] + step * kRow, c.lds + XSLOT * kSlot + (q * kWaves + c.wave) * 1024);
    }

    template <int S4>
    __device__ static void compute(f32x4_t (&acc)[MS][RT], const u32x4_t (&w)[RT], const uint32_t (&sg)[RT],
                                   const uint8_t* xs, int li, int g) {
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
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xs + r * kRow + swz(r, 4 * g + i) * 16);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[ms][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[rt], acc[ms][rt], 0, 0, 0);
            }
        }
    }

    // Loads issued after X_s by the time step s starts, R < 0 meaning a step
    // before the last D and R >= 0 the R-th of them: X_{s+1} .. X_{s+D-2} and
    // W_{s+1} .. W_{s+D-1}, cut off at the last step.
    static constexpr int after_x(int R) {
        const int nw = R < 0 ? D - 1 : D - 1 - R;
        const int nx = R < 0 ? D - 2 : (D - 1 - R < D - 2 ? D - 1 - R : D - 2);
        return nx * kNx + nw * kNw;
    }

    // Step s (ring slot SLOT == s mod D, S4 == s mod 4).  R < 0: a step
    // before the last D, which issues the activations of step s+D-1 into the
    // slot that step s-1 read and the weights of step s+D; R >= 0: the R-th
    // (from 0) of the last D steps, of which only the first still has
    // activations to issue.  X_s is older than the after_x(R) loads issued
    // since, and W_s older still, so waiting for at most that many
    // outstanding loads means both have landed.
    template <int SLOT, int S4, int R>
    __device__ static void step(const Ctx& c, f32x4_t (&acc)[MS][RT], u32x4_t (&w)[RT], uint32_t (&sg)[RT], int s,
                                int li, int g) {
        step_barrier<after_x(R)>();
        pin();
        if (R <= 0) issue_x<(SLOT + D - 1) % D>(c, s + D - 1);
        pin();
        compute<S4>(acc, w, sg, c.lds + SLOT * kSlot, li, g);
        pin();
        if (R < 0) issue_w(c, w, sg, s + D);
        pin();
    }

    // Prologue loads W_J X_J .. W_{D-2} X_{D-2} (compile-time slots).
    template <int J>
    __device__ static void prologue(const Ctx& c, u32x4_t (&w)[D][RT], uint32_t (&sg)[D][RT]) {
        if constexpr (J < D - 1) {
            issue_w(c, w[J], sg[J], J);
            pin();
            issue_x<J>(c, J);
            pin();
            prologue<J + 1>(c, w, sg);
        }
    }

    // Steps s+J .. s+D-1 of one ring turn (s a multiple of D, and D a
    // multiple of 4 or D == 2 == n, so s+J == J mod 4); TAIL: the last D
    // steps of the pass.
    template <int J, bool TAIL>
    __device__ static void steps(const Ctx& c, f32x4_t (&acc)[MS][RT], u32x4_t (&w)[D][RT], uint32_t (&sg)[D][RT],
                                 int s, int li, int g) {
        if constexpr (J < D) {
            step<J, J % 4, TAIL ? J : -1>(c, acc, w[J], sg[J], s + J, li, g);
            steps<J + 1, TAIL>(c, acc, w, sg, s, li, g);
        }
    }

    // One work unit: the M (<= 64) pairs of a chunk of expert e, column tile
    // nt.  pairs[i] (i < M; global or LDS memory) is the chunk's i-th pair id
    // t*k + j; m0 is the chunk's first row in expert-sorted order (the rows of
    // h).  Gate/up reads x rows pairs[i] / k and writes h rows m0 + i; down
    // reads h rows m0 + i and writes o rows pairs[i].
    // pre() runs right before the first loads of the pipeline are issued,
    // late() right after its last weight loads (before the last D steps,
    // which issue no weights: a memory operation started there has those
    // steps to complete before the unit ends; vector-memory operations
    // complete in order, so one issued before the first loads would hold up
    // the first step instead).
    template <typename Pre, typename Late>
    __device__ static void run(const GemmArgs& a, uint8_t* lds, int e, int nt, const int32_t* pairs, int m0, int M,
                               Pre&& pre, Late&& late) {
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
        c.wave = wave;
        // Source row of chunk row r: rows past the chunk's last pair repeat
        // it; their results are computed and never stored.
        auto src_row = [&](int r) {
            const int idx = min(r, M - 1);
            return MODE == kGateUp ? pairs[idx] / a.k_top : m0 + idx;
        };
        // Direct-to-LDS load q of this wave fills the 1 KB at slot offset
        // (q * 4 + wave) KB: rows kRowsPerKb * (q * 4 + wave) + lane /
        // kChunksPerRow, physical chunk lane % kChunksPerRow, which holds the
        // logical chunk that swz() maps there (swz is an involution).
#pragma unroll
        for (int q = 0; q < kNx; ++q) {
            const int r = kRowsPerKb * (q * kWaves + wave) + lane / kChunksPerRow;
            const int lchunk = swz(r, lane % kChunksPerRow);
            c.xoff[q] = (uint32_t)src_row(r) * (uint32_t)(a.K * 2) + (uint32_t)(lchunk * 16);
        }
        // down: pair indices (output rows) of this lane's rows, loaded up
        // front so that the epilogue does not wait on them
        int32_t pr[MS][4];
        if constexpr (MODE == kDown) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int r = 0; r < 4; ++r) pr[ms][r] = pairs[min(ms * 16 + 4 * g + r, M - 1)];
        }

        f32x4_t acc[MS][RT];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[ms][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const int n = c.ns;                    // a multiple of D (K = 256: D = 2 = n)
        u32x4_t w[D][RT];
        uint32_t sg[D][RT];
        pre();
        pin();
        prologue<0>(c, w, sg);
        issue_w(c, w[D - 1], sg[D - 1], D - 1);
        pin();

        int s = 0;
        for (; s < n - D; s += D) steps<0, false>(c, acc, w, sg, s, li, g);
        late();
        pin();
        steps<0, true>(c, acc, w, sg, s, li, g);

        // Epilogue.  Lane holds D[token 4g + r][column li] of every (ms, rt).
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = ms * 16 + 4 * g + r;
                if (idx < M) {
                    if constexpr (MODE == kGateUp) {
                        const size_t orow = (size_t)(m0 + idx);
                        uint16_t* h = reinterpret_cast<uint16_t*>(a.h_out);
#pragma unroll
                        for (int rt = 0; rt < RT / 2; ++rt) {
                            const float hv = silu(acc[ms][rt][r]) * acc[ms][rt + RT / 2][r];
                            uint16_t* dst = h + orow * a.ldo + col0 + rt * 16 + li;
                            if constexpr (H_COHERENT)
                                __hip_atomic_store(dst, f32_to_bf16_rne(hv), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            else
                                *dst = f32_to_bf16_rne(hv);
                        }
                    } else {
                        const size_t orow = (size_t)pr[ms][r];
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) a.o_out[orow * a.ldo + col0 + rt * 16 + li] = acc[ms][rt][r];
                    }
                }
            }
        }
    }
};

// One unit with the sub-tile count MS picked from the chunk's pair count;
// pre() runs right before the pipeline's first loads, late() right after
// its last weight loads.  shared: the expert has other chunks whose units
// of the same weight tile run alongside; the unit then loads its weights
// with kSharedWeightAux, in the full-chunk shape whatever its pair count
// (one more body instead of four: rows past the chunk's last pair are
// computed and never stored).
template <int MODE, int RT, int D, bool H_COHERENT = false, typename Pre, typename Late>
__device__ __forceinline__ void run_unit(const GemmArgs& a, uint8_t* lds, int e, int nt, const int32_t* pairs,
                                         int m0, int rows, Pre&& pre, Late&& late, bool shared = false) {
    if (shared) {
        Pipe<MODE, RT, kMaxMs, D, H_COHERENT, kSharedWeightAux>::run(a, lds, e, nt, pairs, m0, rows, pre, late);
        return;
    }
    switch (min(kMaxMs, (rows + 15) / 16)) {
        case 1: Pipe<MODE, RT, 1, D, H_COHERENT>::run(a, lds, e, nt, pairs, m0, rows, pre, late); break;
        case 2: Pipe<MODE, RT, 2, D, H_COHERENT>::run(a, lds, e, nt, pairs, m0, rows, pre, late); break;
        case 3: Pipe<MODE, RT, 3, D, H_COHERENT>::run(a, lds, e, nt, pairs, m0, rows, pre, late); break;
        default: Pipe<MODE, RT, 4, D, H_COHERENT>::run(a, lds, e, nt, pairs, m0, rows, pre, late); break;
    }
}

// Weight tiles per wave.  4 (gate/up: 2 gate + 2 up, 128 h columns per
// workgroup; down: 256 output columns) normally; 2 when the batch has at most
// one pair per expert on average: every touched expert is then one small
// chunk, the grid is about one round of 4-tile workgroups, and the last of
// them would stream alone -- halving the tile doubles the workgroups.
inline int tiles_per_wave(const Dims& dm) { return dm.P <= dm.E ? 2 : 4; }

// Column tiles (units) per chunk of one projection.
template <int MODE, int RT>
constexpr int col_tiles(int N) { return N / (kWaves * (MODE == kGateUp ? RT / 2 : RT) * 16); }

}  // namespace stream
}  // namespace moe
