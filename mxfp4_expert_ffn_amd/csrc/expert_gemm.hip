// Expert projections: packed MXFP4 weights streamed from HBM, decoded in
// registers and multiplied on the matrix cores.
//
// The pages' point is that decoding a huge MoE is bound by the bytes of
// expert weights it must stream, which FP4 on the experts cuts
// (ai.appwright.xyz "投機的デコード", section "第1層：FP4量子化（モデル側）";
// techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 — MoE에만 걸린
// 양자화"), and that the next tile should stream in while the current one
// computes (dothoosh.com article, section "TileRT: عصر فشار بر GPU").  So
// every kernel here is one pipelined HBM pass over the weights of the
// experts a verify batch touches:
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
//   Weights run D steps ahead in a register ring; activations run D - 1 steps ahead in an LDS ring filled by direct-to-LDS loads (no
//   register staging), in a layout whose 16-byte chunks are XOR-swizzled by
//   row so that the MFMA operand reads are free of bank conflicts.
//
//   The 32 nibbles of a block feed four v_mfma_f32_16x16x32_bf16 steps: the
//   hardware scaled convert turns 8 nibbles and the block's E8M0 scale into
//   the 8 bf16 of the B operand (exact).  The reduction index only has to
//   agree between A and B, so the A operand (activations) is read in the
//   same block order.
//
//   Gate/up: tiles 0..RT/2-1 come from W_gate and RT/2.. from W_up, so the
//   gate and up accumulators of a (token, column) sit in the same lane and
//   SwiGLU h = silu(g) * u runs in the epilogue; h is stored in bf16, rows in
//   expert-sorted order.  Down: A = those h rows; the epilogue multiplies by
//   the pair's routing weight and stores float32 per pair (combined later in
//   a fixed order, so the result is deterministic).
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
constexpr int kSlotBytes = kMaxMs * 16 * 256;  // one LDS ring slot: 64 rows x 128 bf16
constexpr int kRsrcWord3 = 0x00020000;         // gfx9 raw buffer descriptor, dword 3

enum { kGateUp = 0, kDown = 1 };

struct GemmArgs {
    const uint16_t* act;        // gate/up: x [T][K]; down: h [P][K] (sorted rows)
    const uint8_t* w0;          // gate / down packed
    const uint8_t* s0;
    const uint8_t* w1;          // up packed (gate/up only)
    const uint8_t* s1;
    const int32_t* offsets;     // [E+1]
    const int32_t* sorted;      // [P]
    const int32_t* chunks;      // [n][2]: (expert, first pair of the chunk within the expert)
    const int32_t* nchunks;     // device count of chunks
    const float* topk_w;        // [P]
    uint16_t* h_out;            // [P][f]
    float* o_out;               // [P][d]
    int32_t K;                  // reduction length
    int32_t N;                  // rows per weight matrix
    int32_t n_tiles;            // column tiles per expert
    int32_t k_top;
    int32_t ldo;                // output row length
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

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

template <int MODE, int RT, int MS, int D>
struct Pipe {
    static constexpr int kHalf = MODE == kGateUp ? RT / 2 : RT;
    static constexpr int kColsPerWave = kHalf * 16;
    static constexpr int kNx = MS;         // direct-to-LDS loads per wave per step

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

    struct Ctx {
        __amdgpu_buffer_rsrc_t rw[2], rs[2];
        int32_t lane16, lane4;            // lane offsets within a 1 KB tile step / 256 B scale group
        int32_t tile0;                    // first 16-row tile of this wave (per matrix)
        int32_t ns, ng;                   // K steps, scale groups
        const uint8_t* xbase;             // activation rows (bytes)
        uint32_t xoff[MS];                // this lane's direct-to-LDS source offsets
        uint8_t* lds;
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
        for (int q = 0; q < MS; ++q)
            __builtin_amdgcn_global_load_lds(
                c.xbase + c.xoff[q] + step * (kKStep * 2),
                (lds_void*)(c.lds + slot * kSlotBytes + (q * kWaves + c.wave) * 1024), 16, 0, 0);
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
            const int chunk = (4 * g + i) ^ li;
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const bf16x8_t a =
                    *reinterpret_cast<const bf16x8_t*>(xs + (ms * 16 + li) * 256 + chunk * 16);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[ms][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[rt], acc[ms][rt], 0, 0, 0);
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
        compute<S4>(acc, w, sg, c.lds + SLOT * kSlotBytes, li, g);
        pin();
        if (R < 0) issue_w(c, w, sg, s + D);
        pin();
    }

    __device__ static void run(const GemmArgs& a, uint8_t* lds, int e, int nt, int m0, int c0, int M) {
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
        c.xbase = reinterpret_cast<const uint8_t*>(a.act);
        c.lds = lds;
        c.wave = wave;
        // Direct-to-LDS load q of this wave fills LDS rows 4 * (q * 4 + wave) +
        // lane / 16 at physical chunk lane % 16, which holds logical chunk
        // (lane % 16) ^ (row % 16).  Rows past the chunk's last pair repeat
        // it: their results are computed and never stored.
#pragma unroll
        for (int q = 0; q < MS; ++q) {
            const int r = 4 * (q * kWaves + wave) + lane / 16;
            const int idx = min(c0 + r, M - 1);
            const int row = MODE == kGateUp ? a.sorted[m0 + idx] / a.k_top : m0 + idx;
            const int lchunk = (lane % 16) ^ (r % 16);
            c.xoff[q] = (uint32_t)row * (uint32_t)(a.K * 2) + (uint32_t)(lchunk * 16);
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
                if (idx >= M) continue;
                const size_t orow = (size_t)(m0 + idx);
                if (MODE == kGateUp) {
#pragma unroll
                    for (int rt = 0; rt < RT / 2; ++rt) {
                        const float hv = silu(acc[ms][rt][r]) * acc[ms][rt + RT / 2][r];
                        a.h_out[orow * a.ldo + col0 + rt * 16 + li] = f32_to_bf16_rne(hv);
                    }
                } else {
                    const float wgt = a.topk_w[a.sorted[m0 + idx]];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        a.o_out[orow * a.ldo + col0 + rt * 16 + li] = wgt * acc[ms][rt][r];
                }
            }
        }
    }
};

template <int MODE, int RT, int D>
__global__ __launch_bounds__(kThreads, 2) void k_expert(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[D * kSlotBytes];
    const int unit = blockIdx.x;
    const int chunk = unit / a.n_tiles;
    const int nt = unit % a.n_tiles;
    if (chunk >= __builtin_amdgcn_readfirstlane(*a.nchunks)) return;     // uniform per workgroup
    // workgroup-uniform values: keep them in scalar registers so that the
    // buffer descriptors built from them are scalar too
    const int e = __builtin_amdgcn_readfirstlane(a.chunks[2 * chunk]);
    const int c0 = __builtin_amdgcn_readfirstlane(a.chunks[2 * chunk + 1]);
    const int m0 = __builtin_amdgcn_readfirstlane(a.offsets[e]);
    const int M = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - m0;
    const int nsub = min(kMaxMs, (M - c0 + 15) / 16);
    switch (nsub) {
        case 1: Pipe<MODE, RT, 1, D>::run(a, lds, e, nt, m0, c0, M); break;
        case 2: Pipe<MODE, RT, 2, D>::run(a, lds, e, nt, m0, c0, M); break;
        case 3: Pipe<MODE, RT, 3, D>::run(a, lds, e, nt, m0, c0, M); break;
        default: Pipe<MODE, RT, 4, D>::run(a, lds, e, nt, m0, c0, M); break;
    }
}

constexpr int kRtGateUp = 4;     // 2 gate + 2 up tiles per wave: 128 h columns per workgroup
constexpr int kRtDown = 4;       // 4 tiles per wave: 256 output columns per workgroup

template <int MODE, int RT>
hipError_t launch(const GemmArgs& a, int max_units, hipStream_t s) {
    const int nsteps = a.K / kKStep;          // 2 (K = 256) or a multiple of 4
    const dim3 grid(max_units), block(kThreads);
    if (nsteps % 4 == 0)
        hipLaunchKernelGGL((k_expert<MODE, RT, 4>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_expert<MODE, RT, 2>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

int gateup_cols_per_block() { return kWaves * (kRtGateUp / 2) * 16; }
int down_cols_per_block() { return kWaves * kRtDown * 16; }

hipError_t launch_gateup(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm,
                         const Workspace& ws, hipStream_t s) {
    GemmArgs a{};
    a.act = x;
    a.w0 = w.w_gate; a.s0 = w.w_gate_scale;
    a.w1 = w.w_up;   a.s1 = w.w_up_scale;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.topk_w = ws.topk_w;
    a.h_out = ws.h; a.o_out = nullptr;
    a.K = dm.d; a.N = dm.f; a.n_tiles = dm.f / gateup_cols_per_block();
    a.k_top = dm.k; a.ldo = dm.f;
    return launch<kGateUp, kRtGateUp>(a, max_chunks(dm) * a.n_tiles, s);
}

hipError_t launch_down(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    GemmArgs a{};
    a.act = ws.h;
    a.w0 = w.w_down; a.s0 = w.w_down_scale;
    a.w1 = nullptr;  a.s1 = nullptr;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.topk_w = ws.topk_w;
    a.h_out = nullptr; a.o_out = ws.o;
    a.K = dm.f; a.N = dm.d; a.n_tiles = dm.d / down_cols_per_block();
    a.k_top = dm.k; a.ldo = dm.d;
    return launch<kDown, kRtDown>(a, max_chunks(dm) * a.n_tiles, s);
}

}  // namespace moe
