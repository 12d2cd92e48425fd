// Expert projections: packed MXFP4 weights streamed from HBM, decoded in
// registers and multiplied on the matrix cores.
//
// The pages' point is that decoding a huge MoE is bound by the bytes of
// expert weights it must stream, which FP4 on the experts cuts
// (ai.appwright.xyz "投機的デコード", section "第1層：FP4量子化（モデル側）";
// techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 — MoE에만 걸린
// 양자화").  So every kernel here is organised around one HBM pass over the
// weights of the experts a verify batch touches:
//
//   workgroup = (active expert, tile of output columns); 4 wavefronts, each
//   owning RT tiles of 16 weight rows.  A lane owns one weight row of each
//   tile and, per 128-wide K step, one 16-byte MX block of it (lane group g
//   = lane / 16 takes block 4s + g), so one load instruction reads 64
//   contiguous bytes of 16 rows and each block's scale is one byte.
//
//   The 32 nibbles of a block feed four v_mfma_f32_16x16x32_bf16 steps: the
//   hardware scaled convert turns 8 nibbles and the block's E8M0 scale into
//   the 8 bf16 of the B operand (exact).  The reduction index only has to
//   agree between A and B, so the A operand (activations, staged in LDS) is
//   read in the same block order.
//
//   Gate/up: tiles 0..RT/2-1 come from W_gate and RT/2.. from W_up, so the
//   gate and up accumulators of a (token, column) sit in the same lane and
//   SwiGLU h = silu(g) * u runs in the epilogue; h is stored in bf16, rows in
//   expert-sorted order.  Down: A = those h rows; the epilogue multiplies by
//   the pair's routing weight and stores float32 per pair (combined later in
//   a fixed order, so the result is deterministic).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxMs = 4;                 // token sub-tiles of 16 per chunk
constexpr int kLdsRow = kKStep + 8;       // bf16 per LDS row (pad: 272 B stride)

enum { kGateUp = 0, kDown = 1 };

struct GemmArgs {
    const uint16_t* act;        // gate/up: x [T][K]; down: h [P][K] (sorted rows)
    const uint8_t* w0;          // gate / down packed
    const uint8_t* s0;
    const uint8_t* w1;          // up packed (gate/up only)
    const uint8_t* s1;
    const int32_t* offsets;     // [E+1]
    const int32_t* sorted;      // [P]
    const int32_t* active;      // [E+1]
    const float* topk_w;        // [P]
    uint16_t* h_out;            // [P][f]
    float* o_out;               // [P][d]
    int32_t K;                  // reduction length
    int32_t N;                  // rows per weight matrix
    int32_t n_tiles;            // column tiles per expert
    int32_t E;
    int32_t k_top;
    int32_t ldo;                // output row length
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int MODE, int RT, int MS>
struct Tile {
    static constexpr int kColsPerWave = (MODE == kGateUp ? RT / 2 : RT) * 16;

    // Loads of one K step: the lane's 16-byte block of each row tile and its scale byte.
    struct WStage {
        u32x4_t w[RT];
        uint32_t s[RT];
    };

    __device__ static void load_w(WStage& st, const uint8_t* const (&wp)[RT],
                                  const uint8_t* const (&sp)[RT], int step) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            st.w[rt] = *reinterpret_cast<const u32x4_t*>(wp[rt] + (size_t)step * (kKStep / 2));
            st.s[rt] = sp[rt][step * (kKStep / kBlock)];
        }
    }

    __device__ static void load_x(u32x4_t (&xr)[MS], const uint16_t* const (&arow)[MS], int step,
                                  int c16) {
#pragma unroll
        for (int q = 0; q < MS; ++q)
            xr[q] = *reinterpret_cast<const u32x4_t*>(arow[q] + (size_t)step * kKStep + c16 * 8);
    }

    __device__ static void store_x(uint16_t* xs, const u32x4_t (&xr)[MS], int tid) {
#pragma unroll
        for (int q = 0; q < MS; ++q) {
            const int r = q * 16 + tid / 16;
            *reinterpret_cast<u32x4_t*>(xs + r * kLdsRow + (tid % 16) * 8) = xr[q];
        }
    }

    __device__ static void compute(f32x4_t (&acc)[MS][RT], const WStage& st, const uint16_t* xs,
                                   int li, int g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x8_t b[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) b[rt] = decode8_bf16(st.w[rt][i], e8m0_as_scale(st.s[rt]));
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const bf16x8_t a =
                    *reinterpret_cast<const bf16x8_t*>(xs + (ms * 16 + li) * kLdsRow + g * kBlock + 8 * i);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[ms][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[rt], acc[ms][rt], 0, 0, 0);
            }
        }
    }

    // One chunk of up to MS*16 tokens of expert e against this workgroup's columns.
    __device__ static void run(const GemmArgs& a, uint16_t* lds, int e, int nt, int m0, int c0, int M) {
        const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
        const int li = lane % 16, g = lane / 16;
        const int col0 = nt * (kWaves * kColsPerWave) + wave * kColsPerWave;
        const size_t rowbytes = (size_t)a.K / 2, rowscales = (size_t)a.K / kBlock;

        const uint8_t* wp[RT];
        const uint8_t* sp[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            int r;
            const uint8_t *W, *S;
            if (MODE == kGateUp) {
                constexpr int half = RT / 2;
                r = col0 + (rt % half) * 16 + li;
                W = rt < half ? a.w0 : a.w1;
                S = rt < half ? a.s0 : a.s1;
            } else {
                r = col0 + rt * 16 + li;
                W = a.w0;
                S = a.s0;
            }
            const size_t row = (size_t)e * a.N + r;
            wp[rt] = W + row * rowbytes + g * 16;
            sp[rt] = S + row * rowscales + g;
        }

        // Rows past the expert's last token repeat its last row: their
        // accumulators are computed but never stored.
        const uint16_t* arow[MS];
#pragma unroll
        for (int q = 0; q < MS; ++q) {
            const int idx = min(c0 + q * 16 + tid / 16, M - 1);
            const size_t row = MODE == kGateUp ? (size_t)(a.sorted[m0 + idx] / a.k_top) : (size_t)(m0 + idx);
            arow[q] = a.act + row * a.K;
        }

        uint16_t* xs0 = lds;
        uint16_t* xs1 = lds + kMaxMs * 16 * kLdsRow;
        f32x4_t acc[MS][RT];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[ms][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Software pipeline, two K steps per iteration so that the register
        // stages are addressed statically: weights run two steps ahead of
        // the MFMAs, activations one step ahead of the LDS buffer they fill.
        // nsteps is even (K % 256 == 0), so the steady-state loop issues the
        // same loads on every pass.
        const int nsteps = a.K / kKStep;
        const int c16 = tid % 16;
        WStage st0, st1;
        u32x4_t xr[MS];
        // Loads are issued in the steady-state order (activations of a step,
        // then weights of the same step) so that the loop-entry wait counts
        // match the loop-carried ones.
        load_w(st0, wp, sp, 0);
        load_x(xr, arow, 0, c16);
        store_x(xs0, xr, tid);
        load_x(xr, arow, 1, c16);
        load_w(st1, wp, sp, 1);
        __syncthreads();

        for (int s = 0; s < nsteps - 2; s += 2) {
            store_x(xs1, xr, tid);
            load_x(xr, arow, s + 2, c16);
            compute(acc, st0, xs0, li, g);
            load_w(st0, wp, sp, s + 2);
            __syncthreads();
            store_x(xs0, xr, tid);
            load_x(xr, arow, s + 3, c16);
            compute(acc, st1, xs1, li, g);
            load_w(st1, wp, sp, s + 3);
            __syncthreads();
        }
        store_x(xs1, xr, tid);
        compute(acc, st0, xs0, li, g);
        __syncthreads();
        compute(acc, st1, xs1, li, g);

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

template <int MODE, int RT>
__global__ __launch_bounds__(kThreads, 2) void k_expert(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kMaxMs * 16 * kLdsRow];
    const int slot = blockIdx.x / a.n_tiles;
    const int nt = blockIdx.x % a.n_tiles;
    if (slot >= a.active[a.E]) return;                 // uniform per workgroup
    const int e = a.active[slot];
    const int m0 = a.offsets[e];
    const int M = a.offsets[e + 1] - m0;
    for (int c0 = 0; c0 < M; c0 += kMaxMs * 16) {
        const int nsub = min(kMaxMs, (M - c0 + 15) / 16);
        switch (nsub) {
            case 1: Tile<MODE, RT, 1>::run(a, lds, e, nt, m0, c0, M); break;
            case 2: Tile<MODE, RT, 2>::run(a, lds, e, nt, m0, c0, M); break;
            case 3: Tile<MODE, RT, 3>::run(a, lds, e, nt, m0, c0, M); break;
            default: Tile<MODE, RT, 4>::run(a, lds, e, nt, m0, c0, M); break;
        }
        __syncthreads();                               // LDS reuse by the next chunk
    }
}

constexpr int kRtGateUp = 4;     // 2 gate + 2 up tiles per wave: 128 h columns per workgroup
constexpr int kRtDown = 4;       // 4 tiles per wave: 256 output columns per workgroup

}  // namespace

int gateup_cols_per_block() { return kWaves * (kRtGateUp / 2) * 16; }
int down_cols_per_block() { return kWaves * kRtDown * 16; }

hipError_t launch_gateup(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm,
                         const Workspace& ws, hipStream_t s) {
    GemmArgs a{};
    a.act = x;
    a.w0 = w.w_gate; a.s0 = w.w_gate_scale;
    a.w1 = w.w_up;   a.s1 = w.w_up_scale;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.active = ws.active; a.topk_w = ws.topk_w;
    a.h_out = ws.h; a.o_out = nullptr;
    a.K = dm.d; a.N = dm.f; a.n_tiles = dm.f / gateup_cols_per_block();
    a.E = dm.E; a.k_top = dm.k; a.ldo = dm.f;
    const int max_active = dm.E < dm.P ? dm.E : dm.P;
    hipLaunchKernelGGL((k_expert<kGateUp, kRtGateUp>), dim3(max_active * a.n_tiles), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    GemmArgs a{};
    a.act = ws.h;
    a.w0 = w.w_down; a.s0 = w.w_down_scale;
    a.w1 = nullptr;  a.s1 = nullptr;
    a.offsets = ws.offsets; a.sorted = ws.sorted_pairs; a.active = ws.active; a.topk_w = ws.topk_w;
    a.h_out = nullptr; a.o_out = ws.o;
    a.K = dm.f; a.N = dm.d; a.n_tiles = dm.d / down_cols_per_block();
    a.E = dm.E; a.k_top = dm.k; a.ldo = dm.d;
    const int max_active = dm.E < dm.P ? dm.E : dm.P;
    hipLaunchKernelGGL((k_expert<kDown, kRtDown>), dim3(max_active * a.n_tiles), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
