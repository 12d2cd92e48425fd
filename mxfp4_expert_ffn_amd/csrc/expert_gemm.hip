// Expert projections for bf16 activations, one launch per phase: gate/up +
// SwiGLU over every (chunk, column tile) unit, then down.  The pipeline of
// one unit is in stream_pipe.hpp.
#include "stream_pipe.hpp"

namespace moe {
namespace stream {
namespace {

// RT = 4 fits two workgroups per CU (registers), RT = 2 three.
template <int MODE, int RT, int D>
__global__ __launch_bounds__(kThreads, RT >= 4 ? 2 : 3) void k_expert(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[D * kSlot];
    // Work unit = (chunk, column tile).  With a per-XCD table (batches of
    // more pairs than experts), workgroup g runs on XCD g mod kXcds (the
    // GPU's round-robin) and takes the units of that XCD's chunk list in
    // order (xcd_unit: a hot expert's chunks interleaved by column tile);
    // otherwise unit g of the global list, chunk-major: the column tiles of
    // a chunk (same activation rows) are adjacent, hottest expert first.
    // The record and the chunk count are read together, so the weight loads
    // wait on one round trip; workgroup-uniform values are kept in scalar
    // registers so that the buffer descriptors built from them are scalar
    // too.
    int e, start, rows, nt;
    bool shared = false;
    if (a.xtab) {
        XcdUnit w;
        if (!xcd_unit(a.xtab, a.xstride, blockIdx.x % kXcds, blockIdx.x / kXcds, a.n_tiles, w)) return;
        e = w.e; start = w.start; rows = w.rows; nt = w.nt; shared = w.m > 1;
    } else {
        const int slot = blockIdx.x / a.n_tiles;
        nt = blockIdx.x % a.n_tiles;
        const int* rec = a.chunks + kChunkRec * slot;
        e = __builtin_amdgcn_readfirstlane(rec[0]);
        start = __builtin_amdgcn_readfirstlane(rec[1]);
        rows = __builtin_amdgcn_readfirstlane(rec[2]);
        if (slot >= __builtin_amdgcn_readfirstlane(*a.nchunks)) return;     // uniform per workgroup
    }
    // the chunk's pairs sit at sorted positions start .. start + rows - 1
    run_unit<MODE, RT, D>(a, lds, e, nt, a.sorted + start, start, rows, [] {}, [] {}, shared);
}

template <int MODE, int RT>
hipError_t launch_rt(GemmArgs a, const Dims& dm, hipStream_t s) {
    a.n_tiles = a.N / (kWaves * (MODE == kGateUp ? RT / 2 : RT) * 16);
    const int nsteps = a.K / kKStep;          // 2 (K = 256) or a multiple of 4
    // the per-XCD table pays where experts have several chunks or a chunk
    // several rows; at most one pair per expert on average it would only
    // add workgroups (its bound is looser than the global list's)
    a.xstride = xcd_slots(dm);
    if (dm.P <= dm.E) a.xtab = nullptr;
    const dim3 grid(a.xtab ? kXcds * a.xstride * a.n_tiles : max_chunks(dm) * a.n_tiles), block(kThreads);
    if (nsteps % 4 == 0)
        hipLaunchKernelGGL((k_expert<MODE, RT, 4>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_expert<MODE, RT, 2>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch(const GemmArgs& a, const Dims& dm, hipStream_t s) {
    return tiles_per_wave(dm) == 2 ? launch_rt<MODE, 2>(a, dm, s) : launch_rt<MODE, 4>(a, dm, s);
}

}  // namespace
}  // namespace stream

using stream::GemmArgs;
using stream::kDown;
using stream::kGateUp;

hipError_t launch_gateup(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm,
                         const Workspace& ws, hipStream_t s) {
    GemmArgs a{};
    a.act = reinterpret_cast<const uint8_t*>(x);
    a.w0 = w.w_gate; a.s0 = w.w_gate_scale;
    a.w1 = w.w_up;   a.s1 = w.w_up_scale;
    a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks; a.xtab = ws.xtab;
    a.h_out = ws.h; a.o_out = nullptr;
    a.K = dm.d; a.N = dm.f;
    a.k_top = dm.k; a.ldo = dm.f;
    return stream::launch<kGateUp>(a, dm, s);
}

hipError_t launch_down(const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws, hipStream_t s) {
    GemmArgs a{};
    a.act = ws.h;
    a.w0 = w.w_down; a.s0 = w.w_down_scale;
    a.w1 = nullptr;  a.s1 = nullptr;
    a.sorted = ws.sorted_pairs; a.chunks = ws.chunks; a.nchunks = ws.nchunks; a.xtab = ws.xtab;
    a.h_out = nullptr; a.o_out = ws.o;
    a.K = dm.f; a.N = dm.d;
    a.k_top = dm.k; a.ldo = dm.d;
    return stream::launch<kDown>(a, dm, s);
}

}  // namespace moe
