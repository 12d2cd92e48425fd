// The expert layer after routing as ONE launch: gate/up + SwiGLU and the
// down projection run as work units of a single grid, so the two phases
// overlap instead of each draining the GPU before the next launch ramps up.
// Two forms (fused_chain_form picks one per batch):
//
//   - ticketed (k_chain; batches with more pairs than experts): one
//     workgroup per unit, each taking a ticket (see k_chain);
//   - persistent (k_fused; at most one pair per expert on average): a grid
//     of as many workgroups as the GPU holds loops over the units, as
//     described below.
//
// Both run after the per-phase routing and permutation launches (the
// permutation also lists each XCD's chunks), whose first launch also clears
// the counters here.
//
// The unit bodies compile to the per-phase kernels' schedule only where a
// workgroup runs one unit: inside a loop over units the compiler keeps one
// activation fragment register and waits on every LDS read, which is what
// the persistent form pays for its smaller grid.
//
// The pages' runtime keeps a single engine kernel resident on the GPU so
// that microsecond operators pay no launch or synchronisation gap between
// them, and streams the next tile while the current one computes
// (techllm.github.io "Xiaomi MiMo x TileRT", section "3. TileRT — GPU에 상주하는
// 런타임"; dothoosh.com article, section "TileRT: عصر فشار بر GPU").  On gfx950
// the same idea takes this form:
//
//   - k_fused (as many workgroups as the GPU holds at once): every
//     workgroup takes units from one queue (one atomic per unit, taken a
//     unit ahead): first the gate/up units (chunk, column tile), then the
//     down units in chunk order, so the workgroups that finish gate/up first
//     take the down work of the chunks that finished first.  A down unit of
//     chunk c waits only for the gate/up units of chunk c (a counter per
//     chunk), which running workgroups hold and finish without waiting on
//     anything.  Down work starts while gate/up still streams the weights of
//     later chunks.
//   - Every wait is bounded: past the limit the kernel raises an error word
//     in the workspace and its workgroups exit normally (a grid larger than
//     what the GPU holds, for example because another kernel occupies it,
//     can only delay the units of workgroups not yet started).
//   - The gate/up -> down handoff crosses XCDs, whose L2 caches are not kept
//     coherent with each other: gate/up stores h with device-coherent
//     (agent-scope) stores, every wave waits for them, and then one lane
//     bumps the chunk's counter; the consumer's lane 0 polls with agent-scope
//     loads and invalidates its caches (agent-scope acquire) before the
//     workgroup reads h.  (Writing the whole L2 back after every gate/up
//     unit instead, the usual release, measured ~18 us slower at 256
//     tokens.)
//   - The counters are cleared by the routing launch that precedes these
//     kernels in every call (no memset, so the call stays capturable).
//
// The unit bodies are the per-phase kernels' own pipeline (stream_pipe.hpp),
// so every h and o value is bit-identical to the multi-launch path.
#include "layer.hpp"
#include "route_core.hpp"
#include "stream_pipe.hpp"

namespace moe {
namespace fused {
namespace {

using stream::GemmArgs;
using stream::kDown;
using stream::kGateUp;
using stream::kSlot;
using stream::kThreads;
using stream::kWaves;

// ctl[] words.  Each counter sits on a 256-byte line of its own, so the
// polls of waiting workgroups and the atomics on other counters do not queue
// behind each other at one memory channel.
constexpr int kLine = 64;                       // ints per 256 bytes
// (line 0 is spare)
enum { kError = kLine, kDownQueue = 2 * kLine, kTicket = 3 * kLine, kChunkDone = kTicket + kXcds * kLine };
static_assert(kError == kFusedErrorWord, "the host reads the error word at this index");

struct FusedArgs {
    GemmArgs gu, dn;
    int32_t* ctl;              // counters (cleared by the routing launch)
    const int32_t* sorted;     // [P] the permutation (pair ids in expert order)
    const int32_t* chunks;     // global chunk list (expert, first sorted position, pairs, 0)
    const int32_t* nchunks;
    int32_t ntg, ntd;          // column tiles per chunk: gate/up, down
    int32_t spin_limit;        // poll rounds before a wait gives up; < 0: every wait gives up at once
    const int32_t* xtab;       // per-XCD chunk table (ticketed form)
    int32_t xstride;
};

__device__ __forceinline__ int32_t load_agent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (one lane) until *p >= target.  False if the error flag is up (read
// every 32 polls) or the poll limit runs out (then it raises the flag).
__device__ bool wait_geq(const FusedArgs& f, const int32_t* p, int32_t target) {
    for (int i = 0;; ++i) {
        if (f.spin_limit >= 0 && load_agent(p) >= target) return true;
        if (i % 32 == 31 && load_agent(f.ctl + kError) != 0) return false;
        if (i >= f.spin_limit) {
            __hip_atomic_fetch_or(f.ctl + kError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

// Every wave waits for its own stores (the h rows, stored device-coherent),
// then the workgroup meets and lane 0 adds 1 to the chunk's counter.
__device__ __forceinline__ void publish(int32_t* p) {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));        // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0 waits for *p >= target and acquires (its invalidation covers the
// CU's vector L1 and the XCD's L2, which the workgroup's waves share); the
// barrier then orders every wave's later reads after it.  Uniform result:
// false when the wait failed.
__device__ __forceinline__ bool await(const FusedArgs& f, const int32_t* p, int32_t target, int32_t* s_flag) {
    if (threadIdx.x == 0) {
        const bool ok = wait_geq(f, p, target);
        if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_flag = ok;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_flag) != 0;
}

template <int RT, int DG, int DD>
__global__ __launch_bounds__(kThreads, 2) void k_fused(FusedArgs f) {
    constexpr int kRing = DG > DD ? DG : DD;
    // One LDS object: the ring, then two handoff words.  (A second
    // __shared__ object costs the compiler its proof that a step's operand
    // reads do not alias the direct-to-LDS loads in flight, and it then
    // drains every load before each step's reads.)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * kSlot + 2 * sizeof(int32_t)];
    int32_t& s_flag = *reinterpret_cast<int32_t*>(lds + kRing * kSlot);
    int32_t& s_next = *reinterpret_cast<int32_t*>(lds + kRing * kSlot + sizeof(int32_t));
    const int nc = __builtin_amdgcn_readfirstlane(*f.nchunks);
    const int nG = nc * f.ntg, nD = nc * f.ntd;
    // One queue hands out every unit: tickets 0 .. nG-1 are the gate/up
    // units (chunk-major), then the down units in chunk order.  Each
    // workgroup takes its next ticket once the current unit has issued its
    // last weight loads (lane 0; handed over through LDS at the end), so
    // the queue's latency runs under the unit's last steps.  A down unit waits only for gate/up units
    // of its chunk, and a workgroup sees a ticket past the gate/up units
    // only after every gate/up ticket went to a running workgroup: every
    // wait ends, however many workgroups the GPU holds at once (another
    // kernel may occupy part of it).  Two loops keep the two pipelines'
    // registers apart.
    if (threadIdx.x == 0) s_next = __hip_atomic_fetch_add(f.ctl + kDownQueue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int v = __builtin_amdgcn_readfirstlane(s_next);
    int next = 0;
    auto take = [&] {
        if (threadIdx.x == 0) next = __hip_atomic_fetch_add(f.ctl + kDownQueue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    while (v < nG) {
        const int chunk = v / f.ntg, nt = v % f.ntg;
        const int32_t* rec = f.chunks + kChunkRec * chunk;
        const int e = __builtin_amdgcn_readfirstlane(rec[0]);
        const int m0 = __builtin_amdgcn_readfirstlane(rec[1]);
        const int rows = __builtin_amdgcn_readfirstlane(rec[2]);
        // the chunk's pairs sit at sorted positions m0 .. m0 + rows - 1
        stream::run_unit<kGateUp, RT, DG, true>(f.gu, lds, e, nt, f.sorted + m0, m0, rows, [] {}, take);
        publish(f.ctl + kChunkDone + kLine * chunk);
        if (threadIdx.x == 0) s_next = next;
        __syncthreads();               // s_next holds the next ticket; the LDS ring is free again
        v = __builtin_amdgcn_readfirstlane(s_next);
    }
    while (v < nG + nD) {
        const int w = v - nG;
        const int chunk = w / f.ntd, nt = w % f.ntd;
        const int32_t* rec = f.chunks + kChunkRec * chunk;
        const int e = __builtin_amdgcn_readfirstlane(rec[0]);
        const int m0 = __builtin_amdgcn_readfirstlane(rec[1]);
        const int rows = __builtin_amdgcn_readfirstlane(rec[2]);
        if (!await(f, f.ctl + kChunkDone + kLine * chunk, f.ntg, &s_flag)) return;
        stream::run_unit<kDown, RT, DD>(f.dn, lds, e, nt, f.sorted + m0, m0, rows, [] {}, take);
        if (threadIdx.x == 0) s_next = next;
        __syncthreads();               // s_next holds the next ticket; the LDS ring is free again
        v = __builtin_amdgcn_readfirstlane(s_next);
    }
}

// Ticketed form: one unit per workgroup.  Workgroup b takes the next
// ticket of counter b mod kXcds (so each counter serves exactly its share of
// the grid whatever the dispatch order) and runs unit `ticket` of that
// XCD's list in the per-XCD chunk table: first the gate/up units of its
// chunks, then their down units in the same order (xcd_unit: expert by
// expert, a hot expert's chunks interleaved by column tile).  A down
// unit waits only for gate/up units of its chunk, which sit earlier in the
// same list: their tickets were taken first, by workgroups that are running
// or done and never wait, so every wait ends.  With the GPU's round-robin
// dispatch, a list's units also run on one XCD and share its L2.
template <int RT, int DG, int DD>
__global__ __launch_bounds__(kThreads, 2) void k_chain(FusedArgs f) {
    constexpr int kRing = DG > DD ? DG : DD;
    // one LDS object (see k_fused): the ring, then two words
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * kSlot + 2 * sizeof(int32_t)];
    int32_t& s_flag = *reinterpret_cast<int32_t*>(lds + kRing * kSlot);
    int32_t& s_tick = *reinterpret_cast<int32_t*>(lds + kRing * kSlot + sizeof(int32_t));
    const int x = blockIdx.x % kXcds;
    if (threadIdx.x == 0)
        s_tick = __hip_atomic_fetch_add(f.ctl + kTicket + kLine * x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int nslots = __builtin_amdgcn_readfirstlane(f.xtab[x]);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_tick);
    const int nG = nslots * f.ntg, nD = nslots * f.ntd;
    const bool gateup = t < nG;
    if (!gateup && t - nG >= nD) return;                 // past the list: nothing to do
    XcdUnit w;
    xcd_unit(f.xtab, f.xstride, x, gateup ? t : t - nG, gateup ? f.ntg : f.ntd, w);   // t < nG + nD: in the list
    // the chunk's pairs sit at sorted positions w.start .. w.start + w.rows - 1
    if (gateup) {
        stream::run_unit<kGateUp, RT, DG, true>(f.gu, lds, w.e, w.nt, f.sorted + w.start, w.start, w.rows, [] {},
                                                [] {}, w.m > 1);
        publish(f.ctl + kChunkDone + kLine * w.chunk);
    } else {
        if (!await(f, f.ctl + kChunkDone + kLine * w.chunk, f.ntg, &s_flag)) return;
        stream::run_unit<kDown, RT, DD>(f.dn, lds, w.e, w.nt, f.sorted + w.start, w.start, w.rows, [] {}, [] {},
                                        w.m > 1);
    }
}

// ---------------------------------------------------------------------------
// The layer of one verify block (at most 64 pairs over at most 128 experts)
// in two launches: this persistent kernel, with no launch in front of it,
// and the combine after it.
//
//   - Every workgroup routes all T tokens and permutes the P pairs itself,
//     in LDS (route_core.hpp: the same code, so the same bits, as the
//     routing launches), from the block's logits staged in LDS by one
//     coalesced pass.  That costs a workgroup about what reading the chunk
//     count and record did, and no workgroup waits for another to publish
//     the permutation.  Workgroup 0 also writes the routing to the workspace
//     (the routing outputs of the call, and the weights the combine reads).
//   - Units come from one queue as in k_fused: gate/up units first, then
//     down units in chunk order, each waiting for its chunk's gate/up tiles;
//     the per-pair outputs go to the workspace for the combine launch.
//   - Counters: the stream's state block (the queue, a counter per chunk,
//     the error word and the epoch).  The combine launch clears them for the
//     stream's next call, so that call needs no clearing launch in front of
//     it; a wait that gives up stores epoch + 1 in the error word.
//
// Also measured, and slower: the combine inside this kernel as well, either
// by the down unit that completes a column tile (a store drain and an atomic
// with return after every down unit: 81 us against 71 us for k_fused at 8
// tokens) or by every workgroup once a counter of finished down units is
// full (hundreds of workgroups polling one line: 116 us).
struct LayerArgs {
    GemmArgs gu, dn;
    const float* logits;       // [T][E]
    Dims dm;
    int32_t* st;               // the stream's state block
    // the call's routing outputs in the workspace (written by workgroup 0)
    int32_t *ids, *offsets, *sorted, *active, *chunks, *nchunks;
    float* wts;
    int32_t ntg, ntd;
    int32_t spin_limit;
};

// LDS beside the unit ring: routing and permutation of the block.
constexpr int kLyWords = 0;                                        // flag, next ticket, epoch
constexpr int kLySc = 16;                                          // RankScratch<1>[kWaves]
constexpr int kLyIds = kLySc + kWaves * (int)sizeof(route::RankScratch<1>);
constexpr int kLyWts = kLyIds + kChunk * 4;
constexpr int kLyCnt = kLyWts + kChunk * 4;                       // [128]
constexpr int kLyExo = kLyCnt + 2 * kWave * 4;                     // [128]
constexpr int kLyKeys = kLyExo + 2 * kWave * 4;                    // uint64 [64] or int [128]
constexpr int kLyOff = kLyKeys + kWave * 8;                        // [E + 1]
constexpr int kLyAct = kLyOff + (2 * kWave + 4) * 4;               // [E + 1]
constexpr int kLySorted = kLyAct + (2 * kWave + 4) * 4;            // [P]
constexpr int kLyChunks = kLySorted + kChunk * 4;                  // [64][kChunkRec]
constexpr int kLyNch = kLyChunks + kChunk * kChunkRec * 4;
constexpr int kLyLogits = kLyNch + 16;                             // [T][E] router logits
constexpr int kLyBytes = kLyLogits + kLayerMaxLogits * 4;
static_assert(kLayerMaxLogits % kThreads == 0, "whole logit loads per thread");
static_assert(kLySc % 16 == 0 && kLyKeys % 8 == 0 && sizeof(route::RankScratch<1>) % 16 == 0, "LDS alignment");

// Workgroup barrier ordering LDS accesses only (no wait for outstanding
// global memory operations).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait (one lane) until *p >= target; false once a wait of this call gave
// up (its error word holds `tag`), or when the poll limit runs out (then
// this one raises it).
__device__ bool layer_wait(const LayerArgs& a, const int32_t* p, int32_t target, int32_t tag) {
    for (int i = 0;; ++i) {
        if (a.spin_limit >= 0 && load_agent(p) >= target) return true;
        if (i % 32 == 31 && load_agent(a.st + kLayerError) == tag) return false;
        if (i >= a.spin_limit) {
            __hip_atomic_store(a.st + kLayerError, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

// NV: logits per lane of a routing wave (E <= 64 * NV): ranking for one, as
// the routing launches do up to 64 experts; k argmax rounds for two, as they
// do up to 128.
template <int RT, int DG, int DD, int NV>
__global__ __launch_bounds__(kThreads, 2) void k_layer(LayerArgs a) {
    static_assert(NV == 1 || NV == 2, "up to 128 experts");
    constexpr int kRing = DG > DD ? DG : DD;
    // one LDS object (see k_fused): the unit ring, then the block's routing
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * kSlot + kLyBytes];
    uint8_t* ly = lds + kRing * kSlot;
    int32_t* s_words = reinterpret_cast<int32_t*>(ly + kLyWords);
    route::RankScratch<1>* sc = reinterpret_cast<route::RankScratch<1>*>(ly + kLySc);
    int32_t* s_ids = reinterpret_cast<int32_t*>(ly + kLyIds);
    float* s_wts = reinterpret_cast<float*>(ly + kLyWts);
    int32_t* s_off = reinterpret_cast<int32_t*>(ly + kLyOff);
    int32_t* s_act = reinterpret_cast<int32_t*>(ly + kLyAct);
    int32_t* s_sorted = reinterpret_cast<int32_t*>(ly + kLySorted);
    int32_t* s_chunks = reinterpret_cast<int32_t*>(ly + kLyChunks);
    int32_t* s_nch = reinterpret_cast<int32_t*>(ly + kLyNch);
    float* s_lg = reinterpret_cast<float*>(ly + kLyLogits);
    const Dims dm = a.dm;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

    // The block's logits (up to kLayerMaxLogits / kThreads per thread) into
    // LDS; then lane 0 takes the first ticket and reads the epoch, whose
    // results are used only after the routing and the permutation.  Until
    // then the workgroup meets at barriers that order LDS only: a barrier
    // that also ordered global memory would wait for the atomic, which every
    // workgroup issues at once.
    constexpr int kLg = kLayerMaxLogits / kThreads;
    float lgv[kLg];
#pragma unroll
    for (int q = 0; q < kLg; ++q) {
        const int i = tid + q * kThreads;
        lgv[q] = i < dm.T * dm.E ? a.logits[i] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kLg; ++q) s_lg[tid + q * kThreads] = lgv[q];
    int first = 0, epoch = 0;
    if (tid == 0) {
        first = __hip_atomic_fetch_add(a.st + kLayerQueue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        epoch = load_agent(a.st + kLayerEpoch);
    }
    lds_barrier();
    // one wave per token ranks its logits, then wave 0 permutes the pairs
    for (int t = wave; t < dm.T; t += kWaves) {
        if constexpr (NV == 1)
            route::route_token_rank<1>(s_lg, dm, t, lane, sc[wave], s_ids, s_wts, nullptr);
        else
            route::route_token_argmax<NV>(s_lg, dm, t, lane, s_ids, s_wts);
    }
    lds_barrier();
    if (wave == 0) {
        int32_t* cnt = reinterpret_cast<int32_t*>(ly + kLyCnt);
        int32_t* exo = reinterpret_cast<int32_t*>(ly + kLyExo);
        if constexpr (NV == 1)
            route::sort_wave(dm, s_ids, cnt, exo, reinterpret_cast<uint64_t*>(ly + kLyKeys), lane, s_off, s_sorted,
                             s_act, s_chunks, s_nch, nullptr, 0);
        else
            route::sort_wave2(dm, s_ids, cnt, exo, reinterpret_cast<int32_t*>(ly + kLyKeys), lane, s_off, s_sorted,
                              s_act, s_chunks, s_nch);
    }
    if (tid == 0) {
        s_words[1] = first;
        s_words[2] = epoch;
    }
    lds_barrier();
    const int nc = __builtin_amdgcn_readfirstlane(*s_nch);
    const int32_t tag = __builtin_amdgcn_readfirstlane(s_words[2]) + 1;
    if (blockIdx.x == 0) {
        for (int i = tid; i < dm.P; i += kThreads) {
            a.ids[i] = s_ids[i];
            a.wts[i] = s_wts[i];
            a.sorted[i] = s_sorted[i];
        }
        for (int i = tid; i < dm.E; i += kThreads) a.offsets[i] = s_off[i];
        for (int i = tid; i < nc; i += kThreads) a.active[i] = s_act[i];
        for (int i = tid; i < nc * kChunkRec; i += kThreads) a.chunks[i] = s_chunks[i];
        if (tid == 0) {
            a.offsets[dm.E] = dm.P;
            a.active[dm.E] = nc;
            *a.nchunks = nc;
        }
    }

    const int nG = nc * a.ntg, nD = nc * a.ntd;
    int v = __builtin_amdgcn_readfirstlane(s_words[1]);
    int next = 0;
    auto take = [&] {
        if (tid == 0) next = __hip_atomic_fetch_add(a.st + kLayerQueue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    while (v < nG) {
        const int chunk = v / a.ntg, nt = v % a.ntg;
        const int32_t* rec = s_chunks + kChunkRec * chunk;
        const int e = __builtin_amdgcn_readfirstlane(rec[0]);
        const int m0 = __builtin_amdgcn_readfirstlane(rec[1]);
        const int rows = __builtin_amdgcn_readfirstlane(rec[2]);
        stream::run_unit<kGateUp, RT, DG, true>(a.gu, lds, e, nt, s_sorted + m0, m0, rows, [] {}, take);
        publish(a.st + kLayerChunkDone + kLayerLine * chunk);
        if (tid == 0) s_words[1] = next;
        __syncthreads();
        v = __builtin_amdgcn_readfirstlane(s_words[1]);
    }
    while (v < nG + nD) {
        const int w = v - nG;
        const int chunk = w / a.ntd, nt = w % a.ntd;
        const int32_t* rec = s_chunks + kChunkRec * chunk;
        const int e = __builtin_amdgcn_readfirstlane(rec[0]);
        const int m0 = __builtin_amdgcn_readfirstlane(rec[1]);
        const int rows = __builtin_amdgcn_readfirstlane(rec[2]);
        if (tid == 0) {
            const bool ok = layer_wait(a, a.st + kLayerChunkDone + kLayerLine * chunk, a.ntg, tag);
            if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_words[0] = ok;
        }
        __syncthreads();
        if (!__builtin_amdgcn_readfirstlane(s_words[0])) return;
        stream::run_unit<kDown, RT, DD>(a.dn, lds, e, nt, s_sorted + m0, m0, rows, [] {}, take);
        if (tid == 0) s_words[1] = next;
        __syncthreads();               // s_words[1] holds the next ticket; the LDS ring is free again
        v = __builtin_amdgcn_readfirstlane(s_words[1]);
    }
}

__global__ void k_layer_clear(int32_t* st) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < kLayerStateInts; i += gridDim.x * blockDim.x) st[i] = 0;
}

template <int NV, int DG, int DD>
hipError_t launch_layer_variant(const LayerArgs& a, int items, hipStream_t s) {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (cached[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_layer<2, DG, DD, NV>),
                                                         kThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidValue;
        cached[dev] = per_cu * cus > 0 ? per_cu * cus : 1;
    }
    const int grid = items < cached[dev] ? items : cached[dev];
    hipLaunchKernelGGL((k_layer<2, DG, DD, NV>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int RT, int DG, int DD>
hipError_t launch_chain(const FusedArgs& f, const Dims& dm, hipStream_t s) {
    // every counter gets xstride * (ntg + ntd) workgroups: at least the
    // units of the longest list
    const dim3 grid(kXcds * f.xstride * (f.ntg + f.ntd));
    hipLaunchKernelGGL((k_chain<RT, DG, DD>), grid, dim3(kThreads), 0, s, f);
    return hipGetLastError();
}

template <int RT, int DG, int DD>
hipError_t launch_variant(const FusedArgs& f, int items, hipStream_t s) {
    // grid = the workgroups the GPU holds at once (no more are useful: each
    // loops over items), found once per device
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (cached[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_fused<RT, DG, DD>),
                                                         kThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidValue;
        cached[dev] = per_cu * cus > 0 ? per_cu * cus : 1;
    }
    const int grid = items < cached[dev] ? items : cached[dev];
    hipLaunchKernelGGL((k_fused<RT, DG, DD>), dim3(grid), dim3(kThreads), 0, s, f);
    return hipGetLastError();
}

}  // namespace
}  // namespace fused

int fused_ctl_ints(const Dims& dm) { return fused::kChunkDone + fused::kLine * max_chunks(dm); }

bool fused_supported(const Dims& dm) { return dm.P <= kFusedMaxPairs; }

namespace fused {
namespace {

FusedArgs make_args(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws,
                    int spin_limit) {
    using namespace stream;
    FusedArgs f{};
    const int RT = tiles_per_wave(dm);
    f.gu.act = reinterpret_cast<const uint8_t*>(x);
    f.gu.w0 = w.w_gate; f.gu.s0 = w.w_gate_scale;
    f.gu.w1 = w.w_up;   f.gu.s1 = w.w_up_scale;
    f.gu.h_out = ws.h;
    f.gu.K = dm.d; f.gu.N = dm.f; f.gu.k_top = dm.k; f.gu.ldo = dm.f;
    f.dn.act = ws.h;
    f.dn.w0 = w.w_down; f.dn.s0 = w.w_down_scale;
    f.dn.o_out = ws.o;
    f.dn.K = dm.f; f.dn.N = dm.d; f.dn.k_top = dm.k; f.dn.ldo = dm.d;
    f.ctl = ws.fctl;
    f.sorted = ws.sorted_pairs; f.chunks = ws.chunks; f.nchunks = ws.nchunks;
    f.ntg = RT == 2 ? col_tiles<kGateUp, 2>(dm.f) : col_tiles<kGateUp, 4>(dm.f);
    f.ntd = RT == 2 ? col_tiles<kDown, 2>(dm.d) : col_tiles<kDown, 4>(dm.d);
    f.gu.n_tiles = f.ntg;
    f.dn.n_tiles = f.ntd;
    f.spin_limit = spin_limit;
    f.xtab = ws.xtab;
    f.xstride = xcd_slots(dm);
    return f;
}

}  // namespace
}  // namespace fused


// The ticketed form wins where experts have several pairs (256 tokens:
// 138 against 151 us for the persistent kernel, 145 for the per-phase
// launches); at most one pair per expert on average the persistent kernel
// (74 against 78 us at 8 tokens), whose grid is only the resident
// workgroups.
bool fused_chain_form(const Dims& dm) { return dm.P > dm.E; }

hipError_t launch_fused(const uint16_t* x, const moe_mxfp4_weights& w, const Dims& dm, const Workspace& ws,
                        int spin_limit, hipStream_t s) {
    using namespace stream;
    const fused::FusedArgs f = fused::make_args(x, w, dm, ws, spin_limit);
    const int RT = tiles_per_wave(dm);
    if (fused_chain_form(dm)) {
        const bool g4 = (dm.d / kKStep) % 4 == 0, d4 = (dm.f / kKStep) % 4 == 0;
        if (RT == 2) {
            if (g4 && d4) return fused::launch_chain<2, 4, 4>(f, dm, s);
            if (g4) return fused::launch_chain<2, 4, 2>(f, dm, s);
            if (d4) return fused::launch_chain<2, 2, 4>(f, dm, s);
            return fused::launch_chain<2, 2, 2>(f, dm, s);
        }
        if (g4 && d4) return fused::launch_chain<4, 4, 4>(f, dm, s);
        if (g4) return fused::launch_chain<4, 4, 2>(f, dm, s);
        if (d4) return fused::launch_chain<4, 2, 4>(f, dm, s);
        return fused::launch_chain<4, 2, 2>(f, dm, s);
    }
    const int items = max_chunks(dm) * (f.ntg + f.ntd);
    const bool g4 = (dm.d / kKStep) % 4 == 0, d4 = (dm.f / kKStep) % 4 == 0;
    if (RT == 2) {
        if (g4 && d4) return fused::launch_variant<2, 4, 4>(f, items, s);
        if (g4) return fused::launch_variant<2, 4, 2>(f, items, s);
        if (d4) return fused::launch_variant<2, 2, 4>(f, items, s);
        return fused::launch_variant<2, 2, 2>(f, items, s);
    }
    if (g4 && d4) return fused::launch_variant<4, 4, 4>(f, items, s);
    if (g4) return fused::launch_variant<4, 4, 2>(f, items, s);
    if (d4) return fused::launch_variant<4, 2, 4>(f, items, s);
    return fused::launch_variant<4, 2, 2>(f, items, s);
}

bool layer_supported(const Dims& dm) {
    return dm.E <= 2 * kWave && dm.P <= kChunk && dm.P <= dm.E && stream::tiles_per_wave(dm) == 2 &&
           dm.T * dm.E <= kLayerMaxLogits;
}

hipError_t launch_layer(const uint16_t* x, const float* logits, const moe_mxfp4_weights& w, const Dims& dm,
                        const Workspace& ws, int32_t* state, int spin_limit, hipStream_t s) {
    if (!layer_supported(dm)) return hipErrorInvalidValue;
    const fused::FusedArgs f = fused::make_args(x, w, dm, ws, spin_limit);
    fused::LayerArgs a{};
    a.gu = f.gu;
    a.dn = f.dn;
    a.logits = logits;
    a.dm = dm;
    a.st = state;
    a.ids = ws.topk_ids; a.wts = ws.topk_w; a.offsets = ws.offsets; a.sorted = ws.sorted_pairs;
    a.active = ws.active; a.chunks = ws.chunks; a.nchunks = ws.nchunks;
    a.ntg = f.ntg;
    a.ntd = f.ntd;
    a.spin_limit = spin_limit;
    // every active expert is one chunk
    const int items = (dm.P < dm.E ? dm.P : dm.E) * (a.ntg + a.ntd);
    const bool g4 = (dm.d / kKStep) % 4 == 0, d4 = (dm.f / kKStep) % 4 == 0;
    if (dm.E > kWave) {
        if (g4 && d4) return fused::launch_layer_variant<2, 4, 4>(a, items, s);
        if (g4) return fused::launch_layer_variant<2, 4, 2>(a, items, s);
        if (d4) return fused::launch_layer_variant<2, 2, 4>(a, items, s);
        return fused::launch_layer_variant<2, 2, 2>(a, items, s);
    }
    if (g4 && d4) return fused::launch_layer_variant<1, 4, 4>(a, items, s);
    if (g4) return fused::launch_layer_variant<1, 4, 2>(a, items, s);
    if (d4) return fused::launch_layer_variant<1, 2, 4>(a, items, s);
    return fused::launch_layer_variant<1, 2, 2>(a, items, s);
}

hipError_t launch_layer_clear(int32_t* state, hipStream_t s) {
    hipLaunchKernelGGL(fused::k_layer_clear, dim3(16), dim3(256), 0, s, state);
    return hipGetLastError();
}

}  // namespace moe
