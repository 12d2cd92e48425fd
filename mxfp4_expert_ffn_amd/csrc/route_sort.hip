// Top-k routing and the token -> expert permutation.
//
// Routing: techllm.github.io "Xiaomi MiMo x TileRT", section "3. TileRT",
// names the expert-routing step whose pattern the runtime knows ahead; the
// pages give no rule, so: the k largest logits (ties to the lower expert
// index), weights = softmax over the k selected logits.  Up to 64 experts,
// a wave ranks all of a token's logits at once (each lane counts the logits
// that beat its own); beyond that, k rounds of a wave-wide argmax.
//
// Permutation: a stable counting sort of the pairs p = t*k + j by expert,
// built from wavefront ballots (lanes holding the same expert find each
// other with one ballot per expert-id bit), per-wave LDS histograms and a
// prefix scan.  Positions never come from atomics, so the order is
// deterministic; the only atomic adds sum integer ranks, whose total does not
// depend on their order.  Sizes: up to 64 pairs, one wave after the routing
// in the same launch; up to 8192, one workgroup (fused with the routing for
// up to 16 tokens); beyond, tiles of 2048 pairs in three launches.
#include "route_core.hpp"

#include <float.h>
#include <limits.h>

namespace moe {
namespace {

using namespace route;

constexpr int kRouteWaves = 4;          // tokens per routing workgroup
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kPrefetch = 8;            // rounds of pair ids loaded ahead per wave

// One wavefront per token, E <= 64 * NV.
// Clear zero[0 .. nzero) with every thread of the grid (the persistent
// kernel's work counters, which must start at zero in every call).
__device__ __forceinline__ void clear_counters(int32_t* __restrict__ zero, int nzero) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nzero; i += gridDim.x * blockDim.x) zero[i] = 0;
}

template <int NV>
__global__ __launch_bounds__(kRouteWaves * kWave) void k_route_rank(const float* __restrict__ logits,
                                                                    Dims dm, int32_t* __restrict__ ids,
                                                                    float* __restrict__ wts,
                                                                    int32_t* __restrict__ zero, int nzero) {
    __shared__ RankScratch<NV> sc[kRouteWaves];
    clear_counters(zero, nzero);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kRouteWaves + wave;
    if (t >= dm.T) return;                       // whole wave exits; waves share no LDS
    route_token_rank<NV>(logits, dm, t, lane, sc[wave], ids, wts, nullptr);
}

// One wavefront per token, E <= 64 * NV.  Lane l holds logits l, l+64, ...
template <int NV>
__global__ __launch_bounds__(kRouteWaves * kWave) void k_route(const float* __restrict__ logits,
                                                               Dims dm, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts,
                                                               int32_t* __restrict__ zero, int nzero) {
    clear_counters(zero, nzero);
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kRouteWaves + threadIdx.x / kWave;
    if (t >= dm.T) return;                       // whole wave exits together
    route_token_argmax<NV>(logits, dm, t, lane, ids, wts);
}


// Bitmask of the lanes of this wave whose `key` equals mine (valid lanes only).
__device__ __forceinline__ uint64_t match_peers(int key, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Visit the pairs [p0, p1) of one wave in ascending order, kPrefetch rounds
// of 64 at a time (their id loads overlap), and call f(valid, e, rank,
// peers, p) per lane and pair: rank = lanes of this round before it with the
// same expert, peers = those lanes' mask.  keep: the round's ids, reused
// instead of reloading when `reuse` (one round per wave).
template <typename F>
__device__ __forceinline__ void wave_pairs(const int32_t* __restrict__ ids, int p0, int p1, int nbits, int lane,
                                           bool reuse, int (&keep)[kPrefetch], F&& f) {
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int base = p0; base < p1; base += kPrefetch * kWave) {
        if (!reuse) {
#pragma unroll
            for (int q = 0; q < kPrefetch; ++q) {
                const int p = base + q * kWave + lane;
                keep[q] = p < p1 ? ids[p] : 0;
            }
        }
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            if (base + q * kWave >= p1) break;            // uniform: past this wave's pairs
            const int p = base + q * kWave + lane;
            const bool valid = p < p1;
            const uint64_t peers = match_peers(keep[q], valid, nbits);
            f(valid, keep[q], __popcll(peers & lt_mask), __popcll(peers), p);
        }
    }
}


// From the per-expert pair counts (LDS counts[E4], zero past E) of all P
// pairs, with every thread of a kSortThreads workgroup: expert offsets
// [E+1] (also left in LDS exoff[E]), the active experts by descending count
// (ties to the lower index) with their number at active[E], and the chunk
// records, expert by expert in that order, with their number.  Returns the
// exclusive offset of expert `threadIdx.x` (0 past E).  LDS: keys[E] +
// act[E] + rnk[E] + exoff[E] + 32 ints of scratch.
__device__ int expert_lists(const int32_t* counts, uint64_t* keys, int32_t* act, int32_t* rnk, int32_t* exoff,
                            int32_t* wsum, int E, int P, int chunk_rows,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                            int32_t* __restrict__ chunks, int32_t* __restrict__ nchunks,
                            int32_t* __restrict__ xtab, int xstride) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    int32_t* wsum2 = wsum + kSortWaves;
    // exclusive scan of counts over experts (E <= 512 <= 1024 threads), and
    // each expert's unique ranking key: pair count, then lower index first
    const int c = tid < E ? counts[tid] : 0;
    if (tid < E) {
        keys[tid] = ((uint64_t)(uint32_t)c << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)tid);
        rnk[tid] = 0;
    }
    const int incl = wave_inclusive_scan(c, lane);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - c;
    if (tid < E) {
        offsets[tid] = excl;
        exoff[tid] = excl;
    }
    // rank of an active expert = number of experts whose key is larger,
    // counted in slices: thread (slice j, expert e) compares key e with the
    // keys of slice j and adds what it finds to rnk[e] (integer adds: the
    // total does not depend on their order)
    {
        const int ep = (E + kWave - 1) / kWave * kWave;    // experts rounded up to whole waves
        const int nsl = kSortThreads / ep;                  // slices, >= 2 (E <= 512)
        const int e = tid % ep, j = tid / ep;
        if (e < E && j < nsl && counts[e] > 0) {
            const uint64_t mine = keys[e];
            const int len = (E + nsl - 1) / nsl;
            const int hi = min(E, (j + 1) * len);
            int r = 0;
            for (int e2 = j * len; e2 < hi; ++e2) r += keys[e2] > mine;
            if (r > 0) atomicAdd(&rnk[e], r);
        }
    }
    // number of active experts = number of nonzero counts
    const int nz = __popcll(__ballot(tid < E && c > 0));
    if (lane == 0) wsum2[wave] = nz;
    __syncthreads();
    int na = 0;
    for (int w = 0; w < kSortWaves; ++w) na += wsum2[w];
    if (tid == 0) {
        offsets[E] = P;
        active[E] = na;
    }
    if (tid < E && c > 0) {
        const int r = rnk[tid];
        active[r] = tid;
        act[r] = tid;
    }
    __syncthreads();                                   // act[] complete (and wsum's reads done)
    // work chunks of <= chunk_rows pairs, expert by expert in rank order
    const int nch = tid < na ? (counts[act[tid]] + chunk_rows - 1) / chunk_rows : 0;
    const int nincl = wave_inclusive_scan(nch, lane);
    if (lane == kWave - 1) wsum[wave] = nincl;
    __syncthreads();
    int cbefore = 0;
    for (int w = 0; w < wave; ++w) cbefore += wsum[w];
    if (tid < na) {
        // record: expert, position of the chunk's first pair in sorted_pairs,
        // pairs in the chunk, 0
        const int first = cbefore + nincl - nch;
        const int e = act[tid], n = counts[e], base = exoff[e];
        for (int q = 0; q < nch; ++q) {
            int32_t* rec = chunks + kChunkRec * (first + q);
            rec[0] = e;
            rec[1] = base + q * chunk_rows;
            rec[2] = min(chunk_rows, n - q * chunk_rows);
            rec[3] = 0;
        }
        rnk[tid] = first;                              // ranks are no longer needed: first chunk of rank tid
    }
    if (tid == kSortThreads - 1) *nchunks = cbefore + nincl;
    __syncthreads();
    // per-XCD chunk table: the experts in rank order (chunk counts never
    // increase with rank), each to the XCD with the fewest chunks so far,
    // the lowest index on ties -- greedy list scheduling, whose largest list
    // holds at most floor(nchunks / kXcds) plus one expert's chunks.  Equal
    // counts come in runs, and greedy deals a run to the XCDs at the lowest
    // load one each, in index order, before any load above it: so wave 0
    // places the experts in rounds, one expert per XCD at the lowest load,
    // or whole levels of a run when every XCD is at the lowest load (lane
    // x < kXcds holds XCD x's load, lane i the count of rank r0 + i of the
    // current block of ranks).  keys[] (free after the ranking) receives
    // each rank's (XCD << 24 | first slot).
    int32_t* xasg = reinterpret_cast<int32_t*>(keys);
    if (wave == 0) {
        int load = 0;                                   // lane x < kXcds: XCD x's chunks so far
        for (int r0 = 0; r0 < na; r0 += kWave) {
            const int rr = r0 + lane;
            const int mv = rr < na ? (counts[act[rr]] + chunk_rows - 1) / chunk_rows : 0;
            const int nb = min(kWave, na - r0);
            int pos = 0;                                // next rank of the block to place
            while (pos < nb) {
                const int m = __builtin_amdgcn_readlane(mv, pos);
                // the run of ranks with this count, from pos to the block's end at most
                const uint64_t run = __ballot(lane >= pos && lane < nb && mv == m);
                const int nrun = (int)__builtin_popcountll(run);
                // the XCDs at the lowest load (lane reads into scalar
                // registers, not cross-lane shuffles through LDS)
                int lo = __builtin_amdgcn_readlane(load, 0);
#pragma unroll
                for (int k = 1; k < kXcds; ++k) lo = min(lo, __builtin_amdgcn_readlane(load, k));
                const uint64_t takers = __ballot(lane < kXcds && load == lo);
                const int ntake = (int)__builtin_popcountll(takers);
                if (ntake == kXcds && nrun >= kXcds) {
                    // every XCD at the lowest load: greedy deals whole levels
                    // of the run, item p to XCD p mod kXcds at load lo +
                    // (p / kXcds) m, so place them in one round
                    const int lv = nrun / kXcds, p = lane - pos;
                    if (p >= 0 && p < lv * kXcds) xasg[r0 + lane] = ((p % kXcds) << 24) | (lo + (p / kXcds) * m);
                    if (lane < kXcds) load += lv * m;
                    pos += lv * kXcds;
                    continue;
                }
                const int before = (int)__builtin_popcountll(takers & ((1ull << lane) - 1));   // lower-indexed takers
                const int cnt = ntake < nrun ? ntake : nrun;
                if (lane < kXcds && load == lo && before < cnt) {
                    xasg[r0 + pos + before] = (lane << 24) | load;
                    load += m;
                }
                pos += cnt;
            }
        }
        if (lane < kXcds) xtab[lane] = load;
    }
    __syncthreads();
    if (tid < na) {
        const int a = xasg[tid], x = a >> 24, slot = a & 0xFFFFFF;
        const int e = act[tid], n = counts[e];
        const int m = (n + chunk_rows - 1) / chunk_rows;
        int32_t* rec = xtab + kXtabHead + kXtabRec * ((size_t)x * xstride + slot);
        for (int q = 0; q < m; ++q) {
            rec[kXtabRec * q + 0] = e;
            rec[kXtabRec * q + 1] = exoff[e] + q * chunk_rows;
            rec[kXtabRec * q + 2] = min(chunk_rows, n - q * chunk_rows);
            rec[kXtabRec * q + 3] = rnk[tid] + q;    // the chunk's index in the global list
            rec[kXtabRec * q + 4] = q;
            rec[kXtabRec * q + 5] = m;
        }
    }
    return tid < E ? excl : 0;
}

// LDS of the single-workgroup sort: keys[E] (8 bytes) + hist[kSortWaves][E]
// + counts[E rounded up to 4] + act[E] + rnk[E] + exoff[E] + 32 ints,
// rounded up to 16 bytes.
__host__ __device__ inline size_t sort_lds_bytes(int E) {
    const size_t E4 = (size_t)(E + 3) & ~(size_t)3;
    const size_t b = sizeof(uint64_t) * E + sizeof(int32_t) * (kSortWaves * (size_t)E + E4 + 3 * (size_t)E + 2 * kSortWaves);
    return (b + 15) & ~(size_t)15;
}

// The permutation by one kSortThreads workgroup, up to kSortSingleMax pairs,
// ids read from `ids` (global or LDS); sm64: the LDS of sort_lds_bytes(E).
__device__ __forceinline__ void sort_single(const Dims& dm, const int32_t* __restrict__ ids, uint64_t* sm64,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                            int32_t* __restrict__ active, int32_t* __restrict__ chunks,
                            int32_t* __restrict__ nchunks, int chunk_rows, int32_t* __restrict__ xtab,
                            int xstride) {
    const int E = dm.E, P = dm.P;
    const int E4 = (E + 3) & ~3;
    uint64_t* keys = sm64;                            // [E]
    int32_t* sm = reinterpret_cast<int32_t*>(sm64 + E);
    int32_t* hist = sm;                               // [kSortWaves][E]
    int32_t* counts = sm + kSortWaves * E;            // [E4], zero past E
    int32_t* act = counts + E4;                       // [E] active experts in rank order
    int32_t* rnk = act + E;                           // [E] their ranks
    int32_t* exoff = rnk + E;                         // [E] expert offsets
    int32_t* wsum = exoff + E;                        // [32]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

    for (int i = tid; i < kSortWaves * E; i += kSortThreads) hist[i] = 0;
    __syncthreads();

    const int nbits = id_bits(E);
    const int per_wave = ((P + kSortWaves * kWave - 1) / (kSortWaves * kWave)) * kWave;
    const int p0 = wave * per_wave;
    const int p1 = min(P, p0 + per_wave);
    int32_t* my = hist + wave * E;
    // a wave whose pairs fit one prefetch round keeps their ids in registers
    // for the scatter instead of loading them again
    const bool one_round = per_wave <= kPrefetch * kWave;
    int keep[kPrefetch];

    // 1) per-wave histograms
    wave_pairs(ids, p0, p1, nbits, lane, false, keep,
               [&](bool valid, int e, int rank, int n, int) { if (valid && rank == 0) my[e] += n; });
    __syncthreads();

    // 2) per-expert totals; hist[w][e] becomes the count of waves before w
    for (int e = tid; e < E; e += kSortThreads) {
        int v[kSortWaves];
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) v[w] = hist[w * E + e];
        int run = 0;
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) {
            hist[w * E + e] = run;
            run += v[w];
        }
        counts[e] = run;
    }
    if (tid >= E && tid < E4) counts[tid] = 0;
    __syncthreads();
    expert_lists(counts, keys, act, rnk, exoff, wsum, E, P, chunk_rows, offsets, active, chunks, nchunks, xtab,
                 xstride);

    // 3) scatter in the same visiting order: stable within each expert
    //    (position = expert offset + pairs of earlier waves and rounds + rank)
    wave_pairs(ids, p0, p1, nbits, lane, one_round, keep,
               [&](bool valid, int e, int rank, int n, int p) {
                   if (valid) {
                       sorted[exoff[e] + my[e] + rank] = p;
                       if (rank == 0) my[e] += n;
                   }
               });
}

__global__ __launch_bounds__(kSortThreads) void k_sort(Dims dm, const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ chunks,
                                                       int32_t* __restrict__ nchunks, int chunk_rows,
                                                       int32_t* __restrict__ xtab, int xstride) {
    extern __shared__ uint64_t sm64[];
    sort_single(dm, ids, sm64, offsets, sorted, active, chunks, nchunks, chunk_rows, xtab, xstride);
}

// Small batches (T <= kFusedMaxTokens, E <= 64): routing and the permutation
// in one workgroup.  Wave w routes token w and keeps its ids in LDS, where
// the sort then reads them: one launch instead of two, and no round trip of
// the ids through memory between them.  One token per wave: ranking a
// token's logits is 64 x 64 compares, and the 16 waves share one CU's four
// SIMDs, so every further token per wave costs about 4 us (22 against 13 us
// for the two launches at 64 tokens), while the routing launch spreads the
// tokens over many CUs.  LDS after the sort's: ids[P] (rounded to 16 bytes),
// then one ranking scratch per wave.
constexpr int kFusedMaxTokens = kSortWaves;

__global__ __launch_bounds__(kSortThreads) void k_route_sort(const float* __restrict__ logits, Dims dm,
                                                             int32_t* __restrict__ ids, float* __restrict__ wts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted,
                                                             int32_t* __restrict__ active,
                                                             int32_t* __restrict__ chunks,
                                                             int32_t* __restrict__ nchunks, int chunk_rows,
                                                             int32_t* __restrict__ xtab, int xstride,
                                                             int32_t* __restrict__ zero, int nzero) {
    extern __shared__ uint64_t sm64[];
    clear_counters(zero, nzero);
    uint8_t* extra = reinterpret_cast<uint8_t*>(sm64) + sort_lds_bytes(dm.E);
    int32_t* ids_lds = reinterpret_cast<int32_t*>(extra);
    RankScratch<1>* sc = reinterpret_cast<RankScratch<1>*>(extra + (((size_t)dm.P * sizeof(int32_t) + 15) & ~(size_t)15));
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    for (int t = wave; t < dm.T; t += kSortWaves) route_token_rank<1>(logits, dm, t, lane, sc[wave], ids, wts, ids_lds);
    __syncthreads();
    sort_single(dm, ids_lds, sm64, offsets, sorted, active, chunks, nchunks, chunk_rows, xtab, xstride);
}


// Batches of at most 64 pairs over at most 64 experts: routing (one wave per
// token) and then sort_wave on wave 0 -- one barrier in all, against the
// single-workgroup sort's barrier per phase.  Block = min(T, 16) waves.
__global__ __launch_bounds__(kSortThreads) void k_route_sort_tiny(const float* __restrict__ logits, Dims dm,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ wts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted,
                                                                  int32_t* __restrict__ active,
                                                                  int32_t* __restrict__ chunks,
                                                                  int32_t* __restrict__ nchunks,
                                                                  int32_t* __restrict__ xtab, int xstride,
                                                                  int32_t* __restrict__ zero, int nzero) {
    __shared__ RankScratch<1> sc[kSortWaves];
    clear_counters(zero, nzero);
    __shared__ int32_t ids_lds[kWave];
    __shared__ int32_t cnt[kWave];
    __shared__ int32_t exo[kWave];
    __shared__ uint64_t keys[kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
    for (int t = wave; t < dm.T; t += nw) route_token_rank<1>(logits, dm, t, lane, sc[wave], ids, wts, ids_lds);
    __syncthreads();
    if (wave == 0)
        sort_wave(dm, ids_lds, cnt, exo, keys, lane, offsets, sorted, active, chunks, nchunks, xtab, xstride);
}

// Many pairs: tiles of kSortTile pairs, one 256-thread workgroup each (the
// 4 waves split the tile in order).  k_sort_hist stores each tile's expert
// histogram; k_sort_scan turns them into every tile's first position per
// expert and writes the expert lists; k_sort_scatter places the pairs.  The
// visiting order is the single-workgroup one (tiles, waves, rounds, lanes in
// pair order), so the result is the same stable permutation.
constexpr int kTileWaves = 4;
constexpr int kSortTile = kTileWaves * kPrefetch * kWave;
static_assert(kSortTile == 2048, "sort_tiles() counts tiles of 2048 pairs");

__global__ __launch_bounds__(kTileWaves * kWave) void k_sort_hist(Dims dm, const int32_t* __restrict__ ids,
                                                                  int32_t* __restrict__ part) {
    extern __shared__ int32_t sm[];                   // [kTileWaves][E]
    const int E = dm.E, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    for (int i = tid; i < kTileWaves * E; i += kTileWaves * kWave) sm[i] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * kSortTile + wave * kPrefetch * kWave;
    const int p1 = min(dm.P, p0 + kPrefetch * kWave);
    int keep[kPrefetch];
    int32_t* my = sm + wave * E;
    wave_pairs(ids, p0, p1, id_bits(E), lane, false, keep,
               [&](bool valid, int e, int rank, int n, int) { if (valid && rank == 0) my[e] += n; });
    __syncthreads();
    for (int e = tid; e < E; e += kTileWaves * kWave) {
        int c = 0;
        for (int w = 0; w < kTileWaves; ++w) c += sm[w * E + e];
        part[(size_t)blockIdx.x * E + e] = c;
    }
}

__global__ __launch_bounds__(kSortThreads) void k_sort_scan(Dims dm, int ntiles, int32_t* __restrict__ part,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ active,
                                                            int32_t* __restrict__ chunks,
                                                            int32_t* __restrict__ nchunks, int chunk_rows,
                                                            int32_t* __restrict__ xtab, int xstride) {
    extern __shared__ uint64_t sm64[];
    const int E = dm.E, E4 = (E + 3) & ~3, tid = threadIdx.x;
    uint64_t* keys = sm64;                            // [E]
    int32_t* sm = reinterpret_cast<int32_t*>(sm64 + E);
    int32_t* counts = sm;                             // [E4]
    int32_t* act = counts + E4;                       // [E]
    int32_t* rnk = act + E;                           // [E]
    int32_t* exoff = rnk + E;                         // [E]
    int32_t* wsum = exoff + E;                        // [32]
    // per expert: exclusive prefix over tiles (tile-major part[b][e])
    if (tid < E) {
        int run = 0;
        int b = 0;
        for (; b + 8 <= ntiles; b += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = part[(size_t)(b + i) * E + tid];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                part[(size_t)(b + i) * E + tid] = run;
                run += v[i];
            }
        }
        for (; b < ntiles; ++b) {
            const int v = part[(size_t)b * E + tid];
            part[(size_t)b * E + tid] = run;
            run += v;
        }
        counts[tid] = run;
    } else if (tid < E4) {
        counts[tid] = 0;
    }
    __syncthreads();
    const int excl = expert_lists(counts, keys, act, rnk, exoff, wsum, E, dm.P, chunk_rows, offsets, active, chunks,
                                  nchunks, xtab, xstride);
    if (tid < E)
        for (int b = 0; b < ntiles; ++b) part[(size_t)b * E + tid] += excl;
}

__global__ __launch_bounds__(kTileWaves * kWave) void k_sort_scatter(Dims dm, const int32_t* __restrict__ ids,
                                                                     const int32_t* __restrict__ part,
                                                                     int32_t* __restrict__ sorted) {
    extern __shared__ int32_t sm[];                   // [kTileWaves][E]
    const int E = dm.E, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    for (int i = tid; i < kTileWaves * E; i += kTileWaves * kWave) sm[i] = 0;
    __syncthreads();
    const int nbits = id_bits(E);
    const int p0 = blockIdx.x * kSortTile + wave * kPrefetch * kWave;
    const int p1 = min(dm.P, p0 + kPrefetch * kWave);
    int keep[kPrefetch];
    int32_t* my = sm + wave * E;
    wave_pairs(ids, p0, p1, nbits, lane, false, keep,
               [&](bool valid, int e, int rank, int n, int) { if (valid && rank == 0) my[e] += n; });
    __syncthreads();
    // my[w][e] <- first position of wave w's pairs of expert e
    for (int e = tid; e < E; e += kTileWaves * kWave) {
        int run = part[(size_t)blockIdx.x * E + e];
        for (int w = 0; w < kTileWaves; ++w) {
            const int c = sm[w * E + e];
            sm[w * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    wave_pairs(ids, p0, p1, nbits, lane, true, keep,
               [&](bool valid, int e, int rank, int n, int p) {
                   if (valid) {
                       sorted[my[e] + rank] = p;
                       if (rank == 0) my[e] += n;
                   }
               });
}

}  // namespace

hipError_t launch_route(const float* logits, const Dims& dm, const Workspace& ws, hipStream_t s, int32_t* zero,
                        int nzero) {
    const int grid = (dm.T + kRouteWaves - 1) / kRouteWaves;
    // ranking costs E compares per logit (each a 4-cycle wave64 VALU op):
    // it wins for one logit per lane; with two (E <= 128) it already takes
    // 1.3-1.4x as long as the k argmax rounds
    if (dm.E <= kWave)
        hipLaunchKernelGGL(k_route_rank<1>, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                           ws.topk_ids, ws.topk_w, zero, nzero);
    else if (dm.E <= 2 * kWave)
        hipLaunchKernelGGL(k_route<2>, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                           ws.topk_ids, ws.topk_w, zero, nzero);
    else if (dm.E <= 4 * kWave)
        hipLaunchKernelGGL(k_route<4>, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                           ws.topk_ids, ws.topk_w, zero, nzero);
    else
        hipLaunchKernelGGL(k_route<8>, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                           ws.topk_ids, ws.topk_w, zero, nzero);
    return hipGetLastError();
}

bool route_sort_fused(const Dims& dm) {
    return dm.E <= kWave && dm.T <= kFusedMaxTokens && dm.P <= kSortSingleMax;
}

hipError_t launch_route_sort(const float* logits, const Dims& dm, const Workspace& ws, int chunk_rows,
                             hipStream_t s, int32_t* zero, int nzero) {
    if (dm.P <= kWave && dm.P <= chunk_rows) {        // dm.E <= 64 holds for every fused batch
        const int waves = dm.T < kSortWaves ? dm.T : kSortWaves;
        hipLaunchKernelGGL(k_route_sort_tiny, dim3(1), dim3(waves * kWave), 0, s, logits, dm, ws.topk_ids,
                           ws.topk_w, ws.offsets, ws.sorted_pairs, ws.active, ws.chunks, ws.nchunks, ws.xtab,
                           xcd_slots(dm), zero, nzero);
        return hipGetLastError();
    }
    const size_t lds = sort_lds_bytes(dm.E) + (((size_t)dm.P * sizeof(int32_t) + 15) & ~(size_t)15) +
                       kSortWaves * sizeof(RankScratch<1>);
    hipLaunchKernelGGL(k_route_sort, dim3(1), dim3(kSortThreads), lds, s, logits, dm, ws.topk_ids, ws.topk_w,
                       ws.offsets, ws.sorted_pairs, ws.active, ws.chunks, ws.nchunks, chunk_rows, ws.xtab,
                       xcd_slots(dm), zero, nzero);
    return hipGetLastError();
}

hipError_t launch_sort(const Dims& dm, const Workspace& ws, int chunk_rows, hipStream_t s) {
    const size_t E = dm.E, E4 = (E + 3) & ~3;
    if (dm.P <= kSortSingleMax) {
        hipLaunchKernelGGL(k_sort, dim3(1), dim3(kSortThreads), sort_lds_bytes(dm.E), s, dm, ws.topk_ids, ws.offsets,
                           ws.sorted_pairs, ws.active, ws.chunks, ws.nchunks,
                           chunk_rows, ws.xtab, xcd_slots(dm));
        return hipGetLastError();
    }
    const int ntiles = sort_tiles(dm.P);
    const size_t tile_lds = sizeof(int32_t) * kTileWaves * E;
    hipLaunchKernelGGL(k_sort_hist, dim3(ntiles), dim3(kTileWaves * kWave), tile_lds, s, dm, ws.topk_ids,
                       ws.sort_part);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(kSortThreads), sizeof(uint64_t) * E + sizeof(int32_t) * (E4 + 3 * E + 2 * kSortWaves), s, dm,
                       ntiles, ws.sort_part, ws.offsets, ws.active, ws.chunks, ws.nchunks, chunk_rows, ws.xtab,
                       xcd_slots(dm));
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(k_sort_scatter, dim3(ntiles), dim3(kTileWaves * kWave), tile_lds, s, dm, ws.topk_ids,
                       ws.sort_part, ws.sorted_pairs);
    return hipGetLastError();
}

}  // namespace moe
