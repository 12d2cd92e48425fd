// Top-k routing and the token -> expert permutation.
//
// Routing: techllm.github.io "Xiaomi MiMo x TileRT", section "3. TileRT",
// names the expert-routing step whose pattern the runtime knows ahead; the
// pages give no rule, so: the k largest logits (ties to the lower expert
// index), weights = softmax over the k selected logits.
//
// Permutation: a stable counting sort of the pairs p = t*k + j by expert,
// built from wavefront ballots (lanes holding the same expert find each
// other with one ballot per expert-id bit), per-wave LDS histograms and a
// prefix scan -- no atomics, so the order is deterministic.
#include "common.hpp"

#include <float.h>
#include <limits.h>

namespace moe {
namespace {

constexpr int kRouteWaves = 4;          // tokens per routing workgroup
constexpr int kMaxPerLane = 8;          // E <= 512
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kPrefetch = 8;            // rounds of pair ids loaded ahead per wave

// One wavefront per token.  Lane l holds logits l, l+64, ...
__global__ __launch_bounds__(kRouteWaves * kWave) void k_route(const float* __restrict__ logits,
                                                               Dims dm, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts) {
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kRouteWaves + threadIdx.x / kWave;
    if (t >= dm.T) return;                       // whole wave exits together
    const float* l = logits + (size_t)t * dm.E;
    float v[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < dm.E ? l[e] : 0.0f;
    }
    uint32_t taken = 0;
    int my_id = 0;
    float my_val = 0.0f, top_val = 0.0f;
    for (int j = 0; j < dm.k; ++j) {
        // best untaken logit of this lane (lowest index on ties: i ascends)
        float bv = -FLT_MAX;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + kWave * i;
            if (e < dm.E && !((taken >> i) & 1u) && (bi == INT_MAX || v[i] > bv)) {
                bv = v[i];
                bi = e;
            }
        }
        // butterfly: every lane ends with the wave-wide best (value desc, index asc)
#pragma unroll
        for (int off = kWave / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi != INT_MAX && (bi == INT_MAX || ov > bv || (ov == bv && oi < bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi % kWave == lane) taken |= 1u << (bi / kWave);
        if (lane == j) {
            my_id = bi;
            my_val = bv;
        }
        if (j == 0) top_val = bv;
    }
    const float ex = lane < dm.k ? expf(my_val - top_val) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane < dm.k) {
        ids[(size_t)t * dm.k + lane] = my_id;
        wts[(size_t)t * dm.k + lane] = ex / sum;
    }
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
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

// Single workgroup.  LDS: hist[kSortWaves][E] + counts[E] + 16 ints.
__global__ __launch_bounds__(kSortThreads) void k_sort(Dims dm, const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted,
                                                       int32_t* __restrict__ inverse,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ chunks,
                                                       int32_t* __restrict__ nchunks) {
    extern __shared__ int32_t sm[];
    const int E = dm.E, P = dm.P;
    int32_t* hist = sm;                               // [kSortWaves][E]
    int32_t* counts = sm + kSortWaves * E;            // [E]
    int32_t* act = counts + E;                        // [E] active experts in rank order
    int32_t* wsum = act + E;                          // [16]
    int32_t* wsum2 = wsum + kSortWaves;               // [16]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    for (int i = tid; i < kSortWaves * E; i += kSortThreads) hist[i] = 0;
    __syncthreads();

    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int per_wave = ((P + kSortWaves * kWave - 1) / (kSortWaves * kWave)) * kWave;
    const int p0 = wave * per_wave;
    const int p1 = min(P, p0 + per_wave);
    int32_t* my = hist + wave * E;

    // 1) per-wave histograms, pairs visited in ascending order; the ids of
    //    kPrefetch rounds are loaded together so that their latencies overlap
    for (int base = p0; base < p1; base += kPrefetch * kWave) {
        int ev[kPrefetch];
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            const int p = base + q * kWave + lane;
            ev[q] = p < p1 ? ids[p] : 0;
        }
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            if (base + q * kWave >= p1) break;            // uniform: past this wave's pairs
            const int p = base + q * kWave + lane;
            const bool valid = p < p1;
            const uint64_t peers = match_peers(ev[q], valid, nbits);
            const int rank = __popcll(peers & lt_mask);
            if (valid && rank == 0) my[ev[q]] += __popcll(peers);
        }
    }
    __syncthreads();

    // 2) per-expert totals; hist[w][e] becomes the count of waves before w
    for (int e = tid; e < E; e += kSortThreads) {
        int run = 0;
        for (int w = 0; w < kSortWaves; ++w) {
            const int c = hist[w * E + e];
            hist[w * E + e] = run;
            run += c;
        }
        counts[e] = run;
    }
    __syncthreads();

    // exclusive scan of counts over experts (E <= 512 <= 1024 threads)
    const int c = tid < E ? counts[tid] : 0;
    const int incl = wave_inclusive_scan(c, lane);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - c;
    if (tid < E) {
        offsets[tid] = excl;
        for (int w = 0; w < kSortWaves; ++w) hist[w * E + tid] += excl;
        // active experts by descending pair count, ties to the lower index
        if (c > 0) {
            int r = 0;
            for (int e2 = 0; e2 < E; ++e2) {
                const int c2 = counts[e2];
                r += (c2 > c) || (c2 == c && e2 < tid);
            }
            active[r] = tid;
            act[r] = tid;
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
    // work chunks of <= kChunk pairs, expert by expert in rank order
    const int nch = tid < na ? (counts[act[tid]] + kChunk - 1) / kChunk : 0;
    const int nincl = wave_inclusive_scan(nch, lane);
    __syncthreads();                                   // wsum is reused below
    if (lane == kWave - 1) wsum[wave] = nincl;
    __syncthreads();
    int cbefore = 0;
    for (int w = 0; w < wave; ++w) cbefore += wsum[w];
    if (tid < na) {
        // record: expert, first pair of the chunk, first chunk of the expert, chunks of the expert
        const int first = cbefore + nincl - nch;
        for (int q = 0; q < nch; ++q) {
            int32_t* rec = chunks + kChunkRec * (first + q);
            rec[0] = act[tid];
            rec[1] = q * kChunk;
            rec[2] = first;
            rec[3] = nch;
        }
    }
    if (tid == kSortThreads - 1) *nchunks = cbefore + nincl;
    __syncthreads();

    // 3) scatter in the same visiting order: stable within each expert
    for (int base = p0; base < p1; base += kPrefetch * kWave) {
        int ev[kPrefetch];
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            const int p = base + q * kWave + lane;
            ev[q] = p < p1 ? ids[p] : 0;
        }
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            if (base + q * kWave >= p1) break;            // uniform: past this wave's pairs
            const int p = base + q * kWave + lane;
            const bool valid = p < p1;
            const int e = ev[q];
            const uint64_t peers = match_peers(e, valid, nbits);
            const int rank = __popcll(peers & lt_mask);
            const int pos = valid ? my[e] + rank : 0;
            if (valid) {
                sorted[pos] = p;
                inverse[p] = pos;
            }
            if (valid && rank == 0) my[e] += __popcll(peers);
        }
    }
}

}  // namespace

hipError_t launch_route(const float* logits, const Dims& dm, const Workspace& ws, hipStream_t s) {
    const int grid = (dm.T + kRouteWaves - 1) / kRouteWaves;
    hipLaunchKernelGGL(k_route, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                       ws.topk_ids, ws.topk_w);
    return hipGetLastError();
}

hipError_t launch_sort(const Dims& dm, const Workspace& ws, hipStream_t s) {
    const size_t lds = sizeof(int32_t) * ((size_t)kSortWaves * dm.E + 2 * dm.E + 2 * kSortWaves);
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(kSortThreads), lds, s, dm, ws.topk_ids, ws.offsets,
                       ws.sorted_pairs, ws.inverse, ws.active, ws.chunks, ws.nchunks);
    return hipGetLastError();
}

}  // namespace moe
