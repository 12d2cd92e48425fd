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

// One wavefront per token, E <= 64 * NV.  Lane l holds logits l and l + 64.
// The rank of logit e is the number of logits that come before it in the
// order (value descending, expert index ascending); the experts of ranks
// 0..k-1 are the selection, already in order.
template <int NV>
__global__ __launch_bounds__(kRouteWaves * kWave) void k_route_rank(const float* __restrict__ logits,
                                                                    Dims dm, int32_t* __restrict__ ids,
                                                                    float* __restrict__ wts) {
    __shared__ float sv[kRouteWaves][NV * kWave];
    __shared__ int32_t sid[kRouteWaves][kMaxTopK];
    __shared__ float sval[kRouteWaves][kMaxTopK];
    __shared__ float sex[kRouteWaves][kMaxTopK];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kRouteWaves + wave;
    if (t >= dm.T) return;                       // whole wave exits; waves share no LDS
    const float* l = logits + (size_t)t * dm.E;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        // padding sorts after every logit: it never beats one (-inf included)
        v[i] = e < dm.E ? l[e] : -INFINITY;
        sv[wave][e] = v[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int rank[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) rank[i] = 0;
    const float4* row = reinterpret_cast<const float4*>(sv[wave]);
#pragma unroll 4
    for (int q = 0; q < NV * kWave / 4; ++q) {
        const float4 u4 = row[q];
        const float u[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e2 = 4 * q + j;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                rank[i] += (u[j] > v[i]) || (u[j] == v[i] && e2 < lane + kWave * i);
        }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        if (e < dm.E && rank[i] < dm.k) {
            sid[wave][rank[i]] = e;
            sval[wave][rank[i]] = v[i];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float ex = 0.0f;
    if (lane < dm.k) {
        ex = expf(sval[wave][lane] - sval[wave][0]);
        sex[wave][lane] = ex;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < dm.k) {
        float sum = 0.0f;
        for (int j = 0; j < dm.k; ++j) sum += sex[wave][j];
        ids[(size_t)t * dm.k + lane] = sid[wave][lane];
        wts[(size_t)t * dm.k + lane] = ex / sum;
    }
}

// One wavefront per token, any E <= 512.  Lane l holds logits l, l+64, ...
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

// Single workgroup.  LDS: hist[kSortWaves][E] + counts[E rounded up to 4]
// + act[E] + 32 ints.
__global__ __launch_bounds__(kSortThreads) void k_sort(Dims dm, const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted,
                                                       const float* __restrict__ topk_w,
                                                       float* __restrict__ sorted_w,
                                                       int32_t* __restrict__ inverse,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ chunks,
                                                       int32_t* __restrict__ nchunks, int chunk_rows) {
    extern __shared__ int32_t sm[];
    const int E = dm.E, P = dm.P;
    int32_t* hist = sm;                               // [kSortWaves][E]
    const int E4 = (E + 3) & ~3;
    int32_t* counts = sm + kSortWaves * E;            // [E4], zero past E
    int32_t* act = counts + E4;                       // [E] active experts in rank order
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
    // a wave whose pairs fit one prefetch round keeps their ids in registers
    // for the scatter instead of loading them again
    const bool one_round = per_wave <= kPrefetch * kWave;
    int keep[kPrefetch];
    float keepw[kPrefetch];

    // 1) per-wave histograms, pairs visited in ascending order; the ids of
    //    kPrefetch rounds are loaded together so that their latencies overlap
    for (int base = p0; base < p1; base += kPrefetch * kWave) {
        int ev[kPrefetch];
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            const int p = base + q * kWave + lane;
            ev[q] = p < p1 ? ids[p] : 0;
            keep[q] = ev[q];
            keepw[q] = p < p1 ? topk_w[p] : 0.0f;
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
    if (tid >= E && tid < E4) counts[tid] = 0;
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
            const int4* c4 = reinterpret_cast<const int4*>(counts);
            for (int q = 0; q < E4 / 4; ++q) {
                const int4 cc = c4[q];
                const int e2 = 4 * q;
                r += (cc.x > c) || (cc.x == c && e2 < tid);
                r += (cc.y > c) || (cc.y == c && e2 + 1 < tid);
                r += (cc.z > c) || (cc.z == c && e2 + 2 < tid);
                r += (cc.w > c) || (cc.w == c && e2 + 3 < tid);
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
    // work chunks of <= chunk_rows pairs, expert by expert in rank order
    const int nch = tid < na ? (counts[act[tid]] + chunk_rows - 1) / chunk_rows : 0;
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
            rec[1] = q * chunk_rows;
            rec[2] = first;
            rec[3] = nch;
        }
    }
    if (tid == kSortThreads - 1) *nchunks = cbefore + nincl;
    __syncthreads();

    // 3) scatter in the same visiting order: stable within each expert
    for (int base = p0; base < p1; base += kPrefetch * kWave) {
        int ev[kPrefetch];
        float wv[kPrefetch];
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            const int p = base + q * kWave + lane;
            ev[q] = one_round ? keep[q] : (p < p1 ? ids[p] : 0);
            wv[q] = one_round ? keepw[q] : (p < p1 ? topk_w[p] : 0.0f);
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
                sorted_w[pos] = wv[q];
                inverse[p] = pos;
            }
            if (valid && rank == 0) my[e] += __popcll(peers);
        }
    }
}

}  // namespace

hipError_t launch_route(const float* logits, const Dims& dm, const Workspace& ws, hipStream_t s) {
    const int grid = (dm.T + kRouteWaves - 1) / kRouteWaves;
    // ranking costs E compares per logit: it wins for one logit per lane;
    // with more, the k argmax rounds are cheaper
    if (dm.E <= kWave)
        hipLaunchKernelGGL(k_route_rank<1>, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                           ws.topk_ids, ws.topk_w);
    else
        hipLaunchKernelGGL(k_route, dim3(grid), dim3(kRouteWaves * kWave), 0, s, logits, dm,
                           ws.topk_ids, ws.topk_w);
    return hipGetLastError();
}

hipError_t launch_sort(const Dims& dm, const Workspace& ws, int chunk_rows, hipStream_t s) {
    const size_t lds = sizeof(int32_t) * ((size_t)kSortWaves * dm.E + ((dm.E + 3) & ~3) + dm.E + 2 * kSortWaves);
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(kSortThreads), lds, s, dm, ws.topk_ids, ws.offsets,
                       ws.sorted_pairs, ws.topk_w, ws.sorted_w, ws.inverse, ws.active, ws.chunks, ws.nchunks, chunk_rows);
    return hipGetLastError();
}

}  // namespace moe
