// Routing of one token by one wavefront and the permutation of a batch of
// at most 64 pairs by one wavefront: shared by the routing launches
// (route_sort.hip) and the expert kernel that routes a verify block itself
// (fused.hip k_layer), which runs them inside every workgroup.
//
// Routing: techllm.github.io "Xiaomi MiMo x TileRT", section "3. TileRT",
// names the expert-routing step; the pages give no rule, so: the k largest
// logits (ties to the lower expert index), weights = softmax over the k
// selected logits.  Permutation: a stable counting sort of the pairs
// p = t*k + j by expert (ballots on the expert-id bits, no atomics), the
// active experts ranked by descending count (ties to the lower index).
#pragma once

#include "common.hpp"

#include <float.h>
#include <limits.h>

namespace moe {
namespace route {

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave LDS scratch of the ranking router.
template <int NV>
struct alignas(16) RankScratch {                 // sk is read two keys at a time
    uint64_t sk[NV * kWave];
    int32_t sid[kMaxTopK];
    float sval[kMaxTopK];
    float sex[kMaxTopK];
};

// The routing order of a logit as one unsigned 64-bit key, larger first:
// the float's bits mapped to an unsigned integer that orders as the floats
// do (the sign bit flipped for positive values, every bit for negative
// ones; -0 taken as +0, which compares equal to it), then the expert index
// inverted, so that of two equal values the lower index comes first.  For
// finite and infinite logits, key order is the order (value descending,
// index ascending) that float compares give; NaN logits are not supported.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Routing of token t by one wavefront, E <= 64 * NV.  Lane l holds logits l
// and l + 64.  The rank of logit e is the number of logits that come before
// it in the order (value descending, expert index ascending), counted with
// one 64-bit key compare per logit (route_key); the experts of ranks
// 0..k-1 are the selection, already in order.  Writes ids/weights of the
// token's k slots (and the ids to ids_lds when given).
template <int NV>
__device__ __forceinline__ void route_token_rank(const float* __restrict__ logits, const Dims& dm, int t, int lane,
                                 RankScratch<NV>& sc, int32_t* __restrict__ ids, float* __restrict__ wts,
                                 int32_t* ids_lds) {
    const float* l = logits + (size_t)t * dm.E;
    float v[NV];
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        // padding sorts after every logit: it never beats one (-inf included)
        v[i] = e < dm.E ? l[e] : -INFINITY;
        key[i] = route_key(v[i], e);
        sc.sk[e] = key[i];
    }
    wave_sync_lds();
    int rank[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) rank[i] = 0;
    typedef __attribute__((ext_vector_type(2))) uint64_t u64x2_t;
    const u64x2_t* row = reinterpret_cast<const u64x2_t*>(sc.sk);
#pragma unroll 8
    for (int q = 0; q < NV * kWave / 2; ++q) {
        const u64x2_t u2 = row[q];
#pragma unroll
        for (int i = 0; i < NV; ++i) rank[i] += (u2.x > key[i]) + (u2.y > key[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        if (e < dm.E && rank[i] < dm.k) {
            sc.sid[rank[i]] = e;
            sc.sval[rank[i]] = v[i];
        }
    }
    wave_sync_lds();
    float ex = 0.0f;
    if (lane < dm.k) {
        ex = expf(sc.sval[lane] - sc.sval[0]);
        sc.sex[lane] = ex;
    }
    wave_sync_lds();
    if (lane < dm.k) {
        // the k terms added in slot order, read four at a time
        float sum = 0.0f;
        const float4* sx = reinterpret_cast<const float4*>(sc.sex);
        for (int j = 0; j < dm.k; j += 4) {
            const float4 s4 = sx[j / 4];
            sum += s4.x;
            if (j + 1 < dm.k) sum += s4.y;
            if (j + 2 < dm.k) sum += s4.z;
            if (j + 3 < dm.k) sum += s4.w;
        }
        const int id = sc.sid[lane];
        ids[(size_t)t * dm.k + lane] = id;
        wts[(size_t)t * dm.k + lane] = ex / sum;
        if (ids_lds) ids_lds[t * dm.k + lane] = id;
    }
    wave_sync_lds();                             // the scratch may be reused for the next token
}


// Wave-wide sum.  Within each row of 16 lanes, DPP moves pair lanes 1 apart,
// then 2 apart (quad permutes), then the two halves of each 8 (half-mirror)
// and of the row (mirror); the four row sums are then read from lanes 0, 16,
// 32, 48.  Every lane gets the same bits: each step adds the partner's
// value, and a + b == b + a.
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// The logit a route_key came from (-0 comes back as +0, which changes no
// difference to another logit but the sign of a zero one, and exp(+-0) = 1).
__device__ __forceinline__ float route_key_value(uint64_t key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// The larger of a lane's key and the key of the lane DPP control CTRL names.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_key(uint64_t k) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > k ? o : k;
}

// The largest key of the wave, in every lane: the pairings of wave_sum within
// each row of 16, then the four row results folded.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    k = dpp_max_key<0xB1>(k);       // quad_perm [1, 0, 3, 2]
    k = dpp_max_key<0x4E>(k);       // quad_perm [2, 3, 0, 1]
    k = dpp_max_key<0x141>(k);      // row_half_mirror
    k = dpp_max_key<0x140>(k);      // row_mirror
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; ++row) {
        const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * row) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 16 * row);
        r = o > r ? o : r;
    }
    return r;
}

// Routing of token t by one wavefront by k rounds of a wave-wide maximum of
// route_keys, E <= 64 * NV (lane l holds logits l, l + 64, ...): the same
// selection as route_token_rank (value descending, index ascending), with
// one 64-bit compare per pairing and no branches, cheaper than ranking once
// a lane holds two or more logits; weights = softmax over the k selected,
// the k terms summed with wave_sum.  Writes ids/weights of the token's k
// slots (global or LDS).  Every key of a logit is above 0, the key of
// padding and of logits already taken.
template <int NV>
__device__ __forceinline__ void route_token_argmax(const float* __restrict__ logits, const Dims& dm, int t, int lane,
                                                   int32_t* __restrict__ ids, float* __restrict__ wts) {
    const float* l = logits + (size_t)t * dm.E;
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        key[i] = e < dm.E ? route_key(l[e], e) : 0;
    }
    int my_id = 0;
    float my_val = 0.0f, top_val = 0.0f;
    for (int j = 0; j < dm.k; ++j) {
        uint64_t b = key[0];
#pragma unroll
        for (int i = 1; i < NV; ++i) b = key[i] > b ? key[i] : b;
        b = wave_max_key(b);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (key[i] == b) key[i] = 0;             // taken
        const float bv = route_key_value(b);
        if (lane == j) {
            my_id = (int)(0xFFFFFFFFu - (uint32_t)b);
            my_val = bv;
        }
        if (j == 0) top_val = bv;
    }
    const float ex = lane < dm.k ? expf(my_val - top_val) : 0.0f;
    const float sum = wave_sum(ex);
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

__device__ __forceinline__ int id_bits(int E) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    return nbits;
}

// The permutation of at most 64 pairs over at most 64 experts by one
// wavefront, with no workgroup barrier: lane p holds pair p, lane e expert e.
// Same outputs as sort_single (a stable counting sort; experts ranked by
// descending count, ties to the lower index).  A chunk never splits, since
// the caller guarantees P <= chunk_rows, so active expert r is chunk record r.
// ids: P expert ids (LDS); scratch: 64 counts, 64 offsets, 64 keys (used as
// 64 ints).  The
// outputs may be global or LDS memory; xtab == nullptr skips the per-XCD table.
__device__ __forceinline__ void sort_wave(const Dims& dm, const int32_t* ids, int32_t* cnt, int32_t* exo,
                                          uint64_t* keys, int lane, int32_t* __restrict__ offsets,
                                          int32_t* __restrict__ sorted, int32_t* __restrict__ active,
                                          int32_t* __restrict__ chunks, int32_t* __restrict__ nchunks,
                                          int32_t* __restrict__ xtab, int xstride) {
    const int E = dm.E, P = dm.P;
    const bool valid = lane < P;
    const int ep = valid ? ids[lane] : 0;
    // lanes holding the same expert: one ballot per id bit
    uint64_t peers = __ballot(valid);
    for (int b = 0, nb = id_bits(E); b < nb; ++b) {
        const bool bit = (ep >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
    const int rank = __popcll(peers & below);          // earlier pairs of the same expert
    cnt[lane] = 0;
    wave_sync_lds();
    if (valid && rank == 0) cnt[ep] = __popcll(peers);
    wave_sync_lds();
    const int c = lane < E ? cnt[lane] : 0;
    const int excl = wave_inclusive_scan(c, lane) - c;
    exo[lane] = excl;
    if (lane < E) offsets[lane] = excl;
    // rank of an active expert in the order (count descending, index
    // ascending) = active experts with a larger count + those with the same
    // count and a lower index.  Lanes of equal count find each other with one
    // ballot per count bit (counts <= 64); a suffix sum over the histogram of
    // counts gives the larger ones.
    uint64_t same = __ballot(c > 0);
    for (int b = 0; b < 7; ++b) {
        const bool bit = (c >> b) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    const int eq_below = __popcll(same & below);
    int32_t* hist = reinterpret_cast<int32_t*>(keys);      // [64]: active experts of count lane + 1
    hist[lane] = 0;
    wave_sync_lds();
    if (c > 0 && eq_below == 0) hist[c - 1] = __popcll(same);
    wave_sync_lds();
    const int h = hist[lane];
    const int hin = wave_inclusive_scan(h, lane);
    const int ge = __builtin_amdgcn_readlane(hin, kWave - 1) - hin + h;   // active experts of count >= lane + 1
    const int gt = __shfl(ge, c < kWave ? c : 0);                          // ... of count > c (c < 64)
    const int r = (c < kWave ? gt : 0) + eq_below;
    const int na = __popcll(__ballot(lane < E && c > 0));
    if (lane < E && c > 0) {
        active[r] = lane;
        int32_t* rec = chunks + kChunkRec * r;
        rec[0] = lane;
        rec[1] = excl;
        rec[2] = c;
        rec[3] = 0;
        // per-XCD table (the layout of expert_lists): one chunk per expert,
        // so the greedy assignment deals rank r to XCD r mod kXcds, slot
        // r / kXcds
        if (xtab) {
            int32_t* xr = xtab + kXtabHead + kXtabRec * ((size_t)(r % kXcds) * xstride + r / kXcds);
            xr[0] = lane;
            xr[1] = excl;
            xr[2] = c;
            xr[3] = r;
            xr[4] = 0;
            xr[5] = 1;
        }
    }
    if (xtab && lane < kXcds) xtab[lane] = na / kXcds + (lane < na % kXcds);
    if (lane == 0) {
        offsets[E] = P;
        active[E] = na;
        *nchunks = na;
    }
    if (valid) sorted[exo[ep] + rank] = lane;
}

}  // namespace route
}  // namespace moe

namespace moe {
namespace route {

// sort_wave for up to 128 experts: lane e holds experts e and e + 64 (the
// same outputs: a stable counting sort, experts ranked by descending count,
// ties to the lower index, each active expert one chunk).  P <= 64, so
// counts fit 7 bits and the ranks come from the same ballots and count
// histogram as sort_wave, per half: an expert of the high half also has
// every low-half expert of its count before it.  ids: P expert ids (LDS);
// scratch: cnt[128], exo[128], hist[128].
__device__ __forceinline__ void sort_wave2(const Dims& dm, const int32_t* ids, int32_t* cnt, int32_t* exo,
                                           int32_t* hist, int lane, int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ sorted, int32_t* __restrict__ active,
                                           int32_t* __restrict__ chunks, int32_t* __restrict__ nchunks) {
    const int E = dm.E, P = dm.P;
    const bool valid = lane < P;
    const int ep = valid ? ids[lane] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0, nb = id_bits(E); b < nb; ++b) {
        const bool bit = (ep >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
    const int rank = __popcll(peers & below);          // earlier pairs of the same expert
    cnt[lane] = 0;
    cnt[lane + kWave] = 0;
    wave_sync_lds();
    if (valid && rank == 0) cnt[ep] = __popcll(peers);
    wave_sync_lds();
    const int c0 = lane < E ? cnt[lane] : 0;
    const int c1 = lane + kWave < E ? cnt[lane + kWave] : 0;
    const int i0 = wave_inclusive_scan(c0, lane), i1 = wave_inclusive_scan(c1, lane);
    const int excl0 = i0 - c0, excl1 = __builtin_amdgcn_readlane(i0, kWave - 1) + i1 - c1;
    exo[lane] = excl0;
    exo[lane + kWave] = excl1;
    if (lane < E) offsets[lane] = excl0;
    if (lane + kWave < E) offsets[lane + kWave] = excl1;
    uint64_t same0 = __ballot(c0 > 0), same1 = __ballot(c1 > 0);
    for (int b = 0; b < 7; ++b) {
        const bool b0 = (c0 >> b) & 1, b1 = (c1 >> b) & 1;
        const uint64_t m0 = __ballot(b0), m1 = __ballot(b1);
        same0 &= b0 ? m0 : ~m0;
        same1 &= b1 ? m1 : ~m1;
    }
    const int eq0 = __popcll(same0 & below), eq1 = __popcll(same1 & below);
    hist[lane] = 0;                                    // [c - 1]: low-half experts of count c
    hist[lane + kWave] = 0;                            // [64 + c - 1]: high-half ones
    wave_sync_lds();
    if (c0 > 0 && eq0 == 0) hist[c0 - 1] = __popcll(same0);
    if (c1 > 0 && eq1 == 0) hist[kWave + c1 - 1] = __popcll(same1);
    wave_sync_lds();
    const int hl = hist[lane], h = hl + hist[lane + kWave];
    const int hin = wave_inclusive_scan(h, lane);
    const int ge = __builtin_amdgcn_readlane(hin, kWave - 1) - hin + h;   // experts of count >= lane + 1
    const int gt0 = __shfl(ge, c0 < kWave ? c0 : 0), gt1 = __shfl(ge, c1 < kWave ? c1 : 0);
    const int lo1 = __shfl(hl, c1 > 0 ? c1 - 1 : 0);                    // low-half experts of count c1
    const int r0 = (c0 < kWave ? gt0 : 0) + eq0;
    const int r1 = (c1 < kWave ? gt1 : 0) + lo1 + eq1;
    const int na = __popcll(__ballot(c0 > 0)) + __popcll(__ballot(c1 > 0));
    if (c0 > 0) {
        active[r0] = lane;
        int32_t* rec = chunks + kChunkRec * r0;
        rec[0] = lane;
        rec[1] = excl0;
        rec[2] = c0;
        rec[3] = 0;
    }
    if (c1 > 0) {
        active[r1] = lane + kWave;
        int32_t* rec = chunks + kChunkRec * r1;
        rec[0] = lane + kWave;
        rec[1] = excl1;
        rec[2] = c1;
        rec[3] = 0;
    }
    if (lane == 0) {
        offsets[E] = P;
        active[E] = na;
        *nchunks = na;
    }
    if (valid) sorted[exo[ep] + rank] = lane;
}

}  // namespace route
}  // namespace moe
