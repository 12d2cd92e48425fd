// DFlash verify acceptance: rejection sampling over a drafted block.
//
// The pages make the verification of a drafted block lossless with a final
// rejection-sampling pass (techllm.github.io "Xiaomi MiMo x TileRT", section
// "2. DFlash") without printing the rule; this is standard speculative
// sampling.  Position j's draft token x is accepted when u_j * p_draft[j][x]
// < p_target[j][x] (float32; a token outside [0, V) is rejected); the first
// rejection ends the block and the next token is drawn from max(0,
// p_target[j] - p_draft[j]) (float32 per element), or from p_target[j] if
// that residual has no positive entry; after G acceptances it is drawn from
// p_target[G].  A draw takes integer weights q_i = rint(2^32 w_i) (zero for
// w_i <= 0 or NaN), S = sum q_i, threshold = floor(S * r24 / 2^24) with r24
// = floor(2^24 r) clamped to [0, 2^24 - 1], and returns the first i whose
// inclusive prefix sum exceeds the threshold.  Integer sums make the result
// independent of the order of the additions, so any split of the row over
// threads gives the same index.
//
// Two launches.  k_block_sums covers the whole chip: workgroup (s, b) takes
// blocks [16 s, 16 s + 16) of sequence b's row (a block is 256 entries, one
// float4 per lane), each of its 4 waves 4 blocks with all loads issued
// before any sum; every wave redoes the G acceptance tests itself (a few
// cached loads) to know which row to read, and one writes the count.
// k_pick, one workgroup per sequence, scans the block sums of its row,
// finds the block that holds the threshold and reads that block again to
// the exact entry; if the residual has no mass it sums the target row
// itself and draws from that.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kBlk = 4 * kWave;            // entries per block sum
constexpr int kBlocksPerWave = 4;
constexpr int kSumWaves = 4;
constexpr int kBlocksPerGroup = kBlocksPerWave * kSumWaves;
constexpr int kPickWaves = 4;
constexpr int kPickThreads = kPickWaves * kWave;

struct AcceptArgs {
    const int32_t* draft;       // [B][G]
    const float* p_draft;       // [B][G][V]
    const float* p_target;      // [B][G+1][V]
    const float* u;             // [B][G]
    const float* r;             // [B]
    int32_t* n_accepted;        // [B]
    int32_t* next_token;        // [B]
    int32_t* jbuf;              // workspace: accepted count per sequence [B]
    uint64_t* bsum;             // workspace: block sums [B][nblk]
    int32_t G, V, nblk;
};

// Accepted prefix length of sequence b, uniform over the wave (lane j tests
// position j; G <= 64).
__device__ __forceinline__ int accept_count(const AcceptArgs& a, int b, int lane) {
    bool reject = false;
    if (lane < a.G) {
        const int x = a.draft[(size_t)b * a.G + lane];
        if (x < 0 || x >= a.V) {
            reject = true;
        } else {
            const float pd = a.p_draft[((size_t)b * a.G + lane) * a.V + x];
            const float pt = a.p_target[((size_t)b * (a.G + 1) + lane) * a.V + x];
            const float up = a.u[(size_t)b * a.G + lane] * pd;
            reject = !(up < pt);
        }
    }
    const uint64_t rej = __ballot(reject);
    return rej ? __ffsll((unsigned long long)rej) - 1 : a.G;
}

// rint(2^32 w) for w > 0, else 0.  Scaling by 2^32 is exact in float32 as
// in double, and so is rounding a float to an integer, so this equals the
// double-precision definition for every w below 2^32.
__device__ __forceinline__ uint64_t qweight(float w) {
    return w > 0.0f ? (uint64_t)__builtin_rintf(w * 4294967296.0f) : 0;
}

// Four consecutive entries starting at i (zero past V).  VEC: V % 4 == 0 and
// 16-byte aligned rows, so the four are all inside or all outside.
template <bool VEC>
__device__ __forceinline__ float4 load4(const float* row, int i, int V) {
    if constexpr (VEC) {
        if (i < V) return *reinterpret_cast<const float4*>(row + i);
        return float4{0.f, 0.f, 0.f, 0.f};
    } else {
        float4 v;
        v.x = i < V ? row[i] : 0.f;
        v.y = i + 1 < V ? row[i + 1] : 0.f;
        v.z = i + 2 < V ? row[i + 2] : 0.f;
        v.w = i + 3 < V ? row[i + 3] : 0.f;
        return v;
    }
}

// Integer weights of four entries: the residual max(0, t - d) (RES) or t.
template <bool RES>
__device__ __forceinline__ void weights4(const float4& t, const float4& d, uint64_t q[4]) {
    if constexpr (RES) {
        q[0] = qweight(t.x - d.x);
        q[1] = qweight(t.y - d.y);
        q[2] = qweight(t.z - d.z);
        q[3] = qweight(t.w - d.w);
    } else {
        q[0] = qweight(t.x);
        q[1] = qweight(t.y);
        q[2] = qweight(t.z);
        q[3] = qweight(t.w);
    }
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint64_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

// Sums of NB consecutive blocks starting at blk0 of one row, written to
// out[blk] (lane 0) for the blocks below nblk.
template <bool VEC, bool RES, int NB>
__device__ __forceinline__ void wave_block_sums(const float* pt, const float* pd, int V, int nblk, int blk0,
                                                uint64_t* out, int lane) {
    float4 t[NB], d[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) t[i] = load4<VEC>(pt, (blk0 + i) * kBlk + 4 * lane, V);
    if constexpr (RES) {
#pragma unroll
        for (int i = 0; i < NB; ++i) d[i] = load4<VEC>(pd, (blk0 + i) * kBlk + 4 * lane, V);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        uint64_t q[4];
        weights4<RES>(t[i], d[i], q);
        const uint64_t s = wave_sum_u64(q[0] + q[1] + q[2] + q[3]);
        if (lane == 0 && blk0 + i < nblk) out[blk0 + i] = s;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kSumWaves * kWave) void k_block_sums(AcceptArgs a) {
    const int b = blockIdx.y, lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int j = accept_count(a, b, lane);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.jbuf[b] = j;
    const float* pt = a.p_target + ((size_t)b * (a.G + 1) + j) * a.V;
    const int blk0 = (blockIdx.x * kSumWaves + wave) * kBlocksPerWave;
    uint64_t* out = a.bsum + (size_t)b * a.nblk;
    if (j < a.G) {
        const float* pd = a.p_draft + ((size_t)b * a.G + j) * a.V;
        wave_block_sums<VEC, true, kBlocksPerWave>(pt, pd, a.V, a.nblk, blk0, out, lane);
    } else {
        wave_block_sums<VEC, false, kBlocksPerWave>(pt, nullptr, a.V, a.nblk, blk0, out, lane);
    }
}

// Finds the block holding the threshold of r among bs[0..nblk) with the
// whole workgroup.  Returns false (uniformly) when the sum is zero; else
// sets blk and thr_in (the threshold minus the mass before that block).
__device__ bool locate(const uint64_t* bs, int nblk, float r, uint64_t* wtot, int* sh_blk, uint64_t* sh_thr,
                       int& blk, uint64_t& thr_in) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int per = (nblk + kPickThreads - 1) / kPickThreads;
    const int lo = min(nblk, tid * per), hi = min(nblk, lo + per);
    uint64_t local = 0;
    for (int k = lo; k < hi; ++k) local += bs[k];
    const uint64_t incl = wave_incl_scan_u64(local, lane);
    if (lane == kWave - 1) wtot[wave] = incl;
    if (tid == 0) *sh_blk = -1;
    __syncthreads();
    uint64_t S = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kPickWaves; ++w) {
        if (w < wave) before += wtot[w];
        S += wtot[w];
    }
    if (S == 0) return false;
    uint64_t r24 = 0;
    if (r > 0.0f) {
        const float f = floorf(r * 16777216.0f);     // exact: a scaled float, then floor
        r24 = f >= 16777215.0f ? 16777215u : (uint64_t)f;
    }
    // floor(S * r24 / 2^24) with a 128-bit product (S < 2^64, r24 < 2^24)
    const uint64_t plo = S * r24, phi = __umul64hi(S, r24);
    const uint64_t thr = (phi << 40) | (plo >> 24);
    const uint64_t excl = before + incl - local;
    if (excl <= thr && thr < excl + local) {
        uint64_t run = excl;
        for (int k = lo; k < hi; ++k) {
            if (thr < run + bs[k]) {
                *sh_blk = k;
                *sh_thr = thr - run;
                break;
            }
            run += bs[k];
        }
    }
    __syncthreads();
    blk = *sh_blk;
    thr_in = *sh_thr;
    return blk >= 0 && blk < nblk;                  // always, as thr < S: one range holds it
}

// First entry of block blk whose prefix within the block exceeds thr_in
// (which is below the block's sum), with one wave.
template <bool VEC, bool RES>
__device__ int pick_in_block(const float* pt, const float* pd, int V, int blk, uint64_t thr_in, int lane) {
    const int i = blk * kBlk + 4 * lane;
    const float4 t = load4<VEC>(pt, i, V);
    float4 d{0.f, 0.f, 0.f, 0.f};
    if constexpr (RES) d = load4<VEC>(pd, i, V);
    uint64_t q[4];
    weights4<RES>(t, d, q);
    const uint64_t mine = q[0] + q[1] + q[2] + q[3];
    const uint64_t incl = wave_incl_scan_u64(mine, lane);
    const uint64_t hit = __ballot(incl > thr_in);
    if (hit == 0) return -1;                         // not reached: thr_in is below the block's sum
    const int l = __ffsll((unsigned long long)hit) - 1;
    // in lane l: the first of its four entries that takes the sum past thr_in
    int idx = i + 3;
    uint64_t run = incl - mine;
    bool done = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        run += q[e];
        if (!done && run > thr_in) {
            idx = i + e;
            done = true;
        }
    }
    return __shfl(idx, l);
}

template <bool VEC>
__global__ __launch_bounds__(kPickThreads) void k_pick(AcceptArgs a) {
    __shared__ uint64_t wtot[kPickWaves];
    __shared__ uint64_t sh_thr;
    __shared__ int sh_blk;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int j = a.jbuf[b];
    const float* pt = a.p_target + ((size_t)b * (a.G + 1) + j) * a.V;
    const float* pd = j < a.G ? a.p_draft + ((size_t)b * a.G + j) * a.V : nullptr;
    uint64_t* bs = a.bsum + (size_t)b * a.nblk;
    const float r = a.r[b];
    int blk = 0;
    uint64_t thr_in = 0;
    bool found = locate(bs, a.nblk, r, wtot, &sh_blk, &sh_thr, blk, thr_in);
    bool res = pd != nullptr;
    if (!found && res) {
        // the residual has no mass: block sums of the target row, then draw
        __syncthreads();                             // every thread has read wtot
        for (int k0 = wave * kBlocksPerWave; k0 < a.nblk; k0 += kPickWaves * kBlocksPerWave)
            wave_block_sums<VEC, false, kBlocksPerWave>(pt, nullptr, a.V, a.nblk, k0, bs, lane);
        __syncthreads();
        found = locate(bs, a.nblk, r, wtot, &sh_blk, &sh_thr, blk, thr_in);
        res = false;
    }
    if (wave != 0) return;
    int tok = -1;
    if (found) tok = res ? pick_in_block<VEC, true>(pt, pd, a.V, blk, thr_in, lane)
                         : pick_in_block<VEC, false>(pt, nullptr, a.V, blk, thr_in, lane);
    if (lane == 0) {
        a.n_accepted[b] = j;
        a.next_token[b] = tok;
    }
}

template <bool VEC>
hipError_t launch_vec(const AcceptArgs& a, int32_t B, hipStream_t s) {
    const dim3 g1((a.nblk + kBlocksPerGroup - 1) / kBlocksPerGroup, B);
    hipLaunchKernelGGL(k_block_sums<VEC>, g1, dim3(kSumWaves * kWave), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_pick<VEC>, dim3(B), dim3(kPickThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

size_t dflash_workspace_bytes(int32_t B, int32_t V) {
    const size_t nblk = ((size_t)V + kBlk - 1) / kBlk;
    return (((size_t)B * 4 + 255) / 256) * 256 + (size_t)B * nblk * 8;
}

hipError_t launch_dflash_accept(int32_t B, int32_t G, int32_t V, const int32_t* draft, const float* p_draft,
                                const float* p_target, const float* u, const float* r, int32_t* n_accepted,
                                int32_t* next_token, void* workspace, hipStream_t s) {
    AcceptArgs a{};
    a.draft = draft; a.p_draft = p_draft; a.p_target = p_target; a.u = u; a.r = r;
    a.n_accepted = n_accepted; a.next_token = next_token;
    a.jbuf = static_cast<int32_t*>(workspace);
    a.bsum = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + (((size_t)B * 4 + 255) / 256) * 256);
    a.G = G; a.V = V; a.nblk = (V + kBlk - 1) / kBlk;
    // float4 loads need every row 16-byte aligned: V % 4 == 0 (the bases
    // are 16-byte aligned by the caller's contract)
    return V % 4 == 0 ? launch_vec<true>(a, B, s) : launch_vec<false>(a, B, s);
}

}  // namespace moe
