/*
 * moe_mxfp4.h -- C ABI of the MXFP4 Mixture-of-Experts expert FFN for
 * speculative-decoding verify steps, on AMD Instinct MI355X (gfx950).
 *
 * What one forward call computes (the expert layer of a verify step):
 *   1. top-k routing of every token from its router logits;
 *   2. a stable token-to-expert permutation of the (token, slot) pairs;
 *   3. decode of the MXFP4 expert weights -- 4-bit E2M1 elements with one
 *      E8M0 power-of-two scale per block of 32 along the reduction dimension;
 *   4. gate/up projection with SwiGLU;
 *   5. down projection and the routing-weighted combine of the k experts.
 *
 * Passages this follows (sources are web pages about Xiaomi's
 * MiMo-V2.5-Pro-UltraSpeed):
 *   - ai.appwright.xyz, tag page "投機的デコード", section
 *     "第1層：FP4量子化（モデル側）": only the MoE experts are MXFP4, block size
 *     32; decoding is bound by weight footprint and bandwidth.
 *   - techllm.github.io, "Xiaomi MiMo x TileRT ... 1000 tokens per second",
 *     section "1. MXFP4 — MoE에만 걸린 양자화" (experts hold most weights, FP4
 *     cuts footprint and bandwidth), section "2. DFlash" (draft blocks of up
 *     to 8 tokens, verified by the target model), section "3. TileRT" (the
 *     expert-routing pattern; microsecond operators where launch gaps matter).
 *   - dothoosh.com, "Xiaomi: 1000 tokens per second for a 1T model"
 *     (Persian), section "جزئیات پیاده‌سازی DFlash": block size capped at 8.
 * The pages give no routing rule, activation, layout or API.  Readings taken
 * here: softmax over the k selected logits; SwiGLU h = silu(W_gate a) *
 * (W_up a); the packed layout below; the element/scale bit meanings and the
 * scale rule of the OCP Microscaling Formats (MX) v1.0 specification.
 *
 * Conventions for every entry point:
 *   - Pointers documented as "device" are HIP device pointers (from
 *     hipMalloc or a torch CUDA tensor); all others are host pointers.
 *   - Device buffers must be 16-byte aligned.  The library never allocates,
 *     frees or copies caller memory; it only reads inputs and writes outputs
 *     and the caller-provided workspace.
 *   - `hip_stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Work is queued on it asynchronously; apart from moe_mxfp4_stage_times
 *     (which waits for its last timing event) no call synchronises the
 *     device or copies device data to the host, so forward calls can be
 *     captured into a HIP graph.
 *   - Every call returns a moe_status.  Argument errors are detected on the
 *     host before anything is queued and leave all state unchanged.  A
 *     failed kernel launch returns MOE_ERR_HIP; faults inside kernels surface
 *     asynchronously at the caller's next synchronisation.
 *   - Preconditions that are NOT checked (undefined results if broken):
 *     finite logits and activations; no E8M0 scale byte 0xFF; products of
 *     decoded weights and activations that stay finite in float32.
 *   - Fault injection, for tests of error propagation: with the environment
 *     variable MOE_MXFP4_FAULT set to a launch site (router, route, sort,
 *     quant, gateup, down, combine, dflash; the fused path's one launch of
 *     both projections is the gateup and the down site), a call that
 *     reaches that site returns MOE_ERR_HIP there without launching, as a
 *     failed launch would;
 *     the kernels queued before it stay queued.  Read on every call.
 *   - Logging: with MOE_MXFP4_LOG set (to anything but "0") when a context
 *     is created, create prints the configuration and each forward call
 *     whose token count differs from the previous call's prints its launch
 *     sequence (the kernel path taken), on stderr.
 *   - Thread safety: apart from the optional stage timing below, a context
 *     is immutable after create; concurrent forward calls on one context are
 *     safe when they use distinct workspaces and outputs and stage timing is
 *     off.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MXFP4_ABI_VERSION 1
#define MOE_MXFP4_BLOCK 32          /* elements per E8M0 scale (MX block) */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,       /* null pointer, bad enum, negative size     */
    MOE_ERR_UNSUPPORTED_SHAPE = 2, /* dims outside what the kernels handle      */
    MOE_ERR_CAPACITY = 3,          /* num_tokens > max_tokens                   */
    MOE_ERR_ALIGNMENT = 4,         /* a device pointer not 16-byte aligned      */
    MOE_ERR_WORKSPACE = 5,         /* workspace missing or too small            */
    MOE_ERR_HIP = 6,               /* a HIP runtime call or launch failed       */
    MOE_ERR_INTERNAL = 7
} moe_status;

/* How the activations enter the projections. */
typedef enum {
    MOE_ACT_BF16 = 0,        /* bf16 hidden states used as they are              */
    MOE_ACT_MXFP8_E4M3 = 1   /* hidden states and h micro-scaled to E4M3 + E8M0  */
} moe_act_mode;

typedef enum { MOE_OUT_BF16 = 0, MOE_OUT_F32 = 1 } moe_out_dtype;

typedef struct {
    uint32_t struct_size;    /* sizeof(moe_mxfp4_config)                        */
    int32_t num_experts;     /* E, 1..512                                       */
    int32_t d_model;         /* d, 256 or a multiple of 512 (see below)         */
    int32_t d_ff;            /* f, 256 or a multiple of 512 (see below)         */
    int32_t top_k;           /* k, 1..min(E, 32)                                */
    int32_t max_tokens;      /* upper bound of num_tokens per forward call, >= 1;
                                the activation rows the projections read must
                                stay below 4 GiB: max_tokens*d and
                                max_tokens*k*f times 2 bytes (bf16) or 1 byte
                                (MXFP8) below 2^32                              */
    int32_t act_mode;        /* moe_act_mode                                    */
    int32_t out_dtype;       /* moe_out_dtype                                   */
    uint32_t flags;          /* reserved, must be 0                             */
} moe_mxfp4_config;

/*
 * Shape limits (moe_mxfp4_create returns MOE_ERR_UNSUPPORTED_SHAPE outside
 * them).  The format itself only needs K (d_model for gate/up, d_ff for
 * down) to be a multiple of the MX block of 32.  The kernels consume K in
 * steps of 128 (four MX blocks, one per group of 16 lanes of a wavefront)
 * through a software pipeline 4 steps deep, or 2 steps deep for K = 256, so
 * every K is 256 or a multiple of 512; every shape of the workloads in the
 * tests and the benchmark (256, 512, 1536, 2048, 4096, 6144) is one.  A
 * caller with another K pads each expert matrix with all-zero MX blocks and
 * the activations with zero columns up to the next allowed K: zero elements
 * add nothing to any dot product, so the result is unchanged.  Also:
 * max_tokens*k <= 2^30 and d_model*d_ff <= 2^30 (one expert matrix is
 * addressed with 32-bit offsets).
 */

/*
 * MXFP4 matrices.  Every expert matrix has one output unit per row and the
 * reduction dimension K along the row: W_gate and W_up are [d_ff][d_model]
 * (K = d_model), W_down is [d_model][d_ff] (K = d_ff).  An element is a
 * 4-bit E2M1 code (sign bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and
 * every block of 32 consecutive elements of a row shares one E8M0 scale
 * byte: value = E2M1(code) * 2^(byte - 127).
 *
 * ROW-MAJOR layout (the interchange form; moe_mxfp4_quantize_weights writes
 * it): packed uint8 [rows][K/2], element k of a row in byte k/2 (LOW nibble
 * = even k, high nibble = odd k); scales uint8 [rows][K/32], byte k/32.
 *
 * TILED layout (what the forward path reads; moe_mxfp4_tile_weights converts
 * row-major to it).  With ns = K/128 steps and ng = ceil(K/512) scale groups,
 * the 16-byte block of row-major row n, MX block b (elements 32b..32b+31, in
 * row-major byte order) is stored at byte
 *     16 * (64 * ((n/16) * ns + b/4) + (n%16) + 16 * (b%4))
 * so each 1 KB holds 16 rows x 128 elements in the order the matrix-core
 * operand consumes them, and a 16-row tile streams contiguously along K.
 * Scale byte (n, b) is stored at byte
 *     4 * (64 * ((n/16) * ng + b/16) + (n%16) + 16 * (b%4)) + (b/4) % 4
 * (unused bytes of a partial last group are zero).  Sizes: packed rows*K/2
 * bytes (as row-major); scales (rows/16) * ng * 256 bytes.  rows % 16 == 0.
 * Several experts' matrices stacked along rows convert in one call.
 *
 * Expert weights handed to the forward path (device, TILED, borrowed: the
 * caller keeps them alive and unchanged until moe_mxfp4_destroy):
 *   w_gate, w_up : E matrices [d_ff][d_model] stacked (rows = E*d_ff)
 *   w_down       : E matrices [d_model][d_ff] stacked (rows = E*d_model)
 * each with its tiled scales.
 */
typedef struct {
    const uint8_t* w_gate;
    const uint8_t* w_gate_scale;
    const uint8_t* w_up;
    const uint8_t* w_up_scale;
    const uint8_t* w_down;
    const uint8_t* w_down_scale;
} moe_mxfp4_weights;

/*
 * Optional routing outputs of a forward call (device pointers; any may be
 * NULL).  Sizes for T tokens, P = T * k pairs, pair id p = t * k + j:
 *   topk_ids       int32 [T][k]  expert of slot j, descending logit, ties to
 *                                the lower expert index
 *   topk_w         float [T][k]  softmax over the k selected logits
 *   expert_offsets int32 [E+1]   pairs of expert e are sorted_pairs[off[e] ..
 *                                off[e+1]); off[0] = 0, off[E] = P
 *   sorted_pairs   int32 [P]     pair ids grouped by expert, ascending within
 *                                each expert (a stable counting sort)
 */
typedef struct {
    int32_t* topk_ids;
    float* topk_w;
    int32_t* expert_offsets;
    int32_t* sorted_pairs;
} moe_mxfp4_routing;

typedef struct moe_mxfp4_ctx moe_mxfp4_ctx;   /* opaque, host memory only */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_mxfp4_status_string(moe_status s);

/* ABI version the library was built with (MOE_MXFP4_ABI_VERSION). */
int32_t moe_mxfp4_abi_version(void);

/*
 * Validate `cfg` and the weight pointers and create a context.  Host only:
 * queues no device work and touches no device memory.  `*out` receives the
 * context (left untouched on error).  Errors: INVALID_ARG (null pointer,
 * struct_size mismatch, bad enum, nonzero flags), UNSUPPORTED_SHAPE (limits
 * in moe_mxfp4_config), ALIGNMENT (a weight pointer not 16-byte aligned).
 */
moe_status moe_mxfp4_create(const moe_mxfp4_config* cfg,
                            const moe_mxfp4_weights* weights,
                            moe_mxfp4_ctx** out);

/* Release a context and its stage-timing events, if any (no device memory
 * is involved).  destroy(NULL) returns MOE_OK. */
moe_status moe_mxfp4_destroy(moe_mxfp4_ctx* ctx);

/*
 * Bytes of device workspace a forward call with `num_tokens` tokens needs
 * (0 for num_tokens <= 0 or a NULL context).  The workspace holds routing,
 * permutation and the per-pair intermediate activations; it is scratch with
 * no state carried between calls.
 */
size_t moe_mxfp4_workspace_bytes(const moe_mxfp4_ctx* ctx, int32_t num_tokens);

/*
 * Run the expert layer for `num_tokens` tokens (0 is a no-op returning
 * MOE_OK).  All buffers are device memory:
 *   hidden         bf16  [T][d_model] (uint16 bit patterns)
 *   router_logits  float [T][E], finite or infinite (NaN logits give an
 *                  unspecified selection)
 *   out            [T][d_model], bf16 (round to nearest even) or float per
 *                  cfg.out_dtype; fully overwritten
 *   workspace      at least moe_mxfp4_workspace_bytes(ctx, T) bytes
 *   debug_out      optional routing outputs (host struct, may be NULL)
 * out = sum over the k selected experts e of w_e * W_down,e ( silu(W_gate,e a)
 * * (W_up,e a) ), where a is the token's hidden state (after an MXFP8 round
 * trip per 32-block in MOE_ACT_MXFP8_E4M3 mode, which also rounds h the same
 * way).  Accumulation is float32; routing ids and the permutation are exact
 * and deterministic; the output is deterministic for a given input.
 * Errors: INVALID_ARG, CAPACITY (T > max_tokens), ALIGNMENT, WORKSPACE, HIP.
 */
moe_status moe_mxfp4_forward(moe_mxfp4_ctx* ctx, const void* hidden,
                             const float* router_logits, int32_t num_tokens,
                             void* out, void* workspace, size_t workspace_bytes,
                             void* hip_stream, const moe_mxfp4_routing* debug_out);

/*
 * moe_mxfp4_forward for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as moe_mxfp4_forward
 * minus the workspace: the call uses a scratch array of
 * MOE_MXFP4_NOALLOC_SCRATCH_BYTES that the library holds in device memory,
 * one per GPU, from the first call on that GPU until the process ends (the
 * first call on a GPU looks up its address; no call allocates or frees).
 * The scratch keeps the last call's contents and every call on a GPU shares
 * it, so calls on one GPU whose executions overlap in time (concurrent
 * streams, or concurrent host threads) race and give undefined results;
 * serialise them (one stream, or events).  Nothing in it needs clearing:
 * every value a call reads from it was written earlier in the same call
 * (the counters of the expert launch that routes in every workgroup are
 * in the stream's state block, which the library also holds without
 * allocating per call: see MOE_MXFP4_PATH).
 * Errors: as moe_mxfp4_forward; WORKSPACE when the call would need more
 * scratch than MOE_MXFP4_NOALLOC_SCRATCH_BYTES (moe_mxfp4_workspace_bytes
 * gives the figure; 256 tokens at d_model 4096, d_ff 1536, top-8 need about
 * 40 MB), checked before anything touches the device.
 */
#define MOE_MXFP4_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_mxfp4_forward_noalloc(moe_mxfp4_ctx* ctx, const void* hidden, const float* router_logits,
                                     int32_t num_tokens, void* out, void* hip_stream,
                                     const moe_mxfp4_routing* debug_out);

/*
 * Kernel paths (bf16 activations).  MOE_MXFP4_PATH, read when a context is
 * created, selects how a forward call runs the steps after routing:
 *   "fused" (default)   gate/up + SwiGLU and down as work units of one
 *                       launch, handing over through counters in the
 *                       workspace, so down work starts while gate/up still
 *                       streams weights; then the combine.  The pages'
 *                       runtime keeps one engine kernel resident so that
 *                       microsecond operators pay no gap between them
 *                       (techllm.github.io "Xiaomi MiMo x TileRT", section
 *                       "3. TileRT").  Routing and the permutation are
 *                       the per-phase launches (the permutation also lists
 *                       each XCD's chunks).  Batches of more pairs than
 *                       experts take the ticketed form: every workgroup of
 *                       the one launch takes a ticket and runs that unit
 *                       (gate/up units first, then down units, each waiting
 *                       for its chunk).  Smaller batches take the
 *                       persistent form: a kernel of as many workgroups as
 *                       the GPU holds, each looping over gate/up units and
 *                       then taking down units from a queue.  Batches up to
 *                       MOE_MXFP4_FUSED_MAX_PAIRS pairs; larger ones run
 *                       "stream".
 *                       For a single verify block (at most 64 pairs over
 *                       at most 128 experts, no more pairs than experts, at
 *                       most 1024 router logits) the routing and the
 *                       permutation run inside that one launch instead:
 *                       every workgroup routes the block's tokens and
 *                       permutes its pairs itself (the same code as the
 *                       routing launches), so the call is two launches,
 *                       that one and the combine.  The launch's counters
 *                       live in a state block that the library keeps per
 *                       (GPU, stream) in device memory of its own (16 per
 *                       GPU, held until the process ends); the combine
 *                       launch clears it for the stream's next call, and the
 *                       first call on a stream (or one after a call whose
 *                       combine launch failed, or after a capture) clears
 *                       it with one small extra launch.  Streams beyond the
 *                       16th on a GPU route in launches of their own.  A
 *                       call captured into a graph keeps the block of the
 *                       stream it was captured on: replays of that graph
 *                       must not overlap other calls that use the same
 *                       block (as calls sharing a workspace must not).
 *   "fused_launches"    "fused" with the routing and permutation always in
 *                       launches of their own.
 *   "stream"            one launch per phase: permutation, gate/up +
 *                       SwiGLU, down, combine.
 * All give bit-identical outputs.  Any other value makes create fail with
 * MOE_ERR_INVALID_ARG.  MXFP8 mode has one path (the dense kernels).
 *
 * The fused kernels' waits for other workgroups are bounded; past the
 * bound (or with MOE_MXFP4_SPIN_LIMIT set to a negative value, read on every
 * call, for tests of this path) they raise an error word, the workgroups
 * exit normally and the call's outputs are undefined.
 * moe_mxfp4_device_status waits for hip_stream and writes to *status (host)
 * the error word of the most recent call with `num_tokens` tokens: where the
 * routing runs inside the expert launch (see "fused"), of the most recent
 * such call on hip_stream on the current GPU (the word sits in the stream's
 * state block; workspace is not read); otherwise of the most recent such call
 * on `workspace` (device).
 * 0 = no wait gave up; always 0 on paths without such waits.  Errors:
 * INVALID_ARG, CAPACITY, HIP.
 */
#define MOE_MXFP4_FUSED_MAX_PAIRS 8192

moe_status moe_mxfp4_device_status(const moe_mxfp4_ctx* ctx, const void* workspace, int32_t num_tokens,
                                   int32_t* status, void* hip_stream);

/*
 * Router projection, the step in front of the routing:
 *   logits[t][e] = sum_i hidden[t][i] * w_router[e][i]
 * with bf16 inputs and float32 accumulation on the matrix cores, in an order
 * that does not depend on timing (deterministic).  The pages keep every
 * module outside the experts in FP8 or its original precision
 * (techllm.github.io "Xiaomi MiMo x TileRT", section "1. MXFP4 — MoE에만 걸린
 * 양자화") and route every token to its experts (same page, section
 * "3. TileRT"); they give no router form, and this is the plain linear map
 * (no bias).  All buffers are device memory:
 *   hidden    bf16  [T][d_model] (uint16 bit patterns)
 *   w_router  bf16  [E][d_model]: row e is expert e's router vector
 *   logits    float [T][E], fully overwritten
 * T = 0 is a no-op returning MOE_OK.
 * Errors: INVALID_ARG, CAPACITY (T > max_tokens), ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_router_logits(const moe_mxfp4_ctx* ctx, const void* hidden,
                                   const void* w_router, int32_t num_tokens,
                                   float* logits, void* hip_stream);

/*
 * moe_mxfp4_forward with the router projection in front: the logits are
 * computed from hidden and w_router (as moe_mxfp4_router_logits) into the
 * workspace, which moe_mxfp4_workspace_bytes already covers, and the call
 * continues as moe_mxfp4_forward with them.  Stage timing counts the
 * projection in the routing stage.
 * Errors: as moe_mxfp4_forward (INVALID_ARG for a NULL w_router).
 */
moe_status moe_mxfp4_forward_hidden(moe_mxfp4_ctx* ctx, const void* hidden,
                                    const void* w_router, int32_t num_tokens,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream, const moe_mxfp4_routing* debug_out);

/*
 * DFlash verify acceptance: the rejection-sampling pass that ends a verify
 * step and makes block drafting lossless (techllm.github.io "Xiaomi MiMo x
 * TileRT", section "2. DFlash"; blocks of at most 8 drafted tokens).  The
 * pages do not print the rule; this is standard speculative sampling, per
 * sequence b:
 *   - position j = 0, 1, ... of the block: the draft token x = draft[b][j]
 *     is accepted when u[b][j] * p_draft[b][j][x] < p_target[b][j][x]
 *     (float32); a token outside [0, V) is rejected; the first rejection
 *     ends the block.  n_accepted[b] = the number accepted (0..G).
 *   - next_token[b] is drawn with r[b] from max(0, p_target[b][j] -
 *     p_draft[b][j]) (float32 per entry) after a rejection at j, or from
 *     p_target[b][j] if that residual has no positive entry, or from
 *     p_target[b][G] when the whole block is accepted.
 *   - a draw: integer weights q_i = rint(2^32 w_i) (0 for w_i <= 0 or NaN),
 *     S = sum_i q_i, threshold = floor(S * r24 / 2^24) with r24 = floor(2^24
 *     r) clamped to [0, 2^24 - 1], result = the first i whose inclusive
 *     prefix sum of q exceeds the threshold; -1 if S = 0.  Integer sums make
 *     the result exact and independent of how the row is split over threads.
 * All arrays are device memory, row-major:
 *   draft      int32 [B][G]          drafted tokens
 *   p_draft    float [B][G][V]       drafter distributions at the G positions
 *   p_target   float [B][G+1][V]     target distributions at the G+1 positions
 *   u          float [B][G]          uniforms of the acceptance tests
 *   r          float [B]             uniforms of the draws
 *   n_accepted int32 [B], next_token int32 [B]   outputs
 *   workspace  >= moe_mxfp4_dflash_workspace_bytes(B, V) bytes, caller-owned,
 *              no initial contents needed; calls that overlap in time need
 *              distinct workspaces.
 * Limits: 0 <= G <= 64, 1 <= V <= 2^30, 0 <= B <= 65535 (B = 0 is a no-op).
 * Entries are probabilities: rows need not be normalised, but every row's
 * sum must stay below 2^31.  Not context-bound: no moe_mxfp4_ctx.
 * Errors: INVALID_ARG (null pointer, size out of range), ALIGNMENT,
 * WORKSPACE (too small), HIP.
 */
size_t moe_mxfp4_dflash_workspace_bytes(int32_t batch, int32_t vocab);
moe_status moe_mxfp4_dflash_accept(int32_t batch, int32_t block, int32_t vocab,
                                   const int32_t* draft, const float* p_draft,
                                   const float* p_target, const float* u,
                                   const float* r, int32_t* n_accepted,
                                   int32_t* next_token, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);

/*
 * Measurement probes, for reading roofline fractions against what this GPU
 * sustains as well as against its nominal peaks (not part of the forward
 * path).  One launch on hip_stream; *work (host) receives the algorithmic
 * amount it does, so rate = *work / the caller's timing of the launch.
 *   kind 0  read `bytes` (> 0, multiple of 16) from src (device) once with
 *           16-byte non-temporal loads; *work = bytes.
 *   kind 1  v_mfma_f32_16x16x32_bf16 loop       (*work = flops)
 *   kind 2  v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E2M1 (flops)
 *   kind 3  the same, E2M1 x E2M1 (flops)
 *   kind 4, 5, 6  kinds 1, 2, 3 on random finite operands that change from
 *           one MFMA to the next: under the chip's power limit the clock
 *           depends on how many operand bits toggle, so these are the rates
 *           real data can reach, where kinds 1-3 repeat one operand pair
 * MFMA kinds run 2048 workgroups x 4 waves x 32 `reps` (reps 1 .. 2^20)
 * rounds of 8 independent MFMAs per wave, operands in registers; src and bytes are
 * ignored.  sink (device, 4 bytes) is written only with a value the probes
 * never produce (it keeps the work from being optimised away).
 * Errors: INVALID_ARG (kind, bytes, reps, null sink or src), ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_probe(int32_t kind, const void* src, size_t bytes, int32_t reps,
                           uint32_t* sink, double* work, void* hip_stream);

/*
 * Decode rows [row0, row0 + nrows) of one expert matrix (0 gate, 1 up,
 * 2 down) from the context's TILED weights with the forward path's own
 * in-register FP4 decode, widened to float: out (device) float [nrows][K]
 * in row-major order, K = d_model for gate/up, d_ff for down.  For checking
 * the layout and the decode bit for bit.  Errors: INVALID_ARG (bad expert,
 * matrix or row range, null out), ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_debug_dequant(const moe_mxfp4_ctx* ctx, int32_t expert,
                                   int32_t matrix, int32_t row0, int32_t nrows,
                                   float* out, void* hip_stream);

/*
 * Copy the intermediate activations h of the last forward call that ran
 * with `num_tokens` tokens on `workspace` (device, as passed to that call),
 * for checking its rounding decisions.  Rows are in expert-sorted order: row
 * r belongs to pair sorted_pairs[r] of that call's routing outputs.
 * MOE_ACT_MXFP8_E4M3: h (device) uint8 [P][d_ff] E4M3 codes and h_scales
 * (device) uint8 [P][d_ff/32] E8M0 bytes (the MX blocks run along d_ff);
 * MOE_ACT_BF16: h bf16 [P][d_ff] (uint16 bit patterns), h_scales unused
 * (may be NULL).  P = num_tokens * top_k.  Queued on hip_stream after that
 * call.  Errors: INVALID_ARG (null pointer, num_tokens <= 0), CAPACITY,
 * ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_debug_hidden(const moe_mxfp4_ctx* ctx, const void* workspace, int32_t num_tokens,
                                  void* h, uint8_t* h_scales, void* hip_stream);

/*
 * Per-stage timing of forward calls with HIP events, for measurement.  The
 * pages stress that at these speeds each operator lasts microseconds and the
 * gaps between operators matter (techllm.github.io "Xiaomi MiMo x TileRT",
 * section "3. TileRT"), so the stages are timed one by one.  The stages, in
 * launch order: 0 routing, 1 permutation, 2 MXFP8 quantisation of the
 * activations (empty in bf16 mode), 3 gate/up + SwiGLU, 4 down, 5 combine
 * (routing weights and the sum over the k slots).  Batches of at most 64
 * tokens with at most 64 experts route and permute in one launch, timed as
 * stage 0 (stage 1 is then empty).
 *
 * moe_mxfp4_stage_timing(ctx, capacity): capacity > 0 creates capacity *
 * (MOE_MXFP4_NUM_STAGES + 1) HIP events (host call, never inside forward)
 * and makes each later forward call record one event before the first stage
 * and one after each stage, into slot (call index % capacity); capacity 0
 * destroys the events and stops recording.  Errors: INVALID_ARG, HIP.
 *
 * moe_mxfp4_stage_times(ctx, total_ms, calls): waits for the recorded
 * events, writes the summed milliseconds of each stage over the recorded
 * calls still held (at most capacity) into total_ms (host float
 * [MOE_MXFP4_NUM_STAGES]) and their number into *calls (host), then starts
 * a new count.  A call that returned an error holds no slot: its partly
 * recorded events are never summed, and the next call reuses the slot.  Stage i of a call spans event i to event i+1, so it includes
 * any launch gap before that stage's kernel.  Errors: INVALID_ARG (null
 * pointer, timing not enabled), HIP.  Timing calls are not thread safe.
 */
#define MOE_MXFP4_NUM_STAGES 6
moe_status moe_mxfp4_stage_timing(moe_mxfp4_ctx* ctx, int32_t capacity);
moe_status moe_mxfp4_stage_times(moe_mxfp4_ctx* ctx, float* total_ms, int32_t* calls);

/*
 * Weight preparation (off the forward path): quantise a row-major float
 * matrix w (device) [rows][K] into the ROW-MAJOR packed layout above -- per
 * block of 32 along K, scale 2^(floor(log2(amax)) - 2) clamped to the E8M0
 * range (an all-zero block gets byte 0), elements rounded to the nearest
 * E2M1 value with ties to the even code, saturating at +-6, the sign of a
 * value that rounds to zero kept.  packed (device) uint8 [rows][K/2], scales
 * (device) uint8 [rows][K/32].  K must be a positive multiple of 32.
 * Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_quantize_weights(const float* w, int64_t rows, int64_t K,
                                      uint8_t* packed, uint8_t* scales,
                                      void* hip_stream);

/*
 * MXFP8 quantisation of bf16 activations, the kernel the forward path runs
 * in MOE_ACT_MXFP8_E4M3 mode (exposed for callers that quantise ahead and
 * for checking it bit for bit): x (device) bf16 [rows][K] -> codes (device)
 * uint8 [rows][K] OCP E4M3, scales (device) uint8 [rows][K/32] E8M0.  Per
 * block of 32 along K: scale 2^(floor(log2(amax)) - 8) clamped to the E8M0
 * range (all-zero block: byte 0); element = nearest E4M3 of x / scale, ties
 * to the even code, saturating at +-448, never NaN; a value rounding to zero
 * keeps its sign.  The MX block size 32 is the pages' (ai.appwright.xyz
 * "投機的デコード", section "第1層：FP4量子化（モデル側）"); the element and scale
 * rules are the OCP MX v1.0 ones.  K must be a positive multiple of 32.
 * Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_quantize_act_mxfp8(const void* x, int64_t rows, int64_t K,
                                        uint8_t* codes, uint8_t* scales,
                                        void* hip_stream);

/* Bytes of the TILED scale array of a rows x K matrix (0 if rows % 16 or
 * K % 128 is nonzero or a size is not positive). */
size_t moe_mxfp4_tiled_scale_bytes(int64_t rows, int64_t K);

/*
 * Weight preparation: convert a ROW-MAJOR packed matrix (device packed
 * [rows][K/2], scales [rows][K/32]) to the TILED layout (device tiled_packed
 * rows*K/2 bytes, tiled_scales moe_mxfp4_tiled_scale_bytes(rows, K) bytes).
 * A pure byte permutation; inputs and outputs must not overlap.  rows % 16
 * == 0 and K % 128 == 0.  Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
moe_status moe_mxfp4_tile_weights(const uint8_t* packed, const uint8_t* scales,
                                  int64_t rows, int64_t K, uint8_t* tiled_packed,
                                  uint8_t* tiled_scales, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MXFP4_H */
