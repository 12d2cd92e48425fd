// Host side of the C ABI declared in include/moe_mxfp4.h: argument checks,
// workspace carve-up and the launch sequence of one forward call.
//
// A forward call is five to eight launches on the caller's stream and nothing else
// (no allocation, no host synchronisation, no device-to-host copy), so it can
// be captured into a HIP graph: the pages stress that at microsecond
// operator times the gaps between operators matter (techllm.github.io
// "Xiaomi MiMo x TileRT", section "3. TileRT").
#include <stdint.h>
#include <stdlib.h>

#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "common.hpp"

struct moe_mxfp4_ctx {
    moe_mxfp4_config cfg;
    moe_mxfp4_weights w;
    // optional stage timing: capacity slots of NUM_STAGES + 1 events each
    std::vector<hipEvent_t> events;
    int32_t capacity = 0;
    int64_t ncalls = 0;
};

namespace {

using moe::kMaxExperts;
using moe::kMaxTopK;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
    size_t logits, ids, w, offsets, sorted, active, chunks, nchunks, sort_part, xq, xs, h, hs, o, total;
};

Layout make_layout(const moe_mxfp4_config& c, int64_t T) {
    const size_t P = (size_t)T * c.top_k;
    Layout L{};
    size_t at = 0;
    L.logits = at;  at += round256((size_t)T * c.num_experts * sizeof(float));   // router projection output
    L.ids = at;     at += round256(P * sizeof(int32_t));
    L.w = at;       at += round256(P * sizeof(float));
    L.offsets = at; at += round256((size_t)(c.num_experts + 1) * sizeof(int32_t));
    L.sorted = at;  at += round256(P * sizeof(int32_t));
    L.active = at;  at += round256((size_t)(c.num_experts + 1) * sizeof(int32_t));
    moe::Dims dm{(int32_t)T, c.d_model, c.d_ff, c.num_experts, c.top_k, (int32_t)P};
    L.chunks = at;  at += round256((size_t)moe::max_chunks(dm) * moe::kChunkRec * sizeof(int32_t));
    L.nchunks = at; at += 256;
    L.sort_part = at; at += round256((size_t)moe::sort_tiles((int)P) * c.num_experts * sizeof(int32_t));
    const bool mx8 = c.act_mode == MOE_ACT_MXFP8_E4M3;
    L.xq = at;      at += mx8 ? round256((size_t)T * c.d_model) : 0;
    L.xs = at;      at += mx8 ? round256((size_t)T * (c.d_model / MOE_MXFP4_BLOCK)) : 0;
    L.h = at;       at += round256(P * (size_t)c.d_ff * (mx8 ? 1 : sizeof(uint16_t)));
    L.hs = at;      at += mx8 ? round256(P * (size_t)(c.d_ff / MOE_MXFP4_BLOCK)) : 0;
    L.o = at;       at += round256(P * (size_t)c.d_model * sizeof(float));
    L.total = at;
    return L;
}

// Fault injection for tests of error propagation: with MOE_MXFP4_FAULT set
// to a launch site's name, a call that reaches that site returns MOE_ERR_HIP
// there instead of launching, as a failed launch would.  Sites: router,
// route (the routing or fused routing + permutation launch), sort, quant,
// gateup, down, combine, dflash.  Read on every call, so a test can set and
// clear it between calls.
bool fault_at(const char* site) {
    const char* e = std::getenv("MOE_MXFP4_FAULT");
    return e && std::strcmp(e, site) == 0;
}

moe_status check_config(const moe_mxfp4_config* c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->struct_size != sizeof(moe_mxfp4_config)) return MOE_ERR_INVALID_ARG;
    if (c->flags != 0) return MOE_ERR_INVALID_ARG;
    if (c->act_mode != MOE_ACT_BF16 && c->act_mode != MOE_ACT_MXFP8_E4M3) return MOE_ERR_INVALID_ARG;
    if (c->out_dtype != MOE_OUT_BF16 && c->out_dtype != MOE_OUT_F32) return MOE_ERR_INVALID_ARG;
    if (c->num_experts < 1 || c->top_k < 1 || c->d_model < 1 || c->d_ff < 1 || c->max_tokens < 1)
        return MOE_ERR_INVALID_ARG;
    if (c->num_experts > kMaxExperts || c->top_k > kMaxTopK || c->top_k > c->num_experts)
        return MOE_ERR_UNSUPPORTED_SHAPE;
    // K steps per matrix: 2 or a multiple of 4 (the kernels' pipeline depths)
    for (int32_t K : {c->d_model, c->d_ff})
        if (K != 256 && K % 512 != 0) return MOE_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)c->max_tokens * c->top_k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)c->d_model * c->d_ff > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED_SHAPE;
    // MXFP8 activation codes (x: T x d bytes, h: P x f bytes) are read through
    // buffer resources, whose offsets and record counts are 32-bit
    if (c->act_mode == MOE_ACT_MXFP8_E4M3 &&
        ((int64_t)c->max_tokens * c->d_model >= (int64_t)1 << 32 ||
         (int64_t)c->max_tokens * c->top_k * c->d_ff >= (int64_t)1 << 32))
        return MOE_ERR_UNSUPPORTED_SHAPE;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_mxfp4_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, bad enum or size";
        case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE: dimensions outside the kernels' limits";
        case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY: num_tokens exceeds max_tokens";
        case MOE_ERR_ALIGNMENT: return "MOE_ERR_ALIGNMENT: device pointer not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch or runtime call failed";
        case MOE_ERR_INTERNAL: return "MOE_ERR_INTERNAL";
    }
    return "unknown moe_status";
}

int32_t moe_mxfp4_abi_version(void) { return MOE_MXFP4_ABI_VERSION; }

moe_status moe_mxfp4_create(const moe_mxfp4_config* cfg, const moe_mxfp4_weights* weights,
                            moe_mxfp4_ctx** out) {
    if (!out || !weights) return MOE_ERR_INVALID_ARG;
    const moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    const void* ptrs[6] = {weights->w_gate, weights->w_gate_scale, weights->w_up,
                           weights->w_up_scale, weights->w_down, weights->w_down_scale};
    for (const void* p : ptrs)
        if (!p) return MOE_ERR_INVALID_ARG;
    for (const void* p : ptrs)
        if (!aligned16(p)) return MOE_ERR_ALIGNMENT;
    moe_mxfp4_ctx* ctx = new (std::nothrow) moe_mxfp4_ctx;
    if (!ctx) return MOE_ERR_INTERNAL;
    ctx->cfg = *cfg;
    ctx->w = *weights;
    *out = ctx;
    return MOE_OK;
}

moe_status moe_mxfp4_destroy(moe_mxfp4_ctx* ctx) {
    if (ctx)
        for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
    delete ctx;
    return MOE_OK;
}

moe_status moe_mxfp4_stage_timing(moe_mxfp4_ctx* ctx, int32_t capacity) {
    if (!ctx || capacity < 0) return MOE_ERR_INVALID_ARG;
    for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
    ctx->events.clear();
    ctx->capacity = 0;
    ctx->ncalls = 0;
    if (capacity == 0) return MOE_OK;
    const size_t n = (size_t)capacity * (MOE_MXFP4_NUM_STAGES + 1);
    ctx->events.reserve(n);
    for (size_t i = 0; i < n; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) {
            for (hipEvent_t x : ctx->events) (void)hipEventDestroy(x);
            ctx->events.clear();
            return MOE_ERR_HIP;
        }
        ctx->events.push_back(e);
    }
    ctx->capacity = capacity;
    return MOE_OK;
}

moe_status moe_mxfp4_stage_times(moe_mxfp4_ctx* ctx, float* total_ms, int32_t* calls) {
    if (!ctx || !total_ms || !calls || ctx->capacity == 0) return MOE_ERR_INVALID_ARG;
    const int64_t held = ctx->ncalls < ctx->capacity ? ctx->ncalls : ctx->capacity;
    for (int i = 0; i < MOE_MXFP4_NUM_STAGES; ++i) total_ms[i] = 0.f;
    *calls = (int32_t)held;
    if (held > 0) {
        const int64_t last = (ctx->ncalls - 1) % ctx->capacity;
        if (hipEventSynchronize(ctx->events[last * (MOE_MXFP4_NUM_STAGES + 1) + MOE_MXFP4_NUM_STAGES]) !=
            hipSuccess)
            return MOE_ERR_HIP;
        for (int64_t slot = 0; slot < held; ++slot) {
            hipEvent_t* ev = &ctx->events[slot * (MOE_MXFP4_NUM_STAGES + 1)];
            for (int i = 0; i < MOE_MXFP4_NUM_STAGES; ++i) {
                float ms = 0.f;
                if (hipEventElapsedTime(&ms, ev[i], ev[i + 1]) != hipSuccess) return MOE_ERR_HIP;
                total_ms[i] += ms;
            }
        }
    }
    ctx->ncalls = 0;
    return MOE_OK;
}

size_t moe_mxfp4_workspace_bytes(const moe_mxfp4_ctx* ctx, int32_t num_tokens) {
    if (!ctx || num_tokens <= 0) return 0;
    return make_layout(ctx->cfg, num_tokens).total;
}

}  // extern "C"

namespace {

// One forward call: router logits given (w_router == NULL) or projected from
// the hidden states with w_router into the workspace first.
moe_status forward_impl(moe_mxfp4_ctx* ctx, const void* hidden, const float* router_logits, const void* w_router,
                        int32_t num_tokens, void* out, void* workspace, size_t workspace_bytes,
                        void* hip_stream, const moe_mxfp4_routing* debug_out) {
    if (!ctx || num_tokens < 0) return MOE_ERR_INVALID_ARG;
    const moe_mxfp4_config& c = ctx->cfg;
    if (num_tokens > c.max_tokens) return MOE_ERR_CAPACITY;
    if (num_tokens == 0) return MOE_OK;
    if (!hidden || !(router_logits || w_router) || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(router_logits ? (const void*)router_logits : w_router) || !aligned16(out))
        return MOE_ERR_ALIGNMENT;
    const Layout L = make_layout(c, num_tokens);
    if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGNMENT;
    if (debug_out) {
        const void* dp[4] = {debug_out->topk_ids, debug_out->topk_w, debug_out->expert_offsets,
                             debug_out->sorted_pairs};
        for (const void* p : dp)
            if (p && !aligned16(p)) return MOE_ERR_ALIGNMENT;
    }

    char* base = static_cast<char*>(workspace);
    float* ws_logits = reinterpret_cast<float*>(base + L.logits);
    moe::Workspace ws;
    ws.topk_ids = reinterpret_cast<int32_t*>(base + L.ids);
    ws.topk_w = reinterpret_cast<float*>(base + L.w);
    ws.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    ws.sorted_pairs = reinterpret_cast<int32_t*>(base + L.sorted);
    ws.active = reinterpret_cast<int32_t*>(base + L.active);
    ws.chunks = reinterpret_cast<int32_t*>(base + L.chunks);
    ws.nchunks = reinterpret_cast<int32_t*>(base + L.nchunks);
    ws.sort_part = reinterpret_cast<int32_t*>(base + L.sort_part);
    ws.xq = reinterpret_cast<uint8_t*>(base + L.xq);
    ws.xs = reinterpret_cast<uint8_t*>(base + L.xs);
    ws.h = reinterpret_cast<uint8_t*>(base + L.h);
    ws.hs = reinterpret_cast<uint8_t*>(base + L.hs);
    ws.o = reinterpret_cast<float*>(base + L.o);
    ws.os = reinterpret_cast<uint8_t*>(base + L.o + (size_t)num_tokens * c.top_k * c.d_model * sizeof(uint16_t));

    moe::Dims dm{num_tokens, c.d_model, c.d_ff, c.num_experts, c.top_k, num_tokens * c.top_k};
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const uint16_t* x = static_cast<const uint16_t*>(hidden);

    hipEvent_t* ev = nullptr;
    if (ctx->capacity > 0)
        ev = &ctx->events[(size_t)(ctx->ncalls++ % ctx->capacity) * (MOE_MXFP4_NUM_STAGES + 1)];
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };

    const bool mx8 = c.act_mode == MOE_ACT_MXFP8_E4M3;
    if (mark(0) != hipSuccess) return MOE_ERR_HIP;
    if (w_router) {
        // the projection is timed with the routing stage
        if (fault_at("router") ||
            moe::launch_router(x, static_cast<const uint16_t*>(w_router), ws_logits, dm, s) != hipSuccess)
            return MOE_ERR_HIP;
        router_logits = ws_logits;
    }
    const int chunk_rows = mx8 ? moe::kDenseChunk : moe::kChunk;
    if (moe::route_sort_fused(dm)) {
        // one launch; its time is recorded as the routing stage
        if (fault_at("route") || moe::launch_route_sort(router_logits, dm, ws, chunk_rows, s) != hipSuccess ||
            mark(1) != hipSuccess || mark(2) != hipSuccess)
            return MOE_ERR_HIP;
    } else {
        if (fault_at("route") || moe::launch_route(router_logits, dm, ws, s) != hipSuccess || mark(1) != hipSuccess)
            return MOE_ERR_HIP;
        if (fault_at("sort") || moe::launch_sort(dm, ws, chunk_rows, s) != hipSuccess || mark(2) != hipSuccess)
            return MOE_ERR_HIP;
    }
    if (mx8 && (fault_at("quant") || moe::launch_quant_x8(x, dm, ws, s) != hipSuccess)) return MOE_ERR_HIP;
    if (mark(3) != hipSuccess) return MOE_ERR_HIP;
    if (fault_at("gateup")) return MOE_ERR_HIP;
    const hipError_t gu = mx8 ? moe::launch_gateup_dense(ctx->w, dm, ws, s)
                              : moe::launch_gateup(x, ctx->w, dm, ws, s);
    if (gu != hipSuccess || mark(4) != hipSuccess) return MOE_ERR_HIP;
    if (fault_at("down")) return MOE_ERR_HIP;
    const hipError_t dn = mx8 ? moe::launch_down_dense(ctx->w, dm, ws, s) : moe::launch_down(ctx->w, dm, ws, s);
    if (dn != hipSuccess || mark(5) != hipSuccess) return MOE_ERR_HIP;
    if (fault_at("combine") || moe::launch_finalize(dm, ws, out, c.out_dtype, mx8, s) != hipSuccess ||
        mark(6) != hipSuccess)
        return MOE_ERR_HIP;

    if (debug_out) {
        const size_t P = (size_t)dm.P;
        struct { void* dst; const void* src; size_t n; } cp[4] = {
            {debug_out->topk_ids, ws.topk_ids, P * sizeof(int32_t)},
            {debug_out->topk_w, ws.topk_w, P * sizeof(float)},
            {debug_out->expert_offsets, ws.offsets, (size_t)(c.num_experts + 1) * sizeof(int32_t)},
            {debug_out->sorted_pairs, ws.sorted_pairs, P * sizeof(int32_t)}};
        for (auto& k : cp)
            if (k.dst && hipMemcpyAsync(k.dst, k.src, k.n, hipMemcpyDeviceToDevice, s) != hipSuccess)
                return MOE_ERR_HIP;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_mxfp4_forward(moe_mxfp4_ctx* ctx, const void* hidden, const float* router_logits,
                             int32_t num_tokens, void* out, void* workspace, size_t workspace_bytes,
                             void* hip_stream, const moe_mxfp4_routing* debug_out) {
    if (!router_logits && num_tokens > 0) return MOE_ERR_INVALID_ARG;
    return forward_impl(ctx, hidden, router_logits, nullptr, num_tokens, out, workspace, workspace_bytes,
                        hip_stream, debug_out);
}

moe_status moe_mxfp4_forward_hidden(moe_mxfp4_ctx* ctx, const void* hidden, const void* w_router,
                                    int32_t num_tokens, void* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream, const moe_mxfp4_routing* debug_out) {
    if (!w_router && num_tokens > 0) return MOE_ERR_INVALID_ARG;
    return forward_impl(ctx, hidden, nullptr, w_router, num_tokens, out, workspace, workspace_bytes, hip_stream,
                        debug_out);
}

moe_status moe_mxfp4_router_logits(const moe_mxfp4_ctx* ctx, const void* hidden, const void* w_router,
                                   int32_t num_tokens, float* logits, void* hip_stream) {
    if (!ctx || num_tokens < 0) return MOE_ERR_INVALID_ARG;
    const moe_mxfp4_config& c = ctx->cfg;
    if (num_tokens > c.max_tokens) return MOE_ERR_CAPACITY;
    if (num_tokens == 0) return MOE_OK;
    if (!hidden || !w_router || !logits) return MOE_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(w_router) || !aligned16(logits)) return MOE_ERR_ALIGNMENT;
    moe::Dims dm{num_tokens, c.d_model, c.d_ff, c.num_experts, c.top_k, num_tokens * c.top_k};
    if (moe::launch_router(static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_router), logits, dm,
                           static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_mxfp4_probe(int32_t kind, const void* src, size_t bytes, int32_t reps, uint32_t* sink, double* work,
                           void* hip_stream) {
    if (kind < 0 || kind > 6 || !sink || !work) return MOE_ERR_INVALID_ARG;
    if (kind == 0 && (!src || bytes == 0 || bytes % 16 != 0)) return MOE_ERR_INVALID_ARG;
    if (kind != 0 && (reps < 1 || reps > (1 << 20))) return MOE_ERR_INVALID_ARG;
    if ((kind == 0 && !aligned16(src)) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return MOE_ERR_ALIGNMENT;
    if (moe::launch_probe(kind, src, bytes, reps, sink, work, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

size_t moe_mxfp4_dflash_workspace_bytes(int32_t batch, int32_t vocab) {
    if (batch < 0 || batch > 65535 || vocab < 1 || vocab > (1 << 30)) return 0;
    return moe::dflash_workspace_bytes(batch, vocab);
}

moe_status moe_mxfp4_dflash_accept(int32_t batch, int32_t block, int32_t vocab, const int32_t* draft,
                                   const float* p_draft, const float* p_target, const float* u, const float* r,
                                   int32_t* n_accepted, int32_t* next_token, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
    if (batch < 0 || batch > 65535 || block < 0 || block > 64 || vocab < 1 || vocab > (1 << 30))
        return MOE_ERR_INVALID_ARG;
    if (batch == 0) return MOE_OK;
    if (!p_target || !r || !n_accepted || !next_token || (block > 0 && (!draft || !p_draft || !u)))
        return MOE_ERR_INVALID_ARG;
    const void* ptrs[] = {draft, p_draft, p_target, u, r, n_accepted, next_token};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MOE_ERR_ALIGNMENT;
    if (!workspace || workspace_bytes < moe::dflash_workspace_bytes(batch, vocab)) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGNMENT;
    if (fault_at("dflash") ||
        moe::launch_dflash_accept(batch, block, vocab, draft, p_draft, p_target, u, r, n_accepted, next_token,
                                  workspace, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_mxfp4_debug_dequant(const moe_mxfp4_ctx* ctx, int32_t expert, int32_t matrix,
                                   int32_t row0, int32_t nrows, float* out, void* hip_stream) {
    if (!ctx || !out) return MOE_ERR_INVALID_ARG;
    const moe_mxfp4_config& c = ctx->cfg;
    if (expert < 0 || expert >= c.num_experts || matrix < 0 || matrix > 2) return MOE_ERR_INVALID_ARG;
    const int64_t N = matrix == 2 ? c.d_model : c.d_ff;
    const int64_t K = matrix == 2 ? c.d_ff : c.d_model;
    if (row0 < 0 || nrows < 0 || (int64_t)row0 + nrows > N) return MOE_ERR_INVALID_ARG;
    if (!aligned16(out)) return MOE_ERR_ALIGNMENT;
    if (nrows == 0) return MOE_OK;
    const uint8_t* P = matrix == 0 ? ctx->w.w_gate : matrix == 1 ? ctx->w.w_up : ctx->w.w_down;
    const uint8_t* S = matrix == 0 ? ctx->w.w_gate_scale : matrix == 1 ? ctx->w.w_up_scale : ctx->w.w_down_scale;
    const uint8_t* Pe = P + (int64_t)expert * N * (K / 2);
    const uint8_t* Se = S + (int64_t)expert * moe::tiled_scale_bytes(N, K);
    if (moe::launch_debug_dequant(Pe, Se, K, row0, nrows, out, static_cast<hipStream_t>(hip_stream)) !=
        hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_mxfp4_quantize_weights(const float* w, int64_t rows, int64_t K, uint8_t* packed,
                                      uint8_t* scales, void* hip_stream) {
    if (!w || !packed || !scales || rows < 0 || K <= 0 || K % MOE_MXFP4_BLOCK != 0)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(scales)) return MOE_ERR_ALIGNMENT;
    if (rows == 0) return MOE_OK;
    if (moe::launch_quantize(w, rows, K, packed, scales, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_mxfp4_quantize_act_mxfp8(const void* x, int64_t rows, int64_t K, uint8_t* codes,
                                        uint8_t* scales, void* hip_stream) {
    if (!x || !codes || !scales || rows < 0 || K <= 0 || K % MOE_MXFP4_BLOCK != 0) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_ALIGNMENT;
    if (rows == 0) return MOE_OK;
    if (moe::launch_quant_act8(static_cast<const uint16_t*>(x), rows, K, codes, scales,
                               static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

size_t moe_mxfp4_tiled_scale_bytes(int64_t rows, int64_t K) {
    if (rows <= 0 || K <= 0 || rows % 16 != 0 || K % 128 != 0) return 0;
    return (size_t)moe::tiled_scale_bytes(rows, K);
}

moe_status moe_mxfp4_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t K,
                                  uint8_t* tiled_packed, uint8_t* tiled_scales, void* hip_stream) {
    if (!packed || !scales || !tiled_packed || !tiled_scales || rows < 0 || K <= 0 || rows % 16 != 0 ||
        K % 128 != 0)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(scales) || !aligned16(tiled_packed) || !aligned16(tiled_scales))
        return MOE_ERR_ALIGNMENT;
    if (rows == 0) return MOE_OK;
    if (moe::launch_tile(packed, scales, rows, K, tiled_packed, tiled_scales,
                         static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
