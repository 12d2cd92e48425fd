// Host side of the C ABI declared in include/moe_mxfp4.h: argument checks,
// workspace carve-up and the launch sequence of one forward call.
//
// A forward call is four to eight launches on the caller's stream and nothing else
// (no allocation, no host synchronisation, no device-to-host copy), so it can
// be captured into a HIP graph: the pages stress that at microsecond
// operator times the gaps between operators matter (techllm.github.io
// "Xiaomi MiMo x TileRT", section "3. TileRT").
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "layer.hpp"

struct moe_mxfp4_ctx {
    moe_mxfp4_config cfg;
    moe_mxfp4_weights w;
    // optional stage timing: capacity slots of NUM_STAGES + 1 events each;
    // valid[slot] is set once every event of a call was recorded into it
    std::vector<hipEvent_t> events;
    std::vector<char> valid;
    int32_t capacity = 0;
    int64_t ncalls = 0;
    // MOE_MXFP4_LOG=1 at create: print the launch sequence of a call when
    // it differs from the previous call's
    bool log = false;
    std::atomic<int32_t> logged_tokens{-1};
    // bf16 activations, from MOE_MXFP4_PATH at create: one launch of both
    // projections ("fused", the default: for a single verify block the
    // routing and permutation run inside that launch, else in launches of
    // their own; then the combine), the same with the routing always in
    // launches of its own ("fused_launches"), or one launch per phase
    // ("stream")
    bool fused = false;
    bool layer = false;
};

namespace {

using moe::kMaxExperts;
using moe::kMaxTopK;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
    size_t logits, ids, w, offsets, sorted, active, chunks, nchunks, xtab, sort_part, xq, xs, h, hs, o, fctl,
        total;
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
    L.xtab = at;    at += round256(((size_t)moe::kXtabHead + (size_t)moe::kXcds * moe::xcd_slots(dm) * moe::kXtabRec) *
                                   sizeof(int32_t));
    L.sort_part = at; at += round256((size_t)moe::sort_tiles((int)P) * c.num_experts * sizeof(int32_t));
    const bool mx8 = c.act_mode == MOE_ACT_MXFP8_E4M3;
    L.xq = at;      at += mx8 ? round256((size_t)T * c.d_model) : 0;
    L.xs = at;      at += mx8 ? round256((size_t)T * (c.d_model / MOE_MXFP4_BLOCK)) : 0;
    L.h = at;       at += round256(P * (size_t)c.d_ff * (mx8 ? 1 : sizeof(uint16_t)));
    L.hs = at;      at += mx8 ? round256(P * (size_t)(c.d_ff / MOE_MXFP4_BLOCK)) : 0;
    L.o = at;       at += round256(P * (size_t)c.d_model * sizeof(float));
    // the fused path's counters (bf16 mode)
    const bool fz = !mx8 && moe::fused_supported(dm);
    L.fctl = at;    at += fz ? round256((size_t)moe::fused_ctl_ints(dm) * sizeof(int32_t)) : 0;
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

// Poll rounds before a device-side wait of the fused kernel gives up (each
// round sleeps ~0.1 us).  MOE_MXFP4_SPIN_LIMIT overrides it, for tests of
// the error path: a negative value makes every wait give up at once, so the
// kernel raises its error flag and every workgroup exits normally.  Read on
// every call.
int spin_limit() {
    const char* e = std::getenv("MOE_MXFP4_SPIN_LIMIT");
    return e && *e ? std::atoi(e) : (1 << 22);
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
    // The activation rows the expert kernels read (x: T rows of d, h: P rows
    // of f) are addressed by 32-bit byte offsets: buffer-resource offsets for
    // the MXFP8 codes (1 byte each), direct-to-LDS source offsets for bf16
    // (2 bytes each).  Both arrays must stay below 4 GiB.
    const int64_t act_bytes = c->act_mode == MOE_ACT_MXFP8_E4M3 ? 1 : 2;
    if ((int64_t)c->max_tokens * c->d_model * act_bytes >= (int64_t)1 << 32 ||
        (int64_t)c->max_tokens * c->top_k * c->d_ff * act_bytes >= (int64_t)1 << 32)
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
    const char* path = std::getenv("MOE_MXFP4_PATH");
    if (path && *path && std::strcmp(path, "fused") != 0 && std::strcmp(path, "fused_launches") != 0 &&
        std::strcmp(path, "stream") != 0)
        return MOE_ERR_INVALID_ARG;
    moe_mxfp4_ctx* ctx = new (std::nothrow) moe_mxfp4_ctx;
    if (!ctx) return MOE_ERR_INTERNAL;
    ctx->cfg = *cfg;
    ctx->w = *weights;
    ctx->fused = !(path && std::strcmp(path, "stream") == 0);      // "fused" is the default
    ctx->layer = !(path && *path) || std::strcmp(path, "fused") == 0;
    const char* lg = std::getenv("MOE_MXFP4_LOG");
    ctx->log = lg && *lg && std::strcmp(lg, "0") != 0;
    if (ctx->log)
        std::fprintf(stderr, "moe_mxfp4: create E=%d d=%d f=%d k=%d max_tokens=%d act=%s out=%s path=%s\n",
                     cfg->num_experts, cfg->d_model, cfg->d_ff, cfg->top_k, cfg->max_tokens,
                     cfg->act_mode == MOE_ACT_MXFP8_E4M3 ? "mxfp8" : "bf16",
                     cfg->out_dtype == MOE_OUT_F32 ? "f32" : "bf16",
                     cfg->act_mode == MOE_ACT_MXFP8_E4M3 ? "dense"
                     : ctx->layer                         ? "fused"
                     : ctx->fused                         ? "fused_launches"
                                                          : "stream");
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
    ctx->valid.clear();
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
    ctx->valid.assign((size_t)capacity, 0);
    ctx->capacity = capacity;
    return MOE_OK;
}

moe_status moe_mxfp4_stage_times(moe_mxfp4_ctx* ctx, float* total_ms, int32_t* calls) {
    if (!ctx || !total_ms || !calls || ctx->capacity == 0) return MOE_ERR_INVALID_ARG;
    // slots 0 .. held-1 were written; a slot whose call failed part-way is
    // not valid and is skipped
    const int64_t held = ctx->ncalls < ctx->capacity ? ctx->ncalls : ctx->capacity;
    for (int i = 0; i < MOE_MXFP4_NUM_STAGES; ++i) total_ms[i] = 0.f;
    int32_t counted = 0;
    for (int64_t slot = 0; slot < held; ++slot) {
        if (!ctx->valid[slot]) continue;
        hipEvent_t* ev = &ctx->events[slot * (MOE_MXFP4_NUM_STAGES + 1)];
        if (hipEventSynchronize(ev[MOE_MXFP4_NUM_STAGES]) != hipSuccess) return MOE_ERR_HIP;
        for (int i = 0; i < MOE_MXFP4_NUM_STAGES; ++i) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, ev[i], ev[i + 1]) != hipSuccess) return MOE_ERR_HIP;
            total_ms[i] += ms;
        }
        ++counted;
    }
    *calls = counted;
    ctx->ncalls = 0;
    std::fill(ctx->valid.begin(), ctx->valid.end(), 0);
    return MOE_OK;
}

size_t moe_mxfp4_workspace_bytes(const moe_mxfp4_ctx* ctx, int32_t num_tokens) {
    if (!ctx || num_tokens <= 0) return 0;
    return make_layout(ctx->cfg, num_tokens).total;
}

}  // extern "C"

namespace {

// The optional routing outputs, copied from the workspace on stream s.
moe_status copy_debug(const moe_mxfp4_config& c, const moe::Dims& dm, const moe::Workspace& ws,
                      const moe_mxfp4_routing* debug_out, hipStream_t s) {
    if (!debug_out) return MOE_OK;
    const size_t P = (size_t)dm.P;
    struct { void* dst; const void* src; size_t n; } cp[4] = {
        {debug_out->topk_ids, ws.topk_ids, P * sizeof(int32_t)},
        {debug_out->topk_w, ws.topk_w, P * sizeof(float)},
        {debug_out->expert_offsets, ws.offsets, (size_t)(c.num_experts + 1) * sizeof(int32_t)},
        {debug_out->sorted_pairs, ws.sorted_pairs, P * sizeof(int32_t)}};
    for (auto& k : cp)
        if (k.dst && hipMemcpyAsync(k.dst, k.src, k.n, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return MOE_ERR_HIP;
    return MOE_OK;
}

// State blocks of the layer kernel that routes in every workgroup:
// kLayerPool per device, in a device array (each block cleared by a small
// launch the first time a stream takes it, or after a call whose combine
// launch, which clears the block for the next call, could not be made).  A
// stream keeps its block for the life of the process, so calls on one stream
// find the block their predecessor left clear; calls that may overlap run on
// different streams and so on different blocks.  Blocks are shared by every
// context on the device.  With every block taken, further streams use the
// other launches.  In host code the array's name is a host-side stand-in:
// only the device address found with hipGetSymbolAddress is handed to
// kernels.
constexpr int kLayerPool = 16;
__device__ __align__(256) int32_t layer_pool[kLayerPool * moe::kLayerStateInts];

constexpr int kMaxDevices = 64;
struct LayerPool {
    int32_t* base = nullptr;                 // device address of layer_pool
    hipStream_t stream[kLayerPool] = {};
    bool taken[kLayerPool] = {};
    bool clear[kLayerPool] = {};             // the last call on it made its combine launch
};
std::mutex layer_mu;
LayerPool layer_dev[kMaxDevices];

// The block of stream s on the current device (taken now if `take`), with
// *fresh = true when it must be cleared before use; *clear: its flag, which
// the caller lowers before its launches and raises once the combine launch
// is made.  nullptr if the stream has none and none is left (or on a HIP
// error).
int32_t* layer_state(hipStream_t s, bool take, bool* fresh, bool** clear = nullptr) {
    *fresh = false;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(layer_mu);
    LayerPool& lp = layer_dev[dev];
    if (!lp.base) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(layer_pool)) != hipSuccess || !p) return nullptr;
        lp.base = static_cast<int32_t*>(p);
    }
    for (int i = 0; i < kLayerPool; ++i)
        if (lp.taken[i] && lp.stream[i] == s) {
            *fresh = !lp.clear[i];
            if (clear) *clear = &lp.clear[i];
            return lp.base + (size_t)i * moe::kLayerStateInts;
        }
    if (!take) return nullptr;
    for (int i = 0; i < kLayerPool; ++i)
        if (!lp.taken[i]) {
            lp.taken[i] = true;
            lp.stream[i] = s;
            lp.clear[i] = false;
            *fresh = true;
            if (clear) *clear = &lp.clear[i];
            return lp.base + (size_t)i * moe::kLayerStateInts;
        }
    return nullptr;
}

// The launches of one forward call on stream s, the workspace already
// carved; mark(i) records stage-timing event i (a no-op when timing is off).
template <typename Mark>
moe_status launch_all(moe_mxfp4_ctx* ctx, const uint16_t* x, const float* router_logits, const void* w_router,
                      float* ws_logits, const moe::Dims& dm, const moe::Workspace& ws, void* out,
                      const moe_mxfp4_routing* debug_out, hipStream_t s, Mark mark) {
    const moe_mxfp4_config& c = ctx->cfg;
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
    bool fresh = false, *lclear = nullptr;
    int32_t* lstate =
        !mx8 && ctx->layer && moe::layer_supported(dm) ? layer_state(s, true, &fresh, &lclear) : nullptr;
    if (lstate) {
        // routing, permutation and both projections in one launch (timed as
        // the gate/up stage), then the combine, which clears the stream's
        // state block for its next call; a block not known to be clear is
        // cleared first
        if (fault_at("route") || fault_at("sort") || fault_at("gateup") || fault_at("down")) return MOE_ERR_HIP;
        if (mark(1) != hipSuccess || mark(2) != hipSuccess) return MOE_ERR_HIP;
        *lclear = false;
        if (fresh && moe::launch_layer_clear(lstate, s) != hipSuccess) return MOE_ERR_HIP;
        if (mark(3) != hipSuccess ||
            moe::launch_layer(x, router_logits, ctx->w, dm, ws, lstate, spin_limit(), s) != hipSuccess ||
            mark(4) != hipSuccess || mark(5) != hipSuccess)
            return MOE_ERR_HIP;
        if (fault_at("combine") || moe::launch_finalize_layer(dm, ws, out, c.out_dtype, lstate, s) != hipSuccess)
            return MOE_ERR_HIP;
        // Under stream capture nothing ran: the launches (a clear among them)
        // only enter the graph, so the block is not known to be clear until
        // an eager call has cleared it.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cap) != hipSuccess) return MOE_ERR_HIP;
        *lclear = cap == hipStreamCaptureStatusNone;
        if (mark(6) != hipSuccess) return MOE_ERR_HIP;
        if (ctx->log && ctx->logged_tokens.exchange(dm.T) != dm.T)
            std::fprintf(stderr, "moe_mxfp4: T=%d P=%d E=%d d=%d f=%d k=%d: %sone launch of routing and "
                         "permutation in every workgroup, gate/up + SwiGLU and down; combine (float32 per-pair "
                         "outputs)\n",
                         dm.T, dm.P, dm.E, dm.d, dm.f, dm.k, w_router ? "router projection, " : "");
        return copy_debug(c, dm, ws, debug_out, s);
    }
    if (!mx8 && ctx->fused && moe::fused_supported(dm)) {
        // routing (which clears the fused kernel's counters) and the
        // permutation, then one launch of gate/up and down units (timed as
        // the gate/up stage), then the combine
        const bool chain = moe::fused_chain_form(dm);
        const bool rs = moe::route_sort_fused(dm);
        if (fault_at("route") ||
            (rs ? moe::launch_route_sort(router_logits, dm, ws, chunk_rows, s, ws.fctl, moe::fused_ctl_ints(dm))
                : moe::launch_route(router_logits, dm, ws, s, ws.fctl, moe::fused_ctl_ints(dm))) != hipSuccess ||
            mark(1) != hipSuccess)
            return MOE_ERR_HIP;
        if (!rs && (fault_at("sort") || moe::launch_sort(dm, ws, chunk_rows, s) != hipSuccess)) return MOE_ERR_HIP;
        if (mark(2) != hipSuccess || mark(3) != hipSuccess) return MOE_ERR_HIP;
        // one launch runs both projections: it is the gate/up and the down site
        if (fault_at("gateup") || fault_at("down") ||
            moe::launch_fused(x, ctx->w, dm, ws, spin_limit(), s) != hipSuccess ||
            mark(4) != hipSuccess || mark(5) != hipSuccess)
            return MOE_ERR_HIP;
        if (fault_at("combine") || moe::launch_finalize(dm, ws, out, c.out_dtype, false, s) != hipSuccess ||
            mark(6) != hipSuccess)
            return MOE_ERR_HIP;
        if (ctx->log && ctx->logged_tokens.exchange(dm.T) != dm.T)
            std::fprintf(stderr, "moe_mxfp4: T=%d P=%d E=%d d=%d f=%d k=%d: %s%s, combine (float32 per-pair "
                         "outputs)\n",
                         dm.T, dm.P, dm.E, dm.d, dm.f, dm.k, w_router ? "router projection, " : "",
                         chain ? "routing, permutation + per-XCD chunk lists, one launch of ticketed gate/up and "
                                 "down units"
                               : "routing, permutation, persistent kernel (gate/up + SwiGLU, down)");
        return copy_debug(c, dm, ws, debug_out, s);
    }
    const bool fused_rs = moe::route_sort_fused(dm);
    if (fused_rs) {
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
    const hipError_t gu = mx8 ? moe::launch_gateup_dense(ctx->w, dm, ws, s) : moe::launch_gateup(x, ctx->w, dm, ws, s);
    if (gu != hipSuccess || mark(4) != hipSuccess) return MOE_ERR_HIP;
    if (fault_at("down")) return MOE_ERR_HIP;
    const hipError_t dn = mx8 ? moe::launch_down_dense(ctx->w, dm, ws, s) : moe::launch_down(ctx->w, dm, ws, s);
    if (dn != hipSuccess || mark(5) != hipSuccess) return MOE_ERR_HIP;
    if (fault_at("combine") || moe::launch_finalize(dm, ws, out, c.out_dtype, mx8, s) != hipSuccess ||
        mark(6) != hipSuccess)
        return MOE_ERR_HIP;

    if (ctx->log && ctx->logged_tokens.exchange(dm.T) != dm.T)
        std::fprintf(stderr, "moe_mxfp4: T=%d P=%d E=%d d=%d f=%d k=%d: %s%s%s%s, combine (%s per-pair outputs)\n",
                     dm.T, dm.P, dm.E, dm.d, dm.f, dm.k, w_router ? "router projection, " : "",
                     fused_rs ? "routing+permutation (one launch)" : "routing, permutation",
                     mx8 ? ", MXFP8 quantisation of x" : "",
                     mx8 ? ", dense gate/up + SwiGLU (FP8 x FP4 scaled MFMA), dense down"
                         : ", streaming gate/up + SwiGLU (FP4->bf16 MFMA), streaming down",
                     mx8 ? "fp16-coded" : "float32");

    return copy_debug(c, dm, ws, debug_out, s);
}

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
    ws.xtab = reinterpret_cast<int32_t*>(base + L.xtab);
    ws.sort_part = reinterpret_cast<int32_t*>(base + L.sort_part);
    ws.xq = reinterpret_cast<uint8_t*>(base + L.xq);
    ws.xs = reinterpret_cast<uint8_t*>(base + L.xs);
    ws.h = reinterpret_cast<uint8_t*>(base + L.h);
    ws.hs = reinterpret_cast<uint8_t*>(base + L.hs);
    ws.o = reinterpret_cast<float*>(base + L.o);
    ws.os = reinterpret_cast<uint8_t*>(base + L.o + (size_t)num_tokens * c.top_k * c.d_model * sizeof(uint16_t));
    ws.fctl = reinterpret_cast<int32_t*>(base + L.fctl);

    moe::Dims dm{num_tokens, c.d_model, c.d_ff, c.num_experts, c.top_k, num_tokens * c.top_k};
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const uint16_t* x = static_cast<const uint16_t*>(hidden);

    if (ctx->capacity == 0)
        return launch_all(ctx, x, router_logits, w_router, ws_logits, dm, ws, out, debug_out, s,
                          [](int) { return hipSuccess; });
    // stage timing: the call's events go to slot ncalls % capacity, which
    // counts only if every launch and event of the call succeeded
    const int64_t slot = ctx->ncalls % ctx->capacity;
    hipEvent_t* ev = &ctx->events[(size_t)slot * (MOE_MXFP4_NUM_STAGES + 1)];
    ctx->valid[slot] = 0;
    const moe_status st = launch_all(ctx, x, router_logits, w_router, ws_logits, dm, ws, out, debug_out, s,
                                     [&](int i) { return hipEventRecord(ev[i], s); });
    if (st == MOE_OK) {
        ctx->valid[slot] = 1;
        ++ctx->ncalls;
    }
    return st;
}

// Scratch of moe_mxfp4_forward_noalloc: a device array of fixed size (one
// per GPU, held until the process ends).  In host code `scratch` names a
// host-side stand-in, so its device address is looked up once per device
// with hipGetSymbolAddress and only that address is ever handed to kernels.
__device__ __align__(256) uint8_t scratch[MOE_MXFP4_NOALLOC_SCRATCH_BYTES];

std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (nullptr on a HIP error).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
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

moe_status moe_mxfp4_forward_noalloc(moe_mxfp4_ctx* ctx, const void* hidden, const float* router_logits,
                                     int32_t num_tokens, void* out, void* hip_stream,
                                     const moe_mxfp4_routing* debug_out) {
    if (!ctx || num_tokens < 0) return MOE_ERR_INVALID_ARG;
    if (num_tokens > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    if (num_tokens == 0) return MOE_OK;
    if (!router_logits) return MOE_ERR_INVALID_ARG;
    // size check before anything touches the device
    if (make_layout(ctx->cfg, num_tokens).total > (size_t)MOE_MXFP4_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    if (!hidden || !out) return MOE_ERR_INVALID_ARG;
    void* ws = scratch_for_current_device();
    if (!ws) return MOE_ERR_HIP;
    return forward_impl(ctx, hidden, router_logits, nullptr, num_tokens, out, ws,
                        (size_t)MOE_MXFP4_NOALLOC_SCRATCH_BYTES, hip_stream, debug_out);
}

moe_status moe_mxfp4_forward_hidden(moe_mxfp4_ctx* ctx, const void* hidden, const void* w_router,
                                    int32_t num_tokens, void* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream, const moe_mxfp4_routing* debug_out) {
    if (!w_router && num_tokens > 0) return MOE_ERR_INVALID_ARG;
    return forward_impl(ctx, hidden, nullptr, w_router, num_tokens, out, workspace, workspace_bytes, hip_stream,
                        debug_out);
}

moe_status moe_mxfp4_device_status(const moe_mxfp4_ctx* ctx, const void* workspace, int32_t num_tokens,
                                   int32_t* status, void* hip_stream) {
    if (!ctx || !status || num_tokens < 0) return MOE_ERR_INVALID_ARG;
    if (num_tokens > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    *status = 0;
    const moe::Dims dm{num_tokens, ctx->cfg.d_model, ctx->cfg.d_ff, ctx->cfg.num_experts, ctx->cfg.top_k,
                       num_tokens * ctx->cfg.top_k};
    if (num_tokens == 0 || ctx->cfg.act_mode != MOE_ACT_BF16 || !ctx->fused || !moe::fused_supported(dm))
        return MOE_OK;                                // no device-side waits on this path
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (ctx->layer && moe::layer_supported(dm)) {
        // routing in the expert kernel: the stream's state block (none yet:
        // no call)
        bool fresh = false;
        const int32_t* st = layer_state(s, false, &fresh);
        if (!st) return MOE_OK;
        int32_t ep = 0, err = 0;
        if (hipMemcpyAsync(&ep, st + moe::kLayerEpoch, sizeof(ep), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipMemcpyAsync(&err, st + moe::kLayerError, sizeof(err), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return MOE_ERR_HIP;
        *status = ep != 0 && err == ep;            // raised by the call that advanced the epoch last
        return MOE_OK;
    }
    if (!workspace) return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(ctx->cfg, num_tokens);
    int32_t word = 0;
    const char* src = static_cast<const char*>(workspace) + L.fctl + moe::kFusedErrorWord * sizeof(int32_t);
    if (hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return MOE_ERR_HIP;
    *status = word;
    return MOE_OK;
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

moe_status moe_mxfp4_debug_hidden(const moe_mxfp4_ctx* ctx, const void* workspace, int32_t num_tokens, void* h,
                                  uint8_t* h_scales, void* hip_stream) {
    if (!ctx || !workspace || !h || num_tokens <= 0) return MOE_ERR_INVALID_ARG;
    const moe_mxfp4_config& c = ctx->cfg;
    if (num_tokens > c.max_tokens) return MOE_ERR_CAPACITY;
    const bool mx8 = c.act_mode == MOE_ACT_MXFP8_E4M3;
    if (mx8 && !h_scales) return MOE_ERR_INVALID_ARG;
    if (!aligned16(workspace) || !aligned16(h) || (mx8 && !aligned16(h_scales))) return MOE_ERR_ALIGNMENT;
    const Layout L = make_layout(c, num_tokens);
    const size_t P = (size_t)num_tokens * c.top_k;
    const char* base = static_cast<const char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (hipMemcpyAsync(h, base + L.h, P * c.d_ff * (mx8 ? 1 : 2), hipMemcpyDeviceToDevice, s) != hipSuccess)
        return MOE_ERR_HIP;
    if (mx8 && hipMemcpyAsync(h_scales, base + L.hs, P * (c.d_ff / MOE_MXFP4_BLOCK), hipMemcpyDeviceToDevice, s) !=
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
