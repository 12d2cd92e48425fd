// Declarations of the expert launch that routes a verify block itself
// (fused.hip k_layer) and of the combine launch that follows it.
#pragma once

#include "common.hpp"

namespace moe {

// Layer in two launches (bf16 activations, one verify block: at most 64
// pairs over at most 128 experts, no more pairs than experts, at most
// kLayerMaxLogits router logits): one persistent launch routes the tokens and
// permutes the pairs inside every workgroup and runs the gate/up and down
// units; the combine follows.  The first launch's counters live in a state
// block of kLayerStateInts ints that a stream keeps across calls: the
// combine launch clears them for the stream's next call (a launch after the
// kernel that uses them, so no launch runs in front of it) and advances the
// epoch (calls completed on the block); the error word holds epoch + 1 of
// the last call in which a wait gave up.
constexpr int kLayerMaxLogits = 1024;               // T * E, staged in LDS
constexpr int kLayerLine = 64;                      // ints per 256-byte line
enum {
    kLayerEpoch = 0,
    kLayerError = kLayerLine,
    kLayerQueue = 2 * kLayerLine,
    kLayerChunkDone = 3 * kLayerLine,
    kLayerStateInts = kLayerChunkDone + kChunk * kLayerLine
};
bool layer_supported(const Dims& dm);
// The routing, permutation and both projections; the per-pair outputs go to
// ws.o for launch_finalize_layer.  state: the stream's block.
hipError_t launch_layer(const uint16_t* x, const float* logits, const moe_mxfp4_weights& w, const Dims& dm,
                        const Workspace& ws, int32_t* state, int spin_limit, hipStream_t s);
// Zero a state block (its first use on a device, or after a call whose
// combine launch failed).
hipError_t launch_layer_clear(int32_t* state, hipStream_t s);
// The combine of such a call (as launch_finalize with float32 per-pair
// outputs), which also clears the state block's counters for the stream's
// next call and advances its epoch.
hipError_t launch_finalize_layer(const Dims& dm, const Workspace& ws, void* out, int out_dtype, int32_t* state,
                                 hipStream_t s);

}  // namespace moe
