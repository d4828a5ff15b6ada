// Plainly written ("scalar") variant of the fused decode expert kernel
// (scalar.hip); the grouped GEMMs' plain variants live beside the fast ones in
// prefill.hip and are chosen with PrefillArgs::scalar.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace moe {

// The route (top-k, weights, shared gate) of the step from b.logits into
// b.route_idx / route_w / route_gamma, h [(k + 1)][I] of the k routed
// experts (records at experts + (gid_base + e) * stride) and the shared one,
// then the weighted partial down rows into b.partial exactly as
// launch_expert writes them, for the shapes fused_expert_supported accepts.
// Three launches; one thread per value.
hipError_t launch_expert_scalar(const Geometry& g, const uint8_t* experts, uint64_t stride, int64_t gid_base,
                                const uint8_t* shared_rec, const StepBuffers& b, float* h, hipStream_t s);

}  // namespace moe
