// Launch interface of the router kernels (k_route.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// logits: workspace fp32, route_logit_floats(T, E) of them (few tokens: up to
// 16 partial logits per (token, expert), one per 512-column slice of H).
inline size_t route_logit_floats(int T, int E) { return (size_t)(T <= 16 ? 16 : 1) * T * E; }
hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                        int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s);

}  // namespace qmoe
