// Launch interface of the router kernels (k_route.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// logits: workspace fp32 [T][E], route_logit_floats(T, E) of them (the final
// logits, bias included).
inline size_t route_logit_floats(int T, int E) { return (size_t)T * E; }
hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                        int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s);
// The two halves of launch_route: logits [T][E] (route_logit_parts(T, H) = 1
// part), then the top-k of each token from them.
int route_logit_parts(int T, int H);
hipError_t launch_route_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                               float* logits, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int n_parts, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s);

}  // namespace qmoe
