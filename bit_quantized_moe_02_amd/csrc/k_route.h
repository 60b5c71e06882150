// Launch interface of the router kernels (k_route.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// logits: workspace fp32 [route_logit_parts(T, H)][T][E], route_logit_floats
// (T, E) of them: up to 16 tokens the final logits (one part), beyond
// kLogitSplit partial sums over column ranges (bias in part 0) that the
// top-k kernel adds in part order.
constexpr int kLogitSplit = 4;
inline size_t route_logit_floats(int T, int E) { return (size_t)(T > 16 ? kLogitSplit : 1) * T * E; }
hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                        int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s);
// The two halves of launch_route: the logits (route_logit_parts(T, H)
// parts), then the top-k of each token from them.
int route_logit_parts(int T, int H);
hipError_t launch_route_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                               float* logits, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int n_parts, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s);

}  // namespace qmoe
