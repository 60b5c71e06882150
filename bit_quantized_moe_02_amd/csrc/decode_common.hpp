// Helpers shared by the multi-token decode kernels (k_decode.hip,
// k_decodem.hip): the distinct experts among a batch's T*k choices with the
// bitmask of tokens that chose each, and the weighted split of work items
// over the grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe_dec {

constexpr int kMaxT = 16;
constexpr int kMaxSlots = 256;   // T * k <= 256

// ---------------------------------------------------------------------------
// Distinct experts of the T*k choices, in order of first appearance (slot
// order).  Invalid ids (outside [0, E)) are skipped.
struct ExpertList {
  int n;
  int expert[kMaxSlots];
  uint32_t mask[kMaxSlots];
  int slot_e[kMaxSlots];
};

__device__ inline void build_expert_list(const int32_t* topk_idx, int n_slots, int k, int E, ExpertList* L) {
  const int tid = threadIdx.x;
  for (int i = tid; i < n_slots; i += blockDim.x) {
    const int e = topk_idx[i];
    L->slot_e[i] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  if (tid < 64) {
    int base = 0;
    for (int c0 = 0; c0 < n_slots; c0 += 64) {
      const int i = c0 + tid;
      bool first = false;
      uint32_t mask = 0;
      int e = -1;
      if (i < n_slots) {
        e = L->slot_e[i];
        if (e >= 0) {
          first = true;
          for (int j = 0; j < n_slots; ++j) {
            if (L->slot_e[j] == e) {
              mask |= 1u << (j / k);
              if (j < i) first = false;
            }
          }
        }
      }
      const uint64_t b = __ballot(first);
      if (first) {
        const int pos = base + __popcll(b & ((1ull << tid) - 1ull));
        L->expert[pos] = e;
        L->mask[pos] = mask;
      }
      base += __popcll(b);
    }
    if (tid == 0) L->n = base;
  }
  __syncthreads();
}

// Items [first, last) of workgroup g when n_s shared items of weight w_s come
// first and n_r routed items of weight w_r follow; item i goes to the
// workgroup whose share of the total weight holds the item's midpoint.
__device__ inline int64_t item_start(int64_t g, int64_t G, int64_t n_s, int64_t w_s, int64_t n_r,
                              int64_t w_r) {
  const int64_t W = n_s * w_s + n_r * w_r;
  // first item i with (2 P(i) + w(i)) * G >= 2 g W
  int64_t lo = 0, hi = n_s + n_r;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    int64_t twoM;
    if (mid < n_s) twoM = 2 * mid * w_s + w_s;
    else twoM = 2 * (n_s * w_s + (mid - n_s) * w_r) + w_r;
    if (twoM * G >= 2 * g * W) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

}  // namespace qmoe_dec
