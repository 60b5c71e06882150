// Launch interface of the prefill-shape expert FFN kernels (k_prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

struct PfArgs {
  const uint16_t* x;              // bf16 [T][H]
  const uint16_t* x16;            // fp16 [T][H] copy of x (workspace; written by the launch)
  int T, H, I, Is, I_pad, Is_pad, k, E;
  const int32_t* offsets;         // [E+1]
  const int32_t* sorted_slots;    // [T*k]
  const int32_t* slot_pos;        // [T*k]
  const uint8_t* up;
  const uint8_t* gate;
  const uint8_t* down;
  size_t expert_bytes, expert_bytes_down;
  const uint8_t* sup;             // shared expert, BF16 or Q8 tiles (fmt_s)
  const uint8_t* sgate;
  const uint8_t* sdown;
  int fmt_s, tb_s;
  const int8_t* codebook;
  // workspace
  _Float16* h;                    // [T*k][I]  fp16, grouped (position) order
  _Float16* hs;                   // [T][Is]   fp16
  float* yslot;                   // [T*k][H]  fp32, grouped order
  float* ysh;                     // [T][H]    fp32
  int* xexp;                      // [T]       each token's exponent e (x enters fp16 as x 2^-e, h = h 2^-2e)
  int* epos;                      // [T*k]     e of the token at each grouped position
};

int pf_m_rows();
hipError_t launch_prefill(const PfArgs& a, int fmt_ug, int fmt_dn, const float* topk_w, float* y,
                          hipStream_t s);

}  // namespace qmoe
