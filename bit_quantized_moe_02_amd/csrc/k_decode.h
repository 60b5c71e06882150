// Launch interface of the decode-shape expert FFN kernels (k_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

struct DecArgs {
  const uint16_t* x;          // bf16 [T][H]
  int T, H, I, Is, I_pad, Is_pad, k, E;
  int nw_ug, nw_dn;           // waves per workgroup of the two kernels
  int tb_ug, tb_dn;           // tile bytes of the routed up/gate and down formats
  int fmt_s, tb_s;            // shared expert: MOE_FMT_BF16 or MOE_FMT_Q8, and its tile bytes
  const int32_t* topk_idx;    // [T][k]
  const uint8_t* up;          // routed experts, packed, expert-major
  const uint8_t* gate;
  const uint8_t* down;
  size_t expert_bytes;        // bytes of one packed up (= gate) matrix
  size_t expert_bytes_down;   // bytes of one packed down matrix
  const uint8_t* sup;         // shared expert, BF16 or Q8 tiles (or null)
  const uint8_t* sgate;
  const uint8_t* sdown;
  const int8_t* codebook;     // CB2 table (device)
  // workspace
  _Float16* h;                // [T*k][I]   fp16, slot order
  _Float16* hs;               // [T][Is]    fp16
  float* hsum;                // [T*k][I_pad/16][2]  (sum h, offset sum) per 16 rows
  float* ybuf;                // [T*k][H]   fp32 per-slot down outputs
  float* ysh;                 // [T][H]     fp32 shared-expert output
  int* xexp;                  // [T] each token's exponent e (x enters fp16 as x 2^-e, h is stored as h 2^-2e)
  // Routing inside the single-token CB2 up/gate (null logits: topk_idx is
  // given).  The kernel ranks token t_route's top k from the router's logits
  // [T_route][E] and workgroup 0 writes them to topk_idx_out / topk_w_out
  // (which the down kernel then reads as topk_idx / topk_w).
  const float* logits;
  int n_parts, T_route, t_route;     // n_parts: 1 (final logits)
  int32_t* topk_idx_out;
  float* topk_w_out;
};

size_t dec_upgate_lds(const DecArgs& a, int fmt);
size_t dec_down_lds(const DecArgs& a);
hipError_t launch_dec_upgate(const DecArgs& a, int fmt, int cpw, int grid, hipStream_t s);
hipError_t launch_dec_down(const DecArgs& a, int fmt, int grid, hipStream_t s);
// Single-token path (k_decode1.hip): up/gate then down with the shared
// expert and the weighted combine fused; writes y directly.
// LDS of the single-token down kernel of format fmt_dn with nw waves.
size_t dec1_down_lds(const DecArgs& a, int fmt_dn, int nw);
// LDS of the single-token CB2 up/gate with nw waves (route: it ranks the
// token's experts itself).
size_t dec1_cb2_upgate_lds(int nw, bool route);
// cus = compute units of the device (the grids are sized from it).
hipError_t launch_dec1(const DecArgs& a, int fmt_ug, int fmt_dn, const float* topk_w, float* y,
                       int cus, hipStream_t s);
hipError_t launch_combine(const DecArgs& a, const int32_t* topk_idx, const float* topk_w, float* y,
                          hipStream_t s);
// Batched path (k_decodem.hip): 2..16 tokens, CB2/CB2/K2, H/256 and
// I_pad/256 at most 16 chunks each.
size_t decm_upgate_lds(int nw);
size_t decm_down_lds(const DecArgs& a, int nw);
hipError_t launch_decm(const DecArgs& a, const float* topk_w, float* y, int cus, hipStream_t s);

}  // namespace qmoe
