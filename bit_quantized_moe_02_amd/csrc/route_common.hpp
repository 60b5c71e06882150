// Top-k ranking shared by the router kernels and the single-token up/gate
// kernel that routes its token itself ([digest] "Model weights": routing
// stays unquantized; the function is softmax, top-k, renormalize).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"

namespace qmoe_route {

using qmoe_dev::u32x4;

// Top-k by rank counting, one 1024-thread workgroup per token.  The logit of
// expert e is the sum of n_parts partial logits (in part order).  Each
// (logit, e) becomes a 64-bit key whose integer order is "larger logit first,
// equal logits (+0 and -0 identified) lower index first"; all keys are
// distinct, so the rank of a key -- the number of keys above it -- is its
// position in that order.  Four threads count each key's rank over a quarter
// of the keys each.  The experts of rank < k are kept, and
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) with the sum taken in rank
// order.
__device__ __forceinline__ uint64_t route_key(float l, int e) {
  if (l == 0.0f) l = 0.0f;
  uint32_t b = __builtin_bit_cast(uint32_t, l);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Rank top-k of one token with the first NT threads of the workgroup (NT a
// multiple of 256; every thread reaches the barriers): logit_of(e) gives
// expert e's logit; NT/256 threads count each key's rank over a share of the
// keys; out(j, e, w) receives choice j (thread j, j < k).  Shared scratch
// comes from the caller.
struct TopkLds {
  uint64_t key[1024];
  float lg[1024];
  int part_rank[4][256];
  float kv[16];
  int ki[16];
};

template <int NT, typename LogitOf, typename Out>
__device__ __forceinline__ void rank_topk(TopkLds& sm, int E, int k, LogitOf logit_of, Out out) {
  constexpr int Q = NT / 256;
  const int tid = threadIdx.x;
  const int Ep = (E + 31) & ~31;               // keys padded with 0 (below every real key)
  for (int e = tid; tid < NT && e < Ep; e += NT) {
    float s = 0.f;
    uint64_t kk = 0;
    if (e < E) {
      s = logit_of(e);
      kk = route_key(s, e);
    }
    sm.key[e] = kk;
    sm.lg[e] = s;
  }
  __syncthreads();
  const int q = tid >> 8, el = tid & 255;
  const int span = Ep / Q;                      // multiple of 8
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + el;
    int cnt = 0;
    if (e < E && q < Q) {
      const uint64_t mine = sm.key[e];
      const int i_end = (q + 1) * span;
      // span is a multiple of 8: four 16-byte reads in flight per step
#pragma unroll 2
      for (int i = q * span; i < i_end; i += 8) {
        u32x4 v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = *reinterpret_cast<const u32x4*>(&sm.key[i + 2 * r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint64_t k0 = (uint64_t)v[r].x | ((uint64_t)v[r].y << 32);
          const uint64_t k1 = (uint64_t)v[r].z | ((uint64_t)v[r].w << 32);
          cnt += (k0 > mine) + (k1 > mine);
        }
      }
    }
    if (q < Q) sm.part_rank[q][el] = cnt;
    __syncthreads();
    if (q == 0 && e < E) {
      int rank = 0;
      for (int i = 0; i < Q; ++i) rank += sm.part_rank[i][el];
      if (rank < k) {
        sm.kv[rank] = sm.lg[e];
        sm.ki[rank] = e;
      }
    }
    __syncthreads();
  }
  if (tid < k) {
    const float top = sm.kv[0];
    float z = 0.f;
    for (int j = 0; j < k; ++j) z += expf(sm.kv[j] - top);
    out(tid, sm.ki[tid], expf(sm.kv[tid] - top) / z);
  }
}


// Wave-wide maximum of an unsigned value by DPP, with no LDS traffic: row
// shifts leave each row's maximum in its lane 15, two row broadcasts carry
// the rows' maxima to lane 63, which every lane reads.  Lanes whose DPP
// source lies outside the row, and lanes a mask leaves out, take 0, which
// does not change an unsigned maximum.
template <int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, Ctrl, RowMask, BankMask, false);
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xF, 0xF>(v));   // row_shr:1
  v = max(v, dpp_u32<0x112, 0xF, 0xF>(v));   // row_shr:2
  v = max(v, dpp_u32<0x113, 0xF, 0xF>(v));   // row_shr:3
  v = max(v, dpp_u32<0x114, 0xF, 0xE>(v));   // row_shr:4, lanes 4-15 of each row
  v = max(v, dpp_u32<0x118, 0xF, 0xC>(v));   // row_shr:8, lanes 8-15 of each row
  v = max(v, dpp_u32<0x142, 0xA, 0xF>(v));   // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_u32<0x143, 0xC, 0xF>(v));   // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top k (k <= 16, wave-uniform) of up to 256 route keys held four per lane
// by one wave: k rounds, each finding the wave's largest key (the logit
// part first, then the index part among the lanes that hold that logit)
// and clearing it; out(j, key) receives the j-th largest (wave-uniform).
// Keys are distinct and real keys exceed the padding key 0.
template <typename Out>
__device__ __forceinline__ void wave_topk4(uint64_t (&key)[4], int k, Out out) {
  for (int j = 0; j < k; ++j) {
    const uint64_t a = key[0] > key[1] ? key[0] : key[1];
    const uint64_t b = key[2] > key[3] ? key[2] : key[3];
    const uint64_t lm = a > b ? a : b;
    const uint32_t mh = wave_max_u32_dpp((uint32_t)(lm >> 32));
    const uint32_t ml = wave_max_u32_dpp((uint32_t)(lm >> 32) == mh ? (uint32_t)lm : 0u);
    const uint64_t mk = ((uint64_t)mh << 32) | ml;
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = key[i] == mk ? 0 : key[i];
    out(j, mk);
  }
}

// Wave-wide maximum of a 64-bit key (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  uint32_t b = (uint32_t)(key >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;      // inverse of route_key's map
  return __builtin_bit_cast(float, b);
}

}  // namespace qmoe_route
