// Router: fp32 logits l = x Wr^T (+ bias), then top-k with softmax weights
// renormalized over the kept k ([digest] "Model weights": routing stays
// unquantized; the function is softmax, top-k, renormalize).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.hpp"
#include "route_common.hpp"
#include "k_route.h"
#include "../../include/qmoe.h"
#include "launch_util.h"

using namespace qmoe_dev;
using namespace qmoe_route;

namespace {

// Few tokens (T <= 16): one workgroup per expert, one wave per part of H
// (n_parts parts of whole 512-column slices, one slice per wave when H <=
// 8192, so every load of a wave is in flight at once); each lane takes 8
// consecutive columns of each slice, the wave sums with a butterfly, and the
// parts are added in part order (bias with part 0) into the final logit.
constexpr int kMaxLogitParts = 16;

__global__ __launch_bounds__(64 * kMaxLogitParts) void logits_small_kernel(const uint16_t* x, const float* wr,
                                                                           const float* bias, int T, int H,
                                                                           int E, float* logits) {
  __shared__ float part_sum[kMaxLogitParts][16];
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int part = threadIdx.x >> 6, n_parts = blockDim.x >> 6;
  float acc[16];
  for (int t = 0; t < 16; ++t) acc[t] = 0.f;
  const float* w = wr + (size_t)e * H;
  const int cpp = (H + 512 * n_parts - 1) / (512 * n_parts) * 512;     // columns per part
  const int h_end = min(H, (part + 1) * cpp);
  for (int h0 = part * cpp + 8 * lane; h0 < h_end; h0 += 512) {
    const float4v w0 = *reinterpret_cast<const float4v*>(w + h0);
    const float4v w1 = *reinterpret_cast<const float4v*>(w + h0 + 4);
    for (int t = 0; t < T; ++t) {
      const u32x4 xr = load16(x + (size_t)t * H + h0);
      float s = acc[t];
      s = fmaf(bf2f(xr.x & 0xFFFFu), w0.x, s);
      s = fmaf(bf2f(xr.x >> 16), w0.y, s);
      s = fmaf(bf2f(xr.y & 0xFFFFu), w0.z, s);
      s = fmaf(bf2f(xr.y >> 16), w0.w, s);
      s = fmaf(bf2f(xr.z & 0xFFFFu), w1.x, s);
      s = fmaf(bf2f(xr.z >> 16), w1.y, s);
      s = fmaf(bf2f(xr.w & 0xFFFFu), w1.z, s);
      s = fmaf(bf2f(xr.w >> 16), w1.w, s);
      acc[t] = s;
    }
  }
  for (int t = 0; t < T; ++t) {
    float v = acc[t];
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) part_sum[part][t] = v + ((bias && part == 0) ? bias[e] : 0.f);
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float v = part_sum[0][threadIdx.x];
    for (int p = 1; p < n_parts; ++p) v += part_sum[p][threadIdx.x];
    logits[(size_t)threadIdx.x * E + e] = v;
  }
}

// Many tokens: fp32 matrix cores (v_mfma_f32_16x16x4_f32).  A workgroup of
// 4 waves computes 64 tokens x 32 experts; wave w takes tokens 16w..16w+15
// against two 16-expert tiles.  K is staged through LDS 64 columns at a time
// (x converted bf16 -> fp32 exactly), the next chunk's loads in flight while
// the current one is multiplied.
constexpr int kLgT = 64, kLgE = 32, kLgK = 64;

__device__ __forceinline__ float4v mfma_f32x4(float a, float b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void logits_tiled_kernel(const uint16_t* x, const float* wr,
                                                           const float* bias, int T, int H, int E,
                                                           float* logits) {
  __shared__ float xs[kLgT][kLgK + 1];
  __shared__ float ws[kLgE][kLgK + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.y * kLgT, e0 = blockIdx.x * kLgE;
  // loads of one chunk: x 64 rows x 8 pieces of 8 bf16, w 32 rows x 16 pieces of 4 fp32
  u32x4 xr[2], wv[2];
  auto load_chunk = [&](int k0) {
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 3, c = k0 + (p & 7) * 8;
      xr[i] = (t0 + r < T && c < H) ? load16(x + (size_t)(t0 + r) * H + c) : u32x4{0u, 0u, 0u, 0u};
      const int re = p >> 4, ce = k0 + (p & 15) * 4;
      wv[i] = (e0 + re < E && ce < H) ? load16(wr + (size_t)(e0 + re) * H + ce) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_chunk = [&]() {
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int r = p >> 3, c = (p & 7) * 8;
      for (int q = 0; q < 4; ++q) {
        xs[r][c + 2 * q] = bf2f(xr[i][q] & 0xFFFFu);
        xs[r][c + 2 * q + 1] = bf2f(xr[i][q] >> 16);
      }
      const int re = p >> 4, ce = (p & 15) * 4;
      // (bit-cast the whole vector: a bit-cast of a vector element here read
      // element 0 for every element)
      const float4v f = __builtin_bit_cast(float4v, wv[i]);
      for (int q = 0; q < 4; ++q) ws[re][ce + q] = f[q];
    }
  };
  float4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  load_chunk(0);
  for (int k0 = 0; k0 < H; k0 += kLgK) {
    __syncthreads();
    store_chunk();
    __syncthreads();
    if (k0 + kLgK < H) load_chunk(k0 + kLgK);
    const int kq = lane >> 4, ri = lane & 15;
#pragma unroll 4
    for (int ks = 0; ks < kLgK / 4; ++ks) {
      const float av = xs[16 * wave + ri][4 * ks + kq];
      acc0 = mfma_f32x4(av, ws[ri][4 * ks + kq], acc0);
      acc1 = mfma_f32x4(av, ws[16 + ri][4 * ks + kq], acc1);
    }
  }
  // C[4(lane/16) + i][lane%16]: token row, expert column
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * wave + 4 * (lane >> 4) + i;
    if (t >= T) continue;
    const int ea = e0 + (lane & 15), eb = e0 + 16 + (lane & 15);
    if (ea < E) logits[(size_t)t * E + ea] = acc0[i] + (bias ? bias[ea] : 0.f);
    if (eb < E) logits[(size_t)t * E + eb] = acc1[i] + (bias ? bias[eb] : 0.f);
  }
}

// Top-k of the final logits [T][E], one wave per token (E <= 1024): lane l
// holds the keys of experts 64q + l; each of the k rounds takes the wave's
// largest key (the same 64-bit (logit, index) keys as rank_topk, so the same
// order and ties), the lane that held it drops it, and the kept logits give
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) summed in rank order -- the
// same operations as rank_topk, so the same bits.  No LDS, no barriers.
constexpr int kTopkWaves = 4;
constexpr int kTopkMaxKeys = 16;        // keys per lane: E <= 1024

__global__ __launch_bounds__(64 * kTopkWaves) void topk_kernel(const float* logits, int T, int E, int k,
                                                               int32_t* topk_idx, float* topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nq = (E + 63) / 64;
  uint64_t key[kTopkMaxKeys];
#pragma unroll
  for (int q = 0; q < kTopkMaxKeys; ++q) {
    const int e = 64 * q + lane;
    key[q] = (q < nq && e < E) ? route_key(logits[(size_t)t * E + e], e) : 0;
  }
  float kv[16];
  int ki[16];
  for (int j = 0; j < k; ++j) {
    uint64_t m = 0;
#pragma unroll
    for (int q = 0; q < kTopkMaxKeys; ++q) m = key[q] > m ? key[q] : m;
    m = wave_max_u64(m);
#pragma unroll
    for (int q = 0; q < kTopkMaxKeys; ++q)
      if (key[q] == m) key[q] = 0;
    kv[j] = key_logit(m);
    ki[j] = (int)(0xFFFFFFFFu - (uint32_t)m);
  }
  if (lane == 0) {
    const float top = kv[0];
    float z = 0.f;
    for (int j = 0; j < k; ++j) z += expf(kv[j] - top);
    for (int j = 0; j < k; ++j) {
      topk_idx[(size_t)t * k + j] = ki[j];
      topk_w[(size_t)t * k + j] = expf(kv[j] - top) / z;
    }
  }
}

}  // namespace

namespace qmoe {

int route_logit_parts(int, int) { return 1; }

hipError_t launch_route_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                               float* logits, hipStream_t s) {
  const int n_parts = std::min(kMaxLogitParts, (H + 511) / 512);
  return launch_timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
    if (T <= 16)
      hipLaunchKernelGGL(logits_small_kernel, dim3(E), dim3(64 * n_parts), 0, s, x, wr, bias, T, H, E, logits);
    else
      hipLaunchKernelGGL(logits_tiled_kernel, dim3((E + kLgE - 1) / kLgE, (T + kLgT - 1) / kLgT), dim3(256), 0,
                         s, x, wr, bias, T, H, E, logits);
  });
}

hipError_t launch_route_topk(const float* logits, int n_parts, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s) {
  if (n_parts != 1) return hipErrorInvalidValue;           // the logits kernels write final logits
  return launch_timed(MOE_KERNEL_ROUTE_TOPK, s, [&] {
    hipLaunchKernelGGL(topk_kernel, dim3((T + kTopkWaves - 1) / kTopkWaves), dim3(64 * kTopkWaves), 0, s, logits,
                       T, E, k, topk_idx, topk_w);
  });
}

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                        int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  hipError_t err = launch_route_logits(x, wr, bias, T, H, E, logits, s);
  if (err != hipSuccess) return err;
  return launch_route_topk(logits, route_logit_parts(T, H), T, E, k, topk_idx, topk_w, s);
}

}  // namespace qmoe
