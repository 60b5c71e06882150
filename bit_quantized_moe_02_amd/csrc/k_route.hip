// Router: fp32 logits l = x Wr^T (+ bias), then top-k with softmax weights
// renormalized over the kept k ([digest] "Model weights": routing stays
// unquantized; the function is softmax, top-k, renormalize).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"
#include "k_route.h"
#include "../../include/qmoe.h"
#include "launch_util.h"

using namespace qmoe_dev;

namespace {

// Few tokens (T <= 16): one wave per (expert, quarter of H); each lane takes
// a strided 8-column slice, the wave sums it with a butterfly and writes the
// quarter's partial logit (the top-k kernel adds the quarters in order).
constexpr int kLogitSplit = 4;

__global__ __launch_bounds__(256) void logits_small_kernel(const uint16_t* x, const float* wr,
                                                           const float* bias, int T, int H, int E,
                                                           float* logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int part = blockIdx.y;
  if (e >= E) return;
  float acc[16];
  for (int t = 0; t < 16; ++t) acc[t] = 0.f;
  const float* w = wr + (size_t)e * H;
  const int hq = (H / 8 + kLogitSplit - 1) / kLogitSplit * 8;      // columns per part
  const int h_end = min(H, (part + 1) * hq);
  for (int h0 = part * hq + 8 * lane; h0 < h_end; h0 += 512) {
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
    if (lane == 0) logits[((size_t)part * T + t) * E + e] = v + ((bias && part == 0) ? bias[e] : 0.f);
  }
}

// Many tokens: 64 tokens x 64 experts per workgroup, fp32 FMA on 4x4
// register tiles, K staged through LDS 32 columns at a time.
__global__ __launch_bounds__(256) void logits_tiled_kernel(const uint16_t* x, const float* wr,
                                                           const float* bias, int T, int H, int E,
                                                           float* logits) {
  __shared__ float xs[32][65];
  __shared__ float ws[32][65];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < H; k0 += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      const int r = i >> 5, c = i & 31;
      const int t = t0 + r, e = e0 + r, kk = k0 + c;
      xs[c][r] = (t < T && kk < H) ? bf2f(x[(size_t)t * H + kk]) : 0.f;
      ws[c][r] = (e < E && kk < H) ? wr[(size_t)e * H + kk] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < 32; ++c) {
      float xa[4], wb[4];
      for (int i = 0; i < 4; ++i) xa[i] = xs[c][4 * ty + i];
      for (int j = 0; j < 4; ++j) wb[j] = ws[c][4 * tx + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 4 * ty + i, e = e0 + 4 * tx + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
    }
}

// One wave per token: the logit of expert e is the sum of n_parts partial
// logits (in part order); then k rounds of a wave-wide arg-max over
// (logit, -index) -- larger logit first, equal logits keep the lower expert
// index -- and w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the kept
// logits.  Lane j keeps round j's winner (no register arrays are indexed by
// run-time values).
__global__ __launch_bounds__(256) void topk_kernel(const float* logits, int n_parts, int T, int E, int k,
                                                   int32_t* topk_idx, float* topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    float s = -INFINITY;
    if (e < E) {
      s = logits[(size_t)t * E + e];
      for (int p = 1; p < n_parts; ++p) s += logits[((size_t)p * T + t) * E + e];
    }
    v[i] = s;
  }
  float my_v = -INFINITY, top_v = 0.f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (j == 0) top_v = bv;
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (lane + 64 * i == bi) v[i] = -INFINITY;
  }
  const float p = (lane < k) ? expf(my_v - top_v) : 0.f;
  // z = sum over j = 0..k-1 in j order (lane order), as a serial sum by lane 0
  float z = 0.f;
  for (int j = 0; j < k; ++j) z += __shfl(p, j);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_i;
    topk_w[(size_t)t * k + lane] = p / z;
  }
}

}  // namespace

namespace qmoe {

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                        int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  const int n_parts = T <= 16 ? kLogitSplit : 1;
  hipError_t err = launch_timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
    if (T <= 16)
      hipLaunchKernelGGL(logits_small_kernel, dim3((E + 3) / 4, kLogitSplit), dim3(256), 0, s, x, wr, bias, T,
                         H, E, logits);
    else
      hipLaunchKernelGGL(logits_tiled_kernel, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, s, x,
                         wr, bias, T, H, E, logits);
  });
  if (err != hipSuccess) return err;
  return launch_timed(MOE_KERNEL_ROUTE_TOPK, s, [&] {
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, n_parts, T, E, k, topk_idx,
                       topk_w);
  });
}

}  // namespace qmoe
