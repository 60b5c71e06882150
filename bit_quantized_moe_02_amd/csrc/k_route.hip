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

// Many tokens on bf16 matrix cores.  The fp32 router weights split exactly
// into three bf16 parts (w = w1 + w2 + w3: w1 = bf16(w), w2 = bf16(w - w1),
// w3 = w - w1 - w2, each remainder exact in fp32 and the last one a bf16
// number), so x·w = x·w1 + x·w2 + x·w3 with every product exact in fp32
// (8-bit x 8-bit significands) and fp32 accumulation.  A workgroup of 4 waves
// computes 64 tokens x 32 experts; the experts' weights are split into three
// bf16 planes in LDS 64 columns at a time (double-buffered, the next chunk's
// fp32 loads in flight), each wave reads its 16 token rows of x straight from
// memory (the next chunk's in flight) and runs v_mfma_f32_16x16x32_bf16
// against two 16-expert tiles.  The columns are split into kLogitSplit parts
// (grid z), whose partial logits the top-k kernel adds in part order, so
// that enough workgroups keep loads in flight (the loop is latency-bound).
// Consecutive workgroups go to the 8 XCDs in turn (workgroup L on XCD L % 8,
// each XCD with its own L2): workgroup L runs block b = (L % 8) (N / 8) + L / 8
// of the N blocks (expert block fastest, then token tile, then part), so each
// XCD takes a contiguous run of blocks, a token tile's expert blocks share one
// XCD and its L2 fetches that tile of x once (b = L when 8 does not divide N).
constexpr int kLbT = 64, kLbE = 32, kLbK = 64;
constexpr int kLbRow = kLbK * 2 + 16;                   // bytes per plane row (padded: no bank conflicts)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;          // finite inputs
}

__global__ __launch_bounds__(256) void logits_bf16x3_kernel(const uint16_t* x, const float* wr, const float* bias,
                                                            int T, int H, int E, int n_parts, float* logits) {
  __shared__ __align__(16) uint8_t wp[2][3][kLbE * kLbRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = gridDim.x, L = blockIdx.x;
  const int b = (N & 7) ? L : (L & 7) * (N >> 3) + (L >> 3);
  const int nbe = (E + kLbE - 1) / kLbE, nbt = (T + kLbT - 1) / kLbT;
  const int t0 = (b / nbe) % nbt * kLbT, e0 = b % nbe * kLbE;
  const int part = b / (nbe * nbt);
  const int cpp = (H + kLbK * n_parts - 1) / (kLbK * n_parts) * kLbK;     // columns per part
  const int k_beg = part * cpp, k_end = min(H, k_beg + cpp);
  // staging: thread -> expert row sr, columns sc .. sc + 7 of the chunk
  const int sr = tid >> 3, sc = (tid & 7) * 8;
  const bool srow = e0 + sr < E;
  const float* wrow = wr + (size_t)(srow ? e0 + sr : 0) * H;
  auto load_w = [&](int k0, float4v (&w)[2]) {
    const bool ok = srow && k0 + sc < k_end;              // H is a multiple of 8
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    w[0] = ok ? *reinterpret_cast<const float4v*>(wrow + k0 + sc) : z;
    w[1] = ok ? *reinterpret_cast<const float4v*>(wrow + k0 + sc + 4) : z;
  };
  auto store_w = [&](int buf, const float4v (&w)[2]) {
    uint32_t p1[4], p2[4], p3[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t b1[2], b2[2], b3[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float v = w[i >> 1][2 * (i & 1) + h];
        b1[h] = bf16_rne_bits(v);
        const float r1 = v - __builtin_bit_cast(float, b1[h] << 16);
        b2[h] = bf16_rne_bits(r1);
        const float r2 = r1 - __builtin_bit_cast(float, b2[h] << 16);
        b3[h] = __builtin_bit_cast(uint32_t, r2) >> 16;    // r2 fits in bf16 exactly
      }
      p1[i] = b1[0] | (b1[1] << 16);
      p2[i] = b2[0] | (b2[1] << 16);
      p3[i] = b3[0] | (b3[1] << 16);
    }
    const int off = sr * kLbRow + sc * 2;
    *reinterpret_cast<u32x4*>(&wp[buf][0][off]) = u32x4{p1[0], p1[1], p1[2], p1[3]};
    *reinterpret_cast<u32x4*>(&wp[buf][1][off]) = u32x4{p2[0], p2[1], p2[2], p2[3]};
    *reinterpret_cast<u32x4*>(&wp[buf][2][off]) = u32x4{p3[0], p3[1], p3[2], p3[3]};
  };
  // A: token row at of this wave's 16, 8 columns at 8 (lane / 16) of each 32-column step
  const int at = t0 + 16 * wave + (lane & 15);
  const bool arow = at < T;
  const uint16_t* xrow = x + (size_t)(arow ? at : 0) * H;
  auto load_a = [&](int k0, u32x4 (&a)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = k0 + 32 * s + 8 * (lane >> 4);
      a[s] = (arow && kk < k_end) ? load16(xrow + kk) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  float4v acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float4v wn[2];
  u32x4 an[2], ac[2];
  load_w(k_beg, wn);
  load_a(k_beg, ac);
  store_w(0, wn);
  __syncthreads();
  for (int k0 = k_beg; k0 < k_end; k0 += kLbK) {
    const int buf = ((k0 - k_beg) / kLbK) & 1;
    const bool more = k0 + kLbK < k_end;
    if (more) {
      load_w(k0 + kLbK, wn);
      load_a(k0 + kLbK, an);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const u32x4 bv = *reinterpret_cast<const u32x4*>(
              &wp[buf][p][(16 * n + (lane & 15)) * kLbRow + (32 * s + 8 * (lane >> 4)) * 2]);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ac[s]),
                                                          __builtin_bit_cast(bf16x8_t, bv), acc[n], 0, 0, 0);
        }
    if (more) {
      store_w(buf ^ 1, wn);
      ac[0] = an[0];
      ac[1] = an[1];
    }
    __syncthreads();
  }
  // C[4 (l / 16) + i][l % 16]: token row, expert column
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = e0 + 16 * n + (lane & 15);
    if (e >= E) continue;
    const float b = (bias && part == 0) ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * wave + 4 * (lane >> 4) + i;
      if (t < T) logits[((size_t)part * T + t) * E + e] = acc[n][i] + b;
    }
  }
}

// Top-k of the logits [n_parts][T][E] (parts added in part order), one wave
// per token (E <= 1024): lane l
// holds the keys of experts 64q + l; each of the k rounds takes the wave's
// largest key (the same 64-bit (logit, index) keys as rank_topk, so the same
// order and ties), the lane that held it drops it, and the kept logits give
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) summed in rank order -- the
// same operations as rank_topk, so the same bits.  No LDS, no barriers.
constexpr int kTopkWaves = 4;

template <int NQ, int P>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_kernel(const float* logits, int T, int E, int k,
                                                               int32_t* topk_idx, float* topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  // all NQ x P loads are issued before the first is used (a load whose value
  // is read only inside a branch is waited for alone).  A lane past the last
  // expert reads expert E - 1 and keys logit -inf with its own index e >= E:
  // below every real expert's key (also a real -inf, whose index is
  // smaller), so never taken as k <= E.
  float pv[P][NQ];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int q = 0; q < NQ; ++q) pv[p][q] = logits[((size_t)p * T + t) * E + min(64 * q + lane, E - 1)];
  uint64_t key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float l = pv[0][q];
#pragma unroll
    for (int p = 1; p < P; ++p) l += pv[p][q];
    const int e = 64 * q + lane;
    key[q] = route_key(e < E ? l : -__builtin_inff(), e);
  }
  float kv[16];
  int ki[16];
  for (int j = 0; j < k; ++j) {
    uint64_t m = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) m = key[q] > m ? key[q] : m;
    m = wave_max_u64(m);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
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

// Top-k of a few tokens' single-part logits, one 1024-thread workgroup per
// token ranking every key at once (rank_topk: the same keys and the same
// weight arithmetic as topk_kernel, so the same bits).  Below ~16 tokens the
// wave kernel's k serial rounds of wave maxima cost more than this one's
// barriers.
constexpr int kTopkRankThreads = 1024;

__global__ __launch_bounds__(kTopkRankThreads) void topk_rank_kernel(const float* logits, int E, int k,
                                                                     int32_t* topk_idx, float* topk_w) {
  __shared__ __align__(16) TopkLds sm;
  const int t = blockIdx.x;
  const float* lt = logits + (size_t)t * E;
  int32_t* oi = topk_idx + (size_t)t * k;
  float* ow = topk_w + (size_t)t * k;
  rank_topk<kTopkRankThreads>(sm, E, k, [&](int e) { return lt[e]; }, [&](int j, int e, float w) {
    oi[j] = e;
    ow[j] = w;
  });
}

}  // namespace

namespace qmoe {

int route_logit_parts(int T, int) { return T > 16 ? kLogitSplit : 1; }

hipError_t launch_route_logits(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                               float* logits, hipStream_t s) {
  const int n_parts = std::min(kMaxLogitParts, (H + 511) / 512);
  return launch_timed(MOE_KERNEL_ROUTE_LOGITS, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    if (T <= 16) {
      hipExtLaunchKernelGGL(logits_small_kernel, dim3(E), dim3(64 * n_parts), 0, s, ev0_, ev1_, 0, x, wr, bias, T, H, E, logits);
    } else {
      const int blocks = (E + kLbE - 1) / kLbE * ((T + kLbT - 1) / kLbT) * kLogitSplit;
      hipExtLaunchKernelGGL(logits_bf16x3_kernel, dim3(blocks), dim3(256), 0, s, ev0_, ev1_, 0, x, wr, bias, T, H, E, kLogitSplit,
                         logits);
    }
  });
}

hipError_t launch_route_topk(const float* logits, int n_parts, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s) {
  // keys per lane NQ = ceil(E / 64) rounded up to a power of two (E <= 1024);
  // parts: 1 or kLogitSplit, as the logits kernels write them
  if (E < 1 || E > 1024 || (n_parts != 1 && n_parts != kLogitSplit)) return hipErrorInvalidValue;
  const int nq = (E + 63) / 64;
  const bool split = n_parts != 1;
  void (*fk)(const float*, int, int, int, int32_t*, float*) =
      nq <= 1   ? (split ? topk_kernel<1, kLogitSplit> : topk_kernel<1, 1>)
      : nq <= 2 ? (split ? topk_kernel<2, kLogitSplit> : topk_kernel<2, 1>)
      : nq <= 4 ? (split ? topk_kernel<4, kLogitSplit> : topk_kernel<4, 1>)
      : nq <= 8 ? (split ? topk_kernel<8, kLogitSplit> : topk_kernel<8, 1>)
                : (split ? topk_kernel<16, kLogitSplit> : topk_kernel<16, 1>);
  return launch_timed(MOE_KERNEL_ROUTE_TOPK, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    if (T <= 16 && n_parts == 1)
      hipExtLaunchKernelGGL(topk_rank_kernel, dim3(T), dim3(kTopkRankThreads), 0, s, ev0_, ev1_, 0, logits, E, k, topk_idx, topk_w);
    else
      hipExtLaunchKernelGGL(fk, dim3((T + kTopkWaves - 1) / kTopkWaves), dim3(64 * kTopkWaves), 0, s, ev0_, ev1_, 0, logits, T, E, k,
                         topk_idx, topk_w);
  });
}

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                        int k, float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  hipError_t err = launch_route_logits(x, wr, bias, T, H, E, logits, s);
  if (err != hipSuccess) return err;
  return launch_route_topk(logits, route_logit_parts(T, H), T, E, k, topk_idx, topk_w, s);
}

}  // namespace qmoe
