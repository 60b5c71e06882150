// Single-token decode (T = 1): the whole-layer GEMV pair at batch 1.
//
//   dec1_upgate: h_j = SiLU(Wg_{e_j} x) * (Wu_{e_j} x) for the k routed
//                choices j and h_s = SiLU(Wsg x) * (Wsu x) for the shared expert.
//   dec1_down:   y = sum_j w_j Wd_{e_j} h_j + Wsd h_s, written directly (the
//                weighted combine is fused): for one 16-row tile of y, the k
//                routed down matrices and the shared one form a single
//                stacked GEMV over K = k*I + I_s.
//
// Both split K across the 16 waves of a workgroup and keep every partial
// sum in a fixed order (wave-order LDS reductions, no atomics).
//
// MFMA v_mfma_f32_16x16x32_f16 (A = activations, B = decoded weights): with
// one token only A row m = 0 is non-zero, so C[0][n] sits in lane n < 16.
// For K2 the down projection uses block-diagonal A rows instead: in k-block
// kb, A row 2kb holds the activations of sub-block 2kb and row 2kb+1 those of
// 2kb+1, so after the 8 k-blocks of a super-block C[sb][n] is the partial dot
// of sub-block sb and each K2 sub-block scale is applied once per sub-block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmoe.h"
#include "device_common.hpp"
#include "k_decode.h"
#include "launch_util.h"

using namespace qmoe_dev;
using qmoe::DecArgs;

namespace {

constexpr int kBatch = 8;        // row tiles reduced per barrier (up/gate)

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Same weighted contiguous split of items as the multi-token kernels: item i
// goes to the workgroup whose share of the total weight holds its midpoint.
__device__ int64_t item_start1(int64_t g, int64_t G, int64_t n_s, int64_t w_s, int64_t n_r, int64_t w_r) {
  const int64_t W = n_s * w_s + n_r * w_r;
  int64_t lo = 0, hi = n_s + n_r;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    const int64_t twoM = (mid < n_s) ? 2 * mid * w_s + w_s : 2 * (n_s * w_s + (mid - n_s) * w_r) + w_r;
    if (twoM * G >= 2 * g * W) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Per-wave payload of one routed row tile (both matrices) for CPW K-chunks.

template <int FMT, int CPW>
struct UgPay;

template <int CPW>
struct UgPay<MOE_FMT_CB2, CPW> {
  u32x4 code[2][CPW], scale[2][CPW];
};

template <int CPW>
struct UgPay<MOE_FMT_K4, CPW> {
  u32x4 q0[2][CPW], q1[2][CPW];
  uint32_t s0[2][CPW], s1[2][CPW], s2[2][CPW], dd[2][CPW];
};

template <int FMT, int CPW>
__device__ __forceinline__ void ug_load(UgPay<FMT, CPW>& p, const DecArgs& a, int e, int64_t rt, int wave,
                                        int lane, int n_chunks) {
  const int n = lane & 15;
  for (int mat = 0; mat < 2; ++mat)
    for (int cc = 0; cc < CPW; ++cc) {
      const int chunk = min(wave * CPW + cc, n_chunks - 1);
      const uint8_t* tile = (mat ? a.gate : a.up) + (size_t)e * a.expert_bytes +
                            ((size_t)rt * n_chunks + chunk) * (FMT == MOE_FMT_CB2 ? kCb2Tile : kK4Tile);
      if constexpr (FMT == MOE_FMT_CB2) {
        p.code[mat][cc] = load16(tile + 16 * lane);
        p.scale[mat][cc] = load16(tile + 1024 + 16 * n);
      } else {
        p.q0[mat][cc] = load16(tile + 16 * lane);
        p.q1[mat][cc] = load16(tile + 1024 + 16 * lane);
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
        p.s0[mat][cc] = sp[0];
        p.s1[mat][cc] = sp[1];
        p.s2[mat][cc] = sp[2];
        p.dd[mat][cc] = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
      }
    }
}

template <int FMT, int CPW>
__global__ __launch_bounds__(1024) void dec1_upgate_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  int64_t* range = reinterpret_cast<int64_t*>(smem);
  size_t off = 256;
  uint8_t* val_tab = smem + off;
  uint8_t* flip_tab = val_tab + kCb2TableBytes;
  if (FMT == MOE_FMT_CB2) off += 2 * kCb2TableBytes;
  float* xsum = reinterpret_cast<float*>(smem + off);               // K4: per 32-column block
  if (FMT == MOE_FMT_K4) off += (size_t)(a.H / 32) * 4;
  float* red = reinterpret_cast<float*>(smem + off);                // [kBatch][NW][2][16]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NW = blockDim.x >> 6;
  const int k = a.k, n_chunks = a.H / 256;
  const int64_t n_rt = a.I / 16, n_rts = a.Is / 16;
  const int64_t w_r = (int64_t)2 * a.tb_ug * n_chunks, w_s = (int64_t)2 * kBf16Tile * n_chunks;
  if (tid == 0) {
    range[0] = item_start1(blockIdx.x, gridDim.x, n_rts, w_s, (int64_t)k * n_rt, w_r);
    range[1] = item_start1(blockIdx.x + 1, gridDim.x, n_rts, w_s, (int64_t)k * n_rt, w_r);
  }
  if (FMT == MOE_FMT_CB2) cb2_fill_tables(a.codebook, val_tab, flip_tab, tid, blockDim.x);
  if (FMT == MOE_FMT_K4)
    for (int b = tid; b < a.H / 32; b += blockDim.x) {
      float s = 0.f;
      for (int j = 0; j < 32; ++j) s += (float)(_Float16)bf2f(a.x[b * 32 + j]);
      xsum[b] = s;
    }
  __syncthreads();
  const int64_t lo = range[0], hi = range[1];
  if (lo >= hi) return;

  // A operands: row 0 = x, rows 1..15 zero.
  half8 A[CPW][8];
  const int qq = lane >> 4;
  for (int cc = 0; cc < CPW; ++cc)
    for (int kb = 0; kb < 8; ++kb) {
      const int chunk = wave * CPW + cc;
      u32x4 r = {0, 0, 0, 0};
      if ((lane & 15) == 0 && chunk < n_chunks) r = as_u32x4(bf16x8_to_half8(load16(a.x + chunk * 256 + kb * 32 + qq * 8)));
      A[cc][kb] = as_half8(r);
    }
  const bool wave_has_chunks = wave * CPW < n_chunks;
  const uint8_t* val_lane = val_tab + (lane & 7) * 16;
  const uint8_t* flip_lane = flip_tab + (lane & 7) * 16;
  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  // Reduction of a batch of row tiles: red[b][w][mat][n] -> h, plus the
  // down projection's per-16-row sums X = sum h and O = sum 1024 fp16(h 4^-t).
  auto flush = [&](int64_t first, int nb) {
    __syncthreads();
    if (tid < nb * 16) {
      const int b = tid >> 4, n = tid & 15;
      const int64_t item = first + b;
      float u = 0.f, g = 0.f;
      for (int w = 0; w < NW; ++w) {
        u += red[((b * NW + w) * 2 + 0) * 16 + n];
        g += red[((b * NW + w) * 2 + 1) * 16 + n];
      }
      const _Float16 h16 = (_Float16)(silu(g) * u);
      const float hv = (float)h16;
      if (item < n_rts) {
        a.hs[item * 16 + n] = h16;
      } else {
        const int64_t r = item - n_rts;
        const int j = (int)(r / n_rt);
        const int64_t rt = r % n_rt;
        a.h[(size_t)j * a.I + rt * 16 + n] = h16;
        const int kk = (int)((rt * 16 + n) & 255);
        const int t = k2_slot_t(kk >> 5, (kk & 7) >> 1);
        float X = hv, O = 1024.0f * (float)(_Float16)(hv * __builtin_ldexpf(1.0f, -2 * t));
        for (int o = 8; o >= 1; o >>= 1) {
          X += __shfl_xor(X, o);
          O += __shfl_xor(O, o);
        }
        if (n == 0) {
          float* hsm = a.hsum + ((size_t)j * (a.I_pad / 16) + rt) * 2;
          hsm[0] = X;
          hsm[1] = O;
        }
      }
    }
    __syncthreads();
  };

  int nb = 0;
  int64_t first = lo;
  // --- shared-expert row tiles (bf16)
  const int64_t s_hi = min(hi, n_rts);
  for (int64_t item = lo; item < s_hi; ++item) {
    float v[2] = {0.f, 0.f};
    if (wave_has_chunks) {
      for (int cc = 0; cc < CPW; ++cc) {
        const int chunk = wave * CPW + cc;
        if (chunk >= n_chunks) break;
        u32x4 raw[2][8];
        for (int mat = 0; mat < 2; ++mat) {
          const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)item * n_chunks + chunk) * kBf16Tile;
          for (int kb = 0; kb < 8; ++kb) raw[mat][kb] = load16(tile + 1024 * kb + 16 * lane);
        }
        for (int mat = 0; mat < 2; ++mat) {
          float4v c = zero;
          for (int kb = 0; kb < 8; ++kb) c = mfma_f16(A[cc][kb], bf16x8_to_half8(raw[mat][kb]), c);
          v[mat] += c[0];
        }
      }
    }
    if (lane < 16) {
      red[((nb * NW + wave) * 2 + 0) * 16 + lane] = v[0];
      red[((nb * NW + wave) * 2 + 1) * 16 + lane] = v[1];
    }
    if (++nb == kBatch || item + 1 == s_hi) {
      flush(first, nb);
      first = item + 1;
      nb = 0;
    }
  }
  // --- routed row tiles, the next tile's loads in flight during this one
  int64_t item = max(lo, n_rts);
  if (item >= hi) return;
  auto expert_of = [&](int64_t it) {
    const int j = (int)((it - n_rts) / n_rt);
    return (int)a.topk_idx[j];
  };
  // With one K-chunk per wave the next row tile's loads are issued before
  // this one is computed; with two chunks per wave the registers are needed
  // for the activations and the loads are issued per row tile.
  constexpr bool kPrefetch = CPW == 1;
  UgPay<FMT, CPW> cur, nxt;
  if (kPrefetch) {
    const int e = expert_of(item);
    if (wave_has_chunks && e >= 0 && e < a.E) ug_load<FMT, CPW>(cur, a, e, (item - n_rts) % n_rt, wave, lane, n_chunks);
  }
  for (; item < hi; ++item) {
    if (kPrefetch && item + 1 < hi) {
      const int e1 = expert_of(item + 1);
      if (wave_has_chunks && e1 >= 0 && e1 < a.E)
        ug_load<FMT, CPW>(nxt, a, e1, (item + 1 - n_rts) % n_rt, wave, lane, n_chunks);
    }
    const int e = expert_of(item);
    if (!kPrefetch && wave_has_chunks && e >= 0 && e < a.E)
      ug_load<FMT, CPW>(cur, a, e, (item - n_rts) % n_rt, wave, lane, n_chunks);
    float v[2] = {0.f, 0.f};
    if (wave_has_chunks && e >= 0 && e < a.E) {
      for (int mat = 0; mat < 2; ++mat)
        for (int cc = 0; cc < CPW; ++cc) {
          const int chunk = wave * CPW + cc;
          if (chunk >= n_chunks) break;
          if constexpr (FMT == MOE_FMT_CB2) {
            for (int kb = 0; kb < 8; ++kb) {
              const uint32_t code = (cur.code[mat][cc][kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu;
              const float4v c = mfma_f16(A[cc][kb], cb2_group(code, val_lane, flip_lane), zero);
              v[mat] += h2f((cur.scale[mat][cc][kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu) * c[0];
            }
          } else {
            const float d = h2f(cur.dd[mat][cc] & 0xFFFFu), dmin = h2f(cur.dd[mat][cc] >> 16);
            for (int kb = 0; kb < 8; ++kb) {
              const uint32_t w = kb < 4 ? cur.q0[mat][cc][kb & 3] : cur.q1[mat][cc][kb & 3];
              const float4v c = mfma_f16(A[cc][kb], as_half8(k4_magic(w)), zero);
              const float dsc = d * (float)k4_scale_value(cur.s0[mat][cc], cur.s1[mat][cc], cur.s2[mat][cc], kb);
              const float mn = (float)k4_scale_value(cur.s0[mat][cc], cur.s1[mat][cc], cur.s2[mat][cc], 8 + kb);
              v[mat] += dsc * c[0] - (1024.0f * dsc + dmin * mn) * xsum[chunk * 8 + kb];
            }
          }
        }
    }
    if (lane < 16) {
      red[((nb * NW + wave) * 2 + 0) * 16 + lane] = v[0];
      red[((nb * NW + wave) * 2 + 1) * 16 + lane] = v[1];
    }
    if (++nb == kBatch || item + 1 == hi) {
      flush(first, nb);
      first = item + 1;
      nb = 0;
    }
    if (kPrefetch) cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Down + shared down + combine.  Workgroup = one 16-row tile of y.

template <int FMT>
__global__ __launch_bounds__(1024) void dec1_down_kernel(DecArgs a, const float* topk_w, float* y) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NW = blockDim.x >> 6;
  const int k = a.k, I = a.I, I_pad = a.I_pad, Is = a.Is, Is_pad = a.Is_pad;
  const int n_ck = I_pad / 256, n_cks = Is > 0 ? Is_pad / 256 : 0;
  // LDS: staged activations (fp16), per-16-row sums, routing, reduction
  _Float16* hst = reinterpret_cast<_Float16*>(smem);                        // [k][I_pad] (K2: prescaled)
  _Float16* hss = hst + (size_t)k * I_pad;                                    // [Is_pad]
  size_t off = ((size_t)k * I_pad + Is_pad) * 2;
  off = (off + 15) & ~size_t(15);
  uint8_t* zero16 = smem + off;                                               // 16 zero bytes
  off += 16;
  float* xo = reinterpret_cast<float*>(smem + off);                           // [k][I_pad/16][2]
  off += (size_t)k * (I_pad / 16) * 2 * 4;
  float* wj = reinterpret_cast<float*>(smem + off);                           // [k]
  int* ej = reinterpret_cast<int*>(wj + 16);                                  // [k]
  float* red = reinterpret_cast<float*>(ej + 16);                             // [NW][16]

  for (int i = tid; i < k * I_pad; i += blockDim.x) {
    const int j = i / I_pad, col = i % I_pad;
    _Float16 v = (_Float16)0.0f;
    if (col < I) {
      v = a.h[(size_t)j * I + col];
      if (FMT == MOE_FMT_K2) {
        const int kk = col & 255;
        v = v * (_Float16)__builtin_ldexpf(1.0f, -2 * k2_slot_t(kk >> 5, (kk & 7) >> 1));
      }
    }
    hst[i] = v;
  }
  for (int i = tid; i < Is_pad; i += blockDim.x) hss[i] = (i < Is) ? a.hs[i] : (_Float16)0.0f;
  for (int i = tid; i < k * (I_pad / 16) * 2; i += blockDim.x) {
    const int j = i / ((I_pad / 16) * 2), r = i % ((I_pad / 16) * 2);
    xo[i] = (r / 2 < I / 16) ? a.hsum[(size_t)j * (I_pad / 16) * 2 + r] : 0.f;
  }
  if (tid < 4) reinterpret_cast<uint32_t*>(zero16)[tid] = 0u;
  if (tid < k) {
    const int e = a.topk_idx[tid];
    ej[tid] = (e >= 0 && e < a.E) ? e : -1;
    wj[tid] = topk_w[tid];
  }
  __syncthreads();

  const int64_t rt = blockIdx.x;
  const int n = lane & 15, g4 = lane >> 4, m = lane & 15;
  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float acc = 0.f;
  const int n_units = k * n_ck;
  for (int u = wave; u < n_units; u += NW) {
    const int j = u / n_ck, kc = u % n_ck;
    const int e = ej[j];
    if (e < 0) continue;
    const float wgt = wj[j];
    if constexpr (FMT == MOE_FMT_K2) {
      const uint8_t* tile = a.down + (size_t)e * a.expert_bytes_down + ((size_t)rt * n_ck + kc) * kK2Tile;
      const u32x4 qw = load16(tile + 16 * lane);
      const uint32_t scm = *reinterpret_cast<const uint32_t*>(tile + 1024 + 16 * n + 4 * g4);
      const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 1280 + 4 * n);
      float4v c = zero;
      const _Float16* hbase = hst + (size_t)j * I_pad + kc * 256 + g4 * 8;
      for (int kb = 0; kb < 8; ++kb) {
        const bool active = m == 2 * kb + (g4 >> 1);
        const uint8_t* src = active ? reinterpret_cast<const uint8_t*>(hbase + kb * 32) : zero16;
        c = mfma_f16(as_half8(load16(src)), as_half8(k2_magic(qw, kb)), c);
      }
      // C[4 g4 + i][n] = sub-block 4 g4 + i of this super-block
      const float4v X = *reinterpret_cast<const float4v*>(xo + ((size_t)j * (I_pad / 16) + kc * 16 + 4 * g4) * 2);
      const float4v O = *reinterpret_cast<const float4v*>(xo + ((size_t)j * (I_pad / 16) + kc * 16 + 4 * g4) * 2 + 4);
      // xo is (X, O) interleaved: X of sub-block s at 2s, O at 2s+1
      const float xs[4] = {X[0], X[2], O[0], O[2]};
      const float os[4] = {X[1], X[3], O[1], O[3]};
      float dsum = 0.f, msum = 0.f;
      for (int i = 0; i < 4; ++i) {
        const uint32_t byte = (scm >> (8 * i)) & 0xFFu;
        dsum += (float)(byte & 15u) * (c[i] - os[i]);
        msum += (float)(byte >> 4) * xs[i];
      }
      acc += (wgt * h2f(dd & 0xFFFFu)) * dsum - (wgt * h2f(dd >> 16)) * msum;
    } else {  // K4
      const uint8_t* tile = a.down + (size_t)e * a.expert_bytes_down + ((size_t)rt * n_ck + kc) * kK4Tile;
      const u32x4 q0 = load16(tile + 16 * lane);
      const u32x4 q1 = load16(tile + 1024 + 16 * lane);
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
      const uint32_t s0 = sp[0], s1 = sp[1], s2 = sp[2];
      const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
      const float d = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
      const _Float16* hbase = hst + (size_t)j * I_pad + kc * 256 + g4 * 8;
      float part = 0.f;
      for (int kb = 0; kb < 8; ++kb) {
        const uint8_t* src = (m == 0) ? reinterpret_cast<const uint8_t*>(hbase + kb * 32) : zero16;
        const uint32_t w = kb < 4 ? q0[kb & 3] : q1[kb & 3];
        const float4v c = mfma_f16(as_half8(load16(src)), as_half8(k4_magic(w)), zero);
        const float dsc = d * (float)k4_scale_value(s0, s1, s2, kb);
        const float corr = 1024.0f * dsc + dmin * (float)k4_scale_value(s0, s1, s2, 8 + kb);
        const float* xk = xo + ((size_t)j * (I_pad / 16) + kc * 16 + 2 * kb) * 2;
        part += dsc * c[0] - corr * (xk[0] + xk[2]);
      }
      if (g4 == 0) acc += wgt * part;
    }
  }
  // shared expert: units of half a K-chunk (4 k-blocks)
  for (int u = wave; u < 2 * n_cks; u += NW) {
    const int kc = u >> 1, kb0 = 4 * (u & 1);
    const uint8_t* tile = a.sdown + ((size_t)rt * n_cks + kc) * kBf16Tile;
    u32x4 raw[4];
    for (int q = 0; q < 4; ++q) raw[q] = load16(tile + 1024 * (kb0 + q) + 16 * lane);
    float4v c = zero;
    const _Float16* hbase = hss + kc * 256 + g4 * 8;
    for (int q = 0; q < 4; ++q) {
      const uint8_t* src = (m == 0) ? reinterpret_cast<const uint8_t*>(hbase + (kb0 + q) * 32) : zero16;
      c = mfma_f16(as_half8(load16(src)), bf16x8_to_half8(raw[q]), c);
    }
    acc += c[0];
  }
  // sum the 4 lanes of each output row, then the waves in order
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (tid < 16) {
    float s = 0.f;
    for (int w = 0; w < NW; ++w) s += red[w * 16 + tid];
    y[rt * 16 + tid] = s;
  }
}

}  // namespace

namespace qmoe {

size_t dec1_upgate_lds(const DecArgs& a, int fmt, int nw) {
  size_t off = 256;
  if (fmt == MOE_FMT_CB2) off += 2 * kCb2TableBytes;
  if (fmt == MOE_FMT_K4) off += (size_t)(a.H / 32) * 4;
  return off + (size_t)kBatch * nw * 2 * 16 * 4;
}

size_t dec1_down_lds(const DecArgs& a, int nw) {
  size_t off = ((size_t)a.k * a.I_pad + a.Is_pad) * 2;
  off = (off + 15) & ~size_t(15);
  off += 16 + (size_t)a.k * (a.I_pad / 16) * 2 * 4;
  return off + 16 * 4 + 16 * 4 + (size_t)nw * 16 * 4;
}

hipError_t launch_dec1(const DecArgs& a, int fmt_ug, int fmt_dn, int cpw, const float* topk_w, float* y,
                       int grid_ug, hipStream_t s) {
  const int nw_ug = (a.H / 256 + cpw - 1) / cpw;
  void (*fu)(DecArgs) = nullptr;
  if (fmt_ug == MOE_FMT_CB2) fu = cpw == 1 ? dec1_upgate_kernel<MOE_FMT_CB2, 1> : dec1_upgate_kernel<MOE_FMT_CB2, 2>;
  else fu = cpw == 1 ? dec1_upgate_kernel<MOE_FMT_K4, 1> : dec1_upgate_kernel<MOE_FMT_K4, 2>;
  hipError_t err = ensure_dyn_lds((const void*)fu);
  if (err != hipSuccess) return err;
  const size_t lds_ug = dec1_upgate_lds(a, fmt_ug, nw_ug);
  err = launch_timed(MOE_KERNEL_DECODE_UPGATE, s,
                     [&] { hipLaunchKernelGGL(fu, dim3(grid_ug), dim3(64 * nw_ug), lds_ug, s, a); });
  if (err != hipSuccess) return err;
  constexpr int nw_dn = 16;
  void (*fd)(DecArgs, const float*, float*) =
      fmt_dn == MOE_FMT_K2 ? dec1_down_kernel<MOE_FMT_K2> : dec1_down_kernel<MOE_FMT_K4>;
  err = ensure_dyn_lds((const void*)fd);
  if (err != hipSuccess) return err;
  const size_t lds_dn = dec1_down_lds(a, nw_dn);
  return launch_timed(MOE_KERNEL_DECODE_DOWN, s, [&] {
    hipLaunchKernelGGL(fd, dim3(a.H / 16), dim3(64 * nw_dn), lds_dn, s, a, topk_w, y);
  });
}

}  // namespace qmoe
