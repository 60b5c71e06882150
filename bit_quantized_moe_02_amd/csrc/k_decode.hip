// Decode-shape expert FFN (1..16 tokens): up/gate + SiLU, down, combine.
//
// Layer ([digest] "Model weights"; [digest] overview on sparse activation):
//   y[t] = sum_j w[t,j] * Wd_e (SiLU(Wg_e x_t) * (Wu_e x_t)) + shared(x_t),
// with e = topk_idx[t, j], routed experts quantized (CB2 up/gate + K2 down,
// or K4 for all three), the shared expert in bf16.
//
// Work split.  Every distinct expert among the T*k choices is one "expert
// slot" whose token set is a bitmask; its output rows are cut into row tiles
// of 16 (one MFMA N-tile).  A work item is (expert slot, row tile) -- for
// up/gate it covers the up AND the gate rows so SiLU(g)*u is formed in the
// epilogue -- plus one item per row tile of the shared expert.  Items are
// spread over the grid by weight (bytes they stream), contiguously.
//
// Inside a workgroup the reduction dimension K is split across waves: wave w
// owns K-chunks [w*CPW, (w+1)*CPW) of 256 columns, holds the activations of
// its chunks in registers as MFMA A operands (all T tokens at once, rows
// m >= T zero) and streams the matching packed tile of every item.  Partial
// sums meet in LDS and are summed in wave order (fixed-order, no atomics).
//
// MFMA v_mfma_f32_16x16x32_f16: lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and C[4(l/16)+i][l%16], i = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmoe.h"
#include "decode_common.hpp"
#include "device_common.hpp"
#include "k_decode.h"
#include "launch_util.h"

using namespace qmoe_dev;
using qmoe::DecArgs;
using namespace qmoe_dec;

namespace {

// ---------------------------------------------------------------------------
// Up/gate.

struct UgShared {
  ExpertList L;
  int64_t item_lo, item_hi;
  float hv[kMaxT][16];
  uint32_t xef[kMaxT];     // largest exponent field of each token's x
};

template <int FMT, int CPW>
__global__ __launch_bounds__(1024) void dec_upgate_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  UgShared* S = reinterpret_cast<UgShared*>(smem);
  size_t off = (sizeof(UgShared) + 255) & ~size_t(255);
  uint8_t* val_tab = smem + off;
  uint8_t* flip_tab = val_tab + (FMT == MOE_FMT_CB2 ? kCb2TableBytes : 0);
  off += (FMT == MOE_FMT_CB2) ? 2 * kCb2TableBytes : 0;
  float* xsum = reinterpret_cast<float*>(smem + off);              // K4: [H/32][16]
  off += (FMT == MOE_FMT_K4) ? (size_t)(a.H / 32) * 16 * 4 : 0;
  float* red = reinterpret_cast<float*>(smem + off);               // [NW][2][64][4]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int NW = blockDim.x >> 6;
  const int T = a.T, k = a.k;
  const int n_chunks = a.H / 256;

  if (tid < kMaxT) S->xef[tid] = 0u;
  build_expert_list(a.topk_idx, T * k, k, a.E, &S->L);
  // each token's exponent (integer maxima in LDS: order-independent)
  for (int i = tid; i < T * (a.H / 8); i += blockDim.x)
    atomicMax(&S->xef[i / (a.H / 8)], bf16x8_max_efield(load16(a.x + 8 * (size_t)i)));
  if (FMT == MOE_FMT_CB2) cb2_fill_tables(a.codebook, val_tab, flip_tab, tid, blockDim.x);
  const int64_t n_rt = a.I / 16, n_rts = a.Is / 16;
  const int64_t w_r = (int64_t)2 * a.tb_ug * n_chunks, w_s = (int64_t)2 * a.tb_s * n_chunks;
  if (tid == 0) {
    const int64_t n_r = (int64_t)S->L.n * n_rt;
    S->item_lo = item_start(blockIdx.x, gridDim.x, n_rts, w_s, n_r, w_r);
    S->item_hi = item_start(blockIdx.x + 1, gridDim.x, n_rts, w_s, n_r, w_r);
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < T) a.xexp[tid] = x_exp_of_field(S->xef[tid]);
  if (FMT == MOE_FMT_K4) {
    // per-token sums of x 2^-e over each 32-column block (m >= T: 0)
    for (int i = tid; i < (a.H / 32) * 16; i += blockDim.x) {
      const int blk = i >> 4, m = i & 15;
      float s = 0.f;
      if (m < T) {
        const int xe = x_exp_of_field(S->xef[m]);
        for (int j = 0; j < 32; ++j)
          s += (float)(_Float16)__builtin_ldexpf(bf2f(a.x[(size_t)m * a.H + blk * 32 + j]), -xe);
      }
      xsum[i] = s;
    }
    __syncthreads();
  }
  const int64_t item_lo = S->item_lo, item_hi = S->item_hi;
  if (item_lo >= item_hi) return;

  // A operands: x[m][256 c + 32 kb + 8 qq + j] 2^-e_m as fp16, m = lane % 16.
  half8 A[CPW][8];
  {
    const int m = lane & 15, qq = lane >> 4;
    const int xe = x_exp_of_field(S->xef[m < T ? m : 0]);
    for (int cc = 0; cc < CPW; ++cc) {
      const int chunk = wave * CPW + cc;
      for (int kb = 0; kb < 8; ++kb) {
        u32x4 r = {0, 0, 0, 0};
        if (m < T && chunk < n_chunks) {
          const u32x4 raw = load16(a.x + (size_t)m * a.H + chunk * 256 + kb * 32 + qq * 8);
          r = as_u32x4(bf16x8_to_half8_exp(raw, xe));
        }
        A[cc][kb] = as_half8(r);
      }
    }
  }
  const uint8_t* val_lane = val_tab + (lane & 7) * 16;
  const uint8_t* flip_lane = flip_tab + (lane & 7) * 16;
  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  for (int64_t item = item_lo; item < item_hi; ++item) {
    const bool shared = item < n_rts;
    int64_t rt;
    int e = -1;
    uint32_t mask = 0;
    if (shared) {
      rt = item;
    } else {
      const int64_t r = item - n_rts;
      const int d = (int)(r / n_rt);
      rt = r % n_rt;
      e = S->L.expert[d];
      mask = S->L.mask[d];
    }
    float4v acc[2] = {zero, zero};
    if (wave * CPW < n_chunks) {
      for (int mat = 0; mat < 2; ++mat) {
        for (int cc = 0; cc < CPW; ++cc) {
          const int chunk = wave * CPW + cc;
          if (chunk >= n_chunks) break;
          if (shared && a.fmt_s == MOE_FMT_Q8) {
            // exact codes, each k-block's dots times row n's scale in fp32
            const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)rt * n_chunks + chunk) * kQ8Tile;
            const u32x4 scl = load16(tile + q8_scale_off(lane & 15));
            for (int kb = 0; kb < 8; ++kb) {
              const uint32_t* cp = reinterpret_cast<const uint32_t*>(tile + q8_code_off(kb, lane));
              const float4v c = mfma_f16(A[cc][kb], q8_codes(cp[0], cp[1]), zero);
              acc[mat] += h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu) * c;
            }
          } else if (shared) {
            const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)rt * n_chunks + chunk) * kBf16Tile;
            for (int kb = 0; kb < 8; ++kb) {
              const half8 b = bf16x8_to_half8(load16(tile + 1024 * kb + 16 * lane));
              acc[mat] = mfma_f16(A[cc][kb], b, acc[mat]);
            }
          } else if (FMT == MOE_FMT_CB2) {
            const uint8_t* tile = (mat ? a.gate : a.up) + (size_t)e * a.expert_bytes +
                                  ((size_t)rt * n_chunks + chunk) * kCb2Tile;
            const u32x4 codes = load16(tile + 16 * lane);
            const u32x4 scl = load16(tile + 1024 + 16 * (lane & 15));
            for (int kb = 0; kb < 8; ++kb) {
              const uint32_t code = (codes[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu;
              const half8 b = cb2_group(code, val_lane, flip_lane);
              const float4v c = mfma_f16(A[cc][kb], b, zero);
              const float s = h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu);
              acc[mat] += s * c;
            }
          } else {  // K4
            const uint8_t* tile = (mat ? a.gate : a.up) + (size_t)e * a.expert_bytes +
                                  ((size_t)rt * n_chunks + chunk) * kK4Tile;
            const u32x4 q0 = load16(tile + 16 * lane);
            const u32x4 q1 = load16(tile + 1024 + 16 * lane);
            const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * (lane & 15));
            const uint32_t s0 = sp[0], s1 = sp[1], s2 = sp[2];
            const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * (lane & 15));
            const float d = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
            for (int kb = 0; kb < 8; ++kb) {
              const uint32_t w = (kb < 4) ? q0[kb & 3] : q1[kb & 3];
              const half8 b = as_half8(k4_magic(w));
              const float4v c = mfma_f16(A[cc][kb], b, zero);
              const float dsc = d * (float)k4_scale_value(s0, s1, s2, kb);
              const float corr = 1024.0f * dsc + dmin * (float)k4_scale_value(s0, s1, s2, 8 + kb);
              const float4v X = *reinterpret_cast<const float4v*>(xsum + ((chunk * 8 + kb) * 16 + 4 * (lane >> 4)));
              acc[mat] += dsc * c - corr * X;
            }
          }
        }
      }
    }
    float* r = red + ((size_t)wave * 2) * 256;
    *reinterpret_cast<float4v*>(r + lane * 4) = acc[0];
    *reinterpret_cast<float4v*>(r + 256 + lane * 4) = acc[1];
    __syncthreads();
    for (int p = tid; p < T * 16; p += blockDim.x) {
      const int m = p >> 4, n = p & 15;
      const int l = 16 * (m >> 2) + n, i = m & 3;
      float u = 0.f, g = 0.f;
      for (int w = 0; w < NW; ++w) {
        u += red[((size_t)w * 2) * 256 + l * 4 + i];
        g += red[((size_t)w * 2 + 1) * 256 + l * 4 + i];
      }
      const int xe = x_exp_of_field(S->xef[m]);
      const _Float16 h16 = h_of(g, u, xe, xe);
      S->hv[m][n] = (float)h16;
      const int64_t row = rt * 16 + n;
      if (shared) {
        a.hs[(size_t)m * a.Is + row] = h16;
      } else if (mask & (1u << m)) {
        for (int j = 0; j < k; ++j)
          if (a.topk_idx[m * k + j] == e) a.h[(size_t)(m * k + j) * a.I + row] = h16;
      }
    }
    __syncthreads();
    // per-token sums of the 16 new h values for the down projection's
    // offsets: X = sum h, O = sum 1024 * fp16(h * 4^-t) (t of the K2 slot).
    if (!shared && tid < T && (mask & (1u << tid))) {
      const int m = tid;
      float X = 0.f, O = 0.f;
      for (int n = 0; n < 16; ++n) {
        const float hv = S->hv[m][n];
        X += hv;
        const int kk = (int)((rt * 16 + n) & 255);
        const int t = k2_slot_t(kk >> 5, (kk & 7) >> 1);
        O += 1024.0f * (float)(_Float16)(hv * __builtin_ldexpf(1.0f, -2 * t));
      }
      for (int j = 0; j < k; ++j)
        if (a.topk_idx[m * k + j] == e) {
          float* hs = a.hsum + ((size_t)(m * k + j) * (a.I_pad / 16) + rt) * 2;
          hs[0] = X;
          hs[1] = O;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection.  Items: (expert slot, row tile of H) and shared row tiles.

struct DnShared {
  ExpertList L;
  int64_t item_lo, item_hi;
  int tok[kMaxT];      // tokens of the current item, ascending
  int slot[kMaxT];     // first slot (m*k + j) of each token for this expert
  int n_tok;
};

// Token groups for K2 block-diagonal accumulation: a pass handles up to 8
// tokens; with tp tokens, C rows m = tok * 2As + local sub-block, where As
// k-blocks (2As sub-blocks) are accumulated before scaling.
__device__ __forceinline__ int k2_as(int tp) { return tp == 1 ? 8 : tp == 2 ? 4 : tp <= 4 ? 2 : 1; }

template <int FMT>
__global__ __launch_bounds__(1024) void dec_down_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  DnShared* S = reinterpret_cast<DnShared*>(smem);
  const size_t off = (sizeof(DnShared) + 255) & ~size_t(255);
  float* red = reinterpret_cast<float*>(smem + off);    // [NW][64][4]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NW = blockDim.x >> 6;
  const int T = a.T, k = a.k;
  const int n_chunks = a.I_pad / 256;
  const int n_chunks_s = a.Is_pad / 256;
  build_expert_list(a.topk_idx, T * k, k, a.E, &S->L);
  const int64_t n_rt = a.H / 16;
  const int64_t n_rts = (a.Is > 0) ? a.H / 16 : 0;
  const int64_t w_r = (int64_t)a.tb_dn * n_chunks, w_s = (int64_t)a.tb_s * n_chunks_s;
  if (tid == 0) {
    const int64_t n_r = (int64_t)S->L.n * n_rt;
    S->item_lo = item_start(blockIdx.x, gridDim.x, n_rts, w_s, n_r, w_r);
    S->item_hi = item_start(blockIdx.x + 1, gridDim.x, n_rts, w_s, n_r, w_r);
  }
  __syncthreads();
  const int64_t item_lo = S->item_lo, item_hi = S->item_hi;
  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, g4 = lane >> 4;

  int cur_d = -2;
  for (int64_t item = item_lo; item < item_hi; ++item) {
    const bool shared = item < n_rts;
    int64_t rt;
    int d = -1, e = -1;
    if (shared) {
      rt = item;
    } else {
      const int64_t r = item - n_rts;
      d = (int)(r / n_rt);
      rt = r % n_rt;
      e = S->L.expert[d];
    }
    if (d != cur_d) {
      // token list of this item
      __syncthreads();
      if (tid == 0) {
        int nt = 0;
        if (shared) {
          for (int m = 0; m < T; ++m) { S->tok[nt] = m; S->slot[nt] = -1; ++nt; }
        } else {
          const uint32_t mask = S->L.mask[d];
          for (int m = 0; m < T; ++m)
            if (mask & (1u << m)) {
              int sl = -1;
              for (int j = 0; j < k; ++j)
                if (a.topk_idx[m * k + j] == e) { sl = m * k + j; break; }
              S->tok[nt] = m;
              S->slot[nt] = sl;
              ++nt;
            }
        }
        S->n_tok = nt;
      }
      __syncthreads();
      cur_d = d;
    }
    const int n_tok = S->n_tok;
    float4v acc = zero;   // K4 / BF16: C layout; K2: [pass*2 + entry]
    const int nck = shared ? n_chunks_s : n_chunks;
    const int Kvalid = shared ? a.Is : a.I;
    for (int chunk = wave; chunk < nck; chunk += NW) {
      if (shared) {
        const bool q8 = a.fmt_s == MOE_FMT_Q8;
        const uint8_t* tile = a.sdown + ((size_t)rt * n_chunks_s + chunk) * a.tb_s;
        const u32x4 scl = q8 ? load16(tile + q8_scale_off(n)) : u32x4{0u, 0u, 0u, 0u};
        for (int kb = 0; kb < 8; ++kb) {
          const int col = chunk * 256 + kb * 32 + g4 * 8;
          u32x4 ar = {0, 0, 0, 0};
          const int m = n;  // A row = lane % 16
          if (m < n_tok && col < Kvalid) ar = load16(a.hs + (size_t)S->tok[m] * a.Is + col);
          if (q8) {
            // exact codes, the k-block's dots times row n's scale in fp32
            const uint32_t* cp = reinterpret_cast<const uint32_t*>(tile + q8_code_off(kb, lane));
            const float4v c = mfma_f16(as_half8(ar), q8_codes(cp[0], cp[1]), zero);
            acc += h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu) * c;
          } else {
            const half8 b = bf16x8_to_half8(load16(tile + 1024 * kb + 16 * lane));
            acc = mfma_f16(as_half8(ar), b, acc);
          }
        }
      } else if (FMT == MOE_FMT_K4) {
        const uint8_t* tile = a.down + (size_t)e * a.expert_bytes_down + ((size_t)rt * n_chunks + chunk) * kK4Tile;
        const u32x4 q0 = load16(tile + 16 * lane);
        const u32x4 q1 = load16(tile + 1024 + 16 * lane);
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
        const uint32_t s0 = sp[0], s1 = sp[1], s2 = sp[2];
        const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
        const float dsc0 = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
        for (int kb = 0; kb < 8; ++kb) {
          const int col = chunk * 256 + kb * 32 + g4 * 8;
          u32x4 ar = {0, 0, 0, 0};
          if (n < n_tok && col < Kvalid) ar = load16(a.h + (size_t)S->slot[n] * a.I + col);
          const uint32_t w = (kb < 4) ? q0[kb & 3] : q1[kb & 3];
          const float4v c = mfma_f16(as_half8(ar), as_half8(k4_magic(w)), zero);
          const float dsc = dsc0 * (float)k4_scale_value(s0, s1, s2, kb);
          const float corr = 1024.0f * dsc + dmin * (float)k4_scale_value(s0, s1, s2, 8 + kb);
          float4v X;
          for (int i = 0; i < 4; ++i) {
            const int m = 4 * g4 + i;
            float xs = 0.f;
            if (m < n_tok && chunk * 256 + kb * 32 < Kvalid) {
              const float* hsm = a.hsum + (size_t)S->slot[m] * (a.I_pad / 16) * 2;
              const int b16 = (chunk * 256 + kb * 32) / 16;
              xs = hsm[b16 * 2] + hsm[(b16 + 1) * 2];
            }
            X[i] = xs;
          }
          acc += dsc * c - corr * X;
        }
      } else {  // K2
        const uint8_t* tile = a.down + (size_t)e * a.expert_bytes_down + ((size_t)rt * n_chunks + chunk) * kK2Tile;
        const u32x4 qw = load16(tile + 16 * lane);
        const u32x4 scm = load16(tile + 1024 + 16 * n);
        const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 1280 + 4 * n);
        const float dsup = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
        u32x4 Bm[8];
        for (int kb = 0; kb < 8; ++kb) Bm[kb] = k2_magic(qw, kb);
        const int n_pass = (n_tok + 7) / 8;
        for (int p = 0; p < n_pass; ++p) {
          const int tp = min(8, n_tok - 8 * p);
          const int As = k2_as(tp);
          const int m = n;                       // A row of this lane
          const int a_tok = m / (2 * As), a_sbl = m % (2 * As);
          for (int grp = 0; grp < 8 / As; ++grp) {
            float4v c = zero;
            for (int kl = 0; kl < As; ++kl) {
              const int kb = grp * As + kl;
              u32x4 ar = {0, 0, 0, 0};
              const int col = chunk * 256 + kb * 32 + g4 * 8;
              if (a_tok < tp && a_sbl == 2 * kl + (g4 >> 1) && col < Kvalid) {
                const u32x4 raw = load16(a.h + (size_t)S->slot[8 * p + a_tok] * a.I + col);
                half8 hv = as_half8(raw);
                for (int s = 0; s < 4; ++s) {
                  const _Float16 sc = (_Float16)__builtin_ldexpf(1.0f, -2 * k2_slot_t(kb, s));
                  hv[2 * s] = hv[2 * s] * sc;
                  hv[2 * s + 1] = hv[2 * s + 1] * sc;
                }
                ar = as_u32x4(hv);
              }
              c = mfma_f16(as_half8(ar), as_half8(Bm[kb]), c);
            }
            // C[m][n] for m = 4 g4 + i: token m / 2As, sub-block m % 2As
            for (int i = 0; i < 4; ++i) {
              const int mm = 4 * g4 + i;
              const int tok = mm / (2 * As), sbl = mm % (2 * As);
              if (tok >= tp) continue;
              const int sb = grp * 2 * As + sbl;         // sub-block in the super-block
              if (chunk * 256 + sb * 16 >= Kvalid) continue;
              const uint32_t byte = (scm[sb >> 2] >> (8 * (sb & 3))) & 0xFFu;
              const float sc = (float)(byte & 15u), mn = (float)(byte >> 4);
              const float* hsm = a.hsum + ((size_t)S->slot[8 * p + tok] * (a.I_pad / 16) + chunk * 16 + sb) * 2;
              const float v = dsup * sc * (c[i] - hsm[1]) - dmin * mn * hsm[0];
              const int entry = (As == 1) ? (i >> 1) : 0;
              acc[2 * p + entry] += v;
            }
          }
        }
      }
    }
    // reduce over waves (and lanes) in fixed order
    *reinterpret_cast<float4v*>(red + ((size_t)wave * 64 + lane) * 4) = acc;
    __syncthreads();
    for (int q = tid; q < n_tok * 16; q += blockDim.x) {
      const int ts = q >> 4, nn = q & 15;
      float v = 0.f;
      if (shared || FMT == MOE_FMT_K4) {
        const int l = 16 * (ts >> 2) + nn, i = ts & 3;
        for (int w = 0; w < NW; ++w) v += red[((size_t)w * 64 + l) * 4 + i];
      } else {
        const int p = ts >> 3, tl = ts & 7;
        const int tp = min(8, n_tok - 8 * p);
        const int As = k2_as(tp);
        int g_lo, g_hi, entry = 0;
        if (As == 8) { g_lo = 0; g_hi = 4; }
        else if (As == 4) { g_lo = 2 * tl; g_hi = 2 * tl + 2; }
        else if (As == 2) { g_lo = tl; g_hi = tl + 1; }
        else { g_lo = tl >> 1; g_hi = g_lo + 1; entry = tl & 1; }
        for (int w = 0; w < NW; ++w)
          for (int gg = g_lo; gg < g_hi; ++gg)
            v += red[((size_t)w * 64 + 16 * gg + nn) * 4 + 2 * p + entry];
      }
      const int64_t row = rt * 16 + nn;
      const int m = S->tok[ts];
      if (shared) {
        a.ysh[(size_t)m * a.H + row] = v;
      } else {
        for (int j = 0; j < k; ++j)
          if (a.topk_idx[m * k + j] == e) a.ybuf[(size_t)(m * k + j) * a.H + row] = v;
      }
    }
    __syncthreads();
  }
}

// y[t][h] = (sum_j w[t][j] * ybuf[t*k + j][h] + ysh[t][h]) 2^(2 e_t), j
// ascending (h was stored times 2^-2e_t).
__global__ void combine_kernel(const float* ybuf, const float* ysh, const int32_t* topk_idx,
                               const float* topk_w, const int* xexp, int T, int k, int H, int E, float* y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * H) return;
  const int t = (int)(i / H), h = (int)(i % H);
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    if (e < 0 || e >= E) continue;
    acc += topk_w[t * k + j] * ybuf[(size_t)(t * k + j) * H + h];
  }
  if (ysh) acc += ysh[(size_t)t * H + h];
  y[i] = __builtin_ldexpf(acc, 2 * xexp[t]);
}

}  // namespace

namespace qmoe {

size_t dec_upgate_lds(const DecArgs& a, int fmt) {
  size_t off = (sizeof(UgShared) + 255) & ~size_t(255);
  if (fmt == MOE_FMT_CB2) off += 2 * kCb2TableBytes;
  if (fmt == MOE_FMT_K4) off += (size_t)(a.H / 32) * 16 * 4;
  return off + (size_t)a.nw_ug * 2 * 256 * 4;
}

size_t dec_down_lds(const DecArgs& a) {
  return ((sizeof(DnShared) + 255) & ~size_t(255)) + (size_t)a.nw_dn * 64 * 4 * 4;
}

hipError_t launch_dec_upgate(const DecArgs& a, int fmt, int cpw, int grid, hipStream_t s) {
  const size_t lds = dec_upgate_lds(a, fmt);
  const dim3 block(64 * a.nw_ug);
  void (*fn)(DecArgs) = nullptr;
  if (fmt == MOE_FMT_CB2) fn = cpw == 1 ? dec_upgate_kernel<MOE_FMT_CB2, 1> : dec_upgate_kernel<MOE_FMT_CB2, 2>;
  else fn = cpw == 1 ? dec_upgate_kernel<MOE_FMT_K4, 1> : dec_upgate_kernel<MOE_FMT_K4, 2>;
  hipError_t err = ensure_dyn_lds((const void*)fn);
  if (err != hipSuccess) return err;
  return launch_timed(MOE_KERNEL_DECODE_UPGATE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) { hipExtLaunchKernelGGL(fn, dim3(grid), block, lds, s, ev0_, ev1_, 0, a); });
}

hipError_t launch_dec_down(const DecArgs& a, int fmt, int grid, hipStream_t s) {
  const size_t lds = dec_down_lds(a);
  void (*fn)(DecArgs) = fmt == MOE_FMT_K2 ? dec_down_kernel<MOE_FMT_K2> : dec_down_kernel<MOE_FMT_K4>;
  hipError_t err = ensure_dyn_lds((const void*)fn);
  if (err != hipSuccess) return err;
  return launch_timed(MOE_KERNEL_DECODE_DOWN, s,
                      [&](hipEvent_t ev0_, hipEvent_t ev1_) { hipExtLaunchKernelGGL(fn, dim3(grid), dim3(64 * a.nw_dn), lds, s, ev0_, ev1_, 0, a); });
}

hipError_t launch_combine(const DecArgs& a, const int32_t* topk_idx, const float* topk_w, float* y,
                          hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.H;
  return launch_timed(MOE_KERNEL_DECODE_COMBINE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ev0_, ev1_, 0, a.ybuf,
                       a.Is > 0 ? a.ysh : nullptr, topk_idx, topk_w, a.xexp, a.T, a.k, a.H, a.E, y);
  });
}

}  // namespace qmoe
