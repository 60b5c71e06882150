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
#include "route_common.hpp"
#include "launch_util.h"

using namespace qmoe_dev;
using qmoe::DecArgs;

namespace {

// Expert id of choice j (j uniform over the wave), read as a scalar load:
// its wait counts scalar loads only, so taking an id never waits for the
// weight tiles in flight (a wave's vector loads complete in issue order and
// a vector wait is a count of loads still outstanding).
__device__ __forceinline__ int expert_id(const int32_t* topk_idx, int j) {
  return ((const __attribute__((address_space(4))) int32_t*)topk_idx)[j];
}
__device__ __forceinline__ float choice_weight(const float* topk_w, int j) {
  return ((const __attribute__((address_space(4))) float*)topk_w)[j];
}
// The token's exponent, as the up/gate kernel wrote it (scalar load).
__device__ __forceinline__ int token_exp(const int* xexp) {
  return ((const __attribute__((address_space(4))) int*)xexp)[0];
}

// Raw buffer loads of a tile that may not exist: a load whose offset lies
// past the descriptor's byte count returns zeros and touches no memory, so
// such a tile needs no branch around its loads (a load inside a branch makes
// the compiler wait for every earlier load where the paths join).  base must
// be wave-uniform; word 3 is the untyped-dword setting of this family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Streaming weight loads: non-temporal (each weight byte is read once).
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

constexpr int kBatch = 8;        // row tiles reduced per barrier (up/gate)

// ---------------------------------------------------------------------------
// Shared-expert tiles, BF16 or Q8 (SF = MOE_FMT_BF16 / MOE_FMT_Q8).  Q8
// weights enter the MFMA as their exact 8-bit codes and the per-32 scales
// are applied in fp32 to block dots that each cover one k-block, so the
// single-token paths use the Q8 weights exactly, as they do the BF16 ones.
template <int SF>
constexpr int shared_tile_bytes() { return SF == MOE_FMT_Q8 ? kQ8Tile : kBf16Tile; }

// Half row tile (rows r = 8 hr + (n & 7)) of one matrix: lanes n < 8 take
// row r's even k-blocks, lanes n >= 8 its odd ones, so that A_{2p} | A_{2p+1}
// feeds one MFMA per k-block pair p.  BF16: v[p] = the lane's 8 weights of
// k-block 2p + n/8.  Q8: v[0], v[1] = its two 16-byte code pieces (k-blocks
// {0,2}, {4,6} for n < 8, {1,3}, {5,7} for n >= 8), sc = row r's 8 scales.
struct ShHalf {
  u32x4 v[4];
  u32x4 sc;
};

template <int SF, typename Ld>
__device__ __forceinline__ void sh_half_load(ShHalf& S, Ld ld, int n, int qq, int r) {
  const int c = 16 * qq + r;
  if constexpr (SF == MOE_FMT_Q8) {
    S.v[0] = ld(1024 * (2 * (n >> 3)) + 16 * c);
    S.v[1] = ld(1024 * (2 * (n >> 3) + 1) + 16 * c);
    S.sc = ld(q8_scale_off(r));
  } else {
    for (int p = 0; p < 4; ++p) S.v[p] = ld(1024 * (2 * p + (n >> 3)) + 16 * c);
  }
}

// The half tile times the activations; the lane's part of row r (lanes
// g < 2, others 0): the caller adds lanes n, n ^ 8 and g = 0, 1.  After the
// four MFMAs C[kb][n] holds the dot of k-block kb alone (even kb in lanes
// n < 8, odd kb in lanes n >= 8), which is where a Q8 scale applies.
template <int SF, typename Ap>
__device__ __forceinline__ float sh_half_dot(const ShHalf& S, Ap a_pair, int n, int g) {
  float4v c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    half8 b;
    if constexpr (SF == MOE_FMT_Q8) {
      const u32x4 pc = S.v[p >> 1];
      b = (p & 1) ? q8_codes(pc.z, pc.w) : q8_codes(pc.x, pc.y);
    } else {
      b = bf16x8_to_half8(S.v[p]);
    }
    c = mfma_f16(a_pair(p), b, c);
  }
  float t;
  if constexpr (SF == MOE_FMT_Q8) {
    // lane (g, n): k-blocks 4g, 4g+2 (n < 8) or 4g+1, 4g+3 (n >= 8)
    const uint32_t w0 = (g & 1) ? S.sc.z : S.sc.x, w1 = (g & 1) ? S.sc.w : S.sc.y;
    const int sh = (n >> 3) ? 16 : 0;
    const float d0 = h2f((w0 >> sh) & 0xFFFFu), d1 = h2f((w1 >> sh) & 0xFFFFu);
    t = (n < 8) ? fmaf(d1, c[2], d0 * c[0]) : fmaf(d1, c[3], d0 * c[1]);
  } else {
    t = (n < 8) ? c[0] + c[2] : c[1] + c[3];
  }
  return g >= 2 ? 0.f : t;
}

// Half a K-chunk (k-blocks kb0 .. kb0+3, kb0 = 0 or 4) of row n of a down
// tile, for the lane c = 16 g4 + n.  BF16: v[q] = the lane's 8 weights of
// k-block kb0 + q.  Q8: v[0] = the piece of k-blocks kb0, kb0+2, v[1] = that
// of kb0+1, kb0+3, sc = row n's 8 scales.
struct ShQuarter {
  u32x4 v[4];
  u32x4 sc;
};

template <int SF, typename Ld>
__device__ __forceinline__ void sh_dn_load(ShQuarter& S, Ld ld, int kb0, int lane) {
  if constexpr (SF == MOE_FMT_Q8) {
    const int h = kb0 >> 2;
    S.v[0] = ld(1024 * h + 16 * lane);
    S.v[1] = ld(1024 * (h + 2) + 16 * lane);
    S.sc = ld(q8_scale_off(lane & 15));
  } else {
    for (int q = 0; q < 4; ++q) S.v[q] = ld(1024 * (kb0 + q) + 16 * lane);
  }
}

// B operand of k-block kb0 + q.
template <int SF>
__device__ __forceinline__ half8 sh_dn_b(const ShQuarter& S, int q) {
  if constexpr (SF == MOE_FMT_Q8) {
    const u32x4 pc = S.v[q & 1];
    return (q >> 1) ? q8_codes(pc.z, pc.w) : q8_codes(pc.x, pc.y);
  } else {
    return bf16x8_to_half8(S.v[q]);
  }
}

// Row n's sum from the accumulated C.  BF16: the activations sit in A row 0
// for every q, so C[0][n] is the sum.  Q8: those of k-block kb0 + q sit in
// row q, C[q][n] is that block's dot, scaled here (rows >= 4 are zero).
template <int SF>
__device__ __forceinline__ float sh_dn_sum(const ShQuarter& S, const float4v& c, int kb0) {
  if constexpr (SF == MOE_FMT_Q8) {
    const uint32_t w0 = kb0 ? S.sc.z : S.sc.x, w1 = kb0 ? S.sc.w : S.sc.y;
    float v = h2f(w0 & 0xFFFFu) * c[0];
    v = fmaf(h2f(w0 >> 16), c[1], v);
    v = fmaf(h2f(w1 & 0xFFFFu), c[2], v);
    return fmaf(h2f(w1 >> 16), c[3], v);
  } else {
    return c[0];
  }
}

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
// CB2 up/gate at one token for H > 4096 (17 to 32 K-chunks): kCpw = 2
// K-chunks per wave.  Per-wave payload of one routed row tile (both
// matrices): codes and scales of its chunks.

constexpr int kCpw = 2;

struct UgPay {
  u32x4 code[2][kCpw], scale[2][kCpw];
};

__device__ __forceinline__ void ug_load(UgPay& p, const DecArgs& a, int e, int64_t rt, int wave, int lane,
                                        int n_chunks) {
  const int n = lane & 15;
  for (int mat = 0; mat < 2; ++mat)
    for (int cc = 0; cc < kCpw; ++cc) {
      const int chunk = min(wave * kCpw + cc, n_chunks - 1);
      const uint8_t* tile =
          (mat ? a.gate : a.up) + (size_t)e * a.expert_bytes + ((size_t)rt * n_chunks + chunk) * kCb2Tile;
      p.code[mat][cc] = load16(tile + 16 * lane);
      p.scale[mat][cc] = load16(tile + 1024 + 16 * n);
    }
}

template <int SF>
__global__ __launch_bounds__(1024) void dec1_cb2_wide_upgate_kernel(DecArgs a) {
  constexpr int CPW = kCpw;
  extern __shared__ __align__(16) uint8_t smem[];
  int64_t* range = reinterpret_cast<int64_t*>(smem);
  uint8_t* val_tab = smem + 256;
  uint8_t* flip_tab = val_tab + kCb2TableBytes;
  float* red = reinterpret_cast<float*>(smem + 256 + 2 * kCb2TableBytes);   // [kBatch][NW][2][16]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NW = blockDim.x >> 6;
  const int k = a.k, n_chunks = a.H / 256;
  const int64_t n_rt = a.I / 16, n_rts = a.Is / 16;
  const int64_t w_r = (int64_t)2 * a.tb_ug * n_chunks, w_s = (int64_t)2 * shared_tile_bytes<SF>() * n_chunks;
  uint32_t* xef = reinterpret_cast<uint32_t*>(smem + 16);                     // [NW] largest x exponent field per wave
  if (tid == 0) {
    range[0] = item_start1(blockIdx.x, gridDim.x, n_rts, w_s, (int64_t)k * n_rt, w_r);
    range[1] = item_start1(blockIdx.x + 1, gridDim.x, n_rts, w_s, (int64_t)k * n_rt, w_r);
  }
  // A operands: row 0 = x 2^-xe, rows 1..15 zero; raw bf16 until the
  // token's exponent xe is known (every wave's chunks are needed for it)
  u32x4 xraw[CPW][8];
  const int qq = lane >> 4;
  {
    uint32_t ef = 0;
    for (int cc = 0; cc < CPW; ++cc)
      for (int kb = 0; kb < 8; ++kb) {
        const int chunk = wave * CPW + cc;
        u32x4 r = {0, 0, 0, 0};
        if ((lane & 15) == 0 && chunk < n_chunks) r = load16(a.x + chunk * 256 + kb * 32 + qq * 8);
        xraw[cc][kb] = r;
        ef = max(ef, bf16x8_max_efield(r));
      }
    ef = wave_max_u32(ef);
    if (lane == 0) xef[wave] = ef;
  }
  cb2_fill_tables(a.codebook, val_tab, flip_tab, tid, blockDim.x);
  __syncthreads();
  int xe;
  {
    uint32_t ef = 0;
    for (int w = 0; w < NW; ++w) ef = max(ef, xef[w]);
    xe = x_exp_of_field(ef);
  }
  if (blockIdx.x == 0 && tid == 0) a.xexp[0] = xe;
  const int64_t lo = range[0], hi = range[1];
  if (lo >= hi) return;
  half8 A[CPW][8];
  for (int cc = 0; cc < CPW; ++cc)
    for (int kb = 0; kb < 8; ++kb) A[cc][kb] = bf16x8_to_half8_exp(xraw[cc][kb], xe);
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
      const _Float16 h16 = h_of(g, u, xe, xe);
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
        if constexpr (SF == MOE_FMT_Q8) {
          // codes exact in the MFMA, then each k-block's dot times its scale
          u32x4 raw[2][4], scl[2];
          for (int mat = 0; mat < 2; ++mat) {
            const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)item * n_chunks + chunk) * kQ8Tile;
            for (int i = 0; i < 4; ++i) raw[mat][i] = load16(tile + 1024 * i + 16 * lane);
            scl[mat] = load16(tile + q8_scale_off(lane & 15));
          }
          for (int mat = 0; mat < 2; ++mat)
            for (int kb = 0; kb < 8; ++kb) {
              const u32x4 pc = raw[mat][2 * (kb & 1) + (kb >> 2)];
              const half8 b = ((kb >> 1) & 1) ? q8_codes(pc.z, pc.w) : q8_codes(pc.x, pc.y);
              const float4v c = mfma_f16(A[cc][kb], b, zero);
              v[mat] = fmaf(h2f((scl[mat][kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu), c[0], v[mat]);
            }
        } else {
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
  // (two chunks per wave: the registers hold the activations, so a row
  // tile's loads are issued when it is computed, not one tile ahead)
  UgPay cur;
  for (; item < hi; ++item) {
    const int e = expert_of(item);
    if (wave_has_chunks && e >= 0 && e < a.E) ug_load(cur, a, e, (item - n_rts) % n_rt, wave, lane, n_chunks);
    float v[2] = {0.f, 0.f};
    if (wave_has_chunks && e >= 0 && e < a.E) {
      for (int mat = 0; mat < 2; ++mat)
        for (int cc = 0; cc < CPW; ++cc) {
          const int chunk = wave * CPW + cc;
          if (chunk >= n_chunks) break;
          for (int kb = 0; kb < 8; ++kb) {
            const uint32_t code = (cur.code[mat][cc][kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu;
            const float4v c = mfma_f16(A[cc][kb], cb2_group(code, val_lane, flip_lane), zero);
            v[mat] += h2f((cur.scale[mat][cc][kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu) * c[0];
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
  }
}

// ---------------------------------------------------------------------------
// CB2 up/gate at one token (H <= 4096: one K-chunk of 256 columns per wave).
//
// Work split: every workgroup takes an even share of both kinds of work --
// half row tiles (8 rows) of the bf16 shared expert and whole 16-row tiles
// of the routed experts -- so the LDS-heavy codebook decode is spread over
// all compute units while the shared expert's plain bf16 stream keeps HBM
// busy next to it.
//
// Decode table: the 64 KB (index, half, sign nibble) table of cb2_comb at
// LDS offset 0.
//
// A operands are block-diagonal: A_kb holds x's k-block kb in row kb, so 8
// accumulating MFMAs leave the per-block dots C[kb][n] (kb = 4g + i in lane
// (g, n), g < 2), each then scaled by its own fp16 scale.
//
// Shared-expert half tiles use the same A registers: for k-block pair p,
// lanes with n < 8 load row n of k-block 2p and lanes n >= 8 row n-8 of
// k-block 2p+1, and A_{2p} | A_{2p+1} supplies both activation rows, so one
// MFMA covers two k-blocks of 8 rows with all 64 lanes loading useful bytes.

constexpr int kRedBatch = 8;      // routed row tiles per cross-wave reduction
constexpr int kPrefetch3 = 3;     // routed row tiles in flight per wave

struct Cb2Pay {
  u32x4 code[2];     // up, gate: the lane's 8 group codes
  uint32_t sc[2][2]; // up, gate: fp16 scales of k-blocks 4(g&1) .. 4(g&1)+3 of row n
  bool ok;           // false: the loads were aimed at a stand-in tile, contribute 0
};

// Loads are unconditional (a stand-in tile when the item is out of range or
// its expert id invalid) so they can all be in flight at once.
__device__ __forceinline__ void cb2_pay_load(Cb2Pay& p, const DecArgs& a, int e, int rt, int chunk, int lane,
                                             int n_chunks, bool ok) {
  const int n = lane & 15, g = lane >> 4;
  const size_t t_off = (size_t)e * a.expert_bytes + ((size_t)rt * n_chunks + chunk) * kCb2Tile;
  for (int mat = 0; mat < 2; ++mat) {
    const uint8_t* tile = (mat ? a.gate : a.up) + t_off;
    p.code[mat] = load16_nt(tile + 16 * lane);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 sp = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + 1024 + 16 * n + 8 * (g & 1)));
    p.sc[mat][0] = sp.x;
    p.sc[mat][1] = sp.y;
  }
  p.ok = ok;
}

__device__ __forceinline__ float cb2_scaled(const float4v& c, const uint32_t sc[2], bool ok) {
  float v = h2f(sc[0] & 0xFFFFu) * c[0];
  v = fmaf(h2f(sc[0] >> 16), c[1], v);
  v = fmaf(h2f(sc[1] & 0xFFFFu), c[2], v);
  v = fmaf(h2f(sc[1] >> 16), c[3], v);
  return ok ? v : 0.f;
}

// Route: the token's top k are ranked here from the router's partial
// logits (every workgroup ranks them; workgroup 0 writes them out) while the
// shared expert's tiles are already in flight.  E <= the workgroup's threads.
template <bool Route, int SF>
__global__ __launch_bounds__(1024) void dec1_cb2_upgate_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tab = smem;                                                     // [0, 64 KB)
  const int tid = threadIdx.x, lane = tid & 63, NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* red_r = reinterpret_cast<float*>(smem + kCb2CombBytes);  // [kRedBatch][2][NW][32]
  float* red_s = red_r + kRedBatch * 2 * NW * 32;                         // [NW][2][8]
  uint32_t* xef = reinterpret_cast<uint32_t*>(red_s + NW * 2 * 8);        // [NW] largest x exponent field per wave
  int* ids = reinterpret_cast<int*>(xef + NW);                            // [16] (Route)
  qmoe_route::TopkLds* tk = reinterpret_cast<qmoe_route::TopkLds*>(ids + 16);   // (Route)

  // ---- prologue.  Loads are issued oldest-first in the order they are
  // needed (the router's logits, codebook and x, then the shared tile, then
  // a routed tile).  A wave's loads complete in issue order and a wait is a
  // count of loads still in flight, so these loads are unconditional (lanes
  // that need none load a copy and ignore it): a load inside a divergent
  // branch makes the compiler wait for every earlier load at the join.
  // Route, E <= 256 (a multiple of 4): wave 0 loads all logits, four per
  // lane, and ranks them alone; otherwise thread tid loads the logit of
  // expert tid for the workgroup-wide ranking.  Buffer loads: a lane past E
  // (or a load whose descriptor has no bytes) reads zero, with no branch.
  const bool wave_rank = Route && a.E <= 256 && (a.E & 3) == 0;
  float mylogit = 0.f;
  u32x4 lg4 = {0u, 0u, 0u, 0u};
  if constexpr (Route) {
    const float* lrow = a.logits + (size_t)a.t_route * a.E;
    lg4 = bload16(tile_rsrc(lrow, wave_rank && wave == 0 ? 4 * a.E : 0), 16 * lane);
    mylogit = __builtin_bit_cast(float, bload4(tile_rsrc(lrow, wave_rank ? 0 : 4 * a.E), 4 * tid));
  }
  const int k = a.k, n_chunks = a.H / 256, n_rt = a.I / 16, n_rts = a.Is / 16;
  // (32-bit products: gi * U_r <= 255 * 16 * 1024)
  const unsigned G = gridDim.x, gi = blockIdx.x;
  const unsigned U_s = 2 * n_rts, U_r = k * n_rt;
  const int s_lo = (int)(gi * U_s / G), s_hi = (int)((gi + 1) * U_s / G);
  const int r_lo = (int)(gi * U_r / G), r_hi = (int)((gi + 1) * U_r / G);
  const bool active = wave < n_chunks;       // idle waves (H < 1024) load chunk 0 and discard it
  const int chunk = active ? wave : 0;
  const int n = lane & 15, g = lane >> 4, m = lane & 15, qq = lane >> 4;

  int8_t cbv[4];
  {
    const int8_t* cbp = a.codebook + ((tid & 511) >> 1) * 8 + 4 * (tid & 1);
    for (int i = 0; i < 4; ++i) cbv[i] = cbp[i];
  }
  const u32x4 xr = load16(a.x + chunk * 256 + (m & 7) * 32 + qq * 8);    // used by lanes m < 8

  // wave ranking: the route keys of experts 4 lane .. 4 lane + 3 (0 past E).
  // Every wave waits here until wave 0 has its logits, so that no weight
  // tile is requested before them: the logits are then among the first
  // requests the memory system serves, not queued behind the weight stream
  // (which a compute unit drains in request order).
  uint64_t key[4] = {0, 0, 0, 0};
  if constexpr (Route) {
    const float4v lf = __builtin_bit_cast(float4v, lg4);     // (whole-vector cast)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      key[i] = wave_rank && e < a.E ? qmoe_route::route_key(lf[i], e) : 0;
    }
    if (wave_rank) {
      __builtin_amdgcn_s_waitcnt(0);      // this wave's loads are in (wave 0: the logits)
      __syncthreads();
    }
  }

  // shared half tile loads of both matrices (zeros when the workgroup has
  // no shared item)
  constexpr int kSTile = shared_tile_bytes<SF>();
  ShHalf sraw[2];
  auto issue_shared = [&](int su, bool valid) {
    const int rt = su >> 1, hr = su & 1;
    const int r = 8 * hr + (n & 7);
    for (int mat = 0; mat < 2; ++mat) {
      const uint8_t* tile = valid ? (mat ? a.sgate : a.sup) + ((size_t)rt * n_chunks + chunk) * kSTile
                                  : reinterpret_cast<const uint8_t*>(a.x);
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile, valid ? kSTile : 0);
      sh_half_load<SF>(sraw[mat], [&](int off) { return bload16_nt(rs, off); }, n, qq, r);
    }
  };
  issue_shared(s_lo, s_lo < s_hi);

  if constexpr (Route) {
    auto out = [&](int j, int e, float w) {
      ids[j] = e;
      if (blockIdx.x == 0) {
        a.topk_idx_out[j] = e;
        a.topk_w_out[j] = w;
      }
    };
    if (wave_rank) {
      // wave 0: k rounds of wave-wide maxima over its registers (no LDS
      // passes, no barrier until the result)
      if (wave == 0) {
        qmoe_route::wave_topk4(key, k, [&](int j, uint64_t mk) {
          if (lane == 0) {
            tk->kv[j] = qmoe_route::key_logit(mk);
            tk->ki[j] = ids[j] = (int)(0xFFFFFFFFu - (uint32_t)mk);
          }
        });
        // w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), the sum in rank order
        // as in the workgroup ranking (workgroup 0 writes them out)
        if (blockIdx.x == 0 && lane < k) {
          const float top = tk->kv[0];
          float z = 0.f;
          for (int j = 0; j < k; ++j) z += expf(tk->kv[j] - top);
          a.topk_idx_out[lane] = tk->ki[lane];
          a.topk_w_out[lane] = expf(tk->kv[lane] - top) / z;
        }
      }
    } else {
      auto logit_of = [&](int) { return mylogit; };        // called for e = tid only
      if (blockDim.x >= 1024) qmoe_route::rank_topk<1024>(*tk, a.E, k, logit_of, out);
      else if (blockDim.x >= 512) qmoe_route::rank_topk<512>(*tk, a.E, k, logit_of, out);
      else qmoe_route::rank_topk<256>(*tk, a.E, k, logit_of, out);
    }
    __syncthreads();
  }

  int j_ld = r_lo / n_rt, rt_ld = r_lo - j_ld * n_rt;      // next routed item to load
  Cb2Pay P0, P1, P2;
  auto issue = [&](Cb2Pay& P, int r) {
    int e = -1;
    if (r < r_hi) {
      if constexpr (Route) e = __builtin_amdgcn_readfirstlane(ids[j_ld]);
      else e = expert_id(a.topk_idx, j_ld);
      if (e >= a.E) e = -1;
    }
    const bool ok = e >= 0 && active;
    cb2_pay_load(P, a, ok ? e : 0, ok ? rt_ld : 0, chunk, lane, n_chunks, ok);
    if (++rt_ld == n_rt) {
      rt_ld = 0;
      ++j_ld;
    }
  };
  issue(P0, r_lo);
  {
    // the token's exponent: each wave's largest field, combined after the
    // next barrier (computed only now: its wait for x must not come before
    // the weight loads are issued)
    const uint32_t ef = wave_max_u32(active ? bf16x8_max_efield(xr) : 0u);
    if (lane == 0) xef[wave] = ef;
  }

  // decode table, two steps: the 4 fp16 values of each (idx, half) pair
  // into a staging area, then the 16 sign variants of each, written by
  // consecutive lanes to consecutive entries (no bank conflicts)
  uint2* val4 = reinterpret_cast<uint2*>(red_r);          // [512], reuses the reduction area
  if (tid < 512) val4[tid] = cb2_pair_values(cbv);
  for (int pr = tid + (int)blockDim.x; pr < 512; pr += blockDim.x) {     // workgroups under 512 threads
    int8_t v[4];
    for (int i = 0; i < 4; ++i) v[i] = a.codebook[(pr >> 1) * 8 + 4 * (pr & 1) + i];
    val4[pr] = cb2_pair_values(v);
  }
  __syncthreads();

  // the token's exponent xe; block-diagonal activations x 2^-xe: lane
  // (qq, m) holds x block m (m < 8)
  int xe;
  {
    uint32_t ef = 0;
    for (int w = 0; w < NW; ++w) ef = max(ef, xef[w]);
    xe = x_exp_of_field(ef);
  }
  if (blockIdx.x == 0 && tid == 0) a.xexp[0] = xe;
  half8 A[8];
  {
    const u32x4 xh = active ? as_u32x4(bf16x8_to_half8_exp(xr, xe)) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int kb = 0; kb < 8; ++kb) A[kb] = as_half8(m == kb ? xh : z);
  }
  for (int i = tid; i < 512 * 16; i += blockDim.x) cb2_comb_put(tab, i, val4);
  __syncthreads();

  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  // ---- shared expert half tiles
  for (int su = s_lo; su < s_hi; ++su) {
    if (su != s_lo) issue_shared(su, true);
    float v[2];
    for (int mat = 0; mat < 2; ++mat) {
      float t = sh_half_dot<SF>(
          sraw[mat], [&](int p) { return as_half8(as_u32x4(A[2 * p]) | as_u32x4(A[2 * p + 1])); }, n, g);
      t += __shfl_xor(t, 8);
      t += __shfl_xor(t, 16);
      v[mat] = t;
    }
    if (lane < 8 && active) {
      red_s[(wave * 2 + 0) * 8 + lane] = v[0];
      red_s[(wave * 2 + 1) * 8 + lane] = v[1];
    }
    __syncthreads();
    if (tid < 8) {
      float u = 0.f, gg = 0.f;
      for (int w = 0; w < n_chunks; ++w) {
        u += red_s[(w * 2 + 0) * 8 + tid];
        gg += red_s[(w * 2 + 1) * 8 + tid];
      }
      a.hs[(su >> 1) * 16 + 8 * (su & 1) + tid] = h_of(gg, u, xe, xe);
    }
    __syncthreads();
  }

  // ---- routed row tiles, kPrefetch3 in flight per wave (the second and
  // third are issued only now: their registers held the shared tile)
  issue(P1, r_lo + 1);
  issue(P2, r_lo + 2);
  auto compute = [&](const Cb2Pay& P, int b) {
    float4v cu = zero, cg = zero;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      cu = mfma_f16(A[kb], cb2_comb(P.code[0][kb >> 1], kb & 1, lds_offset(tab)), cu);
      cg = mfma_f16(A[kb], cb2_comb(P.code[1][kb >> 1], kb & 1, lds_offset(tab)), cg);
    }
    if (lane < 32 && active) {
      red_r[((b * 2 + 0) * NW + wave) * 32 + lane] = cb2_scaled(cu, P.sc[0], P.ok);
      red_r[((b * 2 + 1) * NW + wave) * 32 + lane] = cb2_scaled(cg, P.sc[1], P.ok);
    }
  };
  auto flush = [&](int first, int nb) {
    __syncthreads();
    if (tid < nb * 16) {
      const int b = tid >> 4, item = first + b;
      float u = 0.f, gg = 0.f;
      for (int w = 0; w < n_chunks; ++w) {
        u += red_r[((b * 2 + 0) * NW + w) * 32 + n];
        u += red_r[((b * 2 + 0) * NW + w) * 32 + 16 + n];
        gg += red_r[((b * 2 + 1) * NW + w) * 32 + n];
        gg += red_r[((b * 2 + 1) * NW + w) * 32 + 16 + n];
      }
      const _Float16 h16 = h_of(gg, u, xe, xe);
      const float hv = (float)h16;
      const int j = item / n_rt, rt = item - j * n_rt;
      a.h[(size_t)j * a.I + rt * 16 + n] = h16;
      const int kk = (rt * 16 + n) & 255;
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
    __syncthreads();
  };

  int nb = 0, first = r_lo;
  for (int r = r_lo; r < r_hi; r += kPrefetch3) {
    compute(P0, nb);
    issue(P0, r + 3);
    if (++nb == kRedBatch || r + 1 == r_hi) {
      flush(first, nb);
      first = r + 1;
      nb = 0;
    }
    if (r + 1 >= r_hi) break;
    compute(P1, nb);
    issue(P1, r + 4);
    if (++nb == kRedBatch || r + 2 == r_hi) {
      flush(first, nb);
      first = r + 2;
      nb = 0;
    }
    if (r + 2 >= r_hi) break;
    compute(P2, nb);
    issue(P2, r + 5);
    if (++nb == kRedBatch || r + 3 == r_hi) {
      flush(first, nb);
      first = r + 3;
      nb = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// K4 up/gate at one token, H up to 8192.
//
// A unit is one item (a routed 16-row tile or a shared 8-row half tile)
// restricted to a K-part of up to 16 chunks: wave w takes chunk 16 kp + w of
// part kp, and the parts of an item are consecutive units whose per-wave
// sums accumulate until the item's last part.  Routed units are loaded two
// ahead.  x sits in LDS as fp16, followed by a zero block: the
// block-diagonal A operand of k-block kb is one LDS read per lane (the lanes
// of row kb read x's block, the others the zero block), so no registers hold
// activations.  K4 codes go into the MFMA as 1024 + q (exact), and the
// 6-bit scales and mins are applied per k-block to the block dots C_kb with
// the block sums X_kb of x:
//   sum_k x_k w_k = sum_kb [d sc_kb C_kb - (1024 d sc_kb + dmin m_kb) X_kb].

struct K4Pay {
  u32x4 q[2][2];       // up, gate: the lane's words of k-blocks 0-3 and 4-7
  uint32_t s[2][3];    // up, gate: row n's packed 6-bit scales (0-7) and mins (8-15)
  uint32_t dd[2];      // up, gate: row n's fp16 d | dmin << 16
  bool ok;             // false: a stand-in tile, contributes 0
};

__device__ __forceinline__ void k4_pay_load(K4Pay& p, const DecArgs& a, int e, int rt, int chunk, int lane,
                                            int n_chunks, bool ok) {
  const int n = lane & 15;
  const size_t t_off = (size_t)e * a.expert_bytes + ((size_t)rt * n_chunks + chunk) * kK4Tile;
  for (int mat = 0; mat < 2; ++mat) {
    const uint8_t* tile = (mat ? a.gate : a.up) + t_off;
    p.q[mat][0] = load16(tile + 16 * lane);
    p.q[mat][1] = load16(tile + 1024 + 16 * lane);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
    p.s[mat][0] = sp[0];
    p.s[mat][1] = sp[1];
    p.s[mat][2] = sp[2];
    p.dd[mat] = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
  }
  p.ok = ok;
}

// Scaled sum of lane (g, n)'s four block dots (k-blocks 4g .. 4g+3, g < 2).
__device__ __forceinline__ float k4_scaled(const float4v& c, const uint32_t s[3], uint32_t dd, const float* xs, int g) {
  const float d = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kb = 4 * g + i;
    const float dsc = d * (float)k4_scale_value(s[0], s[1], s[2], kb);
    const float mn = dmin * (float)k4_scale_value(s[0], s[1], s[2], 8 + kb);
    v = fmaf(dsc, c[i], v);
    v = fmaf(-fmaf(1024.0f, dsc, mn), xs[kb], v);
  }
  return v;
}

template <int SF>
__global__ __launch_bounds__(1024) void dec1_k4_upgate_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, k = a.k, n_chunks = H / 256, n_kp = (n_chunks + 15) / 16;
  const int n_rt = a.I / 16, n_rts = a.Is / 16;
  _Float16* xs16 = reinterpret_cast<_Float16*>(smem);                      // [H] then a 16-byte zero block
  const int zero_off = 2 * H;
  float* xsum = reinterpret_cast<float*>(smem + zero_off + 16);            // [H / 32]
  float* red_r = xsum + H / 32;                                            // [kRedBatch][2][NW][32]
  float* red_s = red_r + kRedBatch * 2 * NW * 32;                          // [NW][2][8]
  uint32_t* xef = reinterpret_cast<uint32_t*>(red_s + NW * 2 * 8);         // [NW] largest x exponent field per wave

  // (32-bit products: gi * U_r <= 255 * 16 * 1024)
  const unsigned G = gridDim.x, gi = blockIdx.x;
  const unsigned U_s = 2 * n_rts, U_r = k * n_rt;
  const int s_lo = (int)(gi * U_s / G), s_hi = (int)((gi + 1) * U_s / G);
  const int r_lo = (int)(gi * U_r / G), r_hi = (int)((gi + 1) * U_r / G);
  const int n = lane & 15, g = lane >> 4, m = lane & 15, qq = lane >> 4;

  // routed units u = item * n_kp + kp, loaded kPrefetch3 ahead
  const int u_lo = r_lo * n_kp, u_hi = r_hi * n_kp;
  auto issue = [&](K4Pay& P, int u) {
    int e = -1, rt = 0, chunk = 0;
    if (u < u_hi) {
      const int item = u / n_kp, kp = u - item * n_kp;
      const int j = item / n_rt;
      rt = item - j * n_rt;
      chunk = kp * 16 + wave;
      e = expert_id(a.topk_idx, j);
      if (e >= a.E || chunk >= n_chunks) e = -1;
    }
    const bool ok = e >= 0;
    k4_pay_load(P, a, ok ? e : 0, ok ? rt : 0, ok ? chunk : 0, lane, n_chunks, ok);
  };
  K4Pay P0, P1;
  issue(P0, u_lo);
  issue(P1, u_lo + 1);

  // the token's exponent xe, then x 2^-xe -> LDS (fp16) and its 32-column
  // block sums
  {
    uint32_t ef = 0;
    for (int i = tid; i < H / 8; i += blockDim.x) ef = max(ef, bf16x8_max_efield(load16(a.x + 8 * i)));
    ef = wave_max_u32(ef);
    if (lane == 0) xef[wave] = ef;
  }
  if (tid == 0) *reinterpret_cast<u32x4*>(smem + zero_off) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  int xe;
  {
    uint32_t ef = 0;
    for (int w = 0; w < NW; ++w) ef = max(ef, xef[w]);
    xe = x_exp_of_field(ef);
  }
  if (blockIdx.x == 0 && tid == 0) a.xexp[0] = xe;
  for (int i = tid; i < H / 8; i += blockDim.x)
    *reinterpret_cast<u32x4*>(xs16 + 8 * i) = as_u32x4(bf16x8_to_half8_exp(load16(a.x + 8 * i), xe));
  __syncthreads();
  for (int b = tid; b < H / 32; b += blockDim.x) {
    float v = 0.f;
    for (int j = 0; j < 32; ++j) v += (float)xs16[32 * b + j];
    xsum[b] = v;
  }
  __syncthreads();

  // A of k-block kb for chunk c: row kb = x block kb (lanes m == kb), else 0
  auto a_kb = [&](int c, int kb) {
    const int off = (m == kb) ? c * 512 + kb * 64 + qq * 16 : zero_off;
    return *reinterpret_cast<const half8*>(smem + off);
  };
  // A of k-block pair p (rows 2p and 2p+1) for the shared half tiles
  auto a_pair = [&](int c, int p) {
    const int off = (m < 8 && (m >> 1) == p) ? c * 512 + m * 64 + qq * 16 : zero_off;
    return *reinterpret_cast<const half8*>(smem + off);
  };
  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  // ---- shared expert half tiles, K-part by K-part
  for (int su = s_lo; su < s_hi; ++su) {
    const int rt = su >> 1, hr = su & 1;
    const int r = 8 * hr + (n & 7);
    float v[2] = {0.f, 0.f};
    for (int kp = 0; kp < n_kp; ++kp) {
      const int chunk = kp * 16 + wave;
      if (chunk >= n_chunks) continue;
      ShHalf sraw[2];
      for (int mat = 0; mat < 2; ++mat) {
        const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)rt * n_chunks + chunk) * shared_tile_bytes<SF>();
        sh_half_load<SF>(sraw[mat], [&](int off) { return load16(tile + off); }, n, qq, r);
      }
      half8 Ap[4];
      for (int p = 0; p < 4; ++p) Ap[p] = a_pair(chunk, p);
      for (int mat = 0; mat < 2; ++mat) {
        float t = sh_half_dot<SF>(sraw[mat], [&](int p) { return Ap[p]; }, n, g);
        t += __shfl_xor(t, 8);
        t += __shfl_xor(t, 16);
        v[mat] += t;
      }
    }
    if (lane < 8) {
      red_s[(wave * 2 + 0) * 8 + lane] = v[0];
      red_s[(wave * 2 + 1) * 8 + lane] = v[1];
    }
    __syncthreads();
    if (tid < 8) {
      float u = 0.f, gg = 0.f;
      for (int w = 0; w < NW; ++w) {
        u += red_s[(w * 2 + 0) * 8 + tid];
        gg += red_s[(w * 2 + 1) * 8 + tid];
      }
      a.hs[rt * 16 + 8 * hr + tid] = h_of(gg, u, xe, xe);
    }
    __syncthreads();
  }

  // ---- routed units
  auto compute = [&](const K4Pay& P, int u, int b) {
    const int item = u / n_kp, kp = u - item * n_kp;
    const int chunk = min(kp * 16 + wave, n_chunks - 1);
    float4v cu = zero, cg = zero;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const half8 av = a_kb(chunk, kb);
      cu = mfma_f16(av, as_half8(k4_magic(P.q[0][kb >> 2][kb & 3])), cu);
      cg = mfma_f16(av, as_half8(k4_magic(P.q[1][kb >> 2][kb & 3])), cg);
    }
    if (lane < 32) {
      const float* xs = xsum + chunk * 8;
      const float vu = P.ok ? k4_scaled(cu, P.s[0], P.dd[0], xs, g) : 0.f;
      const float vg = P.ok ? k4_scaled(cg, P.s[1], P.dd[1], xs, g) : 0.f;
      float* ru = &red_r[((b * 2 + 0) * NW + wave) * 32 + lane];
      float* rg = &red_r[((b * 2 + 1) * NW + wave) * 32 + lane];
      if (kp == 0) {
        *ru = vu;
        *rg = vg;
      } else {
        *ru += vu;
        *rg += vg;
      }
    }
  };
  auto flush = [&](int first, int nb) {
    __syncthreads();
    if (tid < nb * 16) {
      const int b = tid >> 4, item = first + b;
      float u = 0.f, gg = 0.f;
      for (int w = 0; w < NW; ++w) {
        u += red_r[((b * 2 + 0) * NW + w) * 32 + n];
        u += red_r[((b * 2 + 0) * NW + w) * 32 + 16 + n];
        gg += red_r[((b * 2 + 1) * NW + w) * 32 + n];
        gg += red_r[((b * 2 + 1) * NW + w) * 32 + 16 + n];
      }
      const _Float16 h16 = h_of(gg, u, xe, xe);
      const float hv = (float)h16;
      const int j = item / n_rt, rt = item - j * n_rt;
      a.h[(size_t)j * a.I + rt * 16 + n] = h16;
      const int kk = (rt * 16 + n) & 255;
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
    __syncthreads();
  };
  // every wave writes its reduction slot (zeros when idle), so the flush can
  // sum all NW waves
  int nb = 0, first = r_lo;
  auto done_unit = [&](int u) {
    const int item = u / n_kp, kp = u - item * n_kp;
    if (kp + 1 < n_kp) return;
    if (++nb == kRedBatch || item + 1 == r_hi) {
      flush(first, nb);
      first = item + 1;
      nb = 0;
    }
  };
  for (int u = u_lo; u < u_hi; u += 2) {
    compute(P0, u, nb);
    issue(P0, u + 2);
    done_unit(u);
    if (u + 1 >= u_hi) break;
    compute(P1, u + 1, nb);
    issue(P1, u + 3);
    done_unit(u + 1);
  }
}

size_t dec1_k4_upgate_lds(int H, int nw) {
  return (size_t)2 * H + 16 + (size_t)(H / 32) * 4 + (size_t)kRedBatch * 2 * nw * 32 * 4 + (size_t)nw * 2 * 8 * 4 +
         (size_t)nw * 4;
}

// ---------------------------------------------------------------------------
// Per-wave payload of one routed K4 down unit (one K-chunk of one 16-row tile).
struct DnPay4 {
  u32x4 q0, q1;
  uint32_t s0, s1, s2, dd;
};

__device__ __forceinline__ void dn_load4(DnPay4& p, __amdgpu_buffer_rsrc_t tile, int lane) {
  const int n = lane & 15;
  p.q0 = bload16(tile, 16 * lane);
  p.q1 = bload16(tile, 1024 + 16 * lane);
  p.s0 = bload4(tile, 2048 + 12 * n);
  p.s1 = bload4(tile, 2048 + 12 * n + 4);
  p.s2 = bload4(tile, 2048 + 12 * n + 8);
  p.dd = bload4(tile, 2240 + 4 * n);
}

// K4 down + shared down + combine, activations staged in LDS.  Workgroup = one 16-row tile of y; the k
// routed down matrices and the shared one form one stacked GEMV over
// K = k*I + I_s, split over the waves in units of one 256-column K-chunk
// (routed) or half a chunk (shared).  Every wave issues the loads of all its
// units before the activations are staged, so HBM latency overlaps staging.
constexpr int kDnUnits = 4;    // routed units held in registers per wave
constexpr int kStageVec = 6;   // staged 16-byte vectors per thread per pass

template <int SF>
__global__ __launch_bounds__(1024) void dec1_k4_down_kernel(DecArgs a, const float* topk_w, float* y) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = a.k, I = a.I, I_pad = a.I_pad, Is = a.Is, Is_pad = a.Is_pad;
  const int n_ck = I_pad / 256, n_cks = Is > 0 ? Is_pad / 256 : 0;
  // LDS: staged activations (fp16), per-16-row sums, reduction
  _Float16* hst = reinterpret_cast<_Float16*>(smem);                        // [k][I_pad]
  _Float16* hss = hst + (size_t)k * I_pad;                                    // [Is_pad]
  size_t off = ((size_t)k * I_pad + Is_pad) * 2;
  off = (off + 15) & ~size_t(15);
  uint8_t* zero16 = smem + off;                                               // 16 zero bytes
  off += 16;
  float* xo = reinterpret_cast<float*>(smem + off);                           // [k][I_pad/16][2]
  off += (size_t)k * (I_pad / 16) * 2 * 4;
  float* red = reinterpret_cast<float*>(smem + off);                          // [NW][16]

  const int rt = blockIdx.x;
  const int n = lane & 15, g4 = lane >> 4, m = lane & 15;
  const int n_units = k * n_ck, n_sunits = 2 * n_cks;
  const size_t tb = kK4Tile;

  // ---- loads, oldest first: the first pass of the staged activations, the
  // shared unit, then the routed units wave + NW*i.  A wave's loads complete
  // in issue order, so the staging waits only for the activations, not
  // behind weight tiles.
  DnPay4 P[kDnUnits];
  int uj[kDnUnits], ukc[kDnUnits], ue[kDnUnits];
  // (units past the end or naming an invalid expert load zeros, no memory)
  auto issue_round = [&](int base) {
    for (int i = 0; i < kDnUnits; ++i) {
      const int u = base + wave + NW * i;
      const int j = u / n_ck;
      uj[i] = j;
      ukc[i] = u - j * n_ck;
      const int e = u < n_units ? expert_id(a.topk_idx, j) : -1;
      ue[i] = (e >= 0 && e < a.E) ? e : -1;
      const uint8_t* tile = ue[i] >= 0 ? a.down + (size_t)e * a.expert_bytes_down + ((size_t)rt * n_ck + ukc[i]) * tb
                                       : a.down;
      dn_load4(P[i], tile_rsrc(tile, ue[i] >= 0 ? (int)tb : 0), lane);
    }
  };
  constexpr int kSTile = shared_tile_bytes<SF>();
  ShQuarter sraw;
  int s_kc = -1, s_kb0 = 0;
  auto issue_shared = [&](int su) {
    const bool valid = su < n_sunits;
    s_kc = valid ? su >> 1 : -1;
    s_kb0 = 4 * (su & 1);
    const uint8_t* tile = valid ? a.sdown + ((size_t)rt * n_cks + s_kc) * kSTile : a.down;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile, valid ? kSTile : 0);
    sh_dn_load<SF>(sraw, [&](int off) { return bload16(rs, off); }, s_kb0, lane);
  };

  // ---- staging of the activations: h vectors, per-16-row sums, shared h
  const int cvp = I_pad / 8, cv = I / 8;              // 8-column vectors per slot row
  const int nrp = I_pad / 16, nr = I / 16;            // 16-row sums per slot row
  const int n_hv = k * cvp, n_xv = k * (nrp / 2), n_sv = Is_pad / 8;
  const int n_stage = n_hv + n_xv + n_sv, pass = kStageVec * (int)blockDim.x;
  // One buffer descriptor spans h, hs and hsum (consecutive in the
  // workspace, h first): a lane with nothing to stage loads past its end and
  // gets zeros, so the staging loads need no branch (a load inside a branch
  // makes the compiler wait for every earlier load where the paths join).
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(a.h);
  const int off_hs = (int)(reinterpret_cast<const uint8_t*>(a.hs) - hb);
  const int off_xs = (int)(reinterpret_cast<const uint8_t*>(a.hsum) - hb);
  const __amdgpu_buffer_rsrc_t hrs = tile_rsrc(hb, off_xs + k * nrp * 2 * 4);
  // Offsets and destinations first, then the loads as one straight run.
  // dst: LDS byte offset | 0x10000000 for a sum pair whose second half lies
  // past the end; -1 = nothing.
  auto stage_load = [&](int base, u32x4 (&v)[kStageVec], int (&dst)[kStageVec]) {
    const int nrh = nrp / 2;
    int off[kStageVec];
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const int id = base + tid + i * (int)blockDim.x;
      const bool k0 = id < n_hv, k1 = !k0 && id < n_hv + n_xv, k2 = !k0 && !k1 && id < n_stage;
      const int q = k0 ? id : (k1 ? id - n_hv : id - n_hv - n_xv);
      const int per = k0 ? cvp : nrh;
      const int j = q / per, c = q - j * per;           // kinds 0, 1
      int o = 0x7FFFFFF0;                               // past the end: zeros
      if (k0 && c < cv) o = (j * I + 8 * c) * 2;
      if (k1 && 2 * c < nr) o = off_xs + (j * nrp + 2 * c) * 8;
      if (k2 && q < Is / 8) o = off_hs + 16 * q;
      off[i] = o;
      int d = -1;
      if (k0) {
        d = (j * I_pad + 8 * c) * 2;
      } else if (k1) {
        d = (int)((uint8_t*)(xo + ((size_t)j * nrp + 2 * c) * 2) - smem);
        if (2 * c + 1 >= nr) d |= 0x10000000;
      } else if (k2) {
        d = (int)((uint8_t*)(hss + 8 * q) - smem);
      }
      dst[i] = d;
    }
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) v[i] = bload16(hrs, off[i]);
  };
  auto stage_store = [&](const u32x4 (&v)[kStageVec], const int (&dst)[kStageVec]) {
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      if (dst[i] < 0) continue;
      u32x4 w = v[i];
      if (dst[i] & 0x10000000) w = u32x4{w.x, w.y, 0u, 0u};      // odd tail: one sum pair
      *reinterpret_cast<u32x4*>(smem + (dst[i] & 0x0FFFFFFF)) = w;
    }
  };
  // all passes but the last before any weight load (a loop around loads
  // makes the compiler's later waits conservative); the last pass's stores
  // wait only for its own loads
  const int n_pass = (n_stage + pass - 1) / pass;
  for (int ps = 0; ps + 1 < n_pass; ++ps) {
    u32x4 v[kStageVec];
    int dst[kStageVec];
    stage_load(ps * pass, v, dst);
    stage_store(v, dst);
  }
  {
    u32x4 v[kStageVec];
    int dst[kStageVec];
    stage_load((n_pass - 1) * pass, v, dst);
    issue_shared(wave);
    issue_round(0);
    stage_store(v, dst);
  }
  if (tid < 4) reinterpret_cast<uint32_t*>(zero16)[tid] = 0u;
  __syncthreads();

  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float acc = 0.f;
  // the first round is straight-line code, so each unit waits for its own
  // tile only (a loop around loads makes the compiler's waits conservative)
  auto compute_round = [&]() {
    for (int i = 0; i < kDnUnits; ++i) {
      if (ue[i] < 0) continue;
      const int j = uj[i], kc = ukc[i];
      const float wgt = choice_weight(topk_w, j);
      const DnPay4& p = P[i];
      const _Float16* hbase = hst + (size_t)j * I_pad + kc * 256 + g4 * 8;
      const float d = h2f(p.dd & 0xFFFFu), dmin = h2f(p.dd >> 16);
      float part = 0.f;
      for (int kb = 0; kb < 8; ++kb) {
        const uint8_t* src = (m == 0) ? reinterpret_cast<const uint8_t*>(hbase + kb * 32) : zero16;
        const uint32_t w = kb < 4 ? p.q0[kb & 3] : p.q1[kb & 3];
        const float4v c = mfma_f16(as_half8(load16(src)), as_half8(k4_magic(w)), zero);
        const float dsc = d * (float)k4_scale_value(p.s0, p.s1, p.s2, kb);
        const float corr = 1024.0f * dsc + dmin * (float)k4_scale_value(p.s0, p.s1, p.s2, 8 + kb);
        const float* xk = xo + ((size_t)j * (I_pad / 16) + kc * 16 + 2 * kb) * 2;
        part += dsc * c[0] - corr * (xk[0] + xk[2]);
      }
      if (g4 == 0) acc += wgt * part;
    }
  };
  compute_round();
  for (int base = kDnUnits * NW; base < n_units; base += kDnUnits * NW) {
    issue_round(base);
    compute_round();
  }
  // shared expert: units of half a K-chunk (4 k-blocks)
  for (int su = wave; su < n_sunits; su += NW) {
    if (su != wave) issue_shared(su);
    float4v c = zero;
    const _Float16* hbase = hss + s_kc * 256 + g4 * 8;
    for (int q = 0; q < 4; ++q) {
      // BF16: every k-block's activations in A row 0; Q8: k-block kb0 + q's in row q
      const bool feeds_q = m == (SF == MOE_FMT_Q8 ? q : 0);
      const uint8_t* src = feeds_q ? reinterpret_cast<const uint8_t*>(hbase + (s_kb0 + q) * 32) : zero16;
      c = mfma_f16(as_half8(load16(src)), sh_dn_b<SF>(sraw, q), c);
    }
    acc += sh_dn_sum<SF>(sraw, c, s_kb0);
  }
  // sum the 4 lanes of each output row, then the waves in order
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (tid < 16) {
    float s = 0.f;
    for (int w = 0; w < NW; ++w) s += red[w * 16 + tid];
    y[rt * 16 + tid] = __builtin_ldexpf(s, 2 * token_exp(a.xexp));     // h was stored times 2^-2e
  }
}

// K2 down + shared down + combine, with no staging: each unit's slice of h
// and its per-16-row sums are loaded beside its weight tile (the loads
// complete together), so a unit is computed as soon as its own bytes are
// in and compute overlaps the weight stream; only the final cross-wave sum
// waits for every wave.  Workgroup and units as in dec1_k4_down_kernel.
struct DnDirect {
  u32x4 q;            // the lane's 16 bytes of codes
  uint32_t scm, dd;   // sub-block scales/mins of row n, fp16 d | dmin << 16
  u32x4 hv;           // the lane's 8 h values (lanes that feed k-block m/2), else 0
  float xo;           // lane l < 32: value l of the chunk's 16 (X, O) pairs, else 0
};

template <int SF>
__global__ __launch_bounds__(1024) void dec1_down_k2d_kernel(DecArgs a, const float* topk_w, float* y) {
  extern __shared__ __align__(16) uint8_t smem[];
  float* red = reinterpret_cast<float*>(smem);                              // [NW][16]
  const int tid = threadIdx.x, lane = tid & 63, NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = a.k, I = a.I, I_pad = a.I_pad, Is = a.Is;
  const int n_ck = I_pad / 256, n_cks = Is > 0 ? a.Is_pad / 256 : 0;
  const int nrp = I_pad / 16, nr = I / 16;
  const int rt = blockIdx.x;
  const int n = lane & 15, g4 = lane >> 4, m = lane & 15;
  const int n_units = k * n_ck, n_sunits = 2 * n_cks;
  const bool feeds = (m & 1) == (g4 >> 1);             // row 2 kb + g4/2 of A_kb is sub-block m
  const int kb_act = m >> 1;

  // one descriptor over h, hs and hsum (consecutive in the workspace, h
  // first); loads past its end give zeros and touch no memory
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(a.h);
  const int off_hs = (int)(reinterpret_cast<const uint8_t*>(a.hs) - hb);
  const int off_xs = (int)(reinterpret_cast<const uint8_t*>(a.hsum) - hb);
  const __amdgpu_buffer_rsrc_t hrs = tile_rsrc(hb, off_xs + k * nrp * 2 * 4);
  constexpr int kPast = 0x7FFFFFF0;

  DnDirect P[kDnUnits];
  int uj[kDnUnits], ukc[kDnUnits], ue[kDnUnits];
  auto issue_round = [&](int base) {
    for (int i = 0; i < kDnUnits; ++i) {
      const int u = base + wave + NW * i;
      const int j = u / n_ck, kc = u - j * n_ck;
      uj[i] = j;
      ukc[i] = kc;
      const int e = u < n_units ? expert_id(a.topk_idx, j) : -1;
      ue[i] = (e >= 0 && e < a.E) ? e : -1;
      const bool ok = ue[i] >= 0;
      const uint8_t* tile = ok ? a.down + (size_t)e * a.expert_bytes_down + ((size_t)rt * n_ck + kc) * kK2Tile
                               : a.down;
      const __amdgpu_buffer_rsrc_t tr = tile_rsrc(tile, ok ? kK2Tile : 0);
      P[i].q = bload16(tr, 16 * lane);
      P[i].scm = bload4(tr, 1024 + 16 * n + 4 * g4);
      P[i].dd = bload4(tr, 1280 + 4 * n);
      const int col = kc * 256 + kb_act * 32 + g4 * 8;
      P[i].hv = bload16(hrs, (ok && feeds && col < I) ? (j * I + col) * 2 : kPast);
      // sums past the matrix's last row are read as zero
      const int sbl = kc * 16 + (lane >> 1);
      P[i].xo = __builtin_bit_cast(float, bload4(hrs, (ok && lane < 32 && sbl < nr)
                                                          ? off_xs + (j * nrp + kc * 16) * 8 + 4 * lane
                                                          : kPast));
    }
  };
  // shared unit: half a K-chunk (4 k-blocks).  BF16: lanes m == 0 take
  // their four 8-column pieces of hs (A row 0 for every k-block); Q8: lanes
  // m < 4 take the piece of k-block kb0 + m (A row m for k-block kb0 + m).
  constexpr int kSTile = shared_tile_bytes<SF>();
  constexpr int kShv = SF == MOE_FMT_Q8 ? 1 : 4;
  ShQuarter sraw;
  u32x4 shv[kShv];
  int s_kc = -1, s_kb0 = 0;
  auto issue_shared = [&](int su) {
    const bool valid = su < n_sunits;
    s_kc = valid ? su >> 1 : -1;
    s_kb0 = 4 * (su & 1);
    const uint8_t* tile = valid ? a.sdown + ((size_t)rt * n_cks + s_kc) * kSTile : a.down;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile, valid ? kSTile : 0);
    sh_dn_load<SF>(sraw, [&](int off) { return bload16(rs, off); }, s_kb0, lane);
    if constexpr (SF == MOE_FMT_Q8) {
      const int col = s_kc * 256 + (s_kb0 + (m & 3)) * 32 + g4 * 8;
      shv[0] = bload16(hrs, (valid && m < 4 && col < Is) ? off_hs + col * 2 : kPast);
    } else {
      for (int q = 0; q < 4; ++q) {
        const int col = s_kc * 256 + (s_kb0 + q) * 32 + g4 * 8;
        shv[q] = bload16(hrs, (valid && m == 0 && col < Is) ? off_hs + col * 2 : kPast);
      }
    }
  };
  issue_shared(wave);
  issue_round(0);

  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  float acc = 0.f;
  auto compute_round = [&]() {
    for (int i = 0; i < kDnUnits; ++i) {
      if (ue[i] < 0) continue;
      const int j = uj[i], kc = ukc[i];
      const DnDirect& p = P[i];
      // column pair s of an 8-column group sits at slot t(kb, s): h scaled by 4^-t
      const half8 f = (kb_act & 1)
                          ? half8{0.00390625f16, 0.00390625f16, 1.0f16, 1.0f16, 0.25f16, 0.25f16, 0.0625f16, 0.0625f16}
                          : half8{1.0f16, 1.0f16, 0.25f16, 0.25f16, 0.0625f16, 0.0625f16, 0.015625f16, 0.015625f16};
      const u32x4 hs8 = as_u32x4(as_half8(p.hv) * f);
      float4v c = zero;
      for (int kb = 0; kb < 8; ++kb) c = mfma_f16(as_half8(kb == kb_act ? hs8 : z4), as_half8(k2_magic(p.q, kb)), c);
      // C[4 g4 + q][n] = sub-block 4 g4 + q, whose (X, O) sit in lanes
      // 8 g4 + 2q and 8 g4 + 2q + 1
      float dsum = 0.f, msum = 0.f;
      for (int q = 0; q < 4; ++q) {
        const float xq = __shfl(p.xo, 8 * g4 + 2 * q), oq = __shfl(p.xo, 8 * g4 + 2 * q + 1);
        const uint32_t byte = (p.scm >> (8 * q)) & 0xFFu;
        dsum += (float)(byte & 15u) * (c[q] - oq);
        msum += (float)(byte >> 4) * xq;
      }
      const float wgt = choice_weight(topk_w, j);
      acc += (wgt * h2f(p.dd & 0xFFFFu)) * dsum - (wgt * h2f(p.dd >> 16)) * msum;
    }
  };
  compute_round();
  for (int base = kDnUnits * NW; base < n_units; base += kDnUnits * NW) {
    issue_round(base);
    compute_round();
  }
  for (int su = wave; su < n_sunits; su += NW) {
    if (su != wave) issue_shared(su);
    float4v c = zero;
    for (int q = 0; q < 4; ++q) {
      const u32x4 av = SF == MOE_FMT_Q8 ? (m == q ? shv[0] : z4) : (m == 0 ? shv[q % kShv] : z4);
      c = mfma_f16(as_half8(av), sh_dn_b<SF>(sraw, q), c);
    }
    acc += sh_dn_sum<SF>(sraw, c, s_kb0);
  }
  // sum the 4 lanes of each output row, then the waves in order
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (tid < 16) {
    float sum = 0.f;
    for (int w = 0; w < NW; ++w) sum += red[w * 16 + tid];
    y[rt * 16 + tid] = __builtin_ldexpf(sum, 2 * token_exp(a.xexp));   // h was stored times 2^-2e
  }
}

}  // namespace

namespace qmoe {

size_t dec1_cb2_wide_upgate_lds(int nw) { return 256 + 2 * kCb2TableBytes + (size_t)kBatch * nw * 2 * 16 * 4; }
static_assert(16 + 16 * 4 <= 256, "range and exponent fields fit the first 256 bytes");

size_t dec1_down_lds(const DecArgs& a, int fmt_dn, int nw) {
  if (fmt_dn == MOE_FMT_K2) return (size_t)nw * 16 * 4;  // direct loads: the reduction only
  size_t off = ((size_t)a.k * a.I_pad + a.Is_pad) * 2;
  off = (off + 15) & ~size_t(15);
  off += 16 + (size_t)a.k * (a.I_pad / 16) * 2 * 4;
  return off + (size_t)nw * 16 * 4;
}

size_t dec1_cb2_upgate_lds(int nw, bool route) {
  return (size_t)kCb2CombBytes + (size_t)kRedBatch * 2 * nw * 32 * 4 + (size_t)nw * 2 * 8 * 4 +
         (size_t)nw * 4 + (route ? 16 * 4 + sizeof(qmoe_route::TopkLds) : 0);
}

template <int SF>
static hipError_t launch_dec1_sf(const DecArgs& a, int fmt_ug, int fmt_dn, const float* topk_w, float* y,
                                 int cus, hipStream_t s) {
  hipError_t err;
  const int n_chunks = a.H / 256;
  if (fmt_ug == MOE_FMT_K4) {
    const int nw = n_chunks < 4 ? 4 : (n_chunks > 16 ? 16 : n_chunks);
    const int U_s = 2 * (a.Is / 16), U_r = a.k * (a.I / 16);
    const int most = U_s > U_r ? U_s : U_r;
    const int grid = most < cus ? most : cus;
    err = ensure_dyn_lds((const void*)dec1_k4_upgate_kernel<SF>);
    if (err != hipSuccess) return err;
    const size_t lds = dec1_k4_upgate_lds(a.H, nw);
    err = launch_timed(MOE_KERNEL_DECODE_UPGATE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
      hipExtLaunchKernelGGL(dec1_k4_upgate_kernel<SF>, dim3(grid), dim3(64 * nw), lds, s, ev0_, ev1_, 0, a);
    });
  } else if (fmt_ug == MOE_FMT_CB2 && n_chunks <= 16) {
    const int nw = n_chunks < 4 ? 4 : n_chunks;
    const int U_s = 2 * (a.Is / 16), U_r = a.k * (a.I / 16);
    const int most = U_s > U_r ? U_s : U_r;
    const int grid = most < cus ? most : cus;
    const bool route = a.logits != nullptr;
    void (*fk)(DecArgs) = route ? dec1_cb2_upgate_kernel<true, SF> : dec1_cb2_upgate_kernel<false, SF>;
    err = ensure_dyn_lds((const void*)fk);
    if (err != hipSuccess) return err;
    const size_t lds = dec1_cb2_upgate_lds(nw, route);
    err = launch_timed(MOE_KERNEL_DECODE_UPGATE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
      hipExtLaunchKernelGGL(fk, dim3(grid), dim3(64 * nw), lds, s, ev0_, ev1_, 0, a);
    });
  } else {
    // CB2 with 17 to 32 K-chunks (K4 layers take dec1_k4_upgate_kernel at every H)
    if (fmt_ug != MOE_FMT_CB2 || n_chunks > 16 * kCpw) return hipErrorInvalidValue;
    const int nw_ug = (n_chunks + kCpw - 1) / kCpw;
    const int64_t items = (int64_t)a.k * (a.I / 16) + a.Is / 16;
    const int grid_ug = (int)(items < cus ? items : cus);
    err = ensure_dyn_lds((const void*)dec1_cb2_wide_upgate_kernel<SF>);
    if (err != hipSuccess) return err;
    const size_t lds_ug = dec1_cb2_wide_upgate_lds(nw_ug);
    err = launch_timed(MOE_KERNEL_DECODE_UPGATE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
      hipExtLaunchKernelGGL(dec1_cb2_wide_upgate_kernel<SF>, dim3(grid_ug), dim3(64 * nw_ug), lds_ug, s, ev0_, ev1_, 0, a);
    });
  }
  if (err != hipSuccess) return err;
  // one workgroup per 16-row tile of y: 16 waves while the tiles fit the
  // compute units in one round, else 8 so that two workgroups share a CU and
  // the tiles run in a single round (H = 7168: 26.6 us instead of 33.3 us)
  const int nw_dn = a.H / 16 > cus ? 8 : 16;
  void (*fd)(DecArgs, const float*, float*) = fmt_dn == MOE_FMT_K2 ? dec1_down_k2d_kernel<SF> : dec1_k4_down_kernel<SF>;
  err = ensure_dyn_lds((const void*)fd);
  if (err != hipSuccess) return err;
  const size_t lds_dn = dec1_down_lds(a, fmt_dn, nw_dn);
  return launch_timed(MOE_KERNEL_DECODE_DOWN, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(fd, dim3(a.H / 16), dim3(64 * nw_dn), lds_dn, s, ev0_, ev1_, 0, a, topk_w, y);
  });
}

hipError_t launch_dec1(const DecArgs& a, int fmt_ug, int fmt_dn, const float* topk_w, float* y,
                       int cus, hipStream_t s) {
  return a.fmt_s == MOE_FMT_Q8 ? launch_dec1_sf<MOE_FMT_Q8>(a, fmt_ug, fmt_dn, topk_w, y, cus, s)
                               : launch_dec1_sf<MOE_FMT_BF16>(a, fmt_ug, fmt_dn, topk_w, y, cus, s);
}

}  // namespace qmoe
