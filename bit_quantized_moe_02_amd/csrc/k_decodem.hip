// Batched decode (2..16 tokens, e.g. draft verification), CB2 up/gate and K2
// down, H <= 4096:
//   decm_upgate: h_{t,j} = SiLU(Wg_e x_t) * (Wu_e x_t) for every choice (t, j)
//                of the batch and h_s,t for the shared expert;
//   decm_down:   y_{t,j} = Wd_e h_{t,j} and the shared expert's down;
//   decm_combine: y_t = sum_j w_{t,j} y_{t,j} + y_s,t in j order.
//
// Work items are (distinct expert, 16-row tile) -- its token set is the
// bitmask of tokens that chose the expert -- plus the shared expert's row
// tiles; items are split over the grid by the bytes they stream.  All tokens
// of the batch sit in the 16 MFMA rows (v_mfma_f32_16x16x32_f16), so one
// dequantized weight tile serves every token and the rows of tokens that did
// not choose the expert are computed and dropped.  K is split over the waves
// of a workgroup (one 256-column chunk each) and the partial sums meet in LDS
// in wave order (fixed order, no atomics); the next item's weights are in
// flight while the current one is multiplied.  CB2 up/gate weights become
// fp16 B operands with their scales folded in (one fp16 rounding per
// weight), as in the prefill kernels.  K2 down weights stay exact: the B
// operands are the integers q * sc, and per item and chunk the result is
// d * (h . q sc) - dmin * (sum over sub-blocks of m * X), X being the
// sub-block sums of the staged h rows (as fp16 hi + lo).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmoe.h"
#include "decode_common.hpp"
#include "device_common.hpp"
#include "k_decode.h"
#include "launch_util.h"

using namespace qmoe_dev;
using namespace qmoe_dec;
using qmoe::DecArgs;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

constexpr int kMRB = 2;      // items per cross-wave reduction (up/gate)

// Weight loads of the next items are issued on every path, also past a
// workgroup's last item, so that the compiler can count the loads issued
// after each payload and wait for that payload alone (a vector wait is a
// count of loads still in flight, and a load issued on one path only makes
// every later use wait for all of them).  A payload past the last item reads
// through a descriptor of 0 bytes: its loads return zeros and touch no
// memory.  base must be wave-uniform; word 3 is the untyped-dword setting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 wt_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t wt_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ float4v mfma_bf16(const u32x4& a, const u32x4& b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}

// CB2 group for k-block kb with its fp16 scale folded in.
__device__ __forceinline__ half8 cb2_scaled_b(const u32x4& codes, const u32x4& scl, int kb, const uint8_t* tab) {
  const half8 v = cb2_comb(codes[kb >> 1], kb & 1, lds_offset(tab));
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu));
  return v * s;
}

// K2 B operand of lane (qq, n) for k-block kb as the exact integers q * sc
// (sc = the 4-bit scale of the lane's sub-block 2 kb + qq/2): the magic value
// 1024 * 4^t + q * 4^t times sc * 4^-t, minus 1024 * sc * 4^-t, in one fp16
// fma whose exact result is an integer <= 45.
__device__ __forceinline__ half8 k2_qsc_b(const u32x4& qw, const u32x4& scm, int kb, int qq) {
  const half8 mg = as_half8(k2_magic(qw, kb));
  const int sb = 2 * kb + (qq >> 1);
  const _Float16 sc = (_Float16)(float)((scm[sb >> 2] >> (8 * (sb & 3))) & 15u);
  // per slot pair: a = sc * 4^-t, b = -1024 a (packed two slots at a time)
  half2v a[2], b[2];
  for (int p = 0; p < 2; ++p) {
    const half2v pw = {(_Float16)__builtin_ldexpf(1.0f, -2 * k2_slot_t(kb, 2 * p)),
                       (_Float16)__builtin_ldexpf(1.0f, -2 * k2_slot_t(kb, 2 * p + 1))};
    a[p] = half2v{sc, sc} * pw;
    b[p] = a[p] * half2v{(_Float16)(-1024.0f), (_Float16)(-1024.0f)};
  }
  half8 w;
  for (int s = 0; s < 4; ++s) {
    const half2v as = {a[s >> 1][s & 1], a[s >> 1][s & 1]}, bs = {b[s >> 1][s & 1], b[s >> 1][s & 1]};
    const half2v r = half2v{mg[2 * s], mg[2 * s + 1]} * as + bs;
    w[2 * s] = r[0];
    w[2 * s + 1] = r[1];
  }
  return w;
}

// Min-term B operand of a 16x16x16 MFMA over the 16 sub-blocks of a chunk:
// lane (g, n) holds the 4-bit mins m of sub-blocks 4g .. 4g+3 of row n.
__device__ __forceinline__ half4 k2_min_b(const u32x4& scm, int g) {
  const uint32_t w = scm[g];                       // bytes sc | m << 4 of sub-blocks 4g .. 4g+3
  const uint32_t lo = ((w >> 4) & 0xFu) | ((w >> 12) & 0xFu) << 16;
  const uint32_t hi = ((w >> 20) & 0xFu) | ((w >> 28) & 0xFu) << 16;
  const half2v off = {(_Float16)(-1024.0f), (_Float16)(-1024.0f)};
  const half2v m01 = __builtin_bit_cast(half2v, lo | 0x64006400u) + off;
  const half2v m23 = __builtin_bit_cast(half2v, hi | 0x64006400u) + off;
  return half4{m01[0], m01[1], m23[0], m23[1]};
}

// ---------------------------------------------------------------------------
// Up/gate.  Items: shared row tiles [0, n_rts), then (expert d, row tile rt).

struct UgPayM {
  u32x4 code[2], scl[2];     // up, gate: the lane's group codes, row n's scales (zeros past the last item)
};

template <int SF>
__global__ __launch_bounds__(1024) void decm_upgate_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* tab = smem;                                                      // CB2 table, LDS offset 0
  const int tid = threadIdx.x, lane = tid & 63, NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* red = reinterpret_cast<float*>(smem + kCb2CombBytes);             // [kMRB][NW][2][64][4]
  ExpertList* L = reinterpret_cast<ExpertList*>(red + kMRB * NW * 2 * 256);
  uint32_t* xef = reinterpret_cast<uint32_t*>(L + 1);                      // [NW][16] largest x exponent fields
  int* xe16 = reinterpret_cast<int*>(xef + NW * 16);                        // [16] exponent of token m

  const int T = a.T, k = a.k, n_chunks = a.H / 256, n_rt = a.I / 16, n_rts = a.Is / 16;
  const bool active = wave < n_chunks;        // idle waves (H < 1024) load chunk 0 and discard it
  const int chunk = active ? wave : 0;
  const int m = lane & 15, qq = lane >> 4, n = lane & 15;

  // x of all tokens: A rows m < T (bf16 -> fp16), and the codebook bytes
  u32x4 xr[8];
  for (int kb = 0; kb < 8; ++kb)
    xr[kb] = m < T ? load16(a.x + (size_t)m * a.H + chunk * 256 + kb * 32 + qq * 8) : u32x4{0u, 0u, 0u, 0u};
  int8_t cbv[4] = {0, 0, 0, 0};
  if (tid < 512)
    for (int i = 0; i < 4; ++i) cbv[i] = a.codebook[(tid >> 1) * 8 + 4 * (tid & 1) + i];

  build_expert_list(a.topk_idx, T * k, k, a.E, L);
  const int64_t n_r = (int64_t)L->n * n_rt;
  const int64_t w_r = (int64_t)2 * kCb2Tile * n_chunks, w_s = (int64_t)2 * a.tb_s * n_chunks;
  const int64_t lo = item_start(blockIdx.x, gridDim.x, n_rts, w_s, n_r, w_r);
  const int64_t hi = item_start(blockIdx.x + 1, gridDim.x, n_rts, w_s, n_r, w_r);

  // routed payload prefetch: item r = (d, rt)
  int64_t r_ld = max(lo, (int64_t)n_rts) - n_rts;
  int d_ld = (int)(r_ld / n_rt), rt_ld = (int)(r_ld - (int64_t)d_ld * n_rt);
  const int64_t r_end = hi - n_rts;
  auto issue = [&](UgPayM& P) {
    const bool ok = r_ld < r_end && active;
    const int e = ok ? __builtin_amdgcn_readfirstlane(L->expert[d_ld]) : 0;
    const int rt = ok ? rt_ld : 0;
    const size_t t_off = (size_t)e * a.expert_bytes + ((size_t)rt * n_chunks + chunk) * kCb2Tile;
    for (int mat = 0; mat < 2; ++mat) {
      const __amdgpu_buffer_rsrc_t rs = wt_rsrc((mat ? a.gate : a.up) + t_off, ok ? kCb2Tile : 0);
      P.code[mat] = wt_load16(rs, 16 * lane);
      P.scl[mat] = wt_load16(rs, 1024 + 16 * n);
    }
    ++r_ld;
    if (++rt_ld == n_rt) {
      rt_ld = 0;
      ++d_ld;
    }
  };
  UgPayM P0, P1, P2;
  issue(P0);
  {
    // each token's exponent: the wave's largest field of row m (the 4 lanes
    // qq of row m), combined over the waves after the next barrier (computed
    // only now: its wait for x must not come before the first weight loads)
    uint32_t ef = 0;
    for (int kb = 0; kb < 8; ++kb) ef = max(ef, bf16x8_max_efield(xr[kb]));
    if (!active) ef = 0;
    ef = max(ef, (uint32_t)__shfl_xor((int)ef, 16));
    ef = max(ef, (uint32_t)__shfl_xor((int)ef, 32));
    if (lane < 16) xef[wave * 16 + lane] = ef;
  }

  // CB2 table (the pair values staged in the reduction area)
  uint2* val4 = reinterpret_cast<uint2*>(red);
  if (tid < 512) val4[tid] = cb2_pair_values(cbv);
  for (int pr = tid + (int)blockDim.x; pr < 512; pr += blockDim.x) {
    int8_t v[4];
    for (int i = 0; i < 4; ++i) v[i] = a.codebook[(pr >> 1) * 8 + 4 * (pr & 1) + i];
    val4[pr] = cb2_pair_values(v);
  }
  __syncthreads();
  for (int i = tid; i < 512 * 16; i += blockDim.x) cb2_comb_put(tab, i, val4);
  int xe;                                                                   // exponent of this lane's row m
  {
    uint32_t ef = 0;
    for (int w = 0; w < NW; ++w) ef = max(ef, xef[w * 16 + m]);
    xe = x_exp_of_field(ef);
  }
  if (tid < 16) {
    xe16[tid] = xe;
    if (blockIdx.x == 0 && tid < T) a.xexp[tid] = xe;
  }
  __syncthreads();

  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  // cross-wave sums of a batch of items -> h (routed: every slot (t, j) whose
  // token chose the item's expert), h_s (shared)
  auto flush = [&](int64_t first, int nb) {
    __syncthreads();
    // (a 4-wave workgroup has 256 threads for nb * 256 outputs)
    for (int o = tid; o < nb * 256; o += blockDim.x) {
      const int b = o >> 8, mm = (o >> 4) & 15, nn = o & 15;
      const int cl = 16 * (mm >> 2) + nn, ci = mm & 3;
      float u = 0.f, g = 0.f;
      for (int w = 0; w < n_chunks; ++w) {
        u += red[(((b * NW + w) * 2 + 0) * 64 + cl) * 4 + ci];
        g += red[(((b * NW + w) * 2 + 1) * 64 + cl) * 4 + ci];
      }
      // (32-bit item arithmetic: fewer registers in this loop, whose
      // temporaries would otherwise push the weight loads in flight out of
      // their registers)
      const int item = (int)first + b;
      // (BF16 shared items took raw bf16 x; Q8 shared and routed ones x 2^-e)
      const _Float16 h16 = h_of(g, u, (SF == MOE_FMT_BF16 && item < n_rts) ? 0 : xe16[mm], xe16[mm]);
      if (mm < T) {
        if (item < n_rts) {
          a.hs[(size_t)mm * a.Is + item * 16 + nn] = h16;
        } else {
          const int r = item - n_rts;
          const int dd = r / n_rt, rt = r - dd * n_rt;
          const int e = L->expert[dd];
          if ((L->mask[dd] >> mm) & 1u)
            for (int j = 0; j < k; ++j)
              if (L->slot_e[mm * k + j] == e) a.h[(size_t)(mm * k + j) * a.I + rt * 16 + nn] = h16;
        }
      }
    }
    __syncthreads();
  };

  int nb = 0;
  int64_t first = lo;
  auto done_item = [&](int64_t item, const float4v& cu, const float4v& cg) {
    if (active) {
      *reinterpret_cast<float4v*>(red + (((nb * NW + wave) * 2 + 0) * 64 + lane) * 4) = cu;
      *reinterpret_cast<float4v*>(red + (((nb * NW + wave) * 2 + 1) * 64 + lane) * 4) = cg;
    }
    if (++nb == kMRB || item + 1 == hi) {
      flush(first, nb);
      first = item + 1;
      nb = 0;
    }
  };

  half8 A[8];
  auto make_a = [&]() {
    for (int kb = 0; kb < 8; ++kb) A[kb] = active ? bf16x8_to_half8_exp(xr[kb], xe) : as_half8(u32x4{0u, 0u, 0u, 0u});
  };
  if constexpr (SF == MOE_FMT_Q8) make_a();
  // shared row tiles, one matrix at a time.  BF16: x (bf16) x bf16 weights
  // on bf16 matrix cores.  Q8: x 2^-e (fp16) x the exact codes, each
  // k-block's dots times row n's scale in fp32.
  const int64_t s_hi = min(hi, (int64_t)n_rts);
  for (int64_t item = lo; item < s_hi; ++item) {
    float4v c[2] = {zero, zero};
    for (int mat = 0; mat < 2; ++mat) {
      if constexpr (SF == MOE_FMT_Q8) {
        const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)item * n_chunks + chunk) * kQ8Tile;
        u32x4 raw[4];
        for (int i = 0; i < 4; ++i) raw[i] = load16(tile + 1024 * i + 16 * lane);
        const u32x4 scl = load16(tile + q8_scale_off(n));
        for (int kb = 0; kb < 8; ++kb) {
          const u32x4 pc = raw[2 * (kb & 1) + (kb >> 2)];
          const half8 b = ((kb >> 1) & 1) ? q8_codes(pc.z, pc.w) : q8_codes(pc.x, pc.y);
          const float4v ct = mfma_f16(A[kb], b, zero);
          c[mat] += h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu) * ct;
        }
      } else {
        const uint8_t* tile = (mat ? a.sgate : a.sup) + ((size_t)item * n_chunks + chunk) * kBf16Tile;
        u32x4 raw[8];
        for (int kb = 0; kb < 8; ++kb) raw[kb] = load16(tile + 1024 * kb + 16 * lane);
        for (int kb = 0; kb < 8; ++kb) c[mat] = mfma_bf16(active ? xr[kb] : u32x4{0u, 0u, 0u, 0u}, raw[kb], c[mat]);
      }
    }
    done_item(item, c[0], c[1]);
  }
  // routed items, the next two items' weights in flight
  if constexpr (SF != MOE_FMT_Q8) make_a();
  // (every payload is used on every path, also an idle wave's: a payload
  // whose loads some path never waits for makes the compiler wait for all
  // loads in flight before its registers are reused)
  auto compute = [&](const UgPayM& P, int64_t item) {
    float4v cu = zero, cg = zero;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      cu = mfma_f16(A[kb], cb2_scaled_b(P.code[0], P.scl[0], kb, tab), cu);
      cg = mfma_f16(A[kb], cb2_scaled_b(P.code[1], P.scl[1], kb, tab), cg);
    }
    done_item(item, cu, cg);
  };
  const int64_t r0 = max(lo, (int64_t)n_rts);
  issue(P1);
  for (int64_t item = r0; item < hi; item += 3) {
    issue(P2);
    compute(P0, item);
    if (item + 1 >= hi) break;
    issue(P0);
    compute(P1, item + 1);
    if (item + 2 >= hi) break;
    issue(P1);
    compute(P2, item + 2);
  }
}

// ---------------------------------------------------------------------------
// Down.  Items: shared row tiles of H [0, n_rts), then (expert d, row tile of
// H).  A = the 16 token rows of h for the current expert (or of h_s), staged
// in LDS as fp16 when the workgroup reaches a new expert.

// Down: a round is up to kDnR consecutive row tiles of one expert (or one
// shared row tile).  Wave w owns K chunk w; its slice of the staged A rows
// stays in registers for the whole expert, the next two rounds' weights are
// in flight while the current one computes, and the waves' partial sums are
// reduced once per round.
constexpr int kDnR = 4;
constexpr int kStageLoads = 8;   // h loads per thread in flight while a workgroup stages an expert's rows

struct DnRound {
  u32x4 q[kDnR], scm[kDnR];
  uint32_t dd[kDnR];
};

template <int SF>
__global__ __launch_bounds__(512) void decm_down_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, k = a.k;
  const int n_ck = a.I_pad / 256, n_cks = a.Is > 0 ? a.Is_pad / 256 : 0;
  const int kmax = max(a.I_pad, a.Is_pad);                                  // staged columns
  _Float16* hA = reinterpret_cast<_Float16*>(smem);                           // [16][kmax]
  float* red = reinterpret_cast<float*>(smem + (size_t)16 * kmax * 2);       // [kDnR][NW][64][4]
  ExpertList* L = reinterpret_cast<ExpertList*>(red + kDnR * NW * 256);
  int* slot_of = reinterpret_cast<int*>(L + 1);                              // [16] slot of token m (or -1)
  uint32_t* slot_bits = reinterpret_cast<uint32_t*>(slot_of + 16);           // [16] choices j of token m
  // (an offset from smem, 16-byte aligned: a pointer rounded through an
  // integer would lose its LDS address space, and its reads would become
  // flat loads that wait for every weight load in flight)
  const size_t xsb_off = ((size_t)(reinterpret_cast<uint8_t*>(slot_bits + 16) - smem) + 15) & ~(size_t)15;
  _Float16* xsb = reinterpret_cast<_Float16*>(smem + xsb_off);               // [2][16][kmax/16] hi, lo
  const int nsb = kmax / 16;                                                  // sub-blocks per staged row

  const int n_rt = a.H / 16, n_rts = a.Is > 0 ? a.H / 16 : 0;
  const int m = lane & 15, qq = lane >> 4, n = lane & 15;
  build_expert_list(a.topk_idx, T * k, k, a.E, L);
  const int64_t n_r = (int64_t)L->n * n_rt;
  const int64_t w_r = (int64_t)kK2Tile * n_ck, w_s = (int64_t)a.tb_s * n_cks;
  const int64_t lo = item_start(blockIdx.x, gridDim.x, n_rts, w_s, n_r, w_r);
  const int64_t hi = item_start(blockIdx.x + 1, gridDim.x, n_rts, w_s, n_r, w_r);
  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  // stage the A rows: shared (d = -1: h_s of every token) or expert d
  auto stage = [&](int d) {
    __syncthreads();
    const int K = d < 0 ? a.Is : a.I, Kp = d < 0 ? a.Is_pad : a.I_pad;
    if (tid < 16) {
      int sl = -1;
      uint32_t bits = 0;
      if (tid < T) {
        if (d < 0) {
          sl = tid;
        } else if ((L->mask[d] >> tid) & 1u) {
          for (int j = 0; j < k; ++j)
            if (L->slot_e[tid * k + j] == L->expert[d]) {
              sl = tid * k + j;
              bits |= 1u << j;
            }
        }
      }
      slot_of[tid] = sl;
      slot_bits[tid] = bits;
    }
    __syncthreads();
    // rows of h (or h_s) into hA: eight loads per thread in flight before
    // one wait (a row or column without data reads past the buffer: zeros)
    const _Float16* src = d < 0 ? a.hs : a.h;
    const int vp = Kp / 8, vk = K / 8, total = 16 * vp;
    const int src_bytes = (d < 0 ? T * a.Is : T * k * a.I) * 2;      // <= 1 MiB here
    const __amdgpu_buffer_rsrc_t hr = wt_rsrc(src, src_bytes);
    for (int i0 = 0; i0 < total; i0 += kStageLoads * (int)blockDim.x) {
      u32x4 v[kStageLoads];
#pragma unroll
      for (int u = 0; u < kStageLoads; ++u) {
        const int i = i0 + u * (int)blockDim.x + tid;
        const int mm = min(i / vp, 15), c = i - (i / vp) * vp;
        const int sl = slot_of[mm];
        v[u] = wt_load16(hr, (i < total && sl >= 0 && c < vk) ? (sl * K + 8 * c) * 2 : src_bytes);
      }
#pragma unroll
      for (int u = 0; u < kStageLoads; ++u) {
        const int i = i0 + u * (int)blockDim.x + tid;
        if (i < total) *reinterpret_cast<u32x4*>(hA + (size_t)(i / vp) * kmax + 8 * (i % vp)) = v[u];
      }
    }
    __syncthreads();
    if (d >= 0) {
      // sums X of each row over each 16-column sub-block, as fp16 hi + lo
      for (int i = tid; i < 16 * (Kp / 16); i += blockDim.x) {
        const int mm = i / (Kp / 16), sb = i - mm * (Kp / 16);
        const half8 v0 = *reinterpret_cast<const half8*>(hA + (size_t)mm * kmax + 16 * sb);
        const half8 v1 = *reinterpret_cast<const half8*>(hA + (size_t)mm * kmax + 16 * sb + 8);
        float x = 0.f;
        for (int j = 0; j < 8; ++j) x += (float)v0[j];
        for (int j = 0; j < 8; ++j) x += (float)v1[j];
        const _Float16 xh = (_Float16)x;
        xsb[(size_t)mm * nsb + sb] = xh;
        xsb[(size_t)(16 + mm) * nsb + sb] = (_Float16)(x - (float)xh);
      }
      __syncthreads();
    }
  };

  // reduce `cnt` row tiles (first one rt0) over the first n_waves waves and
  // write their rows: shared ones (e < 0) to ysh, routed ones of expert e to
  // ybuf at every slot of the token that chose the staged expert
  auto finish = [&](const float4v* acc, int cnt, int64_t rt0, int n_waves, int e) {
    for (int j = 0; j < kDnR; ++j)
      if (j < cnt) *reinterpret_cast<float4v*>(red + ((j * NW + wave) * 64 + lane) * 4) = acc[j];
    __syncthreads();
    for (int o = tid; o < cnt * 256; o += blockDim.x) {
      const int j = o >> 8, mm = (o >> 4) & 15, nn = o & 15;
      const int cl = 16 * (mm >> 2) + nn, ci = mm & 3;
      float v = 0.f;
      for (int w = 0; w < n_waves; ++w) v += red[((j * NW + w) * 64 + cl) * 4 + ci];
      const int sl = slot_of[mm];
      if (sl >= 0) {
        const size_t row = (size_t)(rt0 + j) * 16 + nn;
        if (e < 0) {
          a.ysh[(size_t)mm * a.H + row] = v;
        } else {
          for (uint32_t bits = slot_bits[mm]; bits; bits &= bits - 1u)
            a.ybuf[(size_t)(mm * k + __builtin_ctz(bits)) * a.H + row] = v;
        }
      }
    }
    __syncthreads();
  };

  // shared row tiles: h_s (fp16) x bf16 weights converted to fp16, or x the
  // exact Q8 codes with each k-block's dots times row n's scale in fp32
  const int64_t s_hi = min(hi, (int64_t)n_rts);
  if (lo < s_hi) stage(-1);
  const bool s_active = wave < n_cks;
  for (int64_t item = lo; item < s_hi; ++item) {
    float4v acc[1] = {zero};
    if (s_active) {
      if constexpr (SF == MOE_FMT_Q8) {
        const uint8_t* tile = a.sdown + ((size_t)item * n_cks + wave) * kQ8Tile;
        u32x4 raw[4];
        for (int i = 0; i < 4; ++i) raw[i] = load16(tile + 1024 * i + 16 * lane);
        const u32x4 scl = load16(tile + q8_scale_off(n));
        for (int kb = 0; kb < 8; ++kb) {
          const half8 av = as_half8(*reinterpret_cast<const u32x4*>(hA + (size_t)m * kmax + wave * 256 + kb * 32 + qq * 8));
          const u32x4 pc = raw[2 * (kb & 1) + (kb >> 2)];
          const half8 b = ((kb >> 1) & 1) ? q8_codes(pc.z, pc.w) : q8_codes(pc.x, pc.y);
          acc[0] += h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu) * mfma_f16(av, b, zero);
        }
      } else {
        const uint8_t* tile = a.sdown + ((size_t)item * n_cks + wave) * kBf16Tile;
        u32x4 raw[8];
        for (int kb = 0; kb < 8; ++kb) raw[kb] = load16(tile + 1024 * kb + 16 * lane);
        for (int kb = 0; kb < 8; ++kb) {
          const half8 av = as_half8(*reinterpret_cast<const u32x4*>(hA + (size_t)m * kmax + wave * 256 + kb * 32 + qq * 8));
          acc[0] = mfma_f16(av, bf16x8_to_half8(raw[kb]), acc[0]);
        }
      }
    }
    finish(acc, 1, item, n_cks, -1);
  }

  // routed rounds, the next round's weights in flight
  const bool r_active = wave < n_ck;
  const int chunk = r_active ? wave : 0;
  int64_t r_next = max(lo, (int64_t)n_rts) - n_rts;       // next routed item to load
  const int64_t r_end = hi - n_rts;
  // (expert, row tile) of r_next, advanced without a division per round (a
  // round never crosses an expert)
  int d_nx = (int)(r_next / n_rt), rt_nx = (int)(r_next - (int64_t)d_nx * n_rt);
  // issue the loads of the round starting at r_next; returns its size (0:
  // none left, its loads read nothing).  Offsets within one expert's down
  // matrix fit 32 bits (H <= 4096, I <= 2048 here).
  auto issue = [&](DnRound& P, int& d, int& rt0) {
    const bool any = r_next < r_end;
    const int cnt = any ? (int)min((int64_t)min(kDnR, n_rt - rt_nx), r_end - r_next) : 0;
    const int e = any ? __builtin_amdgcn_readfirstlane(L->expert[d_nx]) : 0;
    const __amdgpu_buffer_rsrc_t rs =
        wt_rsrc(a.down + (size_t)e * a.expert_bytes_down + (size_t)chunk * kK2Tile,
                any ? (int)(a.expert_bytes_down - (size_t)chunk * kK2Tile) : 0);
#pragma unroll
    for (int j = 0; j < kDnR; ++j) {
      const int toff = (rt_nx + min(j, max(cnt - 1, 0))) * n_ck * kK2Tile;
      P.q[j] = wt_load16(rs, toff + 16 * lane);
      P.scm[j] = wt_load16(rs, toff + 1024 + 16 * n);
      P.dd[j] = wt_load4(rs, toff + 1280 + 4 * n);
    }
    d = d_nx;
    rt0 = rt_nx;
    r_next += cnt;
    rt_nx += cnt;
    if (rt_nx == n_rt) {
      rt_nx = 0;
      ++d_nx;
    }
    return cnt;
  };
  half8 A[8];
  int cur_d = -1;
  auto compute = [&](const DnRound& P, int cnt, int d, int rt0) {
    if (d != cur_d) {
      stage(d);
      cur_d = d;
      for (int kb = 0; kb < 8; ++kb)
        A[kb] = as_half8(*reinterpret_cast<const u32x4*>(hA + (size_t)m * kmax + chunk * 256 + kb * 32 + qq * 8));
    }
    float4v acc[kDnR];
#pragma unroll
    for (int j = 0; j < kDnR; ++j) acc[j] = zero;
    // sum_k h w = d sum_k h (q sc) - dmin sum_sb m X_sb: the q sc dots on
    // the f16 matrix cores (exact operands), the min term as one 16x16x16
    // product of the sub-block sums (hi + lo) with the mins.  Every tile of
    // the round is computed on every path, also past cnt and on idle waves
    // (finish reduces the first cnt tiles of the first n_ck waves): a
    // payload whose loads some path never waits for makes the compiler wait
    // for all loads in flight before its registers are reused.
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int j = 0; j < kDnR; ++j) acc[j] = mfma_f16(A[kb], k2_qsc_b(P.q[j], P.scm[j], kb, qq), acc[j]);
    const int g = lane >> 4;
    const half4 xh = *reinterpret_cast<const half4*>(xsb + (size_t)m * nsb + 16 * chunk + 4 * g);
    const half4 xl = *reinterpret_cast<const half4*>(xsb + (size_t)(16 + m) * nsb + 16 * chunk + 4 * g);
#pragma unroll
    for (int j = 0; j < kDnR; ++j) {
      const half4 mb = k2_min_b(P.scm[j], g);
      float4v cm = __builtin_amdgcn_mfma_f32_16x16x16f16(xh, mb, zero, 0, 0, 0);
      cm = __builtin_amdgcn_mfma_f32_16x16x16f16(xl, mb, cm, 0, 0, 0);
      const float dd = h2f(P.dd[j] & 0xFFFFu), dm = h2f(P.dd[j] >> 16);
      for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(dd, acc[j][i], -dm * cm[i]);
    }
    finish(acc, cnt, rt0, n_ck, L->expert[d]);
  };
  // three rounds rotate through P0, P1, P2: two in flight while one computes
  DnRound P0, P1, P2;
  int d0 = 0, rt0 = 0, d1 = 0, rt1 = 0, d2 = 0, rt2 = 0;
  int c0 = issue(P0, d0, rt0), c1 = issue(P1, d1, rt1), c2 = 0;
  while (true) {
    if (c0 == 0) break;
    c2 = issue(P2, d2, rt2);
    compute(P0, c0, d0, rt0);
    if (c1 == 0) break;
    c0 = issue(P0, d0, rt0);
    compute(P1, c1, d1, rt1);
    if (c2 == 0) break;
    c1 = issue(P1, d1, rt1);
    compute(P2, c2, d2, rt2);
  }
}

// y[t][h] = sum_j w[t][j] * ybuf[t*k + j][h] + ysh[t][h] in j order (choices
// with an invalid expert id skipped); one workgroup per token, 4 h per thread.
__global__ __launch_bounds__(256) void decm_combine_kernel(const float* ybuf, const float* ysh, const int32_t* topk_idx,
                                                           const float* topk_w, const int* xexp, int k, int H, int E,
                                                           float* y) {
  const int t = blockIdx.x;
  const int e2 = 2 * xexp[t];                  // h was stored times 2^-2e
  for (int h = 4 * threadIdx.x; h < H; h += 4 * blockDim.x) {
    float4v v[16];
    bool ok[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = j < k ? topk_idx[t * k + j] : -1;
      ok[j] = e >= 0 && e < E;
      v[j] = ok[j] ? *reinterpret_cast<const float4v*>(ybuf + (size_t)(t * k + j) * H + h) : float4v{0.f, 0.f, 0.f, 0.f};
    }
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (ok[j]) {
        const float wj = topk_w[t * k + j];
        for (int q = 0; q < 4; ++q) acc[q] += wj * v[j][q];
      }
    if (ysh) {
      const float4v sv = *reinterpret_cast<const float4v*>(ysh + (size_t)t * H + h);
      for (int q = 0; q < 4; ++q) acc[q] += sv[q];
    }
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_ldexpf(acc[q], e2);
    *reinterpret_cast<float4v*>(y + (size_t)t * H + h) = acc;
  }
}

}  // namespace

namespace qmoe {

size_t decm_upgate_lds(int nw) {
  return (size_t)kCb2CombBytes + (size_t)kMRB * nw * 2 * 256 * 4 + sizeof(ExpertList) + (size_t)nw * 16 * 4 + 16 * 4;
}

size_t decm_down_lds(const DecArgs& a, int nw) {
  const size_t kmax = (size_t)(a.I_pad > a.Is_pad ? a.I_pad : a.Is_pad);
  return 16 * kmax * 2 + (size_t)kDnR * nw * 256 * 4 + sizeof(ExpertList) + 16 * 4 + 16 * 4 +
         16 + 2 * 16 * (kmax / 16) * 2;
}

hipError_t launch_decm(const DecArgs& a, const float* topk_w, float* y, int cus, hipStream_t s) {
  const int n_chunks = a.H / 256, n_ck = a.I_pad / 256, n_cks = a.Is > 0 ? a.Is_pad / 256 : 0;
  const int nw_ug = n_chunks < 4 ? 4 : n_chunks;
  int nw_dn = n_ck > n_cks ? n_ck : n_cks;
  if (nw_dn < 4) nw_dn = 4;
  if (nw_ug > 16 || nw_dn > 8) return hipErrorInvalidValue;   // H <= 4096, I and I_s <= 2048
  const bool q8 = a.fmt_s == MOE_FMT_Q8;
  void (*fu)(DecArgs) = q8 ? decm_upgate_kernel<MOE_FMT_Q8> : decm_upgate_kernel<MOE_FMT_BF16>;
  void (*fd)(DecArgs) = q8 ? decm_down_kernel<MOE_FMT_Q8> : decm_down_kernel<MOE_FMT_BF16>;
  hipError_t err = ensure_dyn_lds((const void*)fu);
  if (err != hipSuccess) return err;
  err = launch_timed(MOE_KERNEL_DECODE_UPGATE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(fu, dim3(cus), dim3(64 * nw_ug), decm_upgate_lds(nw_ug), s, ev0_, ev1_, 0, a);
  });
  if (err != hipSuccess) return err;
  err = ensure_dyn_lds((const void*)fd);
  if (err != hipSuccess) return err;
  err = launch_timed(MOE_KERNEL_DECODE_DOWN, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(fd, dim3(cus), dim3(64 * nw_dn), decm_down_lds(a, nw_dn), s, ev0_, ev1_, 0, a);
  });
  if (err != hipSuccess) return err;
  return launch_timed(MOE_KERNEL_DECODE_COMBINE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(decm_combine_kernel, dim3((unsigned)a.T), dim3(256), 0, s, ev0_, ev1_, 0, a.ybuf, a.Is > 0 ? a.ysh : nullptr,
                       a.topk_idx, topk_w, a.xexp, a.k, a.H, a.E, y);
  });
}

}  // namespace qmoe
