// Prefill-shape expert FFN: grouped GEMMs over the tokens of each expert
// ([blog] server logs: prompts are prefilled in chunks of 2048, cap 8192;
// [digest] "Model weights": quantized routed experts, bf16 shared expert).
//
// A workgroup owns (expert, N-tile of rows) and loops over all of the
// expert's tokens (positions in moe_group_tokens order), M_TILES*16 at a
// time.  Each wave owns two 16-row tiles of every weight matrix it touches
// (up and gate together for the first GEMM), dequantizes its tiles of a
// K-chunk exactly once into fp16 MFMA B operands in registers -- the
// quantization scales folded in, one fp16 rounding per weight -- and
// multiplies them against every M-tile.  Token rows are gathered, converted
// to fp16 and staged in LDS in MFMA A-operand order, 256 columns at a time.
// fp16 operands with fp32 accumulation keep the layer within the 2e-3
// tolerance, which bf16 operands do not.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmoe.h"
#include "device_common.hpp"
#include "k_prefill.h"
#include "launch_util.h"

using namespace qmoe_dev;
using qmoe::PfArgs;

namespace {

constexpr int kWaves = 8;     // waves per workgroup
constexpr int kTilesPerWave = 2;
constexpr int kRowsPerWg = kWaves * kTilesPerWave * 16;   // 256

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Stage rows [m0, m0 + M_TILES*16) x columns [col0, col0 + 256) of a
// row-major fp16/bf16 source into A-operand order:
//   byte ((mt*8 + kb)*64 + lane)*16 + 2j holds row 16 mt + lane%16,
//   column 32 kb + 8 (lane/16) + j.
// row_of(r) returns the source row of local row r, or -1 for a zero row.
template <int M_TILES, bool SRC_BF16, typename RowOf>
__device__ __forceinline__ void stage_a(uint8_t* a_lds, const uint16_t* src, int64_t ld, int col0,
                                        int col_valid, RowOf row_of) {
  constexpr int kChunks = M_TILES * 16 * 32;     // 16-byte pieces
  for (int p = threadIdx.x; p < kChunks; p += blockDim.x) {
    const int r = p >> 5, piece = p & 31;        // piece = kb*4 + g
    const int kb = piece >> 2, g = piece & 3;
    const int col = col0 + kb * 32 + g * 8;
    const int64_t row = row_of(r);
    u32x4 v = {0, 0, 0, 0};
    if (row >= 0 && col < col_valid) {
      const u32x4 raw = load16(src + row * ld + col);
      v = SRC_BF16 ? as_u32x4(bf16x8_to_half8(raw)) : raw;
    }
    const int mt = r >> 4, lane = g * 16 + (r & 15);
    *reinterpret_cast<u32x4*>(a_lds + ((mt * 8 + kb) * 64 + lane) * 16) = v;
  }
}

// ---------------------------------------------------------------------------
// B-operand dequantizers for prefill (scale folded in, fp16).

__device__ __forceinline__ half8 pf_cb2(const u32x4& codes, const u32x4& scl, int kb,
                                        const uint8_t* val_lane, const uint8_t* flip_lane) {
  const half8 v = cb2_group((codes[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu, val_lane, flip_lane);
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu));
  return v * s;
}

// K2 weight of slot s: (magic * 4^-t - 1024 * 4^-t) = q exactly, then
// q * fp16(d*sc) - fp16(dmin*m).
__device__ __forceinline__ half8 pf_k2(const u32x4& qw, const u32x4& scm, float d, float dmin, int kb,
                                       int qq) {
  const half8 mg = as_half8(k2_magic(qw, kb));
  const int sb = 2 * kb + (qq >> 1);
  const uint32_t byte = (scm[sb >> 2] >> (8 * (sb & 3))) & 0xFFu;
  const _Float16 dsc = (_Float16)(d * (float)(byte & 15u));
  const _Float16 ndm = (_Float16)(-(dmin * (float)(byte >> 4)));
  half8 w;
  for (int s = 0; s < 4; ++s) {
    const int t = k2_slot_t(kb, s);
    const _Float16 sc = (_Float16)__builtin_ldexpf(1.0f, -2 * t);
    const _Float16 off = (_Float16)(-1024.0f * __builtin_ldexpf(1.0f, -2 * t));
    const _Float16 q0 = mg[2 * s] * sc + off;
    const _Float16 q1 = mg[2 * s + 1] * sc + off;
    w[2 * s] = q0 * dsc + ndm;
    w[2 * s + 1] = q1 * dsc + ndm;
  }
  return w;
}

__device__ __forceinline__ half8 pf_k4(uint32_t word, float d, float dmin, uint32_t sc, uint32_t mn) {
  const half8 mg = as_half8(k4_magic(word));
  const _Float16 dsc = (_Float16)(d * (float)sc);
  const _Float16 ndm = (_Float16)(-(dmin * (float)mn));
  const _Float16 m1024 = (_Float16)(-1024.0f);
  half8 w;
  for (int j = 0; j < 8; ++j) w[j] = (mg[j] + m1024) * dsc + ndm;
  return w;
}

// Per-lane state of one weight tile for one K-chunk (enough to produce the
// B operand of every kb).
struct TileRegs {
  u32x4 a, b;        // CB2: codes, scales | K2: q words, sc/m | K4: q halves 0/1
  uint32_t s0, s1, s2, dd;
};

template <int FMT>
__device__ __forceinline__ TileRegs load_tile(const uint8_t* tile, int lane) {
  TileRegs r;
  const int n = lane & 15;
  if (FMT == MOE_FMT_CB2) {
    r.a = load16(tile + 16 * lane);
    r.b = load16(tile + 1024 + 16 * n);
  } else if (FMT == MOE_FMT_K2) {
    r.a = load16(tile + 16 * lane);
    r.b = load16(tile + 1024 + 16 * n);
    r.dd = *reinterpret_cast<const uint32_t*>(tile + 1280 + 4 * n);
  } else if (FMT == MOE_FMT_K4) {
    r.a = load16(tile + 16 * lane);
    r.b = load16(tile + 1024 + 16 * lane);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
    r.s0 = sp[0];
    r.s1 = sp[1];
    r.s2 = sp[2];
    r.dd = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ half8 tile_b(const TileRegs& r, const uint8_t* tile, int kb, int lane,
                                        const uint8_t* val_lane, const uint8_t* flip_lane) {
  if (FMT == MOE_FMT_CB2) return pf_cb2(r.a, r.b, kb, val_lane, flip_lane);
  if (FMT == MOE_FMT_K2) return pf_k2(r.a, r.b, h2f(r.dd & 0xFFFFu), h2f(r.dd >> 16), kb, lane >> 4);
  if (FMT == MOE_FMT_K4)
    return pf_k4(kb < 4 ? r.a[kb & 3] : r.b[kb & 3], h2f(r.dd & 0xFFFFu), h2f(r.dd >> 16),
                 k4_scale_value(r.s0, r.s1, r.s2, kb), k4_scale_value(r.s0, r.s1, r.s2, 8 + kb));
  return bf16x8_to_half8(load16(tile + 1024 * kb + 16 * lane));   // BF16
}

// ---------------------------------------------------------------------------
// Up/gate.  blockIdx.x = N-tile (256 rows of I), blockIdx.y < E: routed
// expert; blockIdx.y >= E: shared-expert M-chunk blockIdx.y - E.

template <int FMT, int M_TILES>
__global__ __launch_bounds__(512) void pf_upgate_kernel(PfArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* a_lds = smem;                                   // M_TILES * 8 KB
  uint8_t* val_tab = smem + M_TILES * 8192;
  uint8_t* flip_tab = val_tab + kCb2TableBytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool shared = blockIdx.y >= (unsigned)a.E;
  const int e = (int)blockIdx.y;
  int64_t p_begin, p_end;
  if (shared) {
    p_begin = (int64_t)(blockIdx.y - a.E) * M_TILES * 16;
    p_end = min((int64_t)a.T, p_begin + M_TILES * 16);
  } else {
    p_begin = a.offsets[e];
    p_end = a.offsets[e + 1];
  }
  if (p_begin >= p_end) return;
  const int rows_total = shared ? a.Is : a.I;
  const int n_rt = rows_total / 16;
  const int rt0 = blockIdx.x * (kRowsPerWg / 16) + wave * kTilesPerWave;
  if (blockIdx.x * kRowsPerWg >= rows_total) return;
  if (!shared && FMT == MOE_FMT_CB2) {
    cb2_fill_tables(a.codebook, val_tab, flip_tab, tid, blockDim.x);
  }
  const uint8_t* val_lane = val_tab + (lane & 7) * 16;
  const uint8_t* flip_lane = flip_tab + (lane & 7) * 16;
  const int n_chunks = a.H / 256;
  const int tb = shared ? kBf16Tile : (FMT == MOE_FMT_CB2 ? kCb2Tile : kK4Tile);
  const uint8_t* base_u = shared ? a.sup : a.up + (size_t)e * a.expert_bytes;
  const uint8_t* base_g = shared ? a.sgate : a.gate + (size_t)e * a.expert_bytes;
  const int k = a.k;
  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  for (int64_t m0 = p_begin; m0 < p_end; m0 += M_TILES * 16) {
    float4v acc[2][kTilesPerWave][M_TILES];
    for (int mat = 0; mat < 2; ++mat)
      for (int t = 0; t < kTilesPerWave; ++t)
        for (int mt = 0; mt < M_TILES; ++mt) acc[mat][t][mt] = zero;
    for (int chunk = 0; chunk < n_chunks; ++chunk) {
      __syncthreads();
      stage_a<M_TILES, true>(a_lds, a.x, a.H, chunk * 256, a.H, [&](int r) -> int64_t {
        const int64_t p = m0 + r;
        if (p >= p_end) return -1;
        return shared ? p : (int64_t)(a.sorted_slots[p] / k);
      });
      __syncthreads();
      TileRegs tr[2][kTilesPerWave];
      const uint8_t* tp[2][kTilesPerWave];
      for (int mat = 0; mat < 2; ++mat)
        for (int t = 0; t < kTilesPerWave; ++t) {
          const int rt = min(rt0 + t, n_rt - 1);
          tp[mat][t] = (mat ? base_g : base_u) + ((size_t)rt * n_chunks + chunk) * tb;
          if (shared) tr[mat][t] = load_tile<MOE_FMT_BF16>(tp[mat][t], lane);
          else tr[mat][t] = load_tile<FMT>(tp[mat][t], lane);
        }
      for (int kb = 0; kb < 8; ++kb) {
        half8 b[2][kTilesPerWave];
        for (int mat = 0; mat < 2; ++mat)
          for (int t = 0; t < kTilesPerWave; ++t)
            b[mat][t] = shared ? tile_b<MOE_FMT_BF16>(tr[mat][t], tp[mat][t], kb, lane, val_lane, flip_lane)
                               : tile_b<FMT>(tr[mat][t], tp[mat][t], kb, lane, val_lane, flip_lane);
        for (int mt = 0; mt < M_TILES; ++mt) {
          const half8 av = as_half8(*reinterpret_cast<const u32x4*>(a_lds + ((mt * 8 + kb) * 64 + lane) * 16));
          for (int mat = 0; mat < 2; ++mat)
            for (int t = 0; t < kTilesPerWave; ++t) acc[mat][t][mt] = mfma_f16(av, b[mat][t], acc[mat][t][mt]);
        }
      }
    }
    // epilogue: h = SiLU(g) * u for C[m = 4(lane/16) + i][n = lane%16]
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int rt = rt0 + t;
      if (rt >= n_rt) continue;
      const int row = rt * 16 + (lane & 15);
      for (int mt = 0; mt < M_TILES; ++mt)
        for (int i = 0; i < 4; ++i) {
          const int64_t p = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (p >= p_end) continue;
          const _Float16 hv = (_Float16)(silu(acc[1][t][mt][i]) * acc[0][t][mt][i]);
          if (shared) a.hs[p * a.Is + row] = hv;
          else a.h[p * a.I + row] = hv;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Down.  blockIdx.x = N-tile (256 rows of H); blockIdx.y as for up/gate.
// Routed outputs go to yslot[position], shared outputs to ysh[token].

template <int FMT, int M_TILES>
__global__ __launch_bounds__(512) void pf_down_kernel(PfArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* a_lds = smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool shared = blockIdx.y >= (unsigned)a.E;
  const int e = (int)blockIdx.y;
  int64_t p_begin, p_end;
  if (shared) {
    p_begin = (int64_t)(blockIdx.y - a.E) * M_TILES * 16;
    p_end = min((int64_t)a.T, p_begin + M_TILES * 16);
  } else {
    p_begin = a.offsets[e];
    p_end = a.offsets[e + 1];
  }
  if (p_begin >= p_end) return;
  const int n_rt = a.H / 16;
  const int rt0 = blockIdx.x * (kRowsPerWg / 16) + wave * kTilesPerWave;
  const int Kvalid = shared ? a.Is : a.I;
  const int n_chunks = (shared ? a.Is_pad : a.I_pad) / 256;
  const int tb = shared ? kBf16Tile : (FMT == MOE_FMT_K2 ? kK2Tile : kK4Tile);
  const uint8_t* base = shared ? a.sdown : a.down + (size_t)e * a.expert_bytes_down;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(shared ? a.hs : a.h);
  const int64_t ld = Kvalid;
  const float4v zero = {0.f, 0.f, 0.f, 0.f};

  for (int64_t m0 = p_begin; m0 < p_end; m0 += M_TILES * 16) {
    float4v acc[kTilesPerWave][M_TILES];
    for (int t = 0; t < kTilesPerWave; ++t)
      for (int mt = 0; mt < M_TILES; ++mt) acc[t][mt] = zero;
    for (int chunk = 0; chunk < n_chunks; ++chunk) {
      __syncthreads();
      stage_a<M_TILES, false>(a_lds, src, ld, chunk * 256, Kvalid, [&](int r) -> int64_t {
        const int64_t p = m0 + r;
        return p < p_end ? p : -1;
      });
      __syncthreads();
      TileRegs tr[kTilesPerWave];
      const uint8_t* tp[kTilesPerWave];
      for (int t = 0; t < kTilesPerWave; ++t) {
        const int rt = min(rt0 + t, n_rt - 1);
        tp[t] = base + ((size_t)rt * n_chunks + chunk) * tb;
        tr[t] = shared ? load_tile<MOE_FMT_BF16>(tp[t], lane) : load_tile<FMT>(tp[t], lane);
      }
      for (int kb = 0; kb < 8; ++kb) {
        half8 b[kTilesPerWave];
        for (int t = 0; t < kTilesPerWave; ++t)
          b[t] = shared ? tile_b<MOE_FMT_BF16>(tr[t], tp[t], kb, lane, nullptr, nullptr)
                        : tile_b<FMT>(tr[t], tp[t], kb, lane, nullptr, nullptr);
        for (int mt = 0; mt < M_TILES; ++mt) {
          const half8 av = as_half8(*reinterpret_cast<const u32x4*>(a_lds + ((mt * 8 + kb) * 64 + lane) * 16));
          for (int t = 0; t < kTilesPerWave; ++t) acc[t][mt] = mfma_f16(av, b[t], acc[t][mt]);
        }
      }
    }
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int rt = rt0 + t;
      if (rt >= n_rt) continue;
      const int row = rt * 16 + (lane & 15);
      for (int mt = 0; mt < M_TILES; ++mt)
        for (int i = 0; i < 4; ++i) {
          const int64_t p = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (p >= p_end) continue;
          if (shared) a.ysh[p * a.H + row] = acc[t][mt][i];
          else a.yslot[p * a.H + row] = acc[t][mt][i];
        }
    }
  }
}

// y[t][h] = sum_j w[t][j] * yslot[slot_pos[t*k + j]][h] + ysh[t][h].
__global__ void pf_combine_kernel(const float* yslot, const float* ysh, const int32_t* slot_pos,
                                  const float* topk_w, int T, int k, int H, float* y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * H) return;
  const int t = (int)(i / H), h = (int)(i % H);
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int p = slot_pos[t * k + j];
    if (p < 0) continue;
    acc += topk_w[t * k + j] * yslot[(size_t)p * H + h];
  }
  if (ysh) acc += ysh[(size_t)t * H + h];
  y[i] = acc;
}

constexpr int kMTiles = 6;

}  // namespace

namespace qmoe {

int pf_m_rows() { return kMTiles * 16; }

hipError_t launch_prefill(const PfArgs& a, int fmt_ug, int fmt_dn, const float* topk_w, float* y,
                          hipStream_t s) {
  const int n_sh_chunks = a.Is > 0 ? (a.T + kMTiles * 16 - 1) / (kMTiles * 16) : 0;
  const dim3 block(64 * kWaves);
  {
    const int rows = a.Is > a.I ? a.Is : a.I;
    const dim3 grid((rows + kRowsPerWg - 1) / kRowsPerWg, a.E + n_sh_chunks);
    const size_t lds = kMTiles * 8192 + 2 * kCb2TableBytes;
    void (*fn)(PfArgs) = fmt_ug == MOE_FMT_CB2 ? pf_upgate_kernel<MOE_FMT_CB2, kMTiles>
                                               : pf_upgate_kernel<MOE_FMT_K4, kMTiles>;
    hipError_t err = ensure_dyn_lds((const void*)fn);
    if (err != hipSuccess) return err;
    err = launch_timed(MOE_KERNEL_PREFILL_UPGATE, s, [&] { hipLaunchKernelGGL(fn, grid, block, lds, s, a); });
    if (err != hipSuccess) return err;
  }
  {
    const dim3 grid((a.H + kRowsPerWg - 1) / kRowsPerWg, a.E + n_sh_chunks);
    const size_t lds = kMTiles * 8192;
    void (*fn)(PfArgs) = fmt_dn == MOE_FMT_K2 ? pf_down_kernel<MOE_FMT_K2, kMTiles>
                                              : pf_down_kernel<MOE_FMT_K4, kMTiles>;
    hipError_t err = ensure_dyn_lds((const void*)fn);
    if (err != hipSuccess) return err;
    err = launch_timed(MOE_KERNEL_PREFILL_DOWN, s, [&] { hipLaunchKernelGGL(fn, grid, block, lds, s, a); });
    if (err != hipSuccess) return err;
  }
  const int64_t n = (int64_t)a.T * a.H;
  return launch_timed(MOE_KERNEL_PREFILL_COMBINE, s, [&] {
    hipLaunchKernelGGL(pf_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.yslot,
                       a.Is > 0 ? a.ysh : nullptr, a.slot_pos, topk_w, a.T, a.k, a.H, y);
  });
}

}  // namespace qmoe
