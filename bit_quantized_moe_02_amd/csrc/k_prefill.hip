// Prefill-shape expert FFN: grouped GEMMs over the tokens of each expert
// ([blog] server logs: prompts are prefilled in chunks of 2048, cap 8192;
// [digest] "Model weights": quantized routed experts, bf16 shared expert).
//
// A workgroup owns (expert, N-tile of weight rows) and loops over the
// expert's tokens (positions in moe_group_tokens order) 96 at a time; the
// shared expert runs as extra workgroups over 96-token chunks of all tokens.
// Each wave owns 32 weight rows (two 16-row tiles) per matrix and multiplies
// them with v_mfma_f32_32x32x16 against up to three 32-token M-tiles: every
// weight is dequantized once per workgroup pass into an fp16 B operand (the
// quantization scales folded in: one fp16 rounding per CB2 or K4 weight; a K2
// down weight is one fp16 fma of its exact code with fp16 per-sub-block
// factors) and used by 32 tokens per instruction.  M-tiles past the expert's
// last token are skipped.  Token rows go into LDS one 256-column K-chunk at a
// time by LDS DMA (the quantized experts read the fp16 copy of x that
// pf_x16_kernel makes); the next chunk's rows stream into the other LDS
// buffer and its weights into registers while the current chunk is
// multiplied.
// fp16 operands with fp32 accumulation keep the layer within the 2e-3
// tolerance, which bf16 operands do not; the shared expert's up/gate uses
// bf16 operands directly because both x and its weights are exact in bf16.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "../../include/qmoe.h"
#include "device_common.hpp"
#include "k_prefill.h"
#include "launch_util.h"

using namespace qmoe_dev;
using qmoe::PfArgs;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kUgWaves = 8;                              // up/gate workgroup: waves
constexpr int kDnWaves = 8;                              // down workgroup: waves
constexpr int kMT = 3;                                   // 32-token M-tiles per pass
constexpr int kMRows = 32 * kMT;                         // 96 tokens per pass
constexpr int kUgTiles = 1;                              // up/gate: 32-row B tiles per wave and matrix
constexpr int kUgRowsPerWg = kUgWaves * 32 * kUgTiles;     // 256 rows of I
constexpr int kDnTiles = 1;                              // down: 32-row B tiles per wave
constexpr int kDnRowsPerWg = kDnWaves * 32 * kDnTiles;     // 256 rows of H

__device__ __forceinline__ float16v mfma32(const half8& a, const half8& b, const float16v& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float16v mfma32_bf(const u32x4& a, const u32x4& b, const float16v& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// ---------------------------------------------------------------------------
// A staging.  A 256-column chunk of kMRows token rows goes from global memory
// straight into LDS through global_load_lds_dwordx4: one instruction writes
// 1 KB, lane l's 16 bytes at byte 16 l of the wave's LDS destination.  In LDS
// row r keeps its 32 pieces of 8 columns rotated by r: piece c8 at slot
// r*32 + ((c8 + r) & 31).  One instruction fills two rows (lane l: row
// r0 + l/32, slot l%32, i.e. piece (l%32 - r) & 31), and the MFMA reads of a
// step (32 consecutive rows, one piece column) hit 32 distinct 16-byte bank
// groups.  Chunks alternate between two buffers, the next chunk in flight
// while the current one is multiplied; no registers hold staged data.

constexpr int kChunkBytes = kMRows * 512;                // one staged chunk (48 KB)
constexpr int kStageBytes = 2 * kChunkBytes;             // double buffer (96 KB)
template <int NW>
constexpr int dma_per_wave() { return kMRows / 2 / NW; }   // two-row DMA instructions per wave per chunk

__device__ __forceinline__ half8 a_read(const uint8_t* buf, int mt, int kk, int lane) {
  const int r = 32 * mt + (lane & 31), c8 = 2 * kk + (lane >> 5);
  return as_half8(*reinterpret_cast<const u32x4*>(buf + 16 * (r * 32 + ((c8 + r) & 31))));
}

// Source rows of this lane's DMA instructions for the pass starting at m0
// (instruction i of wave w stages rows 2 (w D + i) + {0, 1}, D = kMRows / 2 / NW).  Rows
// past the pass's end repeat its last row: they only feed accumulator rows
// that are never stored.
template <int NW, typename RowOf>
__device__ __forceinline__ void stage_rows(int* rows, int64_t m0, int64_t p_end, RowOf row_of) {
  constexpr int kDmaPerWave = dma_per_wave<NW>();
  const int wave = threadIdx.x >> 6, hl = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int64_t p = m0 + 2 * (wave * kDmaPerWave + i) + hl;
    rows[i] = (int)row_of(p < p_end ? p : p_end - 1);
  }
}

// 16 zero bytes in device memory: the DMA source of every 8-column piece
// that lies past the end of a row.
__device__ __attribute__((aligned(16))) const uint32_t kZeroPiece[4] = {0u, 0u, 0u, 0u};

// Issues the DMA of columns [col0, col0 + 256) of rows[] (2-byte elements,
// row stride ld) into buf.  Pieces at or past col_valid (the padding of a
// row whose length is not a multiple of 256) are read from kZeroPiece: the
// packed weights there need not be zero (a K4 sub-block of 32 columns can be
// half padding, whose codes decode to small non-zero values).
template <int NW>
__device__ __forceinline__ void a_dma(uint8_t* buf, const uint16_t* src, int64_t ld, const int* rows, int col0,
                                      int col_valid) {
  constexpr int kDmaPerWave = dma_per_wave<NW>();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int r0 = 2 * (wave * kDmaPerWave + i), r = r0 + (lane >> 5);
    const int col = col0 + 8 * (((lane & 31) - r) & 31);
    const uint16_t* p = col < col_valid ? src + (int64_t)rows[i] * ld + col
                                        : reinterpret_cast<const uint16_t*>(kZeroPiece);
    __builtin_amdgcn_global_load_lds(p, (__attribute__((address_space(3))) void*)(buf + 512 * r0), 16, 0, 0);
  }
}

// Start of a chunk: this wave's loads (its DMA of the chunk, its registers of
// the chunk's weights) are complete, and after the barrier every wave's are,
// and every wave is done with the chunk before.
__device__ __forceinline__ void chunk_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// B operands.  For a wave's 32 rows starting at weight row-tile rt0 (two
// 16-row tiles), lane l takes row n = l%16 of tile rt0 + (l%32)/16; in step
// kk of a chunk it needs the 8 weights (n, kb = kk/2, qq = 2(kk%2) + l/32,
// j = 0..7), i.e. the group that the tile format keeps at lane c = 16 qq + n.
// So per chunk a lane loads the data of lanes c = 16 (l/32) + n (even kk) and
// c = 16 (2 + l/32) + n (odd kk) plus row n's scales.

struct Cb2B {
  u32x4 c0, c1, sc;
};
struct K4B {
  u32x4 q[2][2];     // [odd kk][half kb/4]
  uint32_t s0, s1, s2, dd;
};
struct K2B {
  u32x4 q0, q1, scm;
  uint32_t dd;
};

template <int FMT>
struct BRegs;
template <>
struct BRegs<MOE_FMT_CB2> {
  using T = Cb2B;
};
template <>
struct BRegs<MOE_FMT_K4> {
  using T = K4B;
};
template <>
struct BRegs<MOE_FMT_K2> {
  using T = K2B;
};

__device__ __forceinline__ void b_load(Cb2B& b, const uint8_t* tile, int lane) {
  const int n = lane & 15, hl = lane >> 5;
  b.c0 = load16(tile + 16 * (16 * hl + n));
  b.c1 = load16(tile + 16 * (16 * (2 + hl) + n));
  b.sc = load16(tile + 1024 + 16 * n);
}
__device__ __forceinline__ void b_load(K4B& b, const uint8_t* tile, int lane) {
  const int n = lane & 15, hl = lane >> 5;
  for (int v = 0; v < 2; ++v)
    for (int h = 0; h < 2; ++h) b.q[v][h] = load16(tile + 1024 * h + 16 * (16 * (2 * v + hl) + n));
  const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
  b.s0 = sp[0];
  b.s1 = sp[1];
  b.s2 = sp[2];
  b.dd = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
}
__device__ __forceinline__ void b_load(K2B& b, const uint8_t* tile, int lane) {
  const int n = lane & 15, hl = lane >> 5;
  b.q0 = load16(tile + 16 * (16 * hl + n));
  b.q1 = load16(tile + 16 * (16 * (2 + hl) + n));
  b.scm = load16(tile + 1024 + 16 * n);
  b.dd = *reinterpret_cast<const uint32_t*>(tile + 1280 + 4 * n);
}

// CB2: table value * fp16 scale (one rounding).
__device__ __forceinline__ half8 b_decode(const Cb2B& b, int kk, const uint8_t* tab) {
  const int kb = kk >> 1;
  const uint32_t w = (kk & 1) ? b.c1[kb >> 1] : b.c0[kb >> 1];
  const half8 v = cb2_comb(w, kb & 1, lds_offset(tab));
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)((b.sc[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu));
  return v * s;
}

// K4: (magic - 1024) = q exactly, then q * d*sc - dmin*m as one fp32 fma
// (both products exact in fp32), rounded to fp16.
__device__ __forceinline__ half8 b_decode(const K4B& b, int kk, const uint8_t*) {
  const int kb = kk >> 1;
  const uint32_t word = b.q[kk & 1][kb >> 2][kb & 3];
  const half8 mg = as_half8(k4_magic(word));
  const float d = h2f(b.dd & 0xFFFFu), dmin = h2f(b.dd >> 16);
  const float dsc = d * (float)k4_scale_value(b.s0, b.s1, b.s2, kb);
  const float ndm = -(dmin * (float)k4_scale_value(b.s0, b.s1, b.s2, 8 + kb));
  const _Float16 m1024 = (_Float16)(-1024.0f);
  half8 w;
  for (int j = 0; j < 8; ++j) w[j] = (_Float16)__builtin_fmaf((float)(mg[j] + m1024), dsc, ndm);
  return w;
}

// K2: code pair of slot s decodes to 1024*4^-t + q exactly after scaling the
// magic value by 4^-t; then q * d*sc - dmin*m as one fp32 fma (both products
// exact in fp32), rounded to fp16.  The lane's
// sub-block is 2 kb + qq/2 = 2 kb + kk%2.
__device__ __forceinline__ half8 b_decode(const K2B& b, int kk, const uint8_t*) {
  const int kb = kk >> 1;
  const half8 mg = as_half8(k2_magic((kk & 1) ? b.q1 : b.q0, kb));
  const int sb = 2 * kb + (kk & 1);
  const uint32_t byte = (b.scm[sb >> 2] >> (8 * (sb & 3))) & 0xFFu;
  const float d = h2f(b.dd & 0xFFFFu), dmin = h2f(b.dd >> 16);
  const float dsc = d * (float)(byte & 15u);
  const float ndm = -(dmin * (float)(byte >> 4));
  half8 w;
  for (int s = 0; s < 4; ++s) {
    const int t = k2_slot_t(kb, s);
    const _Float16 sc = (_Float16)__builtin_ldexpf(1.0f, -2 * t);
    const _Float16 off = (_Float16)(-1024.0f * __builtin_ldexpf(1.0f, -2 * t));
    const _Float16 q0 = mg[2 * s] * sc + off;
    const _Float16 q1 = mg[2 * s + 1] * sc + off;
    w[2 * s] = (_Float16)__builtin_fmaf((float)q0, dsc, ndm);
    w[2 * s + 1] = (_Float16)__builtin_fmaf((float)q1, dsc, ndm);
  }
  return w;
}

// K2 in the grouped GEMM, cheaper per weight: the row's per-sub-block
// factors d*sc and -dmin*m are formed once per chunk as fp16 (packed
// products of exact operands, one rounding each; the lane's sub-block at
// step kk is kk), and a weight is fma(q, d*sc, -dmin*m) in fp16 (q exact,
// one more rounding).
struct K2Fac {
  half2v ds[8];   // d*sc of sub-blocks 2i, 2i+1
  half2v nm[8];   // -dmin*m of sub-blocks 2i, 2i+1
};
__device__ __forceinline__ void k2_factors(const K2B& b, K2Fac& f) {
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(b.dd & 0xFFFFu));
  const _Float16 ndmin = -__builtin_bit_cast(_Float16, (uint16_t)(b.dd >> 16));
  const half2v d2 = {d, d}, nd2 = {ndmin, ndmin}, m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = b.scm[w] & 0x0F0F0F0Fu, hi = (b.scm[w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // bytes 2h and 2h+1 (sub-blocks 4w + 2h, 4w + 2h + 1) into the two
      // halves of a word, as fp16 1024 + nibble, minus 1024
      const uint32_t sel = h ? 0x0C030C02u : 0x0C010C00u;
      const half2v sc = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0u, lo, sel) | 0x64006400u) + m1024;
      const half2v mn = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0u, hi, sel) | 0x64006400u) + m1024;
      f.ds[2 * w + h] = sc * d2;
      f.nm[2 * w + h] = mn * nd2;
    }
  }
}
__device__ __forceinline__ half8 b_decode(const K2B& b, const K2Fac& f, int kk) {
  const int kb = kk >> 1;
  const half8 mg = as_half8(k2_magic((kk & 1) ? b.q1 : b.q0, kb));
  const _Float16 ds = f.ds[kk >> 1][kk & 1], nm = f.nm[kk >> 1][kk & 1];
  const half2v ds2 = {ds, ds}, nm2 = {nm, nm};
  half8 w;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = k2_slot_t(kb, s);
    const _Float16 sc = (_Float16)__builtin_ldexpf(1.0f, -2 * t);
    const _Float16 off = (_Float16)(-1024.0f * __builtin_ldexpf(1.0f, -2 * t));
    const half2v mp = {mg[2 * s], mg[2 * s + 1]};
    const half2v q = __builtin_elementwise_fma(mp, half2v{sc, sc}, half2v{off, off});   // exact
    const half2v r = __builtin_elementwise_fma(q, ds2, nm2);
    w[2 * s] = r[0];
    w[2 * s + 1] = r[1];
  }
  return w;
}

// BF16 tiles: the lane's 16 bytes for step kk (raw bf16).
__device__ __forceinline__ u32x4 bf16_piece(const uint8_t* tile, int kk, int lane) {
  const int n = lane & 15, hl = lane >> 5, kb = kk >> 1, qq = 2 * (kk & 1) + hl;
  return load16(tile + 1024 * kb + 16 * (16 * qq + n));
}

// Q8 tiles: the same lane's 8 codes for step kk and their fp16 scale, as
// {codes 0-3, codes 4-7, scale bits, 0}; q8_piece_b turns them into the
// B operand fp16(d q), the fp16 value of each dequantized weight.
__device__ __forceinline__ u32x4 q8_piece(const uint8_t* tile, int kk, int lane) {
  const int n = lane & 15, hl = lane >> 5, kb = kk >> 1, qq = 2 * (kk & 1) + hl;
  const uint32_t* cp = reinterpret_cast<const uint32_t*>(tile + q8_code_off(kb, 16 * qq + n));
  const uint16_t d = *reinterpret_cast<const uint16_t*>(tile + q8_scale_off(n) + 2 * kb);
  return u32x4{cp[0], cp[1], (uint32_t)d, 0u};
}
__device__ __forceinline__ half8 q8_piece_b(const u32x4& p) { return q8_fold(p.x, p.y, p.z); }

template <int SF>
__device__ __forceinline__ u32x4 shared_piece(const uint8_t* tile, int kk, int lane) {
  if constexpr (SF == MOE_FMT_Q8) return q8_piece(tile, kk, lane);
  else return bf16_piece(tile, kk, lane);
}
template <int SF>
constexpr int shared_tile_bytes() { return SF == MOE_FMT_Q8 ? kQ8Tile : kBf16Tile; }

__device__ __forceinline__ float16v zero16v() {
  float16v z;
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------
// Up/gate, routed experts (CB2 or K4): one (expert, 256-row N-tile of I) per
// workgroup, A = the expert's token rows of x (fp16 copy).

// The 16 k-steps of one staged chunk over MTA live M-tiles.
// A of M-tile mt at step kk: row 32 mt + l%32 sits at byte 16384 mt +
// 512 (l%32), piece rotation (2 kk + l/32 + l%32) & 31 does not depend on mt,
// so one address per step serves every M-tile (the empty asm keeps the
// compiler from hoisting the 16 step addresses into registers).
__device__ __forceinline__ const uint8_t* a_step_addr(const uint8_t* buf, int kk, int lane) {
  int q = (lane >> 5) + (lane & 31);
  asm volatile("" : "+v"(q));
  return buf + 512 * (lane & 31) + 16 * ((2 * kk + q) & 31);
}
__device__ __forceinline__ half8 a_at(const uint8_t* p, int mt) {
  return as_half8(*reinterpret_cast<const u32x4*>(p + 16384 * mt));
}

template <int MTA, typename B>
__device__ __forceinline__ void ug_steps(float16v (&acc)[2][kUgTiles][MTA], const B (&cu)[kUgTiles],
                                         const B (&cg)[kUgTiles], const uint8_t* tab, const uint8_t* buf, int lane) {
  half8 av[MTA];
  {
    const uint8_t* p0 = a_step_addr(buf, 0, lane);
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) av[mt] = a_at(p0, mt);
  }
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    half8 an[MTA];
    if (kk + 1 < 16) {
      const uint8_t* pn = a_step_addr(buf, kk + 1, lane);
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) an[mt] = a_at(pn, mt);
    }
    half8 bu[kUgTiles], bg[kUgTiles];
#pragma unroll
    for (int b = 0; b < kUgTiles; ++b) {
      bu[b] = b_decode(cu[b], kk, tab);
      bg[b] = b_decode(cg[b], kk, tab);
    }
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
      for (int b = 0; b < kUgTiles; ++b) {
        acc[0][b][mt] = mfma32(av[mt], bu[b], acc[0][b][mt]);
        acc[1][b][mt] = mfma32(av[mt], bg[b], acc[1][b][mt]);
      }
    if (kk + 1 < 16)
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) av[mt] = an[mt];
  }
}

template <int MTA, typename B>
__device__ __forceinline__ void ug_steps_bpf(float16v (&acc)[2][kUgTiles][MTA], const B (&cu)[kUgTiles],
                                         const B (&cg)[kUgTiles], const uint8_t* tab, const uint8_t* buf, int lane) {
  // A and B of step kk + 1 are read and decoded while step kk multiplies
  // (CB2: the table reads' latency hides behind the MFMAs; the K4 decode
  // needs the registers)
  half8 av[MTA], bu[kUgTiles], bg[kUgTiles];
  {
    const uint8_t* p0 = a_step_addr(buf, 0, lane);
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) av[mt] = a_at(p0, mt);
#pragma unroll
    for (int b = 0; b < kUgTiles; ++b) {
      bu[b] = b_decode(cu[b], 0, tab);
      bg[b] = b_decode(cg[b], 0, tab);
    }
  }
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    half8 an[MTA], bun[kUgTiles], bgn[kUgTiles];
    if (kk + 1 < 16) {
      const uint8_t* pn = a_step_addr(buf, kk + 1, lane);
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) an[mt] = a_at(pn, mt);
#pragma unroll
      for (int b = 0; b < kUgTiles; ++b) {
        bun[b] = b_decode(cu[b], kk + 1, tab);
        bgn[b] = b_decode(cg[b], kk + 1, tab);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
      for (int b = 0; b < kUgTiles; ++b) {
        acc[0][b][mt] = mfma32(av[mt], bu[b], acc[0][b][mt]);
        acc[1][b][mt] = mfma32(av[mt], bg[b], acc[1][b][mt]);
      }
    if (kk + 1 < 16) {
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) av[mt] = an[mt];
#pragma unroll
      for (int b = 0; b < kUgTiles; ++b) {
        bu[b] = bun[b];
        bg[b] = bgn[b];
      }
    }
  }
}

template <int FMT>
__device__ __forceinline__ void ug_routed(const PfArgs& a, uint8_t* smem, int e, int nt) {
  const int64_t p_begin = a.offsets[e], p_end = a.offsets[e + 1];
  if (p_begin >= p_end) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* tab = smem;                                                 // CB2 table at offset 0
  uint8_t* stage = smem + (FMT == MOE_FMT_CB2 ? kCb2CombBytes : 0);
  if (FMT == MOE_FMT_CB2) cb2_comb_fill(a.codebook, tab, reinterpret_cast<uint2*>(stage), tid, blockDim.x);
  const int n_rt = a.I / 16, n_chunks = a.H / 256, k = a.k;
  const int row0 = nt * kUgRowsPerWg + wave * 32 * kUgTiles;          // the wave's first weight row
  const bool active = row0 < a.I;
  const int tb = FMT == MOE_FMT_CB2 ? kCb2Tile : kK4Tile;
  const uint8_t* tu[kUgTiles];
  const uint8_t* tg[kUgTiles];
  for (int b = 0; b < kUgTiles; ++b) {
    const int rt_l = min((row0 + 32 * b) / 16 + ((lane & 31) >> 4), n_rt - 1);   // clamped: loads stay in the matrix
    tu[b] = a.up + (size_t)e * a.expert_bytes + (size_t)rt_l * n_chunks * tb;
    tg[b] = a.gate + (size_t)e * a.expert_bytes + (size_t)rt_l * n_chunks * tb;
  }
  using B = typename BRegs<FMT>::T;

  // one pass of up to kMRows tokens over MTA M-tiles (the last pass of an
  // expert runs only the M-tiles its tokens fill)
  auto run_pass = [&](auto mta_c, int64_t m0) {
    constexpr int MTA = decltype(mta_c)::value;
    int rows[dma_per_wave<kUgWaves>()];
    stage_rows<kUgWaves>(rows, m0, p_end, [&](int64_t p) { return (int64_t)(a.sorted_slots[p] / k); });
    float16v acc[2][kUgTiles][MTA];
    for (int b = 0; b < kUgTiles; ++b)
      for (int mt = 0; mt < MTA; ++mt) acc[0][b][mt] = acc[1][b][mt] = zero16v();
    B cu[kUgTiles], cg[kUgTiles], nu[kUgTiles], ng[kUgTiles];
    __syncthreads();                                                   // the last pass is done with the buffers
    a_dma<kUgWaves>(stage, a.x16, a.H, rows, 0, a.H);
    for (int b = 0; b < kUgTiles; ++b) {
      b_load(cu[b], tu[b], lane);
      b_load(cg[b], tg[b], lane);
    }
    for (int chunk = 0; chunk < n_chunks; ++chunk) {
      const uint8_t* buf = stage + (chunk & 1) * kChunkBytes;
      chunk_sync();
      if (chunk + 1 < n_chunks) {
        a_dma<kUgWaves>(stage + ((chunk + 1) & 1) * kChunkBytes, a.x16, a.H, rows, (chunk + 1) * 256, a.H);
        for (int b = 0; b < kUgTiles; ++b) {
          b_load(nu[b], tu[b] + (size_t)(chunk + 1) * tb, lane);
          b_load(ng[b], tg[b] + (size_t)(chunk + 1) * tb, lane);
        }
      }
      if (active) {
        if constexpr (FMT == MOE_FMT_CB2) ug_steps_bpf<MTA>(acc, cu, cg, tab, buf, lane);
        else ug_steps<MTA>(acc, cu, cg, tab, buf, lane);
      }
      for (int b = 0; b < kUgTiles; ++b) {
        cu[b] = nu[b];
        cg[b] = ng[b];
      }
    }
    // epilogue: C[m][n], m = 8(i/4) + 4(l/32) + i%4, n = l%32
    for (int b = 0; b < kUgTiles; ++b) {
      const int row = row0 + 32 * b + (lane & 31);
      if (row >= a.I) continue;
      for (int mt = 0; mt < MTA; ++mt)
        for (int i = 0; i < 16; ++i) {
          const int64_t p = m0 + 32 * mt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (p < p_end) {
            const int xe = a.epos[p];
            a.h[p * a.I + row] = h_of(acc[1][b][mt][i], acc[0][b][mt][i], xe, xe);
          }
        }
    }
  };
  for (int64_t m0 = p_begin; m0 < p_end; m0 += kMRows) {
    const int64_t left = p_end - m0;
    if (left > 64) run_pass(std::integral_constant<int, 3>{}, m0);
    else if (left > 32) run_pass(std::integral_constant<int, 2>{}, m0);
    else run_pass(std::integral_constant<int, 1>{}, m0);
  }
}

// Up/gate, shared expert: one (96-token chunk, 256-row N-tile of I_s) per
// workgroup.  BF16: raw bf16 x times bf16 weights on bf16 matrix cores.  Q8:
// the fp16 copy of x (x 2^-e) times fp16(d q).  Weights stream two steps at a
// time, the next two steps' loads in flight.
template <int MTA, int SF>
__device__ __forceinline__ void ug_shared_steps(float16v (&acc)[2][kUgTiles][kMT], const u32x4 (&cu)[kUgTiles][2],
                                                const u32x4 (&cg)[kUgTiles][2], const uint8_t* buf, int k0, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    half8 bu[kUgTiles], bg[kUgTiles];
    if constexpr (SF == MOE_FMT_Q8)
      for (int b = 0; b < kUgTiles; ++b) {
        bu[b] = q8_piece_b(cu[b][q]);
        bg[b] = q8_piece_b(cg[b][q]);
      }
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
      const half8 av = a_read(buf, mt, k0 + q, lane);
#pragma unroll
      for (int b = 0; b < kUgTiles; ++b) {
        if constexpr (SF == MOE_FMT_Q8) {
          acc[0][b][mt] = mfma32(av, bu[b], acc[0][b][mt]);
          acc[1][b][mt] = mfma32(av, bg[b], acc[1][b][mt]);
        } else {
          acc[0][b][mt] = mfma32_bf(as_u32x4(av), cu[b][q], acc[0][b][mt]);
          acc[1][b][mt] = mfma32_bf(as_u32x4(av), cg[b][q], acc[1][b][mt]);
        }
      }
    }
  }
}

template <int SF>
__device__ __forceinline__ void ug_shared(const PfArgs& a, uint8_t* smem, int mc, int nt) {
  const int64_t p_begin = (int64_t)mc * kMRows, p_end = min((int64_t)a.T, p_begin + kMRows);
  if (p_begin >= p_end) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* stage = smem;
  const int n_rt = a.Is / 16, n_chunks = a.H / 256;
  const int row0 = nt * kUgRowsPerWg + wave * 32 * kUgTiles;
  const bool active = row0 < a.Is;
  const uint8_t* tu[kUgTiles];
  const uint8_t* tg[kUgTiles];
  for (int b = 0; b < kUgTiles; ++b) {
    const int rt_l = min((row0 + 32 * b) / 16 + ((lane & 31) >> 4), n_rt - 1);
    tu[b] = a.sup + (size_t)rt_l * n_chunks * shared_tile_bytes<SF>();
    tg[b] = a.sgate + (size_t)rt_l * n_chunks * shared_tile_bytes<SF>();
  }
  const int mta = (int)min((int64_t)kMT, (p_end - p_begin + 31) / 32);
  int rows[dma_per_wave<kUgWaves>()];
  stage_rows<kUgWaves>(rows, p_begin, p_end, [](int64_t p) { return p; });
  float16v acc[2][kUgTiles][kMT];
  for (int b = 0; b < kUgTiles; ++b)
    for (int mt = 0; mt < kMT; ++mt) acc[0][b][mt] = acc[1][b][mt] = zero16v();
  u32x4 cu[kUgTiles][2], cg[kUgTiles][2], nu[kUgTiles][2], ng[kUgTiles][2];
  __syncthreads();
  const uint16_t* xsrc = SF == MOE_FMT_Q8 ? a.x16 : a.x;
  a_dma<kUgWaves>(stage, xsrc, a.H, rows, 0, a.H);
  for (int b = 0; b < kUgTiles; ++b)
    for (int q = 0; q < 2; ++q) {
      cu[b][q] = shared_piece<SF>(tu[b], q, lane);
      cg[b][q] = shared_piece<SF>(tg[b], q, lane);
    }
  const int n_pairs = 8 * n_chunks;
  for (int gp = 0; gp < n_pairs; ++gp) {
    const int chunk = gp >> 3, k0 = 2 * (gp & 7);
    const uint8_t* buf = stage + (chunk & 1) * kChunkBytes;
    if ((gp & 7) == 0) {
      chunk_sync();
      if (chunk + 1 < n_chunks) a_dma<kUgWaves>(stage + ((chunk + 1) & 1) * kChunkBytes, xsrc, a.H, rows, (chunk + 1) * 256, a.H);
    }
    if (gp + 1 < n_pairs) {
      const int c1 = (gp + 1) >> 3, k1 = 2 * ((gp + 1) & 7);
      for (int b = 0; b < kUgTiles; ++b)
        for (int q = 0; q < 2; ++q) {
          nu[b][q] = shared_piece<SF>(tu[b] + (size_t)c1 * shared_tile_bytes<SF>(), k1 + q, lane);
          ng[b][q] = shared_piece<SF>(tg[b] + (size_t)c1 * shared_tile_bytes<SF>(), k1 + q, lane);
        }
    }
    if (active) {
      if (mta >= 3) ug_shared_steps<3, SF>(acc, cu, cg, buf, k0, lane);
      else if (mta == 2) ug_shared_steps<2, SF>(acc, cu, cg, buf, k0, lane);
      else ug_shared_steps<1, SF>(acc, cu, cg, buf, k0, lane);
    }
    for (int b = 0; b < kUgTiles; ++b)
      for (int q = 0; q < 2; ++q) {
        cu[b][q] = nu[b][q];
        cg[b][q] = ng[b][q];
      }
  }
  for (int b = 0; b < kUgTiles; ++b) {
    const int row = row0 + 32 * b + (lane & 31);
    if (row >= a.Is) continue;
    for (int mt = 0; mt < kMT; ++mt)
      for (int i = 0; i < 16; ++i) {
        const int64_t p = p_begin + 32 * mt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (p < p_end) {
          // BF16 took raw bf16 x, Q8 x 2^-e
          const int e = a.xexp[p];
          a.hs[p * a.Is + row] = h_of(acc[1][b][mt][i], acc[0][b][mt][i], SF == MOE_FMT_Q8 ? e : 0, e);
        }
      }
  }
}

// Workgroup -> (N-tile nt, group g) over a 1-D grid of n_nt * roundup(G, 8)
// workgroups.  Consecutive workgroups go to the 8 XCDs in turn, so workgroup
// L runs on XCD L % 8; all n_nt N-tiles of a group are given to the same XCD
// back to back, and the token rows they all stage come through one L2.
// Groups [0, n_sh) are the shared expert's token chunks (the heaviest
// workgroups, dispatched first), then the routed experts.
__device__ __forceinline__ bool pf_tile(int n_nt, int n_groups, int& nt, int& g) {
  const int L = (int)blockIdx.x, x = L & 7, j = L >> 3;
  nt = j % n_nt;
  g = (j / n_nt) * 8 + x;
  return g < n_groups;
}

__host__ __device__ inline int pf_shared_chunks(const PfArgs& a) { return a.Is > 0 ? (a.T + kMRows - 1) / kMRows : 0; }

template <int FMT>
__global__ __launch_bounds__(64 * kUgWaves) void pf_upgate_kernel(PfArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int n_sh = pf_shared_chunks(a);
  const int n_nt = ((a.Is > a.I ? a.Is : a.I) + kUgRowsPerWg - 1) / kUgRowsPerWg;
  int nt, g;
  if (!pf_tile(n_nt, a.E + n_sh, nt, g)) return;
  if (g >= n_sh) {
    if (nt * kUgRowsPerWg >= a.I) return;
    ug_routed<FMT>(a, smem, g - n_sh, nt);
  } else {
    if (nt * kUgRowsPerWg >= a.Is) return;
    if (a.fmt_s == MOE_FMT_Q8) ug_shared<MOE_FMT_Q8>(a, smem, g, nt);
    else ug_shared<MOE_FMT_BF16>(a, smem, g, nt);
  }
}

// One workgroup per token t: its exponent e_t (xexp[t], and epos at the
// grouped positions of its choices) and x16[t] = fp16(x[t] 2^-e_t), the
// routed experts' A operand.  Up to kX16Vec 8-value vectors per thread.
constexpr int kX16Threads = 256, kX16Vec = 4;   // H <= 8192

__global__ __launch_bounds__(kX16Threads) void pf_x16_kernel(const uint16_t* x, uint16_t* x16, int H, int k,
                                                             const int32_t* slot_pos, int* xexp, int* epos) {
  __shared__ uint32_t wmax[kX16Threads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, nv = H / 8;
  const uint16_t* row = x + (size_t)t * H;
  u32x4 v[kX16Vec];
  uint32_t ef = 0;
#pragma unroll
  for (int i = 0; i < kX16Vec; ++i) {
    const int c = tid + i * kX16Threads;
    v[i] = c < nv ? load16(row + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    ef = max(ef, bf16x8_max_efield(v[i]));
  }
  ef = wave_max_u32(ef);
  if ((tid & 63) == 0) wmax[tid >> 6] = ef;
  __syncthreads();
  for (int w = 0; w < kX16Threads / 64; ++w) ef = max(ef, wmax[w]);
  const int xe = x_exp_of_field(ef);
#pragma unroll
  for (int i = 0; i < kX16Vec; ++i) {
    const int c = tid + i * kX16Threads;
    if (c < nv) *reinterpret_cast<u32x4*>(x16 + (size_t)t * H + 8 * c) = as_u32x4(bf16x8_to_half8_exp(v[i], xe));
  }
  if (tid == 0) xexp[t] = xe;
  if (tid < k) {
    const int p = slot_pos[(size_t)t * k + tid];
    if (p >= 0) epos[p] = xe;
  }
}

// ---------------------------------------------------------------------------
// Down: one (expert, 256-row N-tile of H) per workgroup, one 32-row B tile
// per wave, A = the expert's rows of h (positions in grouped order).  Routed
// outputs go to yslot[position], shared outputs to ysh[token].

template <int FMT, int MTA, typename B>
__device__ __forceinline__ void dn_steps(float16v (&acc)[kDnTiles][kMT], const B (&cur)[kDnTiles], const uint8_t* buf,
                                         int lane) {
  // A and B of step kk + 1 are read and decoded while step kk multiplies
  K2Fac fac[kDnTiles];
  if constexpr (FMT == MOE_FMT_K2)
    for (int b = 0; b < kDnTiles; ++b) k2_factors(cur[b], fac[b]);
  auto decode = [&](int b, int kk) {
    if constexpr (FMT == MOE_FMT_K2) return b_decode(cur[b], fac[b], kk);
    else return b_decode(cur[b], kk, nullptr);
  };
  half8 av[MTA], bw[kDnTiles];
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt) av[mt] = a_read(buf, mt, 0, lane);
  for (int b = 0; b < kDnTiles; ++b) bw[b] = decode(b, 0);
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    half8 an[MTA], bn[kDnTiles];
    if (kk + 1 < 16) {
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) an[mt] = a_read(buf, mt, kk + 1, lane);
      for (int b = 0; b < kDnTiles; ++b) bn[b] = decode(b, kk + 1);
    }
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
      for (int b = 0; b < kDnTiles; ++b) acc[b][mt] = mfma32(av[mt], bw[b], acc[b][mt]);
    if (kk + 1 < 16) {
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) av[mt] = an[mt];
      for (int b = 0; b < kDnTiles; ++b) bw[b] = bn[b];
    }
  }
}

template <int FMT>
__device__ __forceinline__ void dn_routed(const PfArgs& a, uint8_t* smem, int e, int nt) {
  const int64_t p_begin = a.offsets[e], p_end = a.offsets[e + 1];
  if (p_begin >= p_end) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* stage = smem;
  const int n_rt = a.H / 16, n_chunks = a.I_pad / 256;
  const int tb = FMT == MOE_FMT_K2 ? kK2Tile : kK4Tile;
  int rt0[kDnTiles];
  const uint8_t* tp[kDnTiles];
  for (int b = 0; b < kDnTiles; ++b) {
    rt0[b] = (nt * kDnRowsPerWg + wave * 32 * kDnTiles + 32 * b) / 16;
    const int rt_l = min(rt0[b] + ((lane & 31) >> 4), n_rt - 1);
    tp[b] = a.down + (size_t)e * a.expert_bytes_down + (size_t)rt_l * n_chunks * tb;
  }
  const uint16_t* hsrc = reinterpret_cast<const uint16_t*>(a.h);
  using B = typename BRegs<FMT>::T;
  for (int64_t m0 = p_begin; m0 < p_end; m0 += kMRows) {
    const int mta = (int)min((int64_t)kMT, (p_end - m0 + 31) / 32);
    int rows[dma_per_wave<kDnWaves>()];
    stage_rows<kDnWaves>(rows, m0, p_end, [](int64_t p) { return p; });
    float16v acc[kDnTiles][kMT];
    for (int b = 0; b < kDnTiles; ++b)
      for (int mt = 0; mt < kMT; ++mt) acc[b][mt] = zero16v();
    B cur[kDnTiles], nxt[kDnTiles];
    __syncthreads();
    a_dma<kDnWaves>(stage, hsrc, a.I, rows, 0, a.I);
    for (int b = 0; b < kDnTiles; ++b) b_load(cur[b], tp[b], lane);
    for (int chunk = 0; chunk < n_chunks; ++chunk) {
      const uint8_t* buf = stage + (chunk & 1) * kChunkBytes;
      chunk_sync();
      if (chunk + 1 < n_chunks) {
        a_dma<kDnWaves>(stage + ((chunk + 1) & 1) * kChunkBytes, hsrc, a.I, rows, (chunk + 1) * 256, a.I);
        for (int b = 0; b < kDnTiles; ++b) b_load(nxt[b], tp[b] + (size_t)(chunk + 1) * tb, lane);
      }
      if (mta >= 3) dn_steps<FMT, 3>(acc, cur, buf, lane);
      else if (mta == 2) dn_steps<FMT, 2>(acc, cur, buf, lane);
      else dn_steps<FMT, 1>(acc, cur, buf, lane);
      for (int b = 0; b < kDnTiles; ++b) cur[b] = nxt[b];
    }
    for (int b = 0; b < kDnTiles; ++b) {
      const int row = rt0[b] * 16 + (lane & 31);
      if (row >= a.H) continue;
      for (int mt = 0; mt < kMT; ++mt)
        for (int i = 0; i < 16; ++i) {
          const int64_t p = m0 + 32 * mt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (p < p_end) a.yslot[p * a.H + row] = acc[b][mt][i];
        }
    }
  }
}

// Shared expert down: hs (fp16) x bf16 weights converted to fp16, or
// fp16(d q) of Q8 weights, in registers, weights streamed a quarter chunk at
// a time.
template <int MTA, int SF>
__device__ __forceinline__ void dn_shared_steps(float16v (&acc)[kDnTiles][kMT], const u32x4 (&cw)[kDnTiles][4],
                                                const uint8_t* buf, int q0, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    half8 bw[kDnTiles];
    for (int b = 0; b < kDnTiles; ++b) bw[b] = SF == MOE_FMT_Q8 ? q8_piece_b(cw[b][q]) : bf16x8_to_half8(cw[b][q]);
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
      const half8 av = a_read(buf, mt, q0 + q, lane);
      for (int b = 0; b < kDnTiles; ++b) acc[b][mt] = mfma32(av, bw[b], acc[b][mt]);
    }
  }
}

template <int SF>
__device__ __forceinline__ void dn_shared(const PfArgs& a, uint8_t* smem, int mc, int nt) {
  const int64_t p_begin = (int64_t)mc * kMRows, p_end = min((int64_t)a.T, p_begin + kMRows);
  if (p_begin >= p_end) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* stage = smem;
  const int n_rt = a.H / 16, n_chunks = a.Is_pad / 256;
  int rt0[kDnTiles];
  const uint8_t* tp[kDnTiles];
  for (int b = 0; b < kDnTiles; ++b) {
    rt0[b] = (nt * kDnRowsPerWg + wave * 32 * kDnTiles + 32 * b) / 16;
    const int rt_l = min(rt0[b] + ((lane & 31) >> 4), n_rt - 1);
    tp[b] = a.sdown + (size_t)rt_l * n_chunks * shared_tile_bytes<SF>();
  }
  const uint16_t* hsrc = reinterpret_cast<const uint16_t*>(a.hs);
  const int mta = (int)min((int64_t)kMT, (p_end - p_begin + 31) / 32);
  int rows[dma_per_wave<kDnWaves>()];
  stage_rows<kDnWaves>(rows, p_begin, p_end, [](int64_t p) { return p; });
  float16v acc[kDnTiles][kMT];
  for (int b = 0; b < kDnTiles; ++b)
    for (int mt = 0; mt < kMT; ++mt) acc[b][mt] = zero16v();
  a_dma<kDnWaves>(stage, hsrc, a.Is, rows, 0, a.Is);
  u32x4 cw[kDnTiles][4], nw[kDnTiles][4];
  for (int b = 0; b < kDnTiles; ++b)
    for (int q = 0; q < 4; ++q) cw[b][q] = shared_piece<SF>(tp[b], q, lane);
  const int n_quarters = 4 * n_chunks;
  for (int gq = 0; gq < n_quarters; ++gq) {
    const int chunk = gq >> 2, q0 = 4 * (gq & 3);
    const uint8_t* buf = stage + (chunk & 1) * kChunkBytes;
    if ((gq & 3) == 0) {
      chunk_sync();
      if (chunk + 1 < n_chunks) a_dma<kDnWaves>(stage + ((chunk + 1) & 1) * kChunkBytes, hsrc, a.Is, rows, (chunk + 1) * 256, a.Is);
    }
    if (gq + 1 < n_quarters) {
      const int c1 = (gq + 1) >> 2, k1 = 4 * ((gq + 1) & 3);
      for (int b = 0; b < kDnTiles; ++b)
        for (int q = 0; q < 4; ++q) nw[b][q] = shared_piece<SF>(tp[b] + (size_t)c1 * shared_tile_bytes<SF>(), k1 + q, lane);
    }
    if (mta >= 3) dn_shared_steps<3, SF>(acc, cw, buf, q0, lane);
    else if (mta == 2) dn_shared_steps<2, SF>(acc, cw, buf, q0, lane);
    else dn_shared_steps<1, SF>(acc, cw, buf, q0, lane);
    for (int b = 0; b < kDnTiles; ++b)
      for (int q = 0; q < 4; ++q) cw[b][q] = nw[b][q];
  }
  for (int b = 0; b < kDnTiles; ++b) {
    const int row = rt0[b] * 16 + (lane & 31);
    if (row >= a.H) continue;
    for (int mt = 0; mt < kMT; ++mt)
      for (int i = 0; i < 16; ++i) {
        const int64_t p = p_begin + 32 * mt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (p < p_end) a.ysh[p * a.H + row] = acc[b][mt][i];
      }
  }
}

template <int FMT>
__global__ __launch_bounds__(64 * kDnWaves) void pf_down_kernel(PfArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int n_sh = pf_shared_chunks(a);
  const int n_nt = (a.H + kDnRowsPerWg - 1) / kDnRowsPerWg;
  int nt, g;
  if (!pf_tile(n_nt, a.E + n_sh, nt, g)) return;
  if (g >= n_sh) dn_routed<FMT>(a, smem, g - n_sh, nt);
  else if (a.fmt_s == MOE_FMT_Q8) dn_shared<MOE_FMT_Q8>(a, smem, g, nt);
  else dn_shared<MOE_FMT_BF16>(a, smem, g, nt);
}

// y[t][h] = sum_j w[t][j] * yslot[slot_pos[t*k + j]][h] + ysh[t][h], summed in
// j order.  One workgroup per token; each thread takes 4 consecutive h and
// issues the loads of all k slots before summing.
constexpr int kMaxK = 16;

__global__ __launch_bounds__(256) void pf_combine_kernel(const float* yslot, const float* ysh,
                                                         const int32_t* slot_pos, const float* topk_w,
                                                         const int* xexp, int T, int k, int H, float* y) {
  const int t = blockIdx.x;
  const int e2 = 2 * xexp[t];                  // h was stored times 2^-2e
  int pos[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
    wj[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
  }
  for (int h = 4 * threadIdx.x; h < H; h += 4 * blockDim.x) {
    float4v v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      v[j] = pos[j] >= 0 ? *reinterpret_cast<const float4v*>(yslot + (size_t)pos[j] * H + h)
                         : float4v{0.f, 0.f, 0.f, 0.f};
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (pos[j] >= 0)
        for (int q = 0; q < 4; ++q) acc[q] += wj[j] * v[j][q];
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

int pf_m_rows() { return kMRows; }

hipError_t launch_prefill(const PfArgs& a, int fmt_ug, int fmt_dn, const float* topk_w, float* y,
                          hipStream_t s) {
  const int n_groups8 = (a.E + pf_shared_chunks(a) + 7) / 8 * 8;
  {
    if (a.H / 8 > kX16Threads * kX16Vec) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pf_x16_kernel, dim3((unsigned)a.T), dim3(kX16Threads), 0, s, a.x, const_cast<uint16_t*>(a.x16),
                       a.H, a.k, a.slot_pos, a.xexp, a.epos);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const int rows = a.Is > a.I ? a.Is : a.I;
    const dim3 grid((unsigned)(((rows + kUgRowsPerWg - 1) / kUgRowsPerWg) * n_groups8));
    const size_t lds = (fmt_ug == MOE_FMT_CB2 ? kCb2CombBytes : 0) + kStageBytes;
    void (*fn)(PfArgs) = fmt_ug == MOE_FMT_CB2 ? pf_upgate_kernel<MOE_FMT_CB2> : pf_upgate_kernel<MOE_FMT_K4>;
    hipError_t err = ensure_dyn_lds((const void*)fn);
    if (err != hipSuccess) return err;
    err = launch_timed(MOE_KERNEL_PREFILL_UPGATE, s,
                       [&](hipEvent_t ev0_, hipEvent_t ev1_) { hipExtLaunchKernelGGL(fn, grid, dim3(64 * kUgWaves), lds, s, ev0_, ev1_, 0, a); });
    if (err != hipSuccess) return err;
  }
  {
    const dim3 grid((unsigned)(((a.H + kDnRowsPerWg - 1) / kDnRowsPerWg) * n_groups8));
    void (*fn)(PfArgs) = fmt_dn == MOE_FMT_K2 ? pf_down_kernel<MOE_FMT_K2> : pf_down_kernel<MOE_FMT_K4>;
    hipError_t err = ensure_dyn_lds((const void*)fn);
    if (err != hipSuccess) return err;
    err = launch_timed(MOE_KERNEL_PREFILL_DOWN, s,
                       [&](hipEvent_t ev0_, hipEvent_t ev1_) { hipExtLaunchKernelGGL(fn, grid, dim3(64 * kDnWaves), (size_t)kStageBytes, s, ev0_, ev1_, 0, a); });
    if (err != hipSuccess) return err;
  }
  return launch_timed(MOE_KERNEL_PREFILL_COMBINE, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(pf_combine_kernel, dim3((unsigned)a.T), dim3(256), 0, s, ev0_, ev1_, 0, a.yslot,
                       a.Is > 0 ? a.ysh : nullptr, a.slot_pos, topk_w, a.xexp, a.T, a.k, a.H, y);
  });
}

}  // namespace qmoe
