// Device helpers shared by the libqmoe kernels: vector types, the fp16 MFMA,
// and the per-lane decoders of the CB2 / K2 / K4 / BF16 tiles that
// include/qmoe.h defines.
//
// Every decoder produces the MFMA B operand of one lane for one k-block kb:
// 8 fp16 values = weights (n, kb, qq, j = 0..7) of the lane c = 16*qq + n, in
// j order, so that the A operand (activations) of the same lane is simply
// x[m][32*kb + 8*qq + j] (scaled per slot where a decoder says so).
//
// Magic-number decode (K2, K4): OR-ing a small integer f into the mantissa
// of fp16 1024.0 (0x6400) gives the fp16 number 1024 + f exactly.  A code q
// sitting at bit 2t of a 16-bit half becomes 1024 + 4^t * q, so the matching
// activation is pre-scaled by 4^-t and the sum over a block is
// sum(x * 4^-t * 1024) + sum(x * q); the first term depends on x alone and
// is removed with a precomputed per-block offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe_dev {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCb2Tile = 1280;
constexpr int kK2Tile = 1344;
constexpr int kK4Tile = 2304;
constexpr int kBf16Tile = 8192;

__device__ __forceinline__ float4v mfma_f16(const half8& a, const half8& b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 as_half8(const u32x4& v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ u32x4 as_u32x4(const half8& v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// fp16 bits -> float
__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf2f(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Two bf16 in one dword -> two fp16 in one dword (exact for |v| in the fp16
// normal range; smaller values round once to the fp16 subnormal grid).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __builtin_bit_cast(float, w << 16);
  const float hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
  half2v h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// 8 consecutive bf16 (16 bytes) -> half8
__device__ __forceinline__ half8 bf16x8_to_half8(const u32x4& v) {
  u32x4 r;
  r.x = bf16x2_to_f16x2(v.x);
  r.y = bf16x2_to_f16x2(v.y);
  r.z = bf16x2_to_f16x2(v.z);
  r.w = bf16x2_to_f16x2(v.w);
  return as_half8(r);
}

// ---------------------------------------------------------------------------
// CB2.  Two LDS tables, each replicated 8 times so that the 8 lanes of an
// LDS read phase always hit different bank groups: entry e of copy c sits at
// byte (8*e + c) * 16.
//   value table: entry idx = the 8 fp16 values T[idx][j] / 4 (exact);
//   flip table:  entry f   = 4 xor masks, word w flips the fp16 sign bits of
//                weights 2w (bit 15) and 2w+1 (bit 31) when flip bits 2w,
//                2w+1 of f are set.
constexpr int kCb2TableBytes = 256 * 8 * 16;

__device__ __forceinline__ void cb2_fill_tables(const int8_t* codebook, uint8_t* val_tab,
                                                uint8_t* flip_tab, int tid, int nthreads) {
  for (int i = tid; i < 256 * 8; i += nthreads) {
    const int e = i >> 3;
    u32x4 v, m;
    uint32_t w[4];
    for (int p = 0; p < 4; ++p) {
      const _Float16 lo = (_Float16)((float)codebook[e * 8 + 2 * p] * 0.25f);
      const _Float16 hi = (_Float16)((float)codebook[e * 8 + 2 * p + 1] * 0.25f);
      w[p] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    uint32_t mk[4];
    for (int p = 0; p < 4; ++p)
      mk[p] = (((uint32_t)e >> (2 * p)) & 1u) << 15 | (((uint32_t)e >> (2 * p + 1)) & 1u) << 31;
    m.x = mk[0]; m.y = mk[1]; m.z = mk[2]; m.w = mk[3];
    *reinterpret_cast<u32x4*>(val_tab + i * 16) = v;
    *reinterpret_cast<u32x4*>(flip_tab + i * 16) = m;
  }
}

// Decode the group with 16-bit code (idx | flip << 8).  val_lane / flip_lane
// point at copy (lane & 7) of each table.
__device__ __forceinline__ half8 cb2_group(uint32_t code, const uint8_t* val_lane,
                                           const uint8_t* flip_lane) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(val_lane + (code & 0xFFu) * 128u);
  const u32x4 m = *reinterpret_cast<const u32x4*>(flip_lane + ((code >> 8) & 0xFFu) * 128u);
  return as_half8(v ^ m);
}

// CB2 combined table (REP x 64 KB, the kernels place it at LDS offset 0):
// entry (idx, half, nib) holds the 4 fp16 values T[idx][4*half+i]/4, negated
// where bit i of nib is set, so a group of 8 weights is two 8-byte reads
// addressed straight from its 16-bit code (idx | flip << 8): half 0 takes flip
// bits 0..3, half 1 bits 4..7.  Copy r of the entry sits at byte
//   ((idx*2 + half)*16 + nib)*8*REP + 8*r,
// and lane l reads copy l % REP: with REP = 2 even and odd lanes read
// disjoint halves of the LDS banks, so random codes collide less.
constexpr int kCb2CombBytes = 256 * 2 * 16 * 8;

template <int REP>
__device__ __forceinline__ half8 cb2_comb(uint32_t w, int odd, const uint8_t* tab_lane) {
  static_assert(REP == 1 || REP == 2, "replication 1 or 2");
  const uint32_t c = odd ? (w >> 16) : (w & 0xFFFFu);
  const uint32_t base = (c & 0xFFu) << (REP == 1 ? 8 : 9);
  const uint32_t a0 = base | (REP == 1 ? ((c >> 5) & 0x78u) : ((c >> 4) & 0xF0u));   // nib = flip & 15
  const uint32_t a1 = base | (REP == 1 ? ((c >> 9) & 0x78u) : ((c >> 8) & 0xF0u));   // nib = flip >> 4
  const uint2 lo = *reinterpret_cast<const uint2*>(tab_lane + a0);
  const uint2 hi = *reinterpret_cast<const uint2*>(tab_lane + 128 * REP + a1);
  return as_half8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// The 4 fp16 values T[idx][4*half .. 4*half+3]/4 of pair pr = 2*idx + half,
// packed as two dwords (from the 4 int8 table entries v).
__device__ __forceinline__ uint2 cb2_pair_values(const int8_t* v) {
  uint32_t w[2];
  for (int p = 0; p < 2; ++p) {
    const _Float16 lo = (_Float16)((float)v[2 * p] * 0.25f), hi = (_Float16)((float)v[2 * p + 1] * 0.25f);
    w[p] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return make_uint2(w[0], w[1]);
}

// Slot i (0 .. 8192*REP - 1, in memory order) of the table, from the pair
// values val4[pr] (cb2_pair_values).
template <int REP>
__device__ __forceinline__ void cb2_comb_put(uint8_t* tab, int i, const uint2* val4) {
  const int pr = i / (16 * REP), nib = (i / REP) & 15;
  const uint2 val = val4[pr];
  const uint32_t m01 = ((uint32_t)(nib & 1) << 15) | ((uint32_t)(nib & 2) << 30);
  const uint32_t m23 = ((uint32_t)(nib & 4) << 13) | ((uint32_t)(nib & 8) << 28);
  *reinterpret_cast<uint2*>(tab + (size_t)i * 8) = make_uint2(val.x ^ m01, val.y ^ m23);
}

// Builds the table with the whole workgroup; val4 is 4 KB of LDS scratch.
// Contains two barriers.
__device__ __forceinline__ void cb2_comb_fill(const int8_t* codebook, uint8_t* tab, uint2* val4, int tid,
                                              int nthreads) {
  for (int pr = tid; pr < 512; pr += nthreads) {
    int8_t v[4];
    for (int i = 0; i < 4; ++i) v[i] = codebook[(pr >> 1) * 8 + 4 * (pr & 1) + i];
    val4[pr] = cb2_pair_values(v);
  }
  __syncthreads();
  for (int i = tid; i < 512 * 16; i += nthreads) cb2_comb_put<1>(tab, i, val4);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// K2: the lane's 16 bytes are 4 words; word kb/2 holds kb.  For even kb the
// code pair of slot s (weights 2s, 2s+1) sits at bits 2s and 2s+16 (t = s);
// for odd kb slot 0 sits at bits 8, 24 (t = 4) and slots 1..3 at bits
// 10+2(s-1), 26+2(s-1), read after a 10-bit right shift (t = s - 1).

__device__ __forceinline__ int k2_slot_t(int kb, int s) {
  return (kb & 1) ? (s == 0 ? 4 : s - 1) : s;
}

// 4 words of magic fp16 pairs for k-block kb: value 1024 + 4^t q.
__device__ __forceinline__ u32x4 k2_magic(const u32x4& words, int kb) {
  const uint32_t w = words[kb >> 1];
  u32x4 r;
  if ((kb & 1) == 0) {
    r.x = (w & 0x00030003u) | 0x64006400u;
    r.y = (w & 0x000C000Cu) | 0x64006400u;
    r.z = (w & 0x00300030u) | 0x64006400u;
    r.w = (w & 0x00C000C0u) | 0x64006400u;
  } else {
    const uint32_t w10 = w >> 10;
    r.x = (w & 0x03000300u) | 0x64006400u;
    r.y = (w10 & 0x00030003u) | 0x64006400u;
    r.z = (w10 & 0x000C000Cu) | 0x64006400u;
    r.w = (w10 & 0x00300030u) | 0x64006400u;
  }
  return r;
}

// ---------------------------------------------------------------------------
// K4: words of half kb/4 (16 bytes per lane), word kb%4 holds kb; slot s
// (weights 2s, 2s+1) at bits 4s and 4s+16 (t = 0): value 1024 + q.
__device__ __forceinline__ u32x4 k4_magic(uint32_t w) {
  u32x4 r;
  r.x = (w & 0x000F000Fu) | 0x64006400u;
  r.y = ((w >> 4) & 0x000F000Fu) | 0x64006400u;
  r.z = ((w >> 8) & 0x000F000Fu) | 0x64006400u;
  r.w = ((w >> 12) & 0x000F000Fu) | 0x64006400u;
  return r;
}

// K4 six-bit value i (0..15) of a row's 12-byte scale stream.
__device__ __forceinline__ uint32_t k4_scale_value(uint32_t s0, uint32_t s1, uint32_t s2, int i) {
  const uint64_t lo = (uint64_t)s0 | ((uint64_t)s1 << 32);
  const int bit = 6 * i;
  uint64_t v;
  if (bit + 6 <= 64) v = lo >> bit;
  else if (bit >= 64) v = (uint64_t)s2 >> (bit - 64);
  else v = (lo >> bit) | ((uint64_t)s2 << (64 - bit));
  return (uint32_t)v & 63u;
}

}  // namespace qmoe_dev
