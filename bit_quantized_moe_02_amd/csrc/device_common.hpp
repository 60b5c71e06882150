// Device helpers shared by the libqmoe kernels: vector types, the fp16 MFMA,
// and the per-lane decoders of the CB2 / K2 / K4 / BF16 / Q8 tiles that
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
constexpr int kQ8Tile = 4352;

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
// Q8 tiles (8-bit codes, one fp16 scale d per 32 weights: w = d q).
// Byte offset of the 8 codes of (n, kb, qq) = lane c's k-block kb: 16-byte
// piece 2*(kb%2) + kb/4 holds k-blocks a and a + 2 of every lane.
__device__ __forceinline__ int q8_code_off(int kb, int c) {
  return 1024 * (2 * (kb & 1) + (kb >> 2)) + 16 * c + 8 * ((kb >> 1) & 1);
}
// Byte offset of row n's 8 fp16 scales (k-block kb at +2 kb).
__device__ __forceinline__ int q8_scale_off(int n) { return 4096 + 16 * n; }

// 8 signed 8-bit codes (two dwords, j = 0..7) -> their exact fp16 values:
// code b becomes the byte b ^ 0x80 = b + 128 in the mantissa of fp16 1024
// (0x64 in the high byte), i.e. 1152 + b, and 1152 is subtracted (exact).
__device__ __forceinline__ half8 q8_codes(uint32_t w0, uint32_t w1) {
  const uint32_t b0 = w0 ^ 0x80808080u, b1 = w1 ^ 0x80808080u;
  const uint32_t hi = 0x64646464u;
  u32x4 r;
  r.x = __builtin_amdgcn_perm(hi, b0, 0x04010400u);   // bytes 0, 1 of b0 under 0x64
  r.y = __builtin_amdgcn_perm(hi, b0, 0x04030402u);   // bytes 2, 3
  r.z = __builtin_amdgcn_perm(hi, b1, 0x04010400u);
  r.w = __builtin_amdgcn_perm(hi, b1, 0x04030402u);
  const _Float16 o = (_Float16)1152.0f;
  return as_half8(r) - half8{o, o, o, o, o, o, o, o};
}

// fp16(d q) for the 8 codes: the fp16 product of two fp16 numbers is the
// exact product rounded once, the fp16 value of the dequantized weight.
__device__ __forceinline__ half8 q8_fold(uint32_t w0, uint32_t w1, uint32_t d_bits) {
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)d_bits);
  return q8_codes(w0, w1) * half8{d, d, d, d, d, d, d, d};
}

// ---------------------------------------------------------------------------
// Per-token power-of-two scaling.  fp16 operands hold x and h in a range far
// narrower than bf16's, so every token t gets an exponent
//   e_t = floor(log2 max_i |x_ti|) - 1, clamped to [-kXExpMax, kXExpMax],
// the routed GEMMs take fp16(x_t * 2^-e_t) (its largest value in [2, 4)),
// and h is stored as fp16(h * 2^-2e_t): since |SiLU(g) u| <= |g| |u| and
// g, u scale with x, the stored h does not depend on the scale of x.  Sums
// are taken on the scaled values and the scale is removed in fp32 (exact:
// a power of two), so outside fp16's range limits the result is the same as
// with unscaled operands.
constexpr int kXExpMax = 60;

// Largest exponent field (bits 7..14) of the 8 bf16 values in v.
__device__ __forceinline__ uint32_t bf16x8_max_efield(const u32x4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, (v[i] >> 7) & 0xFFu);
    m = max(m, (v[i] >> 23) & 0xFFu);
  }
  return m;
}

// e_t from the largest bf16 exponent field of the token (0 for a token of
// zeros or subnormals, which gets the smallest exponent).
__device__ __forceinline__ int x_exp_of_field(uint32_t efield) {
  const int e = (int)efield - 128;
  return e < -kXExpMax ? -kXExpMax : (e > kXExpMax ? kXExpMax : e);
}

// Largest exponent field over a wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// 8 bf16 (16 bytes) times 2^-e -> half8 (the multiplication is exact; the
// fp16 conversion rounds once, only below fp16's normal range).
__device__ __forceinline__ half8 bf16x8_to_half8_exp(const u32x4& v, int e) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_ldexpf(__builtin_bit_cast(float, v[i] << 16), -e);
    const float hi = __builtin_ldexpf(__builtin_bit_cast(float, v[i] & 0xFFFF0000u), -e);
    half2v h = {(_Float16)lo, (_Float16)hi};
    r[i] = __builtin_bit_cast(uint32_t, h);
  }
  return as_half8(r);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// h * 2^-2e as fp16, from the fp32 sums of gate and up taken over inputs
// x * 2^-ea (ea = e for the scaled fp16 operands, 0 for raw bf16 ones):
// g = gsum 2^ea, h 2^-2e = (SiLU(g) 2^-e) (usum 2^(ea - e)).  With e = ea = 0
// this is fp16(SiLU(gsum) usum).
__device__ __forceinline__ _Float16 h_of(float gsum, float usum, int ea, int e) {
  const float g = __builtin_ldexpf(gsum, ea);
  return (_Float16)(__builtin_ldexpf(silu_f(g), -e) * __builtin_ldexpf(usum, ea - e));
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

// CB2 combined table (64 KB, the kernels place it at LDS offset 0): entry
// (idx, half, nib) holds the 4 fp16 values T[idx][4*half+i]/4, negated where
// bit i of nib is set, so a group of 8 weights is two 8-byte reads addressed
// straight from its 16-bit code (idx | flip << 8): half 0 takes flip bits
// 0..3, half 1 bits 4..7.  The entry sits at byte
//   half*32768 + idx*128 + nib*8.
// The sign nibbles are uniform over their 16 values, the indices are not
// (on Gaussian weights a handful of codebook rows take most codes).  The bank
// pair a read lands on follows its offset modulo 256, here
// (idx & 1)*128 + nib*8: 32 bank pairs, set mostly by the uniform nibble
// (an order keyed on idx crowds lanes with the common indices into the same
// banks).  Each offset is a shift, a mask and a bit-field insert of the code,
// the idx*128 term shared by the two.
constexpr int kCb2CombBytes = 256 * 2 * 16 * 8;

// A constant the compiler sees as an unknown scalar (vector) register value:
// expressions over it then select three-operand instructions (v_bfi_b32,
// v_and_or_b32) that take no literal constants, instead of a pair of
// two-operand ones with literals.  The empty asm emits nothing.
__device__ __forceinline__ uint32_t sreg(uint32_t c) {
  asm("" : "+s"(c));
  return c;
}
__device__ __forceinline__ uint32_t vreg(uint32_t c) {
  asm("" : "+v"(c));
  return c;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;

// LDS offset of a workgroup-memory pointer.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// The 8 fp16 table values of the code in the low (odd = 0) or high (odd = 1)
// half of the 32-bit word w.  tab is the table's LDS offset and must be a
// multiple of 32 KB (the entry offset is OR-ed into it): the kernels here
// place the table at offset 0 of their dynamic LDS and declare no static LDS.
__device__ __forceinline__ half8 cb2_comb(uint32_t w, int odd, uint32_t tab) {
  const uint32_t i7 = ((odd ? (w >> 9) : (w << 7)) & 0x7F80u) | tab;        // idx*128
  const uint32_t m = sreg(0x78u);
  const uint32_t lo_a = ((odd ? (w >> 21) : (w >> 5)) & m) | (i7 & ~m);    // + (flip & 15)*8
  const uint32_t hi_a = ((odd ? (w >> 25) : (w >> 9)) & m) | (i7 & ~m);    // + (flip >> 4)*8
  const u32x2 lo = *(lds_u32x2*)(size_t)lo_a;
  const u32x2 hi = *(lds_u32x2*)(size_t)(hi_a + 32768u);
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

// Slot i (0 .. 8191, in memory order: i = (half*256 + idx)*16 + nib) of the
// table, from the pair values val4[pr] (cb2_pair_values), pr = 2*idx + half.
__device__ __forceinline__ void cb2_comb_put(uint8_t* tab, int i, const uint2* val4) {
  const int nib = i & 15;
  const uint2 val = val4[2 * ((i >> 4) & 255) + (i >> 12)];
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
  for (int i = tid; i < 512 * 16; i += nthreads) cb2_comb_put(tab, i, val4);
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

// (a & mask) | c with the mask in a scalar and c in a vector register, one
// v_and_or_b32.
__device__ __forceinline__ uint32_t and_or_b32(uint32_t a, uint32_t mask, uint32_t c) {
  return (a & sreg(mask)) | c;
}

// 4 words of magic fp16 pairs for k-block kb: value 1024 + 4^t q.
__device__ __forceinline__ u32x4 k2_magic(const u32x4& words, int kb) {
  const uint32_t w = words[kb >> 1], m = vreg(0x64006400u);
  u32x4 r;
  if ((kb & 1) == 0) {
    r.x = and_or_b32(w, 0x00030003u, m);
    r.y = and_or_b32(w, 0x000C000Cu, m);
    r.z = and_or_b32(w, 0x00300030u, m);
    r.w = and_or_b32(w, 0x00C000C0u, m);
  } else {
    const uint32_t w10 = w >> 10;
    r.x = and_or_b32(w, 0x03000300u, m);
    r.y = and_or_b32(w10, 0x00030003u, m);
    r.z = and_or_b32(w10, 0x000C000Cu, m);
    r.w = and_or_b32(w10, 0x00300030u, m);
  }
  return r;
}

// ---------------------------------------------------------------------------
// K4: words of half kb/4 (16 bytes per lane), word kb%4 holds kb; slot s
// (weights 2s, 2s+1) at bits 4s and 4s+16 (t = 0): value 1024 + q.
__device__ __forceinline__ u32x4 k4_magic(uint32_t w) {
  const uint32_t m = vreg(0x64006400u);
  u32x4 r;
  r.x = and_or_b32(w, 0x000F000Fu, m);
  r.y = and_or_b32(w >> 4, 0x000F000Fu, m);
  r.z = and_or_b32(w >> 8, 0x000F000Fu, m);
  r.w = and_or_b32(w >> 12, 0x000F000Fu, m);
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
