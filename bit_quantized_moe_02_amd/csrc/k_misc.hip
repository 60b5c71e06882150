// Test decoder of packed matrices and the stable expert grouping of slots.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmoe.h"
#include "device_common.hpp"
#include "k_misc.h"
#include "launch_util.h"

using namespace qmoe_dev;

namespace {

// Decodes packed tiles to fp32 with the FFN kernels' lane decoders: each
// wave takes one tile at a time; lane c writes weights (n, kb, qq, j) of its
// slice.  Every value is the exact format value rounded once to fp32:
//   CB2: s * (T/4, sign flipped), exact;  K2/K4: fma(-dmin, m, d*sc*q), where
//   d*sc*q is exact in fp32 and the fma rounds once;  BF16: the value itself.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* packed, int64_t n_rt, int64_t n_kc,
                                                      const int8_t* codebook, float* out) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* val_tab = smem;
  uint8_t* flip_tab = smem + kCb2TableBytes;
  if (FMT == MOE_FMT_CB2) {
    cb2_fill_tables(codebook, val_tab, flip_tab, threadIdx.x, blockDim.x);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, qq = lane >> 4;
  const int64_t kp = n_kc * 256;
  const int64_t n_tiles = n_rt * n_kc;
  const int waves = (blockDim.x >> 6) * gridDim.x;
  for (int64_t tile_i = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); tile_i < n_tiles;
       tile_i += waves) {
    const int64_t rt = tile_i / n_kc, kc = tile_i % n_kc;
    float* orow = out + (rt * 16 + n) * kp + kc * 256 + qq * 8;
    if (FMT == MOE_FMT_CB2) {
      const uint8_t* tile = packed + tile_i * kCb2Tile;
      const u32x4 codes = load16(tile + 16 * lane);
      const u32x4 scl = load16(tile + 1024 + 16 * n);
      for (int kb = 0; kb < 8; ++kb) {
        const half8 v = cb2_group((codes[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu, val_tab + (lane & 7) * 16,
                                  flip_tab + (lane & 7) * 16);
        const float s = h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu);
        for (int j = 0; j < 8; ++j) orow[kb * 32 + j] = s * (float)v[j];
      }
    } else if (FMT == MOE_FMT_K2) {
      const uint8_t* tile = packed + tile_i * kK2Tile;
      const u32x4 qw = load16(tile + 16 * lane);
      const u32x4 scm = load16(tile + 1024 + 16 * n);
      const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 1280 + 4 * n);
      const float d = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
      for (int kb = 0; kb < 8; ++kb) {
        const half8 v = as_half8(k2_magic(qw, kb));
        const int sb = 2 * kb + (qq >> 1);
        const uint32_t byte = (scm[sb >> 2] >> (8 * (sb & 3))) & 0xFFu;
        const float dsc = d * (float)(byte & 15u), mn = (float)(byte >> 4);
        for (int j = 0; j < 8; ++j) {
          const float q = ((float)v[j] - 1024.0f) * __builtin_ldexpf(1.0f, -2 * k2_slot_t(kb, j >> 1));
          orow[kb * 32 + j] = fmaf(-dmin, mn, dsc * q);
        }
      }
    } else if (FMT == MOE_FMT_K4) {
      const uint8_t* tile = packed + tile_i * kK4Tile;
      const u32x4 q0 = load16(tile + 16 * lane);
      const u32x4 q1 = load16(tile + 1024 + 16 * lane);
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(tile + 2048 + 12 * n);
      const uint32_t s0 = sp[0], s1 = sp[1], s2 = sp[2];
      const uint32_t dd = *reinterpret_cast<const uint32_t*>(tile + 2240 + 4 * n);
      const float d = h2f(dd & 0xFFFFu), dmin = h2f(dd >> 16);
      for (int kb = 0; kb < 8; ++kb) {
        const half8 v = as_half8(k4_magic(kb < 4 ? q0[kb & 3] : q1[kb & 3]));
        const float dsc = d * (float)k4_scale_value(s0, s1, s2, kb);
        const float mn = (float)k4_scale_value(s0, s1, s2, 8 + kb);
        for (int j = 0; j < 8; ++j) orow[kb * 32 + j] = fmaf(-dmin, mn, dsc * ((float)v[j] - 1024.0f));
      }
    } else if (FMT == MOE_FMT_Q8) {
      const uint8_t* tile = packed + tile_i * kQ8Tile;
      const u32x4 scl = load16(tile + q8_scale_off(n));
      for (int kb = 0; kb < 8; ++kb) {
        const uint32_t* cp = reinterpret_cast<const uint32_t*>(tile + q8_code_off(kb, lane));
        const half8 v = q8_codes(cp[0], cp[1]);
        const float d = h2f((scl[kb >> 1] >> (16 * (kb & 1))) & 0xFFFFu);
        for (int j = 0; j < 8; ++j) orow[kb * 32 + j] = d * (float)v[j];
      }
    } else {
      const uint8_t* tile = packed + tile_i * kBf16Tile;
      for (int kb = 0; kb < 8; ++kb) {
        const u32x4 raw = load16(tile + 1024 * kb + 16 * lane);
        for (int j = 0; j < 8; ++j) orow[kb * 32 + j] = bf2f((raw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      }
    }
  }
}

// Stable counting sort of the slots by expert, one workgroup of 16 waves.
// Wave w owns the contiguous slot range [w*S, (w+1)*S): it counts its
// experts, the counts are scanned (expert-major, then wave order), and each
// wave writes its slots in slot order, ranking equal experts inside every
// 64-slot chunk with a lane-order count.  A wave loads the expert ids of
// kGroupBatch chunks together (one memory latency per batch, not per chunk).
constexpr int kGroupWaves = 16;
constexpr int kGroupBatch = 16;

__global__ __launch_bounds__(1024) void group_kernel(const int32_t* topk_idx, int n_slots, int E,
                                                     int32_t* offsets, int32_t* sorted_slots,
                                                     int32_t* slot_pos, int* err_count) {
  extern __shared__ __align__(16) int gsm[];
  int* cnt = gsm;                          // [16][E]: counts, then running cursors
  int* tot = gsm + kGroupWaves * E;        // [E + 1]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kGroupWaves * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int S = (n_slots + kGroupWaves - 1) / kGroupWaves;
  const int s0 = wave * S, s1 = min(n_slots, s0 + S);
  // ids of slots cb + 64 i + lane, i < kGroupBatch (only called with
  // s0 <= cb < s1; a lane past s1 reads slot s1 - 1 and ignores it)
  auto load_ids = [&](int cb, int (&ev)[kGroupBatch]) {
#pragma unroll
    for (int i = 0; i < kGroupBatch; ++i) {
      const int s = cb + 64 * i + lane;
      ev[i] = topk_idx[s < s1 ? s : s1 - 1];
    }
  };
  int bad = 0;
  for (int cb = s0; cb < s1; cb += 64 * kGroupBatch) {
    int ev[kGroupBatch];
    load_ids(cb, ev);
#pragma unroll
    for (int i = 0; i < kGroupBatch; ++i) {
      // (no branch before the id is used: a load whose value is read only
      // inside a branch is moved into it, and then waited for alone)
      const int e = ev[i];
      const bool in = cb + 64 * i + lane < s1, valid = in & (e >= 0) & (e < E);
      if (valid) atomicAdd(&cnt[wave * E + e], 1);
      bad += in & !valid;
    }
  }
  __syncthreads();
  // per expert: cursors = exclusive prefix over waves, totals
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < kGroupWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();
  // exclusive scan of the totals in expert order, by wave 0: lane l sums
  // experts [l*P, l*P + P), the lane sums are scanned across the wave
  if (wave == 0) {
    const int P = (E + 63) / 64, e0 = lane * P, e1 = min(E, e0 + P);
    int part = 0;
    for (int e = e0; e < e1; ++e) part += tot[e];
    int incl = part;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int run = incl - part;
    for (int e = e0; e < e1; ++e) {
      const int c = tot[e];
      tot[e] = run;
      offsets[e] = run;
      run += c;
    }
    if (lane == 63) {
      tot[E] = incl;
      offsets[E] = incl;
    }
  }
  __syncthreads();
  const int id_bits = 32 - __builtin_clz((unsigned)(E > 1 ? E - 1 : 1));   // bits of an id in [0, E)
  for (int cb = s0; cb < s1; cb += 64 * kGroupBatch) {
    int ev[kGroupBatch];
    load_ids(cb, ev);
#pragma unroll
    for (int i = 0; i < kGroupBatch; ++i) {
      const int c0 = cb + 64 * i;
      if (c0 >= s1) break;                       // the same for the whole wave
      const int s = c0 + lane;
      const int e = (s < s1) ? ev[i] : -1;
      const bool valid = e >= 0 && e < E;
      // lanes holding the same id: intersect, bit by bit, the ballots of the
      // lanes that agree with this lane's id bit
      uint64_t match = ~0ull;
      for (int b = 0; b < id_bits; ++b) {
        const uint64_t ones = __ballot((e >> b) & 1);
        match &= ((e >> b) & 1) ? ones : ~ones;
      }
      match &= __ballot(valid);
      const int rank = __popcll(match & ((1ull << lane) - 1ull));
      const int same = __popcll(match);
      int cursor = 0;
      if (valid) cursor = cnt[wave * E + e];
      if (valid) {
        const int pos = tot[e] + cursor + rank;
        sorted_slots[pos] = s;
        slot_pos[s] = pos;
      } else if (s < s1) {
        slot_pos[s] = -1;
      }
      // the last lane of each expert in this chunk advances the cursor
      if (valid && rank == same - 1) cnt[wave * E + e] = cursor + same;
    }
  }
  for (int o = 1; o < 64; o <<= 1) bad += __shfl_xor(bad, o);
  if (lane == 0 && bad) atomicAdd(err_count, bad);
}

// Streaming read of n16 16-byte vectors: each is loaded once, coalesced, with
// kReadUnroll loads in flight per thread, and the XOR of every word goes to
// *out (an integer XOR: order-independent) so no load can be dropped.  A
// plain HBM-bound kernel whose rate is the measured ceiling of the
// bandwidth-bound decode kernels at the same byte count.
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* src, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0 && acc) atomicXor(out, acc);
}

}  // namespace

namespace qmoe {

hipError_t launch_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t s) {
  return launch_timed(MOE_KERNEL_READ, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, s, ev0_, ev1_, 0, (const u32x4*)src,
                          (int64_t)(bytes / 16), out);
  });
}

hipError_t launch_dequant(int fmt, const uint8_t* packed, int64_t rows, int64_t kp, const int8_t* codebook,
                          float* out, hipStream_t s) {
  const int64_t n_rt = rows / 16, n_kc = kp / 256;
  const int64_t n_tiles = n_rt * n_kc;
  const int grid = (int)((n_tiles + 3) / 4 < 1024 ? (n_tiles + 3) / 4 : 1024);
  const size_t lds = (fmt == MOE_FMT_CB2) ? 2 * kCb2TableBytes : 0;
  void (*fn)(const uint8_t*, int64_t, int64_t, const int8_t*, float*) = nullptr;
  switch (fmt) {
    case MOE_FMT_CB2: fn = dequant_kernel<MOE_FMT_CB2>; break;
    case MOE_FMT_K2: fn = dequant_kernel<MOE_FMT_K2>; break;
    case MOE_FMT_K4: fn = dequant_kernel<MOE_FMT_K4>; break;
    case MOE_FMT_Q8: fn = dequant_kernel<MOE_FMT_Q8>; break;
    default: fn = dequant_kernel<MOE_FMT_BF16>; break;
  }
  if (lds > 0) {
    hipError_t err = ensure_dyn_lds((const void*)fn);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, s, packed, n_rt, n_kc, codebook, out);
  return hipGetLastError();
}

size_t group_lds(int E) { return (size_t)(kGroupWaves * E + E + 1) * 4; }

hipError_t launch_group(const int32_t* topk_idx, int n_slots, int E, int32_t* offsets, int32_t* sorted_slots,
                        int32_t* slot_pos, int* err_count, hipStream_t s) {
  const size_t lds = group_lds(E);
  hipError_t err = ensure_dyn_lds((const void*)group_kernel);
  if (err != hipSuccess) return err;
  return launch_timed(MOE_KERNEL_GROUP, s, [&](hipEvent_t ev0_, hipEvent_t ev1_) {
    hipExtLaunchKernelGGL(group_kernel, dim3(1), dim3(64 * kGroupWaves), lds, s, ev0_, ev1_, 0, topk_idx, n_slots, E, offsets,
                       sorted_slots, slot_pos, err_count);
  });
}

}  // namespace qmoe
