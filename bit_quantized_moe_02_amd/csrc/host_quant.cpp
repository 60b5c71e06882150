// Host side of libqmoe: the CB2 codebook, fp64 -> fp16 rounding, the CB2 /
// K2 / K4 / Q8 quantizers and the tile packers, plus the thread-local error
// string.  No HIP dependency: this file builds with the host compiler alone.
//
// The formats and quantizer rules are the ones include/qmoe.h defines; the
// pages only name the formats ([digest] "Model weights": up/gate in a 2-bit
// codebook format, down in a 2-bit K-quant format; [osrepos] "Q4KExperts").
// The arithmetic is fp64 with no contraction into fused multiply-adds
// (built with -ffp-contract=off), so every comparison the quantizers make
// is decided on the same rounded values whatever machine runs it.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <thread>
#include <vector>

#include "../../include/qmoe.h"
#include "qmoe_internal.h"

namespace qmoe {
thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

ProfileHook& profile_hook() {
  static thread_local ProfileHook hook;
  return hook;
}

int tile_bytes(int fmt) {
  switch (fmt) {
    case MOE_FMT_CB2: return 1280;
    case MOE_FMT_K2: return 1344;
    case MOE_FMT_K4: return 2304;
    case MOE_FMT_BF16: return 8192;
    case MOE_FMT_Q8: return 4352;
    default: return 0;
  }
}

namespace {

// ---------------------------------------------------------------------------
// Rounding

// Nearest fp16 to a double, ties to even, in one rounding straight from the
// double's 53-bit significand.  Overflow gives infinity.
uint16_t f64_to_f16(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int biased = (int)((b >> 52) & 0x7FF);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (biased == 0x7FF) return (uint16_t)(sign | 0x7C00 | (frac ? 0x200 : 0));
  if (biased == 0) return sign;                 // fp64 subnormal: far below fp16
  const int e = biased - 1023;                  // x = 1.f * 2^e
  if (e > 15) return (uint16_t)(sign | 0x7C00);
  const uint64_t sig = frac | (1ull << 52);     // 53 significant bits
  // fp16 keeps 11 significant bits when normal (e >= -14); below that the
  // unit in the last place is fixed at 2^-24.
  const int drop = (e >= -14) ? 42 : 42 + (-14 - e);
  if (drop >= 54) return sign;                  // below half the smallest subnormal
  uint64_t kept = sig >> drop;
  const uint64_t rem = sig & ((1ull << drop) - 1);
  const uint64_t half = 1ull << (drop - 1);
  if (rem > half || (rem == half && (kept & 1))) ++kept;
  if (e >= -14) {
    int field = e + 15;
    if (kept == (1ull << 11)) {                 // rounded up to the next binade
      kept >>= 1;
      ++field;
    }
    if (field >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (field << 10) | (kept & 0x3FF));
  }
  return (uint16_t)(sign | kept);               // subnormal (kept == 1024 is the smallest normal)
}

double f16_to_f64(uint16_t h) {
  const int field = (h >> 10) & 0x1F;
  const int frac = h & 0x3FF;
  double v;
  if (field == 0) v = ldexp((double)frac, -24);
  else if (field == 31) v = frac ? NAN : INFINITY;
  else v = ldexp((double)(frac | 0x400), field - 25);
  return (h & 0x8000) ? -v : v;
}

// fp16 of x with a zero result stored as +0.
uint16_t f16_nonneg_zero(double x) {
  uint16_t h = f64_to_f16(x);
  return (h & 0x7FFF) == 0 ? 0 : h;
}

uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// CB2 index search.  The error of entry e for a group is
//   err(e) = (((t(0,b0) + t(1,b1)) + t(2,b2)) + ...) + t(7,b7),
//   t(j,b) = (|w_j| - s*(b ? 0.75 : 0.25))^2,  b_j = (|T[e][j]| == 3),
// a sum taken in j order.  Entries with the same magnitude pattern have the
// same error, so the sums are built once per pattern along a prefix tree
// (each node adds one more term to its parent's partial sum, exactly the
// partial sums of the j-ordered sum) and the entries are scanned per distinct
// pattern in order of their first index; ties keep the lower index.

struct Cb2Table {
  int8_t t[256][8];
  int n_patterns = 0;
  uint8_t pattern[256];       // distinct magnitude patterns, by first index
  uint8_t first_index[256];   // lowest entry with that pattern
};

void cb2_table_init(const int8_t* cb, Cb2Table* tab) {
  memcpy(tab->t, cb, 2048);
  bool seen[256] = {false};
  for (int e = 0; e < 256; ++e) {
    int p = 0;
    for (int j = 0; j < 8; ++j)
      if (cb[e * 8 + j] == 3 || cb[e * 8 + j] == -3) p |= 1 << j;
    if (!seen[p]) {
      seen[p] = true;
      tab->pattern[tab->n_patterns] = (uint8_t)p;
      tab->first_index[tab->n_patterns] = (uint8_t)e;
      ++tab->n_patterns;
    }
  }
}

int cb2_search(const Cb2Table& tab, const float* w, double s) {
  double term[8][2];
  const double v0 = s * 0.25, v1 = s * 0.75;
  for (int j = 0; j < 8; ++j) {
    const double a = fabs((double)w[j]);
    const double d0 = a - v0;
    const double d1 = a - v1;
    term[j][0] = d0 * d0;
    term[j][1] = d1 * d1;
  }
  // level l holds the 2^(l+1) partial sums over j = 0..l, indexed by the
  // bits b_0..b_l (bit j = b_j).
  double cur[256], nxt[256];
  cur[0] = term[0][0];
  cur[1] = term[0][1];
  int width = 2;
  for (int j = 1; j < 8; ++j) {
    for (int p = 0; p < width; ++p) {
      nxt[p] = cur[p] + term[j][0];
      nxt[p | width] = cur[p] + term[j][1];
    }
    width <<= 1;
    memcpy(cur, nxt, sizeof(double) * width);
  }
  double best = cur[tab.pattern[0]];
  int best_e = tab.first_index[0];
  for (int i = 1; i < tab.n_patterns; ++i) {
    const double err = cur[tab.pattern[i]];
    if (err < best) {   // patterns are in first-index order: strict < keeps the lowest
      best = err;
      best_e = tab.first_index[i];
    }
  }
  return best_e;
}

// ---------------------------------------------------------------------------
// Per-tile packers.  `rows` points at 16 rows of kp floats (row stride kp)
// starting at column kc*256; `tile` receives tile_bytes(fmt) bytes.

void put16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
}

bool pack_tile_cb2(const float* rows, int64_t stride, const Cb2Table& tab, uint8_t* tile) {
  for (int n = 0; n < 16; ++n) {
    const float* r = rows + n * stride;
    for (int kb = 0; kb < 8; ++kb) {
      const float* blk = r + 32 * kb;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = std::max(amax, fabs((double)blk[i]));
      const uint16_t sh = f16_nonneg_zero(amax / 0.75);
      if ((sh & 0x7C00) == 0x7C00) return false;      // scale not representable
      put16(tile + 1024 + 16 * n + 2 * kb, sh);
      const double s = f16_to_f64(sh);
      for (int qq = 0; qq < 4; ++qq) {
        const float* g = blk + 8 * qq;
        const int e = cb2_search(tab, g, s);
        uint32_t flip = 0;
        for (int j = 0; j < 8; ++j)
          if ((g[j] < 0.0f) != (tab.t[e][j] < 0)) flip |= 1u << j;
        const int lane = 16 * qq + n;
        put16(tile + 16 * lane + 2 * kb, (uint16_t)(e | (flip << 8)));
      }
    }
  }
  return true;
}

struct KqParams {
  int sub_len, qmax, smax;
};

// Quantizes one 256-weight super-block into q[256], sc[], m[] and d, dmin.
void kquant_superblock(const float* w, const KqParams& p, uint8_t* q, uint8_t* sc, uint8_t* m,
                       uint16_t* d_h, uint16_t* dmin_h) {
  const int nsb = 256 / p.sub_len;
  double a[16], b[16];
  double amax = 0.0, bmax = 0.0;
  for (int s = 0; s < nsb; ++s) {
    const float* x = w + s * p.sub_len;
    double lo = (double)x[0], hi = (double)x[0];
    for (int i = 1; i < p.sub_len; ++i) {
      lo = std::min(lo, (double)x[i]);
      hi = std::max(hi, (double)x[i]);
    }
    lo = std::min(0.0, lo);
    a[s] = (hi - lo) / (double)p.qmax;
    b[s] = 0.0 - lo;
    if (s == 0 || a[s] > amax) amax = a[s];
    if (s == 0 || b[s] > bmax) bmax = b[s];
  }
  *d_h = f16_nonneg_zero(amax / (double)p.smax);
  *dmin_h = f16_nonneg_zero(bmax / (double)p.smax);
  const double d = f16_to_f64(*d_h), dmin = f16_to_f64(*dmin_h);
  for (int s = 0; s < nsb; ++s) {
    const double scv = (d == 0.0) ? 0.0 : std::min((double)p.smax, floor(a[s] / d + 0.5));
    const double mv = (dmin == 0.0) ? 0.0 : std::min((double)p.smax, floor(b[s] / dmin + 0.5));
    sc[s] = (uint8_t)scv;
    m[s] = (uint8_t)mv;
    const double step = d * scv;
    const double off = dmin * mv;
    const float* x = w + s * p.sub_len;
    for (int i = 0; i < p.sub_len; ++i) {
      double qv = 0.0;
      if (step != 0.0) {
        qv = floor(((double)x[i] + off) / step + 0.5);
        qv = std::min((double)p.qmax, std::max(0.0, qv));
      }
      q[s * p.sub_len + i] = (uint8_t)qv;
    }
  }
}

void pack_tile_k2(const float* rows, int64_t stride, uint8_t* tile) {
  const KqParams p{16, 3, 15};
  memset(tile, 0, 1024);
  for (int n = 0; n < 16; ++n) {
    uint8_t q[256], sc[16], m[16];
    uint16_t dh, dmh;
    kquant_superblock(rows + n * stride, p, q, sc, m, &dh, &dmh);
    for (int kk = 0; kk < 256; ++kk) {
      const int kb = kk / 32, qq = (kk % 32) / 8, j = kk % 8;
      const int lane = 16 * qq + n;
      const int bit = 2 * (4 * (kb % 2) + j / 2) + 16 * (j % 2);
      uint8_t* word = tile + 16 * lane + 4 * (kb / 2);
      word[bit / 8] |= (uint8_t)(q[kk] << (bit % 8));
    }
    for (int s = 0; s < 16; ++s) tile[1024 + 16 * n + s] = (uint8_t)(sc[s] | (m[s] << 4));
    put16(tile + 1280 + 4 * n, dh);
    put16(tile + 1280 + 4 * n + 2, dmh);
  }
}

void pack_tile_k4(const float* rows, int64_t stride, uint8_t* tile) {
  const KqParams p{32, 15, 63};
  memset(tile, 0, 2048);
  for (int n = 0; n < 16; ++n) {
    uint8_t q[256], sc[8], m[8];
    uint16_t dh, dmh;
    kquant_superblock(rows + n * stride, p, q, sc, m, &dh, &dmh);
    for (int kk = 0; kk < 256; ++kk) {
      const int kb = kk / 32, qq = (kk % 32) / 8, j = kk % 8;
      const int lane = 16 * qq + n;
      const int bit = 4 * (j / 2) + 16 * (j % 2);
      uint8_t* word = tile + 1024 * (kb / 4) + 16 * lane + 4 * (kb % 4);
      word[bit / 8] |= (uint8_t)(q[kk] << (bit % 8));
    }
    // 16 six-bit values, sc0..sc7 then m0..m7, as a little-endian bit stream
    uint8_t* sb = tile + 2048 + 12 * n;
    memset(sb, 0, 12);
    for (int i = 0; i < 16; ++i) {
      const uint32_t v = (i < 8 ? sc[i] : m[i - 8]) & 63u;
      for (int bit = 0; bit < 6; ++bit)
        if (v & (1u << bit)) sb[(6 * i + bit) / 8] |= (uint8_t)(1u << ((6 * i + bit) % 8));
    }
    put16(tile + 2240 + 4 * n, dh);
    put16(tile + 2240 + 4 * n + 2, dmh);
  }
}

// Q8: per 32 weights d = fp16(max|w| / 127); q = nearest code to w/d with
// ties away from zero, clamped to -127..127.  Codes of (n, kb, qq) go to the
// 16-byte piece i of lane 16*qq + n that holds k-blocks 4*(i%2) + i/2 and that
// plus 2 (i = 2*(kb%2) + kb/4, second half when (kb/2) % 2 == 1).
bool pack_tile_q8(const float* rows, int64_t stride, uint8_t* tile) {
  for (int n = 0; n < 16; ++n) {
    const float* r = rows + n * stride;
    for (int kb = 0; kb < 8; ++kb) {
      const float* blk = r + 32 * kb;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = std::max(amax, fabs((double)blk[i]));
      const uint16_t dh = f16_nonneg_zero(amax / 127.0);
      if ((dh & 0x7C00) == 0x7C00) return false;      // scale not representable
      put16(tile + 4096 + 16 * n + 2 * kb, dh);
      const double d = f16_to_f64(dh);
      const int piece = 2 * (kb % 2) + kb / 4, half = (kb / 2) % 2;
      for (int i = 0; i < 32; ++i) {
        const double x = (double)blk[i];
        double mag = 0.0;
        if (d != 0.0) mag = std::min(127.0, floor(fabs(x) / d + 0.5));
        const int q = x < 0.0 ? -(int)mag : (int)mag;
        const int qq = i / 8, j = i % 8, lane = 16 * qq + n;
        tile[1024 * piece + 16 * lane + 8 * half + j] = (uint8_t)(int8_t)q;
      }
    }
  }
  return true;
}

void pack_tile_bf16(const float* rows, int64_t stride, uint8_t* tile) {
  for (int n = 0; n < 16; ++n)
    for (int kk = 0; kk < 256; ++kk) {
      const int kb = kk / 32, qq = (kk % 32) / 8, j = kk % 8;
      put16(tile + 1024 * kb + 16 * (16 * qq + n) + 2 * j, f32_to_bf16(rows[n * stride + kk]));
    }
}

}  // namespace
}  // namespace qmoe

using namespace qmoe;

extern "C" const char* moe_last_error(void) { return g_last_error.c_str(); }

extern "C" int moe_codebook_generate(uint64_t seed, int8_t* table_out) {
  clear_error();
  if (!table_out) return fail(MOE_ERR_INVALID_ARG, "moe_codebook_generate: table_out is NULL");
  static const int8_t value[4] = {-3, -1, 1, 3};
  uint64_t state = seed;
  for (int i = 0; i < 2048; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    table_out[i] = value[z >> 62];
  }
  return MOE_OK;
}

// True when some fp16 scale of the packed matrix would not be finite: CB2's
// s = fp16(max|w| / 0.75) or Q8's d = fp16(max|w| / 127) over a 32-weight group, or a K-quant super-block's
// d = fp16(max_s a_s / S) or dmin = fp16(max_s b_s / S).  fp16 rounding is
// monotone, so the largest group or sub-block decides; columns past k are the
// zeros the packers pad with.  Checked before any output byte is written.
static bool scale_overflows(int fmt, const float* w, int64_t rows, int64_t k) {
  if (fmt == MOE_FMT_CB2 || fmt == MOE_FMT_Q8) {
    double amax = 0.0;
    for (int64_t i = 0; i < rows * k; ++i) amax = std::max(amax, fabs((double)w[i]));
    return (f16_nonneg_zero(amax / (fmt == MOE_FMT_CB2 ? 0.75 : 127.0)) & 0x7C00) == 0x7C00;
  }
  if (fmt != MOE_FMT_K2 && fmt != MOE_FMT_K4) return false;
  const KqParams p = fmt == MOE_FMT_K2 ? KqParams{16, 3, 15} : KqParams{32, 15, 63};
  double amax = 0.0, bmax = 0.0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < k; c += p.sub_len) {
      const float* x = w + r * k + c;
      const int64_t n = std::min<int64_t>(p.sub_len, k - c);
      double lo = (double)x[0], hi = (double)x[0];
      for (int64_t i = 1; i < n; ++i) {
        lo = std::min(lo, (double)x[i]);
        hi = std::max(hi, (double)x[i]);
      }
      if (n < p.sub_len) hi = std::max(hi, 0.0);       // padded zeros
      lo = std::min(0.0, lo);
      amax = std::max(amax, (hi - lo) / (double)p.qmax);
      bmax = std::max(bmax, 0.0 - lo);
    }
  return (f16_nonneg_zero(amax / (double)p.smax) & 0x7C00) == 0x7C00 ||
         (f16_nonneg_zero(bmax / (double)p.smax) & 0x7C00) == 0x7C00;
}

extern "C" size_t moe_packed_bytes(int fmt, int64_t rows, int64_t k) {
  const int tb = tile_bytes(fmt);
  if (tb == 0 || rows <= 0 || rows % 16 != 0 || k < 1) return 0;
  return (size_t)(rows / 16) * (size_t)(pad256(k) / 256) * (size_t)tb;
}

extern "C" int moe_quantize_pack(int fmt, const float* w, int64_t rows, int64_t k,
                                 const int8_t* codebook, void* out, size_t out_bytes,
                                 int n_threads) {
  clear_error();
  const size_t need = moe_packed_bytes(fmt, rows, k);
  if (need == 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: unknown format or rows not a positive "
                                     "multiple of 16 or k < 1");
  if (!w || !out) return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: NULL pointer");
  if (out_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: out_bytes " + std::to_string(out_bytes) +
                                         " < " + std::to_string(need));
  if (fmt == MOE_FMT_CB2 && !codebook)
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: CB2 needs the codebook");
  if (fmt == MOE_FMT_CB2)
    for (int i = 0; i < 2048; ++i)
      if (codebook[i] != -3 && codebook[i] != -1 && codebook[i] != 1 && codebook[i] != 3)
        return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: codebook values must be in {-3,-1,1,3}");
  for (int64_t i = 0; i < rows * k; ++i)
    if (!std::isfinite(w[i])) return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: non-finite weight");
  if (scale_overflows(fmt, w, rows, k))
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: |w| too large for an fp16 scale");

  const int64_t kp = pad256(k);
  const int64_t n_rt = rows / 16, n_kc = kp / 256;
  const int tb = tile_bytes(fmt);
  Cb2Table tab;
  if (fmt == MOE_FMT_CB2) cb2_table_init(codebook, &tab);
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::min<int64_t>(nt, n_rt);
  std::vector<int> ok(nt, 1);
  auto worker = [&](int tid) {
    std::vector<float> buf(16 * (size_t)kp);
    for (int64_t rt = tid; rt < n_rt; rt += nt) {
      std::fill(buf.begin(), buf.end(), 0.0f);
      for (int n = 0; n < 16; ++n)
        memcpy(buf.data() + n * kp, w + (rt * 16 + n) * k, sizeof(float) * (size_t)k);
      for (int64_t kc = 0; kc < n_kc; ++kc) {
        uint8_t* tile = (uint8_t*)out + (size_t)(rt * n_kc + kc) * tb;
        const float* src = buf.data() + kc * 256;
        switch (fmt) {
          case MOE_FMT_CB2:
            if (!pack_tile_cb2(src, kp, tab, tile)) ok[tid] = 0;
            break;
          case MOE_FMT_K2: pack_tile_k2(src, kp, tile); break;
          case MOE_FMT_K4: pack_tile_k4(src, kp, tile); break;
          case MOE_FMT_Q8:
            if (!pack_tile_q8(src, kp, tile)) ok[tid] = 0;
            break;
          default: pack_tile_bf16(src, kp, tile); break;
        }
      }
    }
  };
  if (nt == 1) {
    worker(0);
  } else {
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t) th.emplace_back(worker, t);
    for (auto& t : th) t.join();
  }
  for (int t = 0; t < nt; ++t)      // (scale_overflows has ruled this out)
    if (!ok[t]) return fail(MOE_ERR_INVALID_ARG, "moe_quantize_pack: |w| too large for an fp16 scale");
  return MOE_OK;
}
