// C ABI of libqmoe (include/qmoe.h): argument checks, workspace layout and
// kernel launches.  Every check happens before anything is enqueued; a
// failing call returns its MOE_ERR_* code with a message and touches no
// output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <string>

#include "../../include/qmoe.h"
#include "k_decode.h"
#include "k_misc.h"
#include "k_prefill.h"
#include "k_route.h"
#include "qmoe_internal.h"

using namespace qmoe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_fail(const char* where, hipError_t e) {
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

int n_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Shape and pointer checks of a weight set; on success fills the derived
// sizes.
struct Geometry {
  int E, H, I, Is, I_pad, Is_pad;
  int fmt_ug, fmt_dn, fmt_s;
  size_t up_bytes, down_bytes;
};

int check_weights(const moe_weights* w, Geometry* g, const char* fn) {
  const std::string f(fn);
  if (!w) return fail(MOE_ERR_INVALID_ARG, f + ": weights is NULL");
  if (w->n_experts < 1 || w->n_experts > 1024)
    return fail(MOE_ERR_INVALID_ARG, f + ": n_experts must be in [1, 1024]");
  if (w->hidden < 256 || w->hidden % 256 != 0 || w->hidden > 8192)
    return fail(MOE_ERR_INVALID_ARG, f + ": hidden must be a multiple of 256 in [256, 8192]");
  if (w->inter < 16 || w->inter % 16 != 0 || w->inter > 16384)
    return fail(MOE_ERR_INVALID_ARG, f + ": inter must be a multiple of 16 in [16, 16384]");
  if (w->shared_inter < 0 || w->shared_inter % 16 != 0 || w->shared_inter > 16384)
    return fail(MOE_ERR_INVALID_ARG, f + ": shared_inter must be 0 or a multiple of 16 (<= 16384)");
  const bool cb2 = w->fmt_up == MOE_FMT_CB2 && w->fmt_gate == MOE_FMT_CB2 && w->fmt_down == MOE_FMT_K2;
  const bool k4 = w->fmt_up == MOE_FMT_K4 && w->fmt_gate == MOE_FMT_K4 && w->fmt_down == MOE_FMT_K4;
  if (!cb2 && !k4)
    return fail(MOE_ERR_UNSUPPORTED, f + ": formats must be (CB2, CB2, K2) or (K4, K4, K4)");
  if (!w->up || !w->gate || !w->down) return fail(MOE_ERR_INVALID_ARG, f + ": expert weight pointer is NULL");
  if (!aligned16(w->up) || !aligned16(w->gate) || !aligned16(w->down))
    return fail(MOE_ERR_INVALID_ARG, f + ": expert weights must be 16-byte aligned");
  if (cb2 && !w->codebook) return fail(MOE_ERR_INVALID_ARG, f + ": CB2 weights need the codebook");
  if (cb2 && !aligned16(w->codebook)) return fail(MOE_ERR_INVALID_ARG, f + ": the codebook must be 16-byte aligned");
  if (w->fmt_shared != MOE_FMT_BF16 && w->fmt_shared != MOE_FMT_Q8)
    return fail(MOE_ERR_UNSUPPORTED, f + ": fmt_shared must be MOE_FMT_BF16 or MOE_FMT_Q8");
  if (w->shared_inter > 0) {
    if (!w->shared_up || !w->shared_gate || !w->shared_down)
      return fail(MOE_ERR_INVALID_ARG, f + ": shared expert pointer is NULL");
    if (!aligned16(w->shared_up) || !aligned16(w->shared_gate) || !aligned16(w->shared_down))
      return fail(MOE_ERR_INVALID_ARG, f + ": shared expert weights must be 16-byte aligned");
  }
  g->E = w->n_experts;
  g->H = w->hidden;
  g->I = w->inter;
  g->Is = w->shared_inter;
  g->I_pad = (int)pad256(w->inter);
  g->Is_pad = (int)pad256(w->shared_inter > 0 ? w->shared_inter : 1);
  g->fmt_ug = w->fmt_up;
  g->fmt_dn = w->fmt_down;
  g->fmt_s = w->fmt_shared;
  g->up_bytes = moe_packed_bytes(w->fmt_up, w->inter, w->hidden);
  g->down_bytes = moe_packed_bytes(w->fmt_down, w->hidden, w->inter);
  return MOE_OK;
}

}  // namespace

// The weight checks of the decode and prefill calls, for other translation
// units (the expert cache validates its host layer with them).
int qmoe::validate_weights(const moe_weights* w, const char* fn) {
  Geometry g;
  return check_weights(w, &g, fn);
}

namespace {

// Up to this many tokens the decode call runs the single-token kernels once
// per token; beyond, the batched kernels that read each distinct expert once.
constexpr int kDecPerTokenMax = 3;

struct DecLayout {
  size_t h, hs, hsum, ybuf, ysh, xexp, total;
};

DecLayout dec_layout(const Geometry& g, int T, int k) {
  DecLayout L;
  size_t off = 0;
  L.h = off;
  off = align_up(off + (size_t)T * k * g.I * 2);
  L.hs = off;
  off = align_up(off + (size_t)T * (g.Is > 0 ? g.Is : 1) * 2);
  L.hsum = off;
  off = align_up(off + (size_t)T * k * (g.I_pad / 16) * 2 * 4);
  L.ybuf = off;
  off = align_up(off + (size_t)T * k * g.H * 4);
  L.ysh = off;
  off = align_up(off + (size_t)T * g.H * 4);
  L.xexp = off;
  off = align_up(off + (size_t)T * 4);
  L.total = off;
  return L;
}

struct PfLayout {
  size_t h, hs, yslot, ysh, xexp, epos, total;
};

PfLayout pf_layout(const Geometry& g, int64_t T, int k) {
  PfLayout L;
  size_t off = 0;
  L.h = off;
  off = align_up(off + (size_t)T * k * g.I * 2);
  L.hs = off;
  off = align_up(off + (size_t)T * (g.Is > 0 ? g.Is : 1) * 2);
  L.yslot = off;
  off = align_up(off + (size_t)T * k * g.H * 4);
  L.ysh = off;
  off = align_up(off + (size_t)T * g.H * 4);
  L.xexp = off;
  off = align_up(off + (size_t)T * 4);
  L.epos = off;
  off = align_up(off + (size_t)T * k * 4);
  L.total = off;
  return L;
}

}  // namespace

// ---------------------------------------------------------------------------

extern "C" size_t moe_route_workspace_bytes(int32_t T, int32_t E) {
  if (T < 1 || E < 1) return 0;
  return align_up(route_logit_floats(T, E) * 4);
}

extern "C" int moe_route(const void* x_bf16, const float* w_router, const float* logit_bias, int32_t T,
                         int32_t H, int32_t E, int32_t k, int32_t* topk_idx, float* topk_w, void* ws,
                         size_t ws_bytes, void* stream) {
  clear_error();
  if (!x_bf16 || !w_router || !topk_idx || !topk_w || !ws)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: NULL pointer");
  if (T < 1 || H < 8 || H % 8 != 0 || E < 1 || E > 1024)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: need T >= 1, H a positive multiple of 8, 1 <= E <= 1024");
  if (k < 1 || k > E || k > 16) return fail(MOE_ERR_INVALID_ARG, "moe_route: need 1 <= k <= min(E, 16)");
  if (!aligned16(x_bf16) || !aligned16(w_router))
    return fail(MOE_ERR_INVALID_ARG, "moe_route: x and w_router must be 16-byte aligned");
  if (ws_bytes < moe_route_workspace_bytes(T, E))
    return fail(MOE_ERR_WORKSPACE, "moe_route: workspace too small");
  hipError_t e = launch_route((const uint16_t*)x_bf16, w_router, logit_bias, T, H, E, k, (float*)ws, topk_idx,
                              topk_w, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("moe_route", e);
  return MOE_OK;
}

extern "C" size_t moe_group_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (T < 1 || k < 1 || E < 1) return 0;
  return kAlign;
}

extern "C" int moe_group_tokens(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_pos, void* ws,
                                size_t ws_bytes, void* stream) {
  clear_error();
  if (!topk_idx || !expert_offsets || !sorted_slots || !slot_pos || !ws)
    return fail(MOE_ERR_INVALID_ARG, "moe_group_tokens: NULL pointer");
  if (T < 1 || k < 1 || k > 16 || E < 1 || E > 1024 || (int64_t)T * k > (1 << 22))
    return fail(MOE_ERR_INVALID_ARG, "moe_group_tokens: need T >= 1, 1 <= k <= 16, 1 <= E <= 1024, T*k <= 2^22");
  if (ws_bytes < moe_group_workspace_bytes(T, k, E))
    return fail(MOE_ERR_WORKSPACE, "moe_group_tokens: workspace too small");
  hipError_t e = launch_group(topk_idx, T * k, E, expert_offsets, sorted_slots, slot_pos, (int*)ws,
                              (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("moe_group_tokens", e);
  return MOE_OK;
}

extern "C" size_t moe_ffn_workspace_bytes(const moe_weights* w, int32_t T, int32_t k, int prefill) {
  Geometry g;
  if (check_weights(w, &g, "moe_ffn_workspace_bytes") != MOE_OK) return 0;
  if (T < 1 || k < 1 || k > 16) return 0;
  if (!prefill) {
    if (T > 16) return 0;
    return dec_layout(g, T, k).total;
  }
  return pf_layout(g, T, k).total;
}

namespace {

// Router output that the decode kernels take instead of given top-k: the
// partial logits of all T tokens; the single-token CB2 up/gate ranks each
// token itself and writes topk_idx / topk_w.
struct DecRoute {
  const float* logits;
  int n_parts;
};

// Checks of the decode entry points that do not depend on routing.
int check_decode(const char* who, const moe_weights* w, Geometry* g, const void* x_bf16, int32_t T, int32_t k,
                 const void* topk_idx, const void* topk_w, const float* y, const void* ws) {
  int rc = check_weights(w, g, who);
  if (rc != MOE_OK) return rc;
  if (!x_bf16 || !topk_idx || !topk_w || !y || !ws) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": NULL pointer");
  if (T < 1 || T > 16) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": T must be in [1, 16]");
  if (k < 1 || k > 16 || k > g->E)
    return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": need 1 <= k <= min(E, 16)");
  if (!aligned16(x_bf16) || !aligned16(ws) || !aligned16(y))
    return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": x, y and ws must be 16-byte aligned");
  return MOE_OK;
}

// The expert FFN for 1..16 tokens.  With route != null, topk_idx / topk_w
// are outputs: the single-token CB2 path ranks each token's experts inside
// its up/gate kernel; every other path runs the top-k kernel first.
int run_decode(const char* who, const moe_weights* w, const Geometry& g, const void* x_bf16, int32_t T,
               int32_t k, int32_t* topk_idx, float* topk_w, float* y, uint8_t* wsb, hipStream_t s,
               const DecRoute* route) {
  const DecLayout L = dec_layout(g, T, k);
  DecArgs a{};
  a.x = (const uint16_t*)x_bf16;
  a.T = T;
  a.H = g.H;
  a.I = g.I;
  a.Is = g.Is;
  a.I_pad = g.I_pad;
  a.Is_pad = g.Is_pad;
  a.k = k;
  a.E = g.E;
  const int n_chunks = g.H / 256;
  const int cpw = n_chunks > 16 ? 2 : 1;
  a.nw_ug = (n_chunks + cpw - 1) / cpw;
  if (a.nw_ug < 4) a.nw_ug = 4;
  int nd = g.I_pad / 256;
  a.nw_dn = nd < 4 ? 4 : (nd > 16 ? 16 : nd);
  a.tb_ug = tile_bytes(g.fmt_ug);
  a.tb_dn = tile_bytes(g.fmt_dn);
  a.topk_idx = topk_idx;
  a.up = (const uint8_t*)w->up;
  a.gate = (const uint8_t*)w->gate;
  a.down = (const uint8_t*)w->down;
  a.expert_bytes = g.up_bytes;
  a.expert_bytes_down = g.down_bytes;
  a.sup = (const uint8_t*)w->shared_up;
  a.sgate = (const uint8_t*)w->shared_gate;
  a.sdown = (const uint8_t*)w->shared_down;
  a.fmt_s = g.fmt_s;
  a.tb_s = tile_bytes(g.fmt_s);
  a.codebook = w->codebook;
  a.h = (_Float16*)(wsb + L.h);
  a.hs = (_Float16*)(wsb + L.hs);
  a.hsum = (float*)(wsb + L.hsum);
  a.ybuf = (float*)(wsb + L.ybuf);
  a.ysh = (float*)(wsb + L.ysh);
  a.xexp = (int*)(wsb + L.xexp);
  const int cus = n_cus();
  if (T <= kDecPerTokenMax && dec1_down_lds(a, g.fmt_dn, 16) <= 160 * 1024) {
    // few tokens: the single-token kernels once per token (exact weights)
    const int nw_cb2 = n_chunks < 4 ? 4 : n_chunks;
    // (one token only: for more, one top-k launch for all of them is cheaper
    // than ranking inside each token's up/gate)
    const bool route_here = route && T == 1 && g.fmt_ug == MOE_FMT_CB2 && n_chunks <= 16 &&
                            g.E <= 64 * nw_cb2 && route->n_parts == 1 &&
                            dec1_cb2_upgate_lds(nw_cb2, true) <= 160 * 1024;
    if (route && !route_here) {
      hipError_t e = launch_route_topk(route->logits, route->n_parts, T, g.E, k, topk_idx, topk_w, s);
      if (e != hipSuccess) return hip_fail(who, e);
    }
    for (int t = 0; t < T; ++t) {
      DecArgs at = a;
      at.T = 1;
      at.x = a.x + (size_t)t * g.H;
      at.topk_idx = topk_idx + (size_t)t * k;
      at.h = a.h + (size_t)t * k * g.I;
      at.hs = a.hs + (size_t)t * g.Is;
      at.hsum = a.hsum + (size_t)t * k * (g.I_pad / 16) * 2;
      at.xexp = a.xexp + t;
      if (route_here) {
        at.logits = route->logits;
        at.n_parts = route->n_parts;
        at.T_route = T;
        at.t_route = t;
        at.topk_idx_out = topk_idx + (size_t)t * k;
        at.topk_w_out = topk_w + (size_t)t * k;
      }
      hipError_t e = launch_dec1(at, g.fmt_ug, g.fmt_dn, topk_w + (size_t)t * k, y + (size_t)t * g.H, cus, s);
      if (e != hipSuccess) return hip_fail(who, e);
    }
    return MOE_OK;
  }
  if (route) {
    hipError_t e = launch_route_topk(route->logits, route->n_parts, T, g.E, k, topk_idx, topk_w, s);
    if (e != hipSuccess) return hip_fail(who, e);
  }
  const int nck = g.I_pad / 256, ncks = g.Is > 0 ? g.Is_pad / 256 : 0;
  const int nw_m = (nck > ncks ? nck : ncks) < 4 ? 4 : (nck > ncks ? nck : ncks);
  if (g.fmt_ug == MOE_FMT_CB2 && n_chunks <= 16 && nck <= 8 && ncks <= 8 &&
      decm_down_lds(a, nw_m) <= 160 * 1024) {
    hipError_t e = launch_decm(a, topk_w, y, cus, s);
    if (e != hipSuccess) return hip_fail(who, e);
    return MOE_OK;
  }
  const int64_t nd_max = (int64_t)(T * k < g.E ? T * k : g.E);
  const int64_t items_ug = nd_max * (g.I / 16) + g.Is / 16;
  const int64_t items_dn = nd_max * (g.H / 16) + (g.Is > 0 ? g.H / 16 : 0);
  const int grid_ug = (int)(items_ug < cus ? items_ug : cus);
  const int grid_dn = (int)(items_dn < 2 * cus ? items_dn : 2 * cus);
  hipError_t e = launch_dec_upgate(a, g.fmt_ug, cpw, grid_ug, s);
  if (e != hipSuccess) return hip_fail(who, e);
  e = launch_dec_down(a, g.fmt_dn, grid_dn, s);
  if (e != hipSuccess) return hip_fail(who, e);
  e = launch_combine(a, topk_idx, topk_w, y, s);
  if (e != hipSuccess) return hip_fail(who, e);
  return MOE_OK;
}

}  // namespace

extern "C" int moe_expert_ffn_decode(const moe_weights* w, const void* x_bf16, int32_t T, int32_t k,
                                     const int32_t* topk_idx, const float* topk_w, float* y, void* ws,
                                     size_t ws_bytes, void* stream) {
  clear_error();
  Geometry g;
  int rc = check_decode("moe_expert_ffn_decode", w, &g, x_bf16, T, k, topk_idx, topk_w, y, ws);
  if (rc != MOE_OK) return rc;
  const DecLayout L = dec_layout(g, T, k);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn_decode: workspace too small (need " + std::to_string(L.total) + ")");
  // (topk_idx and topk_w are only read on this path)
  return run_decode("moe_expert_ffn_decode", w, g, x_bf16, T, k, const_cast<int32_t*>(topk_idx),
                    const_cast<float*>(topk_w), y, (uint8_t*)ws, (hipStream_t)stream, nullptr);
}

extern "C" size_t moe_layer_decode_workspace_bytes(const moe_weights* w, int32_t T, int32_t k) {
  Geometry g;
  if (T < 1 || T > 16 || k < 1 || !w || check_weights(w, &g, "moe_layer_decode_workspace_bytes") != MOE_OK) {
    clear_error();
    return 0;
  }
  return align_up(dec_layout(g, T, k).total) + align_up(route_logit_floats(T, g.E) * 4);
}

namespace {

// Checks of moe_layer_decode beyond check_decode (the workspace aside).
int check_layer_decode(const char* who, const moe_weights* w, Geometry* g, const float* w_router,
                       const void* x_bf16, int32_t T, int32_t k, const void* topk_idx, const void* topk_w,
                       const float* y, const void* ws) {
  int rc = check_decode(who, w, g, x_bf16, T, k, topk_idx, topk_w, y, ws);
  if (rc != MOE_OK) return rc;
  if (!w_router) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": NULL router");
  if (!aligned16(w_router)) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": w_router must be 16-byte aligned");
  return MOE_OK;
}

int run_layer_decode(const char* who, const moe_weights* w, const Geometry& g, const float* w_router,
                     const float* logit_bias, const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx,
                     float* topk_w, float* y, uint8_t* wsb, hipStream_t s);

}  // namespace

extern "C" int moe_layer_decode(const moe_weights* w, const float* w_router, const float* logit_bias,
                                const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx, float* topk_w,
                                float* y, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  Geometry g;
  int rc = check_layer_decode("moe_layer_decode", w, &g, w_router, x_bf16, T, k, topk_idx, topk_w, y, ws);
  if (rc != MOE_OK) return rc;
  if (ws_bytes < moe_layer_decode_workspace_bytes(w, T, k))
    return fail(MOE_ERR_WORKSPACE, "moe_layer_decode: workspace too small (need " +
                                       std::to_string(moe_layer_decode_workspace_bytes(w, T, k)) + ")");
  return run_layer_decode("moe_layer_decode", w, g, w_router, logit_bias, x_bf16, T, k, topk_idx, topk_w, y,
                          (uint8_t*)ws, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// moe_layer_decode_noalloc: the same step with its workspace in a file-scope
// device array.  The array's name is a host-side stand-in in host code; its
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever handed to a kernel.

namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(const char* who, uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(who, e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, std::string(who) + ": device index beyond " + std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(who, e);
    if (!p) return fail(MOE_ERR_HIP, std::string(who) + ": no device address for the scratch array");
    g_scratch_ptr[dev] = (uint8_t*)p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_decode_noalloc(const moe_weights* w, const float* w_router, const float* logit_bias,
                                        const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx,
                                        float* topk_w, float* y, void* stream) {
  clear_error();
  static const char* who = "moe_layer_decode_noalloc";
  Geometry g;
  // (an aligned non-null stand-in for ws: the scratch array replaces it)
  int rc = check_layer_decode(who, w, &g, w_router, x_bf16, T, k, topk_idx, topk_w, y,
                              reinterpret_cast<const void*>(kAlign));
  if (rc != MOE_OK) return rc;
  const size_t need = moe_layer_decode_workspace_bytes(w, T, k);
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE, std::string(who) + ": this layer and T need " + std::to_string(need) +
                                       " bytes of scratch, more than the " + std::to_string(kScratchBytes) +
                                       " the library holds; use moe_layer_decode with a workspace");
  uint8_t* sp = nullptr;
  rc = scratch_address(who, &sp);
  if (rc != MOE_OK) return rc;
  return run_layer_decode(who, w, g, w_router, logit_bias, x_bf16, T, k, topk_idx, topk_w, y, sp,
                          (hipStream_t)stream);
}

namespace {

int run_layer_decode(const char* who, const moe_weights* w, const Geometry& g, const float* w_router,
                     const float* logit_bias, const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx,
                     float* topk_w, float* y, uint8_t* wsb, hipStream_t s) {
  const size_t off_logits = align_up(dec_layout(g, T, k).total);
  float* logits = (float*)(wsb + off_logits);
  hipError_t e = launch_route_logits((const uint16_t*)x_bf16, w_router, logit_bias, T, g.H, g.E, logits, s);
  if (e != hipSuccess) return hip_fail(who, e);
  const DecRoute route{logits, route_logit_parts(T, g.H)};
  return run_decode(who, w, g, x_bf16, T, k, topk_idx, topk_w, y, wsb, s, &route);
}

}  // namespace

extern "C" int moe_expert_ffn_prefill(const moe_weights* w, const void* x_bf16, int32_t T, int32_t k,
                                      const int32_t* topk_idx, const float* topk_w,
                                      const int32_t* expert_offsets, const int32_t* sorted_slots,
                                      const int32_t* slot_pos, float* y, void* ws, size_t ws_bytes,
                                      void* stream) {
  clear_error();
  Geometry g;
  int rc = check_weights(w, &g, "moe_expert_ffn_prefill");
  if (rc != MOE_OK) return rc;
  if (!x_bf16 || !topk_idx || !topk_w || !expert_offsets || !sorted_slots || !slot_pos || !y || !ws)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_prefill: NULL pointer");
  if (T < 1 || (int64_t)T * 16 > (1ll << 26))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_prefill: T must be in [1, 2^22]");
  if (k < 1 || k > 16 || k > g.E) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_prefill: need 1 <= k <= min(E, 16)");
  if (!aligned16(x_bf16) || !aligned16(ws) || !aligned16(y))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_prefill: x, y and ws must be 16-byte aligned");
  const PfLayout L = pf_layout(g, T, k);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn_prefill: workspace too small (need " + std::to_string(L.total) + ")");
  uint8_t* wsb = (uint8_t*)ws;
  PfArgs a{};
  a.x = (const uint16_t*)x_bf16;
  a.T = T;
  a.H = g.H;
  a.I = g.I;
  a.Is = g.Is;
  a.I_pad = g.I_pad;
  a.Is_pad = g.Is_pad;
  a.k = k;
  a.E = g.E;
  a.offsets = expert_offsets;
  a.sorted_slots = sorted_slots;
  a.slot_pos = slot_pos;
  a.up = (const uint8_t*)w->up;
  a.gate = (const uint8_t*)w->gate;
  a.down = (const uint8_t*)w->down;
  a.expert_bytes = g.up_bytes;
  a.expert_bytes_down = g.down_bytes;
  a.sup = (const uint8_t*)w->shared_up;
  a.sgate = (const uint8_t*)w->shared_gate;
  a.sdown = (const uint8_t*)w->shared_down;
  a.fmt_s = g.fmt_s;
  a.tb_s = tile_bytes(g.fmt_s);
  a.codebook = w->codebook;
  a.h = (_Float16*)(wsb + L.h);
  a.hs = (_Float16*)(wsb + L.hs);
  a.yslot = (float*)(wsb + L.yslot);
  a.ysh = (float*)(wsb + L.ysh);
  a.xexp = (int*)(wsb + L.xexp);
  a.epos = (int*)(wsb + L.epos);
  a.x16 = (const uint16_t*)(wsb + L.yslot);   // T*H fp16 fits in yslot, which only the down kernel writes
  hipError_t e = launch_prefill(a, g.fmt_ug, g.fmt_dn, topk_w, y, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("moe_expert_ffn_prefill", e);
  return MOE_OK;
}

extern "C" int moe_profile_next_launch(int kernel_id, void* start_event, void* stop_event) {
  clear_error();
  ProfileHook& hk = profile_hook();
  if (kernel_id == -1) {
    hk.n = 0;
    return MOE_OK;
  }
  if (kernel_id < MOE_KERNEL_ROUTE_LOGITS || kernel_id > MOE_KERNEL_READ)
    return fail(MOE_ERR_INVALID_ARG, "moe_profile_next_launch: unknown kernel id");
  if (!start_event || !stop_event) return fail(MOE_ERR_INVALID_ARG, "moe_profile_next_launch: NULL event");
  if (hk.n >= ProfileHook::kMax) return fail(MOE_ERR_INVALID_ARG, "moe_profile_next_launch: too many pending");
  hk.kernel_id[hk.n] = kernel_id;
  hk.start[hk.n] = start_event;
  hk.stop[hk.n] = stop_event;
  ++hk.n;
  return MOE_OK;
}

extern "C" int moe_debug_dequant(int fmt, const void* packed, int64_t rows, int64_t k, const int8_t* codebook,
                                 float* out, void* stream) {
  clear_error();
  if (moe_packed_bytes(fmt, rows, k) == 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_debug_dequant: bad format or shape");
  if (!packed || !out) return fail(MOE_ERR_INVALID_ARG, "moe_debug_dequant: NULL pointer");
  if (fmt == MOE_FMT_CB2 && !codebook) return fail(MOE_ERR_INVALID_ARG, "moe_debug_dequant: CB2 needs the codebook");
  if (!aligned16(packed)) return fail(MOE_ERR_INVALID_ARG, "moe_debug_dequant: packed must be 16-byte aligned");
  hipError_t e = launch_dequant(fmt, (const uint8_t*)packed, rows, pad256(k), codebook, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("moe_debug_dequant", e);
  return MOE_OK;
}

extern "C" int moe_measure_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream) {
  clear_error();
  if (!src || !out) return fail(MOE_ERR_INVALID_ARG, "moe_measure_read: NULL pointer");
  if (!aligned16(src) || bytes == 0 || bytes % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_measure_read: src must be 16-byte aligned and bytes a positive multiple of 16");
  if (blocks < 0 || blocks > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "moe_measure_read: blocks out of range");
  hipError_t e = launch_read(src, bytes, out, blocks > 0 ? blocks : 4 * n_cus(), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("moe_measure_read", e);
  return MOE_OK;
}
