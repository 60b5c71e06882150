// Expert streaming through an HBM expert cache ([osrepos] "SSD Streaming for
// Large Models": routed MoE experts loaded on demand into a cache of a size
// the user sets).  Host runtime only: the routed experts stay in host
// memory, n_slots of them sit in device slot arrays, and a least-recently-
// used planner (the replacement rule include/qmoe.h states) decides which
// step needs which copies.  The expert FFN then runs over the slots with the
// existing kernels: the cache is an ordinary weight set of n_slots experts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "../../include/qmoe.h"
#include "qmoe_internal.h"

using namespace qmoe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kOrderBits = 20;                    // choice order within a step in a recency stamp
constexpr int kMaxStreamChoices = 16 * 16;        // T * k of one streamed decode step

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int hip_fail(const char* where, hipError_t e) {
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

}  // namespace

struct moe_expert_cache {
  moe_weights host;                  // the layer as given (up/gate/down in host memory)
  moe_weights dev;                   // the slots as a weight set
  int32_t E = 0, n_slots = 0, keep = 0;
  size_t nb_up = 0, nb_dn = 0;       // bytes of one expert's up (= gate) and down matrix
  std::vector<int32_t> slot_of;      // [E]: slot, or -1
  std::vector<int32_t> expert_of;    // [n_slots]: expert, or -1
  std::vector<uint64_t> last_use;    // [n_slots]: step << kOrderBits | order within the step
  uint64_t step = 0;
  int64_t hits = 0, misses = 0;
  // page-locked staging of the streamed decode step, allocated at its first call
  int32_t* h_ids = nullptr;
  int32_t* h_slots = nullptr;
  int32_t* h_miss_e = nullptr;
  int32_t* h_miss_s = nullptr;
  hipEvent_t copied = nullptr;
};

namespace {

size_t slot_layout(const moe_weights* w, int32_t n_slots, size_t* off_gate, size_t* off_down) {
  const size_t nb_up = moe_packed_bytes(w->fmt_up, w->inter, w->hidden);
  const size_t nb_dn = moe_packed_bytes(w->fmt_down, w->hidden, w->inter);
  const size_t up = align_up((size_t)n_slots * nb_up), dn = align_up((size_t)n_slots * nb_dn);
  if (off_gate) *off_gate = up;
  if (off_down) *off_down = 2 * up;
  return 2 * up + dn;
}

int plan_step(moe_expert_cache* c, const int32_t* ids, int32_t n, int32_t* slots_out, int32_t* miss_e,
              int32_t* miss_s, int32_t* n_miss, const char* who) {
  const std::string f(who);
  if (!c || !ids || !slots_out || !miss_e || !miss_s || !n_miss)
    return fail(MOE_ERR_INVALID_ARG, f + ": NULL pointer");
  if (n < 0 || n >= (1 << kOrderBits)) return fail(MOE_ERR_INVALID_ARG, f + ": n out of range");
  // the step's distinct experts in order of first appearance
  std::vector<uint8_t> seen(c->E, 0);
  std::vector<int32_t> need;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = ids[i];
    if (e >= 0 && e < c->E && !seen[e]) {
      seen[e] = 1;
      need.push_back(e);
    }
  }
  const uint64_t st = c->step + 1;
  int n_new = 0;
  for (int32_t e : need) n_new += c->slot_of[e] < 0;
  int n_free = 0;
  for (int32_t s = 0; s < c->n_slots; ++s) n_free += c->expert_of[s] < 0;
  const int n_evict = std::max(0, n_new - n_free);
  // eviction candidates: resident, not needed now, not used in the last keep steps
  std::vector<std::pair<uint64_t, int32_t>> cand;
  for (int32_t s = 0; s < c->n_slots; ++s) {
    const int32_t e = c->expert_of[s];
    if (e < 0 || seen[e]) continue;
    const uint64_t used = c->last_use[s] >> kOrderBits;
    if (c->keep > 0 && used + (uint64_t)c->keep >= st) continue;
    cand.emplace_back(c->last_use[s], s);
  }
  if (n_evict > (int)cand.size())
    return fail(MOE_ERR_INVALID_ARG, f + ": the step needs " + std::to_string(n_new) +
                                         " new experts, but only " + std::to_string(n_free + (int)cand.size()) +
                                         " slots are free or evictable");
  std::partial_sort(cand.begin(), cand.begin() + n_evict, cand.end());
  for (int i = 0; i < n_evict; ++i) {
    const int32_t s = cand[i].second;
    c->slot_of[c->expert_of[s]] = -1;
    c->expert_of[s] = -1;
  }
  int32_t nm = 0, next_free = 0;
  for (size_t i = 0; i < need.size(); ++i) {
    const int32_t e = need[i];
    if (c->slot_of[e] >= 0) {
      ++c->hits;
    } else {
      while (c->expert_of[next_free] >= 0) ++next_free;
      c->expert_of[next_free] = e;
      c->slot_of[e] = next_free;
      miss_e[nm] = e;
      miss_s[nm] = next_free;
      ++nm;
      ++c->misses;
    }
    c->last_use[c->slot_of[e]] = (st << kOrderBits) | (uint64_t)i;
  }
  c->step = st;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = ids[i];
    slots_out[i] = (e >= 0 && e < c->E) ? c->slot_of[e] : -1;
  }
  *n_miss = nm;
  return MOE_OK;
}

}  // namespace

extern "C" size_t moe_expert_cache_slot_bytes(const moe_weights* w, int32_t n_slots) {
  if (!w || n_slots < 1 || n_slots > w->n_experts || validate_weights(w, "moe_expert_cache_slot_bytes") != MOE_OK) {
    clear_error();
    return 0;
  }
  return slot_layout(w, n_slots, nullptr, nullptr);
}

extern "C" int moe_expert_cache_create(const moe_weights* host_layer, int32_t n_slots, int32_t keep, void* slot_mem,
                                       size_t slot_mem_bytes, moe_expert_cache** out) {
  clear_error();
  if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: out is NULL");
  int rc = validate_weights(host_layer, "moe_expert_cache_create");
  if (rc != MOE_OK) return rc;
  if (n_slots < 1 || n_slots > host_layer->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: n_slots must be in [1, n_experts]");
  if (keep < 0 || keep > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: keep out of range");
  size_t off_gate = 0, off_down = 0;
  const size_t need = slot_layout(host_layer, n_slots, &off_gate, &off_down);
  if (!slot_mem || ((uintptr_t)slot_mem % kAlign) != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: slot_mem must be a 256-byte aligned device pointer");
  if (slot_mem_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_cache_create: slot_mem too small (need " + std::to_string(need) + ")");
  moe_expert_cache* c = new moe_expert_cache();
  c->host = *host_layer;
  c->dev = *host_layer;
  c->E = host_layer->n_experts;
  c->n_slots = n_slots;
  c->keep = keep;
  c->nb_up = moe_packed_bytes(host_layer->fmt_up, host_layer->inter, host_layer->hidden);
  c->nb_dn = moe_packed_bytes(host_layer->fmt_down, host_layer->hidden, host_layer->inter);
  uint8_t* base = (uint8_t*)slot_mem;
  c->dev.n_experts = n_slots;
  c->dev.up = base;
  c->dev.gate = base + off_gate;
  c->dev.down = base + off_down;
  c->slot_of.assign(c->E, -1);
  c->expert_of.assign(n_slots, -1);
  c->last_use.assign(n_slots, 0);
  *out = c;
  return MOE_OK;
}

extern "C" int moe_expert_cache_destroy(moe_expert_cache* cache) {
  clear_error();
  if (!cache) return MOE_OK;
  if (cache->h_ids) (void)hipHostFree(cache->h_ids);
  if (cache->copied) (void)hipEventDestroy(cache->copied);
  delete cache;
  return MOE_OK;
}

extern "C" int moe_expert_cache_weights(const moe_expert_cache* cache, moe_weights* out) {
  clear_error();
  if (!cache || !out) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_weights: NULL pointer");
  *out = cache->dev;
  return MOE_OK;
}

extern "C" int moe_expert_cache_plan(moe_expert_cache* cache, const int32_t* ids, int32_t n, int32_t* slots_out,
                                     int32_t* miss_experts, int32_t* miss_slots, int32_t* n_miss) {
  clear_error();
  return plan_step(cache, ids, n, slots_out, miss_experts, miss_slots, n_miss, "moe_expert_cache_plan");
}

extern "C" int moe_expert_cache_fetch(moe_expert_cache* cache, const int32_t* miss_experts, const int32_t* miss_slots,
                                      int32_t n_miss, void* stream) {
  clear_error();
  if (!cache || (n_miss > 0 && (!miss_experts || !miss_slots)))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_fetch: NULL pointer");
  if (n_miss < 0) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_fetch: n_miss < 0");
  for (int32_t i = 0; i < n_miss; ++i)
    if (miss_experts[i] < 0 || miss_experts[i] >= cache->E || miss_slots[i] < 0 || miss_slots[i] >= cache->n_slots)
      return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_fetch: expert or slot out of range");
  const hipStream_t s = (hipStream_t)stream;
  const uint8_t* hu = (const uint8_t*)cache->host.up;
  const uint8_t* hg = (const uint8_t*)cache->host.gate;
  const uint8_t* hd = (const uint8_t*)cache->host.down;
  uint8_t* du = (uint8_t*)cache->dev.up;
  uint8_t* dg = (uint8_t*)cache->dev.gate;
  uint8_t* dd = (uint8_t*)cache->dev.down;
  for (int32_t i = 0; i < n_miss; ++i) {
    const size_t e = (size_t)miss_experts[i], sl = (size_t)miss_slots[i];
    hipError_t err = hipMemcpyAsync(du + sl * cache->nb_up, hu + e * cache->nb_up, cache->nb_up,
                                    hipMemcpyHostToDevice, s);
    if (err == hipSuccess)
      err = hipMemcpyAsync(dg + sl * cache->nb_up, hg + e * cache->nb_up, cache->nb_up, hipMemcpyHostToDevice, s);
    if (err == hipSuccess)
      err = hipMemcpyAsync(dd + sl * cache->nb_dn, hd + e * cache->nb_dn, cache->nb_dn, hipMemcpyHostToDevice, s);
    if (err != hipSuccess) return hip_fail("moe_expert_cache_fetch", err);
  }
  return MOE_OK;
}

extern "C" int moe_expert_cache_state(const moe_expert_cache* cache, int32_t* expert_of_slot, int64_t* hits,
                                      int64_t* misses) {
  clear_error();
  if (!cache) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_state: NULL cache");
  if (expert_of_slot) std::copy(cache->expert_of.begin(), cache->expert_of.end(), expert_of_slot);
  if (hits) *hits = cache->hits;
  if (misses) *misses = cache->misses;
  return MOE_OK;
}

namespace {

struct StreamedLayout {
  size_t route, slots, ffn, total;
};

bool streamed_layout(const moe_expert_cache* c, int32_t T, int32_t k, StreamedLayout* L) {
  if (!c || T < 1 || T > 16 || k < 1 || k > 16) return false;
  const size_t r = moe_route_workspace_bytes(T, c->E);
  const size_t f = moe_ffn_workspace_bytes(&c->dev, T, k, 0);
  if (r == 0 || f == 0) return false;
  L->route = 0;
  L->slots = align_up(r);
  L->ffn = L->slots + align_up((size_t)T * k * 4);
  L->total = L->ffn + align_up(f);
  return true;
}

}  // namespace

extern "C" size_t moe_layer_decode_streamed_workspace_bytes(const moe_expert_cache* cache, int32_t T, int32_t k) {
  StreamedLayout L;
  const bool ok = streamed_layout(cache, T, k, &L);
  clear_error();
  return ok ? L.total : 0;
}

extern "C" int moe_layer_decode_streamed(moe_expert_cache* cache, const float* w_router, const float* logit_bias,
                                         const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx,
                                         float* topk_w, float* y, void* ws, size_t ws_bytes, void* stream,
                                         void* copy_stream) {
  clear_error();
  const char* who = "moe_layer_decode_streamed";
  if (!cache) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": NULL cache");
  if (T < 1 || T > 16 || k < 1 || k > 16) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": T or k out of range");
  if (!ws || ((uintptr_t)ws % kAlign) != 0)
    return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": ws must be a 256-byte aligned device pointer");
  StreamedLayout L;
  if (!streamed_layout(cache, T, k, &L)) return fail(MOE_ERR_INVALID_ARG, std::string(who) + ": bad layer");
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, std::string(who) + ": workspace too small (need " + std::to_string(L.total) + ")");
  const hipStream_t s = (hipStream_t)stream;
  hipError_t err;
  if (!cache->h_ids) {
    // four page-locked int32 arrays of kMaxStreamChoices: choices, slots, misses
    void* p = nullptr;
    err = hipHostMalloc(&p, 4 * kMaxStreamChoices * sizeof(int32_t), hipHostMallocDefault);
    if (err != hipSuccess) return hip_fail(who, err);
    err = hipEventCreateWithFlags(&cache->copied, hipEventDisableTiming);
    if (err != hipSuccess) {
      (void)hipHostFree(p);
      return hip_fail(who, err);
    }
    cache->h_ids = (int32_t*)p;
    cache->h_slots = cache->h_ids + kMaxStreamChoices;
    cache->h_miss_e = cache->h_slots + kMaxStreamChoices;
    cache->h_miss_s = cache->h_miss_e + kMaxStreamChoices;
  }
  uint8_t* wsb = (uint8_t*)ws;
  const int32_t n = T * k;
  int rc = moe_route(x_bf16, w_router, logit_bias, T, cache->host.hidden, cache->E, k, topk_idx, topk_w,
                     wsb + L.route, L.slots - L.route, stream);
  if (rc != MOE_OK) return rc;
  // the choices to the host (this also orders the previous call's copy of
  // the slot ids out of h_slots before it is overwritten)
  err = hipMemcpyAsync(cache->h_ids, topk_idx, (size_t)n * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return hip_fail(who, err);
  int32_t n_miss = 0;
  rc = plan_step(cache, cache->h_ids, n, cache->h_slots, cache->h_miss_e, cache->h_miss_s, &n_miss, who);
  if (rc != MOE_OK) return rc;
  if (n_miss > 0) {
    const hipStream_t cs = copy_stream ? (hipStream_t)copy_stream : s;
    rc = moe_expert_cache_fetch(cache, cache->h_miss_e, cache->h_miss_s, n_miss, cs);
    if (rc != MOE_OK) return rc;
    if (cs != s) {
      err = hipEventRecord(cache->copied, cs);
      if (err == hipSuccess) err = hipStreamWaitEvent(s, cache->copied, 0);
      if (err != hipSuccess) return hip_fail(who, err);
    }
  }
  int32_t* d_slots = (int32_t*)(wsb + L.slots);
  err = hipMemcpyAsync(d_slots, cache->h_slots, (size_t)n * 4, hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return hip_fail(who, err);
  return moe_expert_ffn_decode(&cache->dev, x_bf16, T, k, d_slots, topk_w, y, wsb + L.ffn, L.total - L.ffn, stream);
}
