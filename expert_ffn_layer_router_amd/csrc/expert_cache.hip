// Expert slot cache (host) and the copy of one expert's weights into a slot.
//
// Co-inference page, section 2.2: the weight pool's S slots form an N-way
// set-associative cache of (layer, expert) weights, M ways per set and
// N = S / M sets, with LRU replacement (experts are reused across
// consecutive layers and consecutive tokens).  Section 3.1 and the Strata
// page, section 2.2: the experts a layer will need are copied host -> device
// on a second stream while the GPU computes the current layer.  The cache
// decides which slot holds which expert; the caller enqueues the copies it
// asks for (moe_expert_upload) on its copy stream before the forward that
// reads the slot table.
//
// Set of layer L: L mod N.  Slot = set * M + way.  A request is the experts
// one layer needs for one step: resident ones are hits; each missing one
// takes an empty way of the set (lowest first), else the least recently used
// way holding no expert of the same request (lowest way among equals).  All
// experts of the request are then marked used at this request.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "moe.h"
#include "plan.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {
moe_status api_fail(moe_status st, const char* fmt, ...);  // moe_api.hip: sets moe_last_error()
bool api_check_handle(moe_handle h, const moe_config** cfg);
}  // namespace moe

struct moe_cache {
  int32_t sets = 0, ways = 0, experts = 0;
  std::vector<int64_t> layer;    // per slot: layer of the expert held, -1 when empty
  std::vector<int32_t> expert;   // per slot: the expert held
  std::vector<uint64_t> used;    // per slot: request counter of the last use
  uint64_t clock = 0;
  int64_t hits = 0, misses = 0;
};

namespace {

int32_t find_slot(const moe_cache& c, int64_t layer, int32_t e) {
  const int32_t base = (int32_t)(layer % c.sets) * c.ways;
  for (int32_t w = 0; w < c.ways; ++w)
    if (c.layer[base + w] == layer && c.expert[base + w] == e) return base + w;
  return -1;
}

}  // namespace

MOE_EXPORT moe_status moe_cache_create(int32_t num_sets, int32_t ways, int32_t num_experts, moe_cache_handle* out) {
  if (!out) return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  *out = nullptr;
  if (num_sets < 1 || ways < 1 || num_experts < 1 || (int64_t)num_sets * ways > (1 << 24))
    return moe::api_fail(MOE_ERR_INVALID_ARG, "num_sets=%d, ways=%d, num_experts=%d: need positive values and at most 2^24 slots",
                         num_sets, ways, num_experts);
  moe_cache* c = new (std::nothrow) moe_cache;
  if (!c) return moe::api_fail(MOE_ERR_INVALID_ARG, "out of host memory");
  c->sets = num_sets;
  c->ways = ways;
  c->experts = num_experts;
  const size_t S = (size_t)num_sets * ways;
  c->layer.assign(S, -1);
  c->expert.assign(S, -1);
  c->used.assign(S, 0);
  *out = c;
  return MOE_OK;
}

MOE_EXPORT void moe_cache_destroy(moe_cache_handle c) { delete c; }

MOE_EXPORT moe_status moe_cache_request(moe_cache_handle c, int32_t layer, const int32_t* experts, int32_t n,
                                        int32_t* slots, int32_t* load_experts, int32_t* load_slots,
                                        int32_t* n_loads, int32_t* slot_table) {
  if (!c || (n > 0 && (!experts || !slots || !load_experts || !load_slots)) || !n_loads)
    return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if (layer < 0 || n < 0) return moe::api_fail(MOE_ERR_INVALID_ARG, "layer=%d, n=%d must be >= 0", layer, n);
  // distinct experts in request order; validate before touching the cache
  std::vector<int32_t> wanted;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = experts[i];
    if (e < 0 || e >= c->experts)
      return moe::api_fail(MOE_ERR_INVALID_ARG, "expert %d outside [0, %d)", e, c->experts);
    if (std::find(wanted.begin(), wanted.end(), e) == wanted.end()) wanted.push_back(e);
  }
  if ((int32_t)wanted.size() > c->ways)
    return moe::api_fail(MOE_ERR_INVALID_ARG, "%d distinct experts do not fit %d ways", (int)wanted.size(), c->ways);
  ++c->clock;
  const int32_t base = (int32_t)(layer % c->sets) * c->ways;
  std::vector<int32_t> where(wanted.size(), -1);
  for (size_t i = 0; i < wanted.size(); ++i) {  // hits
    where[i] = find_slot(*c, layer, wanted[i]);
    if (where[i] >= 0) ++c->hits;
  }
  auto taken = [&](int32_t s) { return std::find(where.begin(), where.end(), s) != where.end(); };
  int32_t nl = 0;
  for (size_t i = 0; i < wanted.size(); ++i) {  // misses, in request order
    if (where[i] >= 0) continue;
    ++c->misses;
    int32_t pick = -1;
    for (int32_t w = 0; w < c->ways && pick < 0; ++w)
      if (c->layer[base + w] < 0 && !taken(base + w)) pick = base + w;
    if (pick < 0) {
      for (int32_t w = 0; w < c->ways; ++w) {
        const int32_t s = base + w;
        if (!taken(s) && (pick < 0 || c->used[s] < c->used[pick])) pick = s;
      }
    }
    c->layer[pick] = layer;
    c->expert[pick] = wanted[i];
    where[i] = pick;
    load_experts[nl] = wanted[i];
    load_slots[nl] = pick;
    ++nl;
  }
  for (int32_t s : where) c->used[s] = c->clock;
  for (int32_t i = 0; i < n; ++i)
    slots[i] = where[std::find(wanted.begin(), wanted.end(), experts[i]) - wanted.begin()];
  *n_loads = nl;
  if (slot_table)
    for (int32_t e = 0; e < c->experts; ++e) slot_table[e] = find_slot(*c, layer, e);
  return MOE_OK;
}

MOE_EXPORT moe_status moe_cache_stats(moe_cache_handle c, int64_t* hits, int64_t* misses) {
  if (!c || !hits || !misses) return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  *hits = c->hits;
  *misses = c->misses;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_cache_geometry(uint64_t free_bytes, uint64_t expert_bytes, int32_t ways, int32_t* num_slots,
                                         int32_t* num_sets) {
  if (!num_slots || !num_sets) return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if (expert_bytes == 0 || ways < 1)
    return moe::api_fail(MOE_ERR_INVALID_ARG, "expert_bytes=%llu, ways=%d: need positive values",
                         (unsigned long long)expert_bytes, ways);
  const uint64_t slots = free_bytes / expert_bytes;
  if (slots > (1u << 24)) return moe::api_fail(MOE_ERR_INVALID_ARG, "more than 2^24 slots");
  *num_slots = (int32_t)slots;
  *num_sets = (int32_t)(slots / (uint64_t)ways);
  return MOE_OK;
}

MOE_EXPORT moe_status moe_expert_bytes(moe_handle h, uint64_t* bytes) {
  const moe_config* cfg = nullptr;
  if (!moe::api_check_handle(h, &cfg)) return moe::api_fail(MOE_ERR_INVALID_ARG, "invalid handle");
  if (!bytes) return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  const uint64_t d = (uint64_t)cfg->d_model, f = (uint64_t)cfg->d_ff, bits = (uint64_t)cfg->weight_bits;
  const uint64_t gu_groups = cfg->group_size ? d / cfg->group_size : 1;
  const uint64_t dn_groups = cfg->group_size ? f / cfg->group_size : 1;
  // codes of gate, up and down, then fp16 scale and zero-point of each
  *bytes = 3 * d * f * bits / 8 + 2 * 2 * (2 * f * gu_groups + d * dn_groups);
  return MOE_OK;
}

MOE_EXPORT moe_status moe_expert_upload(moe_handle h, const moe_weights* pool, int32_t slot, const moe_weights* src,
                                        moe_stream stream) {
  const moe_config* cfg = nullptr;
  if (!moe::api_check_handle(h, &cfg)) return moe::api_fail(MOE_ERR_INVALID_ARG, "invalid handle");
  if (!pool || !src) return moe::api_fail(MOE_ERR_INVALID_ARG, "null pointer argument");
  if (slot < 0 || slot >= cfg->num_slots)
    return moe::api_fail(MOE_ERR_INVALID_ARG, "slot %d outside [0, num_slots=%d)", slot, cfg->num_slots);
  const size_t d = (size_t)cfg->d_model, f = (size_t)cfg->d_ff, bits = (size_t)cfg->weight_bits;
  // (s, z) per output row, or per output row and group of group_size inputs
  const size_t gu_groups = cfg->group_size ? d / cfg->group_size : 1;
  const size_t dn_groups = cfg->group_size ? f / cfg->group_size : 1;
  struct Part {
    void* dst;
    const void* src;
    size_t bytes;
  };
  const Part parts[] = {
      {(void*)pool->w_gate, src->w_gate, f * d * bits / 8},   {(void*)pool->w_up, src->w_up, f * d * bits / 8},
      {(void*)pool->w_down, src->w_down, d * f * bits / 8},   {(void*)pool->s_gate, src->s_gate, 2 * f * gu_groups},
      {(void*)pool->z_gate, src->z_gate, 2 * f * gu_groups},  {(void*)pool->s_up, src->s_up, 2 * f * gu_groups},
      {(void*)pool->z_up, src->z_up, 2 * f * gu_groups},      {(void*)pool->s_down, src->s_down, 2 * d * dn_groups},
      {(void*)pool->z_down, src->z_down, 2 * d * dn_groups},
  };
  for (const Part& p : parts)
    if (!p.dst || !p.src) return moe::api_fail(MOE_ERR_INVALID_ARG, "null weight pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (const Part& p : parts) {
    const hipError_t err = hipMemcpyAsync(static_cast<char*>(p.dst) + (size_t)slot * p.bytes, p.src, p.bytes,
                                          hipMemcpyDefault, s);
    if (err != hipSuccess) return moe::api_fail(MOE_ERR_HIP, "copy into slot %d: %s", slot, hipGetErrorString(err));
  }
  return MOE_OK;
}
