// HBM residency cache for an expert bank held in host memory.  The inference path addresses
// experts through stable logical slots while their physical residency moves ("What expert
// offloading actually costs", section "Inside expert paging"); a least-recently-used cache
// serves most expert lookups (theflow.svmpsp.dev related-abstracts list, the router-locality
// study of Qwen3-235B).  A streamed expert costs its bytes every time it is fetched again
// (same first page: the transfer cost recurs with selection frequency), so the planner only
// fetches misses, one contiguous package per miss, on a side stream.
//
// Planning is host work on host ids (the router's choice copied back); fetching enqueues
// hipMemcpyAsync from the page-locked bank plus one small copy of the slot table.
#include <algorithm>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

#include "common.hpp"

struct moe_cache {
  moe_cache_desc d;
  int64_t tick = 0;                          // index of the next lookup group
  std::vector<int32_t> slot_of;              // key -> slot, -1 if absent
  std::vector<int64_t> last;                 // key -> tick of last use
  std::vector<int32_t> key_of_slot;          // slot -> key, -1 if free
  std::set<std::pair<int64_t, int32_t>> lru;  // (tick, key) of resident keys
  std::vector<int64_t> count;                 // key -> use count (LFU_DECAY)
  std::set<std::tuple<int64_t, int64_t, int32_t>> lfu;  // (count, tick, key) of resident keys
  std::set<int32_t> free_slots;
  moe_cache_stats_t st{};
};

using namespace moe;

extern "C" int moe_cache_create(const moe_cache_desc* desc, moe_cache_t** out) {
  if (!desc || !out) return fail(MOE_ERR_INVALID, "moe_cache_create: null pointer");
  const moe_cache_desc& d = *desc;
  if (d.L < 1 || d.E < 1 || d.E > 1024) return fail(MOE_ERR_INVALID, "moe_cache_create: L=%d E=%d", d.L, d.E);
  if (d.capacity < 1 || (int64_t)d.capacity > (int64_t)d.L * d.E)
    return fail(MOE_ERR_INVALID, "moe_cache_create: capacity %d out of 1..L*E", d.capacity);
  if (d.pkg_bytes == 0) return fail(MOE_ERR_INVALID, "moe_cache_create: pkg_bytes 0");
  if (d.policy != MOE_CACHE_LRU && d.policy != MOE_CACHE_LFU_DECAY)
    return fail(MOE_ERR_INVALID, "moe_cache_create: policy %d", d.policy);
  if (d.decay_period < 0) return fail(MOE_ERR_INVALID, "moe_cache_create: decay_period %d", d.decay_period);
  // host_bank == NULL and device_pool == NULL: planning-only cache (moe_cache_fetch refuses it)
  if ((d.host_bank == nullptr) != (d.device_pool == nullptr))
    return fail(MOE_ERR_INVALID, "moe_cache_create: host_bank and device_pool must both be set (or both NULL)");
  if (d.host_bank) {
    if (d.slot_stride < d.pkg_bytes || d.slot_stride % 256)
      return fail(MOE_ERR_INVALID, "moe_cache_create: slot_stride %zu", d.slot_stride);
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, d.host_bank);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(MOE_ERR_NOT_PINNED, "moe_cache_create: host_bank is not page-locked HIP host memory");
    }
  }
  moe_cache* c = new moe_cache();
  c->d = d;
  c->slot_of.assign((size_t)d.L * d.E, -1);
  c->last.assign((size_t)d.L * d.E, -1);
  c->count.assign((size_t)d.L * d.E, 0);
  c->key_of_slot.assign(d.capacity, -1);
  for (int s = 0; s < d.capacity; ++s) c->free_slots.insert(s);
  *out = c;
  return MOE_OK;
}

extern "C" int moe_cache_plan(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan) {
  if (!c || !plan || (n > 0 && !host_ids)) return fail(MOE_ERR_INVALID, "moe_cache_plan: null pointer");
  const int E = c->d.E;
  if (layer < 0 || layer >= c->d.L) return fail(MOE_ERR_INVALID, "moe_cache_plan: layer %d", layer);
  if (n < 0) return fail(MOE_ERR_INVALID, "moe_cache_plan: n=%d", n);
  std::vector<int32_t> ids(host_ids, host_ids + n);
  for (int32_t v : ids)
    if (v < 0 || v >= E) return fail(MOE_ERR_INVALID, "moe_cache_plan: id %d outside [0, %d)", v, E);
  std::sort(ids.begin(), ids.end());
  ids.erase(std::unique(ids.begin(), ids.end()), ids.end());
  if ((int)ids.size() > c->d.capacity)
    return fail(MOE_ERR_CAPACITY, "moe_cache_plan: %zu distinct experts exceed %d slots", ids.size(), c->d.capacity);

  const int64_t g = c->tick++;
  const int32_t kbase = layer * E;
  const bool lfu = c->d.policy == MOE_CACHE_LFU_DECAY;
  auto in_group = [&](int32_t key) {
    return key >= kbase && key < kbase + E && std::binary_search(ids.begin(), ids.end(), key - kbase);
  };
  if (lfu) {
    // decay, then this group's uses; the resident order is rebuilt (halving can create ties)
    if (c->d.decay_period > 0 && g > 0 && g % c->d.decay_period == 0)
      for (int64_t& v : c->count) v >>= 1;
    for (int32_t id : ids) c->count[kbase + id] += 1024;
    c->lfu.clear();
    for (int s = 0; s < c->d.capacity; ++s) {
      const int32_t key = c->key_of_slot[s];
      if (key >= 0) c->lfu.insert({c->count[key], c->last[key], key});
    }
  }
  plan->layer = layer;
  plan->n_ids = (int)ids.size();
  plan->n_hits = plan->n_misses = 0;
  for (int32_t id : ids) {
    const int32_t key = kbase + id;
    if (c->slot_of[key] >= 0) {
      plan->n_hits++;
      if (lfu)
        c->lfu.erase({c->count[key], c->last[key], key});
      else
        c->lru.erase({c->last[key], key});
    } else {
      int32_t slot;
      if (!c->free_slots.empty()) {
        slot = *c->free_slots.begin();
        c->free_slots.erase(c->free_slots.begin());
      } else {
        // the first resident key not in the group (cannot run out: distinct ids <= capacity
        // and every slot is taken)
        int32_t victim;
        if (lfu) {
          auto it = c->lfu.begin();
          while (it != c->lfu.end() && in_group(std::get<2>(*it))) ++it;
          victim = std::get<2>(*it);
          c->lfu.erase(it);
        } else {
          auto it = c->lru.begin();
          while (it != c->lru.end() && in_group(it->second)) ++it;
          victim = it->second;
          c->lru.erase(it);
        }
        slot = c->slot_of[victim];
        c->slot_of[victim] = -1;
        c->key_of_slot[slot] = -1;
        c->st.evictions++;
      }
      c->slot_of[key] = slot;
      c->key_of_slot[slot] = key;
      plan->miss_ids[plan->n_misses] = id;
      plan->miss_slots[plan->n_misses] = slot;
      plan->n_misses++;
    }
    c->last[key] = g;
    if (lfu)
      c->lfu.insert({c->count[key], g, key});
    else
      c->lru.insert({g, key});
  }
  for (int e = 0; e < E; ++e) plan->slot_of_expert[e] = c->slot_of[kbase + e];
  c->st.lookups += plan->n_ids;
  c->st.hits += plan->n_hits;
  c->st.misses += plan->n_misses;
  c->st.bytes_fetched += (int64_t)plan->n_misses * (int64_t)c->d.pkg_bytes;
  return MOE_OK;
}

extern "C" int moe_cache_fetch(moe_cache_t* c, const moe_cache_plan_t* plan, int32_t* dev_slot_of_expert,
                               void* copy_stream, void* done) {
  if (!c || !plan) return fail(MOE_ERR_INVALID, "moe_cache_fetch: null pointer");
  if (!c->d.host_bank) return fail(MOE_ERR_INVALID, "moe_cache_fetch: planning-only cache has no bank");
  if (plan->layer < 0 || plan->layer >= c->d.L) return fail(MOE_ERR_INVALID, "moe_cache_fetch: bad plan");
  hipStream_t s = (hipStream_t)copy_stream;
  const char* bank = (const char*)c->d.host_bank;
  char* pool = (char*)c->d.device_pool;
  for (int i = 0; i < plan->n_misses; ++i) {
    const int id = plan->miss_ids[i], slot = plan->miss_slots[i];
    if (id < 0 || id >= c->d.E || slot < 0 || slot >= c->d.capacity)
      return fail(MOE_ERR_INVALID, "moe_cache_fetch: bad plan entry %d", i);
    const size_t key = (size_t)plan->layer * c->d.E + id;
    hipError_t e = hipMemcpyAsync(pool + (size_t)slot * c->d.slot_stride, bank + key * c->d.pkg_bytes,
                                  c->d.pkg_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "moe_cache_fetch: package copy");
  }
  if (dev_slot_of_expert) {
    hipError_t e = hipMemcpyAsync(dev_slot_of_expert, plan->slot_of_expert, sizeof(int32_t) * c->d.E,
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "moe_cache_fetch: slot table copy");
  }
  if (done) {
    hipError_t e = hipEventRecord((hipEvent_t)done, s);
    if (e != hipSuccess) return hip_fail(e, "moe_cache_fetch: event record");
  }
  return MOE_OK;
}

extern "C" int moe_cache_stats(const moe_cache_t* c, moe_cache_stats_t* out) {
  if (!c || !out) return fail(MOE_ERR_INVALID, "moe_cache_stats: null pointer");
  *out = c->st;
  return MOE_OK;
}

extern "C" void moe_cache_destroy(moe_cache_t* c) { delete c; }
