// HBM residency cache for an expert bank held in host memory.  The inference path addresses
// experts through stable logical slots while their physical residency moves ("What expert
// offloading actually costs", section "Inside expert paging"); a least-recently-used cache
// serves most expert lookups, and a static pin of the popular experts is the other baseline
// (theflow.svmpsp.dev related-abstracts list, the router-locality study of Qwen3-235B); experts
// can be fetched ahead of their use (same list, the Edge0 abstract).  A streamed expert costs its
// bytes every time it is fetched again (first page: the transfer cost recurs with selection
// frequency), so the planner only fetches misses, one contiguous package per miss, on a side
// stream.
//
// Planning is host work on host ids (the router's choice copied back); fetching enqueues copies
// from the page-locked bank (hipMemcpyAsync, or the caller's copy engine) plus one small copy of
// the slot table.  A bank of rANS blobs (moe_cache_set_rans) moves fewer bytes over the link: each
// blob lands in a device staging slot and a decode stream owned by the cache turns it into the plain
// package in its pool slot, while the copy stream carries on with the next blob; the copy stream
// waits for the last decode before it records the fetch's event.
#include <string.h>

#include <algorithm>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

#include "common.hpp"

namespace {
typedef std::tuple<int64_t, int64_t, int32_t> Prio;  // (count or 0, last use, key): smallest is evicted first
}

struct moe_cache {
  moe_cache_desc d;
  int64_t tick = 0;                  // index of the next demand lookup group
  std::vector<int32_t> slot_of;      // key -> slot, -1 if absent
  std::vector<int64_t> last;         // key -> tick of its last demand use (-1: none since it became resident)
  std::vector<int64_t> count;        // key -> use count (LFU_DECAY)
  std::vector<char> pinned;          // key never evicted
  std::vector<char> fresh;           // resident through a prefetch, not used by a demand lookup since
  std::vector<int32_t> key_of_slot;  // slot -> key, -1 if free
  std::set<Prio> order;              // resident keys that may be evicted
  std::set<int32_t> free_slots;
  std::vector<int32_t> last_group;   // keys of the latest demand group (sorted): a prefetch keeps them
  int64_t n_pinned = 0;
  moe_cache_stats_t st{};
  // rANS bank (moe_cache_set_rans): staging ring, decode stream and its events
  bool rans = false;
  char* staging = nullptr;
  size_t staging_stride = 0, raw_bytes = 0;
  int n_stage = 0, next_stage = 0, device = -1;
  hipStream_t dec = nullptr;
  std::vector<hipEvent_t> copied, decoded;  // per staging slot: its blob landed; its decode finished
  std::vector<char> stage_used;             // the slot's `decoded` event has been recorded

  ~moe_cache() {
    if (!dec) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != device) (void)hipSetDevice(device);
    (void)hipStreamSynchronize(dec);
    for (hipEvent_t e : copied) (void)hipEventDestroy(e);
    for (hipEvent_t e : decoded) (void)hipEventDestroy(e);
    (void)hipStreamDestroy(dec);
    if (cur != device && cur >= 0) (void)hipSetDevice(cur);
  }

  bool lfu() const { return d.policy == MOE_CACHE_LFU_DECAY; }
  Prio prio(int32_t key) const { return Prio(lfu() ? count[key] : 0, last[key], key); }
  void hold(int32_t key) {  // key becomes (or stays) an eviction candidate
    if (!pinned[key]) order.insert(prio(key));
  }
  void release(int32_t key) { order.erase(prio(key)); }
  // the first eviction candidate not in `keep` (sorted), or -1
  int32_t victim(const std::vector<int32_t>& keep, const std::vector<int32_t>* keep2 = nullptr) const {
    for (const Prio& p : order) {
      const int32_t key = std::get<2>(p);
      if (std::binary_search(keep.begin(), keep.end(), key)) continue;
      if (keep2 && std::binary_search(keep2->begin(), keep2->end(), key)) continue;
      return key;
    }
    return -1;
  }
  int32_t evict(int32_t key) {  // frees key's slot and returns it
    release(key);
    const int32_t slot = slot_of[key];
    slot_of[key] = -1;
    key_of_slot[slot] = -1;
    fresh[key] = 0;
    st.evictions++;
    return slot;
  }
  int32_t take_slot(int32_t key, int32_t victim_key) {  // a free slot, else the victim's
    int32_t slot;
    if (!free_slots.empty()) {
      slot = *free_slots.begin();
      free_slots.erase(free_slots.begin());
    } else {
      slot = evict(victim_key);
    }
    slot_of[key] = slot;
    key_of_slot[slot] = key;
    return slot;
  }
  // eviction candidates outside `keep` and `keep2` (sorted keys)
  int64_t evictable(const std::vector<int32_t>& keep, const std::vector<int32_t>* keep2 = nullptr) const {
    std::vector<int32_t> all(keep);
    if (keep2) {
      all.insert(all.end(), keep2->begin(), keep2->end());
      std::sort(all.begin(), all.end());
      all.erase(std::unique(all.begin(), all.end()), all.end());
    }
    int64_t held = 0;
    for (int32_t key : all) held += slot_of[key] >= 0 && !pinned[key];
    return (int64_t)order.size() - held;
  }
};

using namespace moe;

namespace {

// distinct ids of a lookup as sorted keys of `layer`, validated
int group_keys(moe_cache_t* c, int layer, const int32_t* host_ids, int n, const char* fn, std::vector<int32_t>& keys) {
  if (!c || (n > 0 && !host_ids)) return fail(MOE_ERR_INVALID, "%s: null pointer", fn);
  if (layer < 0 || layer >= c->d.L) return fail(MOE_ERR_INVALID, "%s: layer %d", fn, layer);
  if (n < 0) return fail(MOE_ERR_INVALID, "%s: n=%d", fn, n);
  keys.clear();
  for (int i = 0; i < n; ++i) {
    const int32_t v = host_ids[i];
    if (v < 0 || v >= c->d.E) return fail(MOE_ERR_INVALID, "%s: id %d outside [0, %d)", fn, v, c->d.E);
    keys.push_back(layer * c->d.E + v);
  }
  std::sort(keys.begin(), keys.end());
  keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
  return MOE_OK;
}

void plan_begin(moe_cache_t* c, int layer, moe_cache_plan_t* plan, int n_ids) {
  plan->layer = layer;
  plan->n_ids = n_ids;
  plan->n_hits = plan->n_misses = 0;
}

void plan_end(moe_cache_t* c, int layer, moe_cache_plan_t* plan) {
  const int E = c->d.E;
  for (int e = 0; e < E; ++e) plan->slot_of_expert[e] = c->slot_of[layer * E + e];
}

void plan_miss(moe_cache_t* c, moe_cache_plan_t* plan, int32_t key, int32_t slot) {
  plan->miss_ids[plan->n_misses] = key % c->d.E;
  plan->miss_slots[plan->n_misses] = slot;
  plan->n_misses++;
  c->st.bytes_fetched += (int64_t)c->d.pkg_bytes;
}

// The resident set after a failed copy: the misses from `from` on were never copied, so they
// are no longer resident (their slots are free and the next lookup of them misses again).
void roll_back(moe_cache_t* c, const moe_cache_plan_t* plan, int from) {
  for (int i = from; i < plan->n_misses; ++i) {
    const int32_t key = plan->layer * c->d.E + plan->miss_ids[i], slot = plan->miss_slots[i];
    if (c->slot_of[key] != slot) continue;  // a later plan already moved it
    if (c->pinned[key]) {
      c->pinned[key] = 0;
      c->n_pinned--;
    }
    c->release(key);
    c->slot_of[key] = -1;
    c->key_of_slot[slot] = -1;
    c->fresh[key] = 0;
    c->free_slots.insert(slot);
    c->st.bytes_fetched -= (int64_t)c->d.pkg_bytes;
  }
}

int hip_copy(void*, void* dst, const void* src, size_t bytes, void* stream) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, (hipStream_t)stream) == hipSuccess ? 0 : 1;
}

}  // namespace

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
    if (!d.copy) {  // the HIP copy engine reads the bank directly: it must be page-locked
      hipPointerAttribute_t attr;
      hipError_t e = hipPointerGetAttributes(&attr, d.host_bank);
      if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(MOE_ERR_NOT_PINNED, "moe_cache_create: host_bank is not page-locked HIP host memory");
      }
    }
  }
  moe_cache* c = new moe_cache();
  c->d = d;
  const size_t nk = (size_t)d.L * d.E;
  c->slot_of.assign(nk, -1);
  c->last.assign(nk, -1);
  c->count.assign(nk, 0);
  c->pinned.assign(nk, 0);
  c->fresh.assign(nk, 0);
  c->key_of_slot.assign(d.capacity, -1);
  for (int s = 0; s < d.capacity; ++s) c->free_slots.insert(s);
  *out = c;
  return MOE_OK;
}

extern "C" int moe_cache_plan(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan) {
  std::vector<int32_t> keys;
  int rc = group_keys(c, layer, host_ids, n, "moe_cache_plan", keys);
  if (rc != MOE_OK) return rc;
  if (!plan) return fail(MOE_ERR_INVALID, "moe_cache_plan: null plan");
  int64_t misses = 0;
  for (int32_t key : keys) misses += c->slot_of[key] < 0;
  if (misses > (int64_t)c->free_slots.size() + c->evictable(keys))
    return fail(MOE_ERR_CAPACITY, "moe_cache_plan: %zu distinct experts (%lld to fetch) do not fit %d slots (%lld pinned)",
                keys.size(), (long long)misses, c->d.capacity, (long long)c->n_pinned);

  const int64_t g = c->tick++;
  if (c->lfu()) {
    // decay, then this group's uses; the eviction order is rebuilt (counts changed)
    if (c->d.decay_period > 0 && g > 0 && g % c->d.decay_period == 0)
      for (int64_t& v : c->count) v >>= 1;
    for (int32_t key : keys) c->count[key] += 1024;
    c->order.clear();
    for (int s = 0; s < c->d.capacity; ++s) {
      const int32_t key = c->key_of_slot[s];
      if (key >= 0) c->hold(key);
    }
  }
  plan_begin(c, layer, plan, (int)keys.size());
  for (int32_t key : keys) {
    if (c->slot_of[key] >= 0) {
      plan->n_hits++;
      if (c->fresh[key]) c->st.prefetch_hits++, c->fresh[key] = 0;
      c->release(key);
    } else {
      const int32_t slot = c->take_slot(key, c->victim(keys));
      plan_miss(c, plan, key, slot);
    }
    c->last[key] = g;
    c->hold(key);
  }
  plan_end(c, layer, plan);
  c->last_group = keys;
  c->st.lookups += plan->n_ids;
  c->st.hits += plan->n_hits;
  c->st.misses += plan->n_misses;
  return MOE_OK;
}

extern "C" int moe_cache_prefetch(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan) {
  std::vector<int32_t> keys;
  int rc = group_keys(c, layer, host_ids, n, "moe_cache_prefetch", keys);
  if (rc != MOE_OK) return rc;
  if (!plan) return fail(MOE_ERR_INVALID, "moe_cache_prefetch: null plan");
  plan_begin(c, layer, plan, (int)keys.size());
  for (int32_t key : keys) {
    if (c->slot_of[key] >= 0) {
      plan->n_hits++;
      continue;
    }
    int32_t v = -1;
    if (c->free_slots.empty()) {
      v = c->victim(keys, &c->last_group);
      if (v < 0) break;  // best effort: nothing left that may go
    }
    const int32_t slot = c->take_slot(key, v);
    c->last[key] = -1;  // an unused prefetch is the first candidate for eviction
    c->fresh[key] = 1;
    c->hold(key);
    plan_miss(c, plan, key, slot);
    c->st.prefetch_fetches++;
  }
  plan_end(c, layer, plan);
  return MOE_OK;
}

extern "C" int moe_cache_pin(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan) {
  std::vector<int32_t> keys;
  int rc = group_keys(c, layer, host_ids, n, "moe_cache_pin", keys);
  if (rc != MOE_OK) return rc;
  if (!plan) return fail(MOE_ERR_INVALID, "moe_cache_pin: null plan");
  int64_t misses = 0;
  for (int32_t key : keys) misses += c->slot_of[key] < 0;
  if (misses > (int64_t)c->free_slots.size() + c->evictable(keys, &c->last_group))
    return fail(MOE_ERR_CAPACITY, "moe_cache_pin: %lld experts to fetch do not fit the unpinned slots", (long long)misses);
  plan_begin(c, layer, plan, (int)keys.size());
  for (int32_t key : keys) {
    if (c->slot_of[key] >= 0) {
      plan->n_hits++;
      c->release(key);
    } else {
      const int32_t slot = c->take_slot(key, c->free_slots.empty() ? c->victim(keys, &c->last_group) : -1);
      plan_miss(c, plan, key, slot);
    }
    c->fresh[key] = 0;
    if (!c->pinned[key]) c->pinned[key] = 1, c->n_pinned++;
  }
  plan_end(c, layer, plan);
  return MOE_OK;
}

extern "C" int moe_cache_set_rans(moe_cache_t* c, void* staging, size_t staging_stride, int staging_slots,
                                  size_t raw_bytes) {
  if (!c || !staging) return fail(MOE_ERR_INVALID, "moe_cache_set_rans: null pointer");
  if (!c->d.host_bank) return fail(MOE_ERR_INVALID, "moe_cache_set_rans: planning-only cache has no bank");
  if (c->rans) return fail(MOE_ERR_INVALID, "moe_cache_set_rans: already set");
  if (staging_slots < 1 || staging_slots > 64)
    return fail(MOE_ERR_INVALID, "moe_cache_set_rans: %d staging slots (1..64)", staging_slots);
  if (staging_stride < c->d.pkg_bytes || staging_stride % 256)
    return fail(MOE_ERR_INVALID, "moe_cache_set_rans: staging_stride %zu (a multiple of 256, >= pkg_bytes %zu)",
                staging_stride, c->d.pkg_bytes);
  if (raw_bytes == 0 || raw_bytes > c->d.slot_stride)
    return fail(MOE_ERR_INVALID, "moe_cache_set_rans: raw_bytes %zu (1..slot_stride %zu)", raw_bytes,
                c->d.slot_stride);
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->dec, hipStreamNonBlocking);
  if (e != hipSuccess) {
    c->dec = nullptr;
    return hip_fail(e, "moe_cache_set_rans: decode stream");
  }
  c->copied.assign(staging_slots, nullptr);
  c->decoded.assign(staging_slots, nullptr);
  for (int r = 0; r < staging_slots && e == hipSuccess; ++r) {
    e = hipEventCreateWithFlags(&c->copied[r], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->decoded[r], hipEventDisableTiming);
  }
  if (e != hipSuccess) return hip_fail(e, "moe_cache_set_rans: events");  // (the destructor frees them)
  c->stage_used.assign(staging_slots, 0);
  c->staging = (char*)staging;
  c->staging_stride = staging_stride;
  c->n_stage = staging_slots;
  c->raw_bytes = raw_bytes;
  c->rans = true;
  return MOE_OK;
}

namespace {

// rANS bank: blob -> staging slot (copy stream) -> decode into the pool slot (decode stream)
int fetch_rans_one(moe_cache* c, moe_copy_fn copy, void* ctx, const char* blob, char* dst, hipStream_t cs) {
  size_t bytes = c->d.pkg_bytes;
  if (!c->d.copy) {  // the bank is host memory: copy the blob's own bytes, not its whole slot
    uint32_t magic;
    uint64_t n, total;
    memcpy(&magic, blob, 4);
    memcpy(&n, blob + 8, 8);
    memcpy(&total, blob + 24, 8);
    if (magic != 0x31534E52u || n != c->raw_bytes || total > bytes || total < 64) return MOE_ERR_INVALID;
    bytes = (size_t)total;
  }
  const int r = c->next_stage;
  c->next_stage = (r + 1) % c->n_stage;
  char* stage = c->staging + (size_t)r * c->staging_stride;
  // the staging slot is free once the decode that read it has finished (a wait on the copy stream
  // costs the link a gap, so none is enqueued for a decode already over)
  if (c->stage_used[r]) {
    const hipError_t q = hipEventQuery(c->decoded[r]);
    if (q == hipErrorNotReady) {
      (void)hipGetLastError();  // (not an error: keep it out of the next launch check)
      if (hipStreamWaitEvent(cs, c->decoded[r], 0) != hipSuccess) return MOE_ERR_HIP;
    } else if (q != hipSuccess) {
      return MOE_ERR_HIP;
    }
  }
  if (copy(ctx, stage, blob, bytes, cs) != 0) return MOE_ERR_HIP;
  if (hipEventRecord(c->copied[r], cs) != hipSuccess || hipStreamWaitEvent(c->dec, c->copied[r], 0) != hipSuccess)
    return MOE_ERR_HIP;
  if (moe::launch_rns_decode_one(stage, dst, c->raw_bytes, c->dec) != MOE_OK) return MOE_ERR_HIP;
  if (hipEventRecord(c->decoded[r], c->dec) != hipSuccess) return MOE_ERR_HIP;
  c->stage_used[r] = 1;
  c->st.bytes_fetched -= (int64_t)(c->d.pkg_bytes - bytes);  // (the stats count the bytes that cross the link)
  return MOE_OK;
}

}  // namespace

extern "C" int moe_cache_fetch(moe_cache_t* c, const moe_cache_plan_t* plan, int32_t* dev_slot_of_expert,
                               void* copy_stream, void* done) {
  if (!c || !plan) return fail(MOE_ERR_INVALID, "moe_cache_fetch: null pointer");
  if (!c->d.host_bank) return fail(MOE_ERR_INVALID, "moe_cache_fetch: planning-only cache has no bank");
  if (plan->layer < 0 || plan->layer >= c->d.L || plan->n_misses < 0 || plan->n_misses > c->d.E)
    return fail(MOE_ERR_INVALID, "moe_cache_fetch: bad plan");
  for (int i = 0; i < plan->n_misses; ++i) {
    const int id = plan->miss_ids[i], slot = plan->miss_slots[i];
    if (id < 0 || id >= c->d.E || slot < 0 || slot >= c->d.capacity)
      return fail(MOE_ERR_INVALID, "moe_cache_fetch: bad plan entry %d", i);
  }
  moe_copy_fn copy = c->d.copy ? c->d.copy : hip_copy;
  void* ctx = c->d.copy ? c->d.copy_ctx : nullptr;
  const char* bank = (const char*)c->d.host_bank;
  char* pool = (char*)c->d.device_pool;
  int last_stage = -1;
  for (int i = 0; i < plan->n_misses; ++i) {
    const size_t key = (size_t)plan->layer * c->d.E + plan->miss_ids[i];
    char* dst = pool + (size_t)plan->miss_slots[i] * c->d.slot_stride;
    const char* src = bank + key * c->d.pkg_bytes;
    int rc = MOE_OK;
    if (c->rans) {
      const int r = c->next_stage;
      rc = fetch_rans_one(c, copy, ctx, src, dst, (hipStream_t)copy_stream);
      if (rc == MOE_OK) last_stage = r;
    } else if (copy(ctx, dst, src, c->d.pkg_bytes, copy_stream) != 0) {
      rc = MOE_ERR_HIP;
    }
    if (rc != MOE_OK) {
      (void)hipGetLastError();
      roll_back(c, plan, i);
      if (last_stage >= 0)  // the decodes already launched still finish before later events of the copy stream
        (void)hipStreamWaitEvent((hipStream_t)copy_stream, c->decoded[last_stage], 0);
      return fail(rc, "moe_cache_fetch: %s of expert %d of layer %d failed; it and the %d misses after it are not "
                  "resident", rc == MOE_ERR_INVALID ? "blob header" : "copy", plan->miss_ids[i], plan->layer,
                  plan->n_misses - i - 1);
    }
  }
  // the pool slots hold the decoded packages once the last decode has finished
  if (last_stage >= 0 && hipStreamWaitEvent((hipStream_t)copy_stream, c->decoded[last_stage], 0) != hipSuccess)
    return fail(MOE_ERR_HIP, "moe_cache_fetch: wait for the decode stream");
  if (dev_slot_of_expert &&
      copy(ctx, dev_slot_of_expert, plan->slot_of_expert, sizeof(int32_t) * c->d.E, copy_stream) != 0) {
    (void)hipGetLastError();
    return fail(MOE_ERR_HIP, "moe_cache_fetch: slot table copy failed");
  }
  if (done) {
    hipError_t e = hipEventRecord((hipEvent_t)done, (hipStream_t)copy_stream);
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
