// Drives the expert-cache planner (demand lookups of both policies, prefetches, pins, a fetch
// through a copy engine that fails halfway, the error paths) and the host encoders, for builds
// with AddressSanitizer and UndefinedBehaviorSanitizer; no GPU is touched.
#include <stdio.h>
#include <string.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/moe.h"

// the cache's rANS bank mode launches a GPU decoder; this host-only build links no kernels, and the
// mode itself is never switched on here (it needs a device stream), so a stand-in that refuses
namespace moe {
int launch_rns_decode_one(const void*, void*, size_t, hipStream_t) { return MOE_ERR_UNSUPPORTED; }
}  // namespace moe

static int copies = 0;
static int fake_copy(void*, void* dst, const void* src, size_t n, void*) {
  if (++copies % 7 == 0) return 1;  // every seventh copy fails
  memcpy(dst, src, n);
  return 0;
}

int main() {
  const int L = 3, E = 40, pkg = 256, cap = 20;
  std::vector<unsigned char> bank((size_t)L * E * pkg, 7), pool((size_t)cap * pkg);
  std::vector<int32_t> table(E);
  for (int policy = 0; policy < 2; ++policy) {
    moe_cache_desc d;
    memset(&d, 0, sizeof d);
    d.host_bank = bank.data();
    d.device_pool = pool.data();
    d.pkg_bytes = pkg;
    d.slot_stride = pkg;
    d.L = L, d.E = E, d.capacity = cap, d.policy = policy, d.decay_period = 5;
    d.copy = fake_copy;
    moe_cache_t* c = nullptr;
    if (moe_cache_create(&d, &c) != MOE_OK) return 2;
    moe_cache_plan_t* p = new moe_cache_plan_t;
    int32_t ids[8];
    const int32_t pin_ids[2] = {1, 2};
    if (moe_cache_pin(c, 0, pin_ids, 2, p) != MOE_OK) return 3;
    for (int g = 0; g < 400; ++g) {
      const int layer = g % L;
      for (int i = 0; i < 8; ++i) ids[i] = (g * 13 + i * i * 5 + layer) % E;
      const int rc = g % 4 == 2 ? moe_cache_prefetch(c, layer, ids, 3, p) : moe_cache_plan(c, layer, ids, 8, p);
      if (rc != MOE_OK) return 4;
      const int f = moe_cache_fetch(c, p, table.data(), nullptr, nullptr);
      if (f != MOE_OK && f != MOE_ERR_HIP) return 5;
    }
    int32_t bad = E;
    if (moe_cache_plan(c, 0, &bad, 1, p) != MOE_ERR_INVALID) return 6;
    if (moe_cache_plan(c, L, ids, 1, p) != MOE_ERR_INVALID) return 7;
    moe_cache_stats_t st;
    if (moe_cache_stats(c, &st) != MOE_OK || st.lookups <= 0) return 8;
    // the rANS bank mode's argument checks (all before a stream would be created)
    unsigned char stage_stub[1];
    if (moe_cache_set_rans(c, nullptr, 256, 4, pkg) != MOE_ERR_INVALID) return 13;
    if (moe_cache_set_rans(c, stage_stub, 128, 4, pkg) != MOE_ERR_INVALID) return 14;
    if (moe_cache_set_rans(c, stage_stub, 256, 0, pkg) != MOE_ERR_INVALID) return 15;
    if (moe_cache_set_rans(c, stage_stub, 256, 4, pkg + 1) != MOE_ERR_INVALID) return 16;
    delete p;
    moe_cache_destroy(c);
  }
  // the host encoder of the lossless code: a hand-worked chunk (largest exponent 128, two escapes)
  // and random bit patterns, sizes and the refusals
  {
    std::vector<uint16_t> v(512 * 6);
    for (size_t i = 0; i < v.size(); ++i) v[i] = (uint16_t)((i * 2654435761u) >> 13);
    v[0] = 0xC000, v[1] = 0x0000, v[2] = 0x3FC0, v[3] = 0x8001;
    for (int i = 4; i < 512; ++i) v[i] = 0x3F80;
    const size_t raw = v.size() * 2, cap = moe_compress_bound(raw);
    std::vector<uint8_t> blob(cap);
    size_t n = 0;
    if (moe_compress_package(v.data(), raw, blob.data(), cap, &n) != MOE_OK || n > cap) return 9;
    uint32_t off1;
    memcpy(&off1, blob.data() + 68, 4);
    if (off1 != 784 || blob[64 + 4 * 7] != 114) return 10;  // first chunk: 768 + 16 bytes, window base 114
    if (moe_compress_package(v.data(), raw, blob.data(), cap - 1, &n) != MOE_ERR_INVALID) return 11;
    if (moe_compress_package(v.data(), 1000, blob.data(), cap, &n) != MOE_ERR_INVALID) return 12;
  }
  // the host rANS encoder over regions shorter and longer than its 32768 streams, empty regions and
  // one-symbol regions: the blob stays within the bound and its header names what was encoded
  {
    const size_t sizes[] = {0, 1, 1000, 32768 + 5, 3 * 32768 + 999};
    for (size_t raw : sizes) {
      std::vector<uint8_t> r(raw);
      for (size_t i = 0; i < raw; ++i) r[i] = (uint8_t)(((i * 2654435761u) >> 20) % 9 == 0 ? i * 7 : 3);
      const size_t cap = moe_compress_rans_bound(raw);
      std::vector<uint8_t> blob(cap);
      const size_t splits[] = {0, raw / 3, raw};
      for (size_t q : splits) {
        size_t n = 0;
        if (moe_compress_rans(r.data(), raw, q, blob.data(), cap, &n) != MOE_OK || n > cap || n % 16) return 17;
        uint64_t hn, hq, ht;
        memcpy(&hn, blob.data() + 8, 8);
        memcpy(&hq, blob.data() + 16, 8);
        memcpy(&ht, blob.data() + 24, 8);
        if (hn != raw || hq != q || ht != n) return 18;
      }
      size_t n = 0;
      if (moe_compress_rans(r.data(), raw, raw + 1, blob.data(), cap, &n) != MOE_ERR_INVALID) return 19;
      if (moe_compress_rans(r.data(), raw, 0, blob.data(), cap - 1, &n) != MOE_ERR_INVALID) return 20;
    }
  }
  printf("planner and encoders: ok (%d copies)\n", copies);
  return 0;
}
