// moe_expert_ffn_noalloc: the grouped expert FFN for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid allocation).  Its
// workspace (activation cast, h, row-tile plans, work counters) is a static device array of fixed
// size instead of a caller buffer.  Each device gets its own copy of the array when the library's
// code object is loaded there; its address is looked up once per device, on the first call made
// with that device current, and kept.  Calls on one device share the array: calls in flight
// together on one device (different streams, or different host threads) race on it.
#include <mutex>

#include "common.hpp"

namespace moe {
namespace {

constexpr size_t kScratchBytes = MOE_FFN_NOALLOC_MAX_WORKSPACE;  // per device
constexpr int kMaxDevices = 64;

// host code must not use this name as a device address: the address comes from hipGetSymbolAddress
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// device address of this device's scratch array (looked up on first use with the device current)
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "moe_expert_ffn_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_expert_ffn_noalloc(const moe_experts* w, const void* x, int xdt, int T, int k,
                                      const int32_t* offsets, const int32_t* perm_src, float* y_perm, int mode,
                                      void* stream) {
  if (!w) return fail(MOE_ERR_INVALID, "moe_expert_ffn_noalloc: null moe_experts");
  if (T < 0 || k < 1 || k > 16) return fail(MOE_ERR_INVALID, "moe_expert_ffn_noalloc: T=%d k=%d", T, k);
  const size_t need = moe_ffn_workspace(w, T, k, mode);
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_expert_ffn_noalloc: T=%d, k=%d needs %zu workspace bytes; the static scratch holds %zu "
                "(use moe_expert_ffn with a workspace)", T, k, need, kScratchBytes);
  void* ws = nullptr;
  int rc = scratch_for_current_device(&ws);
  if (rc != MOE_OK) return rc;
  // (no helper stream: the first use of one would create it)
  return expert_ffn(w, x, xdt, T, k, offsets, perm_src, y_perm, mode, ws, kScratchBytes, stream, false);
}
