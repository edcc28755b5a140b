// Prefill tile kernel for int4g32 weights, gate/up matrix (one kernel per file: they compile in parallel).
#include "ffn_tile.hpp"

namespace moe {
int launch_tile_int4g32_gu(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s) {
  return tile_launch<MOE_W_INT4G32, true>(a, H, I, n, E, s);
}
}  // namespace moe
