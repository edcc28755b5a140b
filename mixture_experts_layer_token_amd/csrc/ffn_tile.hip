// Dispatch of the prefill (MFMA tile) variant of the expert FFN: the kernels themselves are in
// ffn_tile.hpp, one instantiation per ffn_tile_<format>_<matrix>.hip file.
#include "ffn_common.hpp"

namespace moe {

int launch_tile_bf16_gu(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);
int launch_tile_bf16_down(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);
int launch_tile_mxfp4_gu(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);
int launch_tile_mxfp4_down(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);
int launch_tile_int4g32_gu(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);
int launch_tile_int4g32_down(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);

int launch_ffn_tile_part(int fmt, bool gate_up, const FfnArgs& a, int H, int I, int n, int E, hipStream_t s) {
  switch (fmt) {
    case MOE_W_BF16: return gate_up ? launch_tile_bf16_gu(a, H, I, n, E, s) : launch_tile_bf16_down(a, H, I, n, E, s);
    case MOE_W_MXFP4: return gate_up ? launch_tile_mxfp4_gu(a, H, I, n, E, s) : launch_tile_mxfp4_down(a, H, I, n, E, s);
    case MOE_W_INT4G32:
      return gate_up ? launch_tile_int4g32_gu(a, H, I, n, E, s) : launch_tile_int4g32_down(a, H, I, n, E, s);
  }
  return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: no prefill kernel for format %d", fmt);
}

}  // namespace moe
