// Weighted combine: every token collects the outputs of the experts it was sent to ("Mixture of
// experts VRAM: total vs active parameters", section "Expert parallelism on RTX PRO 6000 and
// H200 NVL": dispatch, then collect the results) and weights them by its gate weights; an
// always-on shared expert is added with weight 1 (same page, routing section).
//
// Gather form: one workgroup per token reads its k rows of y_perm through inv_perm and writes
// the token's row once.  fp32 sum in slot order, then the shared row, then one rounding; no
// atomics, so the result is bitwise deterministic.  HBM-bound: 16-byte loads and stores.
#include "common.hpp"

namespace moe {
namespace {

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv, int k, int H,
                                                      const float* __restrict__ shared, void* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int rows[16];
  __shared__ float gates[16];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = inv[(size_t)t * k + threadIdx.x];
    gates[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    // the k rows' loads are issued together, then summed in slot order
    f32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) v[j] = *(const f32x4*)(y + (size_t)rows[j] * H + c);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k) {
        const float g = gates[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(g, v[j][q], acc[q]);
      }
    }
    if (shared) {
      f32x4 v = *(const f32x4*)(shared + (size_t)t * H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += v[q];
    }
    if (BF16_OUT) {
      unsigned short* o = (unsigned short*)out + (size_t)t * H + c;
      uint2 pk;
      pk.x = (unsigned)f32_to_bf16_rne(acc[0]) | ((unsigned)f32_to_bf16_rne(acc[1]) << 16);
      pk.y = (unsigned)f32_to_bf16_rne(acc[2]) | ((unsigned)f32_to_bf16_rne(acc[3]) << 16);
      *(uint2*)o = pk;
    } else {
      *(f32x4*)((float*)out + (size_t)t * H + c) = acc;
    }
  }
}

}  // namespace

int launch_combine(const float* y, const float* w, const int32_t* inv, int T, int k, int H, const float* shared,
                   void* out, int odt, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (H % 4) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: H %% 4 != 0 (H=%d)", H);
  if (k > 16) return fail(MOE_ERR_INVALID, "moe_combine: k=%d exceeds 16", k);
  int threads = 256;
  while (threads > 64 && threads * 4 > H) threads >>= 1;
  if (odt == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(threads), 0, s, y, w, inv, k, H, shared, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(threads), 0, s, y, w, inv, k, H, shared, out);
  MOE_CHECK_LAUNCH("moe_combine launch");
  return MOE_OK;
}

}  // namespace moe
