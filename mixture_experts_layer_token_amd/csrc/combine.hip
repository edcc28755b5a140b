// Weighted combine: every token collects the outputs of the experts it was sent to ("Mixture of
// experts VRAM: total vs active parameters", section "Expert parallelism on RTX PRO 6000 and
// H200 NVL": dispatch, then collect the results) and weights them by its gate weights; an
// always-on shared expert is added with weight 1 (same page, routing section).
//
// Gather form: one workgroup per token reads its k rows of y_perm through inv_perm and writes
// the token's row once.  fp32 sum in slot order, then the shared row, then one rounding; no
// atomics, so the result is bitwise deterministic.  HBM-bound: 16-byte loads and stores.
#include <utility>

#include "common.hpp"

namespace moe {
namespace {

// Every byte is touched once: y_perm and shared are read, out is written, with non-temporal
// hints so that they stream past the caches (11% faster on the Kimi-shaped layer: 8192 tokens,
// top-8, hidden 7168).
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

template <bool BF16_OUT, int K>
__global__ __launch_bounds__(512) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv, int H,
                                                      const float* __restrict__ shared, void* __restrict__ out) {
  const int t = blockIdx.x;
  // the token's k rows of y_perm and gate weights (uniform)
  int rows[K];
  float gates[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = __builtin_amdgcn_readfirstlane(inv[(size_t)t * K + j]);
    gates[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, w[(size_t)t * K + j])));
  }
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    // the k rows' loads are issued together, then summed in slot order
    f32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      // a pair the permutation dropped (inv_perm -1: its expert id was outside [0, E)) adds nothing
      v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (rows[j] >= 0) v[j] = ld_stream((const f32x4*)(y + (size_t)rows[j] * H + c));
    }
    f32x4 sv = {0.f, 0.f, 0.f, 0.f};
    if (shared) sv = ld_stream((const f32x4*)(shared + (size_t)t * H + c));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (rows[j] >= 0)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(gates[j], v[j][q], acc[q]);
    if (shared)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += sv[q];
    if constexpr (BF16_OUT) {
      u32x2 pk;
      pk[0] = (unsigned)f32_to_bf16_rne(acc[0]) | ((unsigned)f32_to_bf16_rne(acc[1]) << 16);
      pk[1] = (unsigned)f32_to_bf16_rne(acc[2]) | ((unsigned)f32_to_bf16_rne(acc[3]) << 16);
      st_stream((u32x2*)((unsigned short*)out + (size_t)t * H + c), pk);
    } else {
      st_stream((f32x4*)((float*)out + (size_t)t * H + c), acc);
    }
  }
}

template <int K>
void launch_k(bool bf16, unsigned T, unsigned threads, const float* y, const float* w, const int32_t* inv, int H,
              const float* shared, void* out, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((combine_kernel<true, K>), dim3(T), dim3(threads), 0, s, y, w, inv, H, shared, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, K>), dim3(T), dim3(threads), 0, s, y, w, inv, H, shared, out);
}

template <int... Ks>
void launch_any_k(int k, bool bf16, unsigned T, unsigned threads, const float* y, const float* w, const int32_t* inv,
                  int H, const float* shared, void* out, hipStream_t s, std::integer_sequence<int, Ks...>) {
  ((k == Ks + 1 ? launch_k<Ks + 1>(bf16, T, threads, y, w, inv, H, shared, out, s) : void()), ...);
}

}  // namespace

int launch_combine(const float* y, const float* w, const int32_t* inv, int T, int k, int H, const float* shared,
                   void* out, int odt, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (H % 4) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: H %% 4 != 0 (H=%d)", H);
  if (k < 1 || k > 16) return fail(MOE_ERR_INVALID, "moe_combine: k=%d outside 1..16", k);
  int threads = 512;
  while (threads > 64 && threads * 4 > H) threads >>= 1;
  launch_any_k(k, odt == MOE_BF16, (unsigned)T, (unsigned)threads, y, w, inv, H, shared, out, s,
               std::make_integer_sequence<int, 16>{});
  MOE_CHECK_LAUNCH("moe_combine launch");
  return MOE_OK;
}

}  // namespace moe
