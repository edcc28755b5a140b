// Top-k selection of one token's logits by one wave (shared by the router kernels and the fused
// route + permutation kernel).
#pragma once

#include <math.h>

#include "common.hpp"

namespace moe {

// The selection compares unsigned keys that order the logits totally: a larger logit has a larger
// key (-0 counts as +0), every NaN has key 1, below -inf, and a chosen entry has key 0, below
// everything.  So a token whose logits hold NaN or infinities still gets k distinct ids in [0, E)
// (finite and infinite logits first, NaN ones last, equal keys -> lower id), and only its own gate
// weights carry the NaN.
__device__ __forceinline__ unsigned logit_key(float v) {
  if (v != v) return 1u;
  unsigned u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(unsigned key) {
  if (key == 1u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Logit (t, e) from the router's KS K-range partials part[KS][T][E]: loaded 16 ranges at a time
// (independent loads in flight together), summed in range order, plus the bias.
__device__ __forceinline__ float split_logit(const float* __restrict__ part, const float* __restrict__ bias, int T,
                                             int E, int KS, int t, int e) {
  float v = 0.f;
  for (int r0 = 0; r0 < KS; r0 += 16) {
    float pv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = r0 + i < KS ? r0 + i : r0;
      pv[i] = part[((size_t)r * T + t) * E + e];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (r0 + i < KS) v = (r0 + i == 0) ? pv[i] : v + pv[i];
  }
  return v + (bias ? bias[e] : 0.f);
}

// Wave-wide reductions without LDS traffic: across the two 32-lane halves and the 16-lane rows by
// gfx950's permlane swaps (with both operands the same register, swap 32 pairs lane l with l +- 32
// and swap 16 pairs row r with r ^ 1), inside a row by DPP rotations by 8 and 4 and two quad
// permutations.  Every lane ends with the result.
template <typename F>
__device__ __forceinline__ void wave_combine_2x32(unsigned& hi, unsigned& lo, F take) {
  {
    const auto a = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    // a[0], a[1] (and b[0], b[1]) hold this lane's value and its partner's, in some order
    hi = a[0], lo = b[0];
    take(a[1], b[1]);
  }
  {
    const auto a = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    hi = a[0], lo = b[0];
    take(a[1], b[1]);
  }
  take((unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, 0x128, 0xF, 0xF, false),   // row_ror:8
       (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, 0x128, 0xF, 0xF, false));
  take((unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, 0x124, 0xF, 0xF, false),   // row_ror:4
       (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, 0x124, 0xF, 0xF, false));
  take((unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, 0x4E, 0xF, 0xF, false),    // quad_perm 2,3,0,1
       (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, 0x4E, 0xF, 0xF, false));
  take((unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, 0xB1, 0xF, 0xF, false),    // quad_perm 1,0,3,2
       (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  unsigned hi = (unsigned)(v >> 32), lo = (unsigned)v;
  wave_combine_2x32(hi, lo, [&](unsigned ohi, unsigned olo) {
    const bool t = ohi > hi || (ohi == hi && olo > lo);
    hi = t ? ohi : hi;
    lo = t ? olo : lo;
  });
  return ((unsigned long long)hi << 32) | lo;
}

// sum over the wave; lane 0's sum (one fixed order) for every lane
__device__ __forceinline__ float wave_sum_f32(float v) {
  unsigned hi = __float_as_uint(v), lo = 0;
  wave_combine_2x32(hi, lo, [&](unsigned ohi, unsigned) { hi = __float_as_uint(__uint_as_float(hi) + __uint_as_float(ohi)); });
  return __uint_as_float(__builtin_amdgcn_readfirstlane(hi));
}

// top-k of one token's E logits in LDS row `lg`; executed by one full wave.  The row is turned into
// keys in place (logit_key), chosen entries get key 0.  Lane j keeps the j-th choice and writes
// ids[j], w[j] (and ids_copy[j] when given).
__device__ inline void wave_topk(float* lg, int E, int k, int32_t* ids, float* w, int32_t* ids_copy = nullptr) {
  const int lane = threadIdx.x & 63;
  unsigned* key = (unsigned*)lg;
  for (int e = lane; e < E; e += 64) key[e] = logit_key(lg[e]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  unsigned my_key = 0;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    // (key, E - 1 - id) as one 64-bit value: its maximum is the largest key, then the lowest id;
    // an unchosen entry (key >= 1) always exists because k <= E
    unsigned long long best = 0;
    for (int e = lane; e < E; e += 64) {
      const unsigned long long c = ((unsigned long long)key[e] << 32) | (unsigned)(E - 1 - e);
      best = c > best ? c : best;
    }
    best = wave_max_u64(best);
    const int be = E - 1 - (int)(unsigned)(best & 0xFFFFFFFFull);
    if (lane == j) my_key = (unsigned)(best >> 32), my_e = be;
    if (lane == 0) key[be] = 0u;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  const float my_v = key_logit(my_key);
  // softmax over the k chosen logits (max = the first choice)
  const float v0 = __shfl(my_v, 0, 64);
  float p = lane < k ? expf(my_v - v0) : 0.f;
  const float z = wave_sum_f32(p);
  if (lane < k) {
    ids[lane] = my_e;
    w[lane] = p / z;
    if (ids_copy) ids_copy[lane] = my_e;
  }
}

}  // namespace moe
