// Stable grouping of the T*k (token, slot) pairs by expert: histogram, exclusive scan, stable
// scatter.  Grouping tokens by the expert they chose is what lets one read of an expert's
// weights serve all of them ("Understanding MoE Inference Costs on Galactus", section "Prompt
// processing is a different phase").
//
// One workgroup of 1024 threads does the whole job (T*k is at most a few times 10^4 for the
// layers served here, so a single CU finishes in microseconds and no inter-block protocol is
// needed):
//   1. LDS histogram with LDS atomics (order-free: only counts);
//   2. exclusive scan of the E <= 1024 counts (one per thread);
//   3. stable scatter in chunks of 1024 flat indices: inside a wave, each lane's rank among
//      lanes with the same expert comes from 10 ballots over the bits of the expert id; the 16
//      waves of a chunk then claim their ranges from a per-expert cursor in wave order.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv) {
  __shared__ int cnt[1024];
  __shared__ int cursor[1024];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // exclusive scan of cnt[0..E): wave-level inclusive scan, then across the 16 waves
  int v = tid < E ? cnt[tid] : 0;
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int excl = base + incl - v;
  if (tid < E) {
    counts[tid] = v;
    offsets[tid] = excl;
    cursor[tid] = excl;
  }
  if (tid == 0) offsets[E] = n;
  __syncthreads();

  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int c0 = 0; c0 < n; c0 += kPermThreads) {
    const int i = c0 + tid;
    const bool valid = i < n;
    int e = valid ? ids[i] : -1;
    if (valid && (unsigned)e >= (unsigned)E) e = -1;  // out-of-range ids are dropped
    // peers: lanes of this wave holding the same expert id
    unsigned long long peers = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      unsigned long long m = __ballot(e >= 0 && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    if (e < 0) peers = 0;
    const int rank = __popcll(peers & below);
    const int total = __popcll(peers);
    for (int w = 0; w < 16; ++w) {
      if (wave == w && e >= 0) {
        // every lane of the wave reads cursor[e] (one LDS instruction) before the last peer
        // advances it (a later instruction of the same wave)
        int pos = cursor[e] + rank;
        perm[pos] = i;
        inv[i] = pos;
        if (rank == total - 1) cursor[e] = pos + 1;
      }
      __syncthreads();
    }
  }
}

}  // namespace

int launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                   int32_t* inv, hipStream_t s) {
  if (E > 1024) return fail(MOE_ERR_INVALID, "moe_permute: E=%d exceeds 1024", E);
  int n = T * k;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, n, E, counts, offsets, perm, inv);
  MOE_CHECK_LAUNCH("moe_permute launch");
  return MOE_OK;
}

}  // namespace moe
