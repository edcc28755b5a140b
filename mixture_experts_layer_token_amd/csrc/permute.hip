// Stable grouping of the T*k (token, slot) pairs by expert: histogram, exclusive scan, stable
// scatter.  Grouping tokens by the expert they chose is what lets one read of an expert's
// weights serve all of them ("Understanding MoE Inference Costs on Galactus", section "Prompt
// processing is a different phase").
//
// Small batches (T*k <= kSingleMax, decode): one workgroup of 1024 threads does the whole job:
//   1. LDS histogram with LDS atomics (order-free: only counts);
//   2. exclusive scan of the E <= 1024 counts (one per thread);
//   3. stable scatter in chunks of 1024 flat indices: inside a wave, each lane's rank among
//      lanes with the same expert comes from 10 ballots over the bits of the expert id; the 16
//      waves of a chunk then claim their ranges from a per-expert cursor in wave order.
// Large batches (prefill): the flat indices are cut into blocks of kBlk; (1) every block counts
// its experts, (2) one workgroup scans the counts per expert over blocks and over experts (the
// offsets, and each block's starting cursor per expert), (3) every block scatters its indices
// in order from those cursors with the same in-block ranking.  Same result, block-parallel.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kBlk = 2048;         // flat indices per block (multi-block path)
constexpr int kSingleMax = 8192;   // largest T*k done by the single workgroup

__device__ void scatter_range(const int32_t* __restrict__ ids, int i0, int i1, int E, int* cursor,
                              int32_t* __restrict__ perm, int32_t* __restrict__ inv);

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
  // the end of the last expert's range is the number of pairs placed (pairs with an id outside
  // [0, E) are dropped), so no range covers an unwritten entry
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    offsets[E] = total;
  }
  __syncthreads();

  scatter_range(ids, 0, n, E, cursor, perm, inv);
}

// Stable scatter of flat indices [i0, i1) (1024 threads), cursor[e] = next position of expert e.
__device__ void scatter_range(const int32_t* __restrict__ ids, int i0, int i1, int E, int* cursor,
                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int c0 = i0; c0 < i1; c0 += kPermThreads) {
    const int i = c0 + tid;
    const bool valid = i < i1;
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
    if (valid && e < 0) inv[i] = -1;  // a dropped pair: its combine term is skipped
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

// (1) per-block expert counts: bcnt[b][e]
__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                  int32_t* __restrict__ bcnt) {
  __shared__ int cnt[1024];
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int i1 = min(n, (b + 1) * kBlk);
  for (int i = b * kBlk + tid; i < i1; i += kPermThreads) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) bcnt[(size_t)b * E + e] = cnt[e];
}

// (2) one workgroup: thread e sums its expert over the blocks, the totals are scanned over
// experts, and bbase[b][e] = offsets[e] + the counts of expert e in blocks before b
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(const int32_t* __restrict__ bcnt, int B, int n, int E,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ bbase) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v = 0;
  if (tid < E)
    for (int b = 0; b < B; ++b) v += bcnt[(size_t)b * E + tid];
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int excl = base + incl - v;
  if (tid < E) {
    counts[tid] = v;
    offsets[tid] = excl;
    int run = excl;
    for (int b = 0; b < B; ++b) {
      bbase[(size_t)b * E + tid] = run;
      run += bcnt[(size_t)b * E + tid];
    }
  }
  if (tid == 0) {  // pairs placed (ids outside [0, E) are dropped)
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    offsets[E] = total;
  }
}

// (3) block b scatters its indices in order, starting expert e at bbase[b][e]
__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                    const int32_t* __restrict__ bbase,
                                                                    int32_t* __restrict__ perm,
                                                                    int32_t* __restrict__ inv) {
  __shared__ int cursor[1024];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kPermThreads) cursor[e] = bbase[(size_t)b * E + e];
  __syncthreads();
  scatter_range(ids, b * kBlk, min(n, (b + 1) * kBlk), E, cursor, perm, inv);
}

}  // namespace

size_t permute_workspace(int T, int k, int E) {
  const long long n = (long long)T * k;
  if (n <= kSingleMax) return 0;
  const long long B = (n + kBlk - 1) / kBlk;
  return (size_t)(2 * B * E) * sizeof(int32_t);  // bcnt and bbase
}

int launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                   int32_t* inv, void* ws, size_t ws_bytes, hipStream_t s) {
  if (E > 1024) return fail(MOE_ERR_INVALID, "moe_permute: E=%d exceeds 1024", E);
  const int n = T * k;
  if (n <= kSingleMax) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, n, E, counts, offsets, perm, inv);
  } else {
    const size_t need = permute_workspace(T, k, E);
    if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu", ws_bytes, need);
    const int B = (n + kBlk - 1) / kBlk;
    int32_t* bcnt = (int32_t*)ws;
    int32_t* bbase = bcnt + (size_t)B * E;
    hipLaunchKernelGGL(perm_count_kernel, dim3(B), dim3(kPermThreads), 0, s, ids, n, E, bcnt);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, s, bcnt, B, n, E, counts, offsets, bbase);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(B), dim3(kPermThreads), 0, s, ids, n, E, bbase, perm, inv);
  }
  MOE_CHECK_LAUNCH("moe_permute launch");
  return MOE_OK;
}

}  // namespace moe
