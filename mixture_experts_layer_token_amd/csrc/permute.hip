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
// Decode batches routed and grouped in one call (moe_route_permute): after the router's partial
// logits, a single workgroup sums them, selects every token's top k (at most 16 tokens, one per
// wave) and groups the pairs from an LDS copy of the ids: one launch and one dependent step less.
#include "common.hpp"
#include "topk.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kBlk = 2048;         // flat indices per block (multi-block path)
constexpr int kSingleMax = 8192;   // largest T*k done by the single workgroup
constexpr int kFusedMaxT = 16;     // largest batch routed and grouped by one workgroup (route_permute):
                                   // one token per wave

__device__ void scatter_range(const int32_t* ids, int i0, int i1, int E, int* cursor, int32_t* __restrict__ perm,
                              int32_t* __restrict__ inv);

// The whole grouping by one workgroup of kPermThreads threads (ids may be in LDS or global memory).
__device__ void group_pairs(const int32_t* ids, int n, int E, int32_t* __restrict__ counts,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
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

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv) {
  group_pairs(ids, n, E, counts, offsets, perm, inv);
}

// Decode-sized batches (T <= kFusedMaxT), router and grouping in one workgroup after the router's
// partial logits (route_split_partials): each of the 16 waves sums the K ranges of a token's logits in
// range order, adds the bias and selects its top k (as route_topk_kernel does), keeping the ids in
// LDS as well; then the workgroup groups the pairs as permute_kernel does.
__global__ __launch_bounds__(kPermThreads) void topk_permute_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, int T, int E, int KS, int k,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ logits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ float lg_all[];  // [16][E] logit rows, then [T * k] ids
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* ids_lds = (int32_t*)(lg_all + 16 * E);
  float* lg = lg_all + (size_t)wave * E;
  for (int t = wave; t < T; t += kPermThreads / 64) {
    for (int e = lane; e < E; e += 64) {
      const float v = split_logit(part, bias, T, E, KS, t, e);
      lg[e] = v;
      if (logits) logits[(size_t)t * E + e] = v;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    wave_topk(lg, E, k, ids + (size_t)t * k, w + (size_t)t * k, ids_lds + t * k);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  __syncthreads();
  group_pairs(ids_lds, T * k, E, counts, offsets, perm, inv);
}

// Stable scatter of flat indices [i0, i1) (1024 threads), cursor[e] = next position of expert e.
__device__ void scatter_range(const int32_t* ids, int i0, int i1, int E, int* cursor,
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
    // only the waves that hold pairs of this chunk take a turn (decode batches: one or a few)
    const int turns = min(kPermThreads / 64, (i1 - c0 + 63) / 64);
    for (int w = 0; w < turns; ++w) {
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

bool route_permute_fused(int T, int H, int E, int k, int xdt) {
  return T <= kFusedMaxT && (long long)T * k <= 1024 && route_split_path(T, H, E, xdt);
}

size_t route_permute_workspace(int T, int H, int E, int k, int xdt) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  if (route_permute_fused(T, H, E, k, xdt)) return al(route_workspace(T, H, E, xdt));
  return al(route_workspace(T, H, E, xdt)) + al(permute_workspace(T, k, E));
}

int launch_route_permute(const void* x, int xdt, int T, int H, const void* wg, const float* bias, int E, int k,
                         int32_t* ids, float* w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* inv, void* ws, size_t ws_bytes, hipStream_t s) {
  const size_t need = route_permute_workspace(T, H, E, k, xdt);
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_ERR_WORKSPACE, "moe_route_permute: workspace %zu < %zu", ws_bytes, need);
  if (E > 1024) return fail(MOE_ERR_INVALID, "moe_route_permute: E=%d exceeds 1024", E);
  if (!route_permute_fused(T, H, E, k, xdt)) {
    const size_t rws = (route_workspace(T, H, E, xdt) + 255) & ~(size_t)255;
    int rc = launch_route(x, xdt, T, H, wg, bias, E, k, ids, w, logits, ws, rws, s);
    if (rc != MOE_OK) return rc;
    return launch_permute(ids, T, k, E, counts, offsets, perm, inv, (char*)ws + rws, ws_bytes - rws, s);
  }
  if (T == 0) return launch_permute(ids, T, k, E, counts, offsets, perm, inv, nullptr, 0, s);
  int KS = 0;
  int rc = route_split_partials(x, T, H, wg, E, (float*)ws, &KS, s);
  if (rc != MOE_OK) return rc;
  // 16 logit rows of E <= 1024 floats and T*k <= 1024 ids: at most 68 KiB of dynamic LDS
  const size_t lds = (size_t)16 * E * sizeof(float) + (size_t)T * k * sizeof(int32_t);
  static bool attr_set[64];  // per device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_permute_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       16 * 1024 * (int)sizeof(float) + 1024 * (int)sizeof(int32_t));
    if (e != hipSuccess) return hip_fail(e, "moe_route_permute: LDS attribute");
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(topk_permute_kernel, dim3(1), dim3(kPermThreads), lds, s, (const float*)ws, bias, T, E, KS, k,
                     ids, w, logits, counts, offsets, perm, inv);
  MOE_CHECK_LAUNCH("moe_route_permute launch");
  return MOE_OK;
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
