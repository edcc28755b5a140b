// Router: logits = x . Wg^T + b, then top-k (descending, ties to the lower expert id) and the
// gate weights softmax-renormalised over the chosen k.  The router is dense and scores every
// expert for every token ("Mixture of experts VRAM: total vs active parameters", section "How
// current MoE models route each token").
//
// bf16 activations: one workgroup per 16 tokens; its 8 waves cover the experts in 16-wide MFMA
// tiles (v_mfma_f32_16x16x32_bf16, fp32 accumulation) and, when there are few tiles, also split
// the hidden dimension; the 16 x E logit block goes to LDS, then each wave selects the top-k of
// 2 tokens with 64-lane shuffle reductions.
// fp32 activations: one workgroup per token, fp32 FMA dot products reduced across the wave.
#include <math.h>

#include "ffn_common.hpp"
#include "topk.hpp"

namespace moe {
namespace {

constexpr int kRouteTokens = 16;    // tokens per workgroup (MFMA M)
constexpr int kTilesPerPass = 8;    // 16-expert tiles each wave accumulates per pass over H
constexpr int kMaxE = 1024;
// The router is split over workgroups (16 x 16 logit tiles, K ranges) while T * E <= kSplitMaxTE:
// each workgroup re-reads its 16 rows of x and of Wg from L2, which is cheap until the product
// is large; larger batches use the MFMA tile kernel (one read per 192 x 256 tile).
constexpr long long kSplitMaxTE = 1 << 20;

// 8 waves: G groups of expert tiles x R ranges of H (G * R = 8).  Few experts (decode shapes):
// all waves split H, so every wave has a short run of loads in flight; many experts: waves split
// the expert tiles.  Partial logits of the R ranges are summed in LDS in fixed order.
constexpr int kRouteThreads = 512;

__global__ __launch_bounds__(kRouteThreads) void route_bf16_kernel(const unsigned short* __restrict__ x,
                                                                   const unsigned short* __restrict__ wg,
                                                                   const float* __restrict__ bias, int T, int H,
                                                                   int E, int k, int G, int32_t* __restrict__ ids,
                                                                   float* __restrict__ w,
                                                                   float* __restrict__ logits) {
  extern __shared__ float lds[];  // [R][16][Epad]
  const int Epad = ((E + 15) / 16) * 16 + 1;
  const int R = 8 / G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave % G, rng = wave / G;
  const int t0 = blockIdx.x * kRouteTokens;
  const int m = lane & 15, kq = (lane >> 4) * 8;
  const int n_tiles = (E + 15) / 16;
  const int nks = H / 32;
  const int ks0 = rng * nks / R, ks1 = (rng + 1) * nks / R;
  const bool row_ok = t0 + m < T;
  const unsigned short* xrow = x + (size_t)(row_ok ? t0 + m : 0) * H + kq;
  float* part = lds + (size_t)rng * kRouteTokens * Epad;

  for (int first = grp; first < n_tiles; first += G * kTilesPerPass) {
    f32x4 acc[kTilesPerPass];
    const unsigned short* brow[kTilesPerPass];
    bool bok[kTilesPerPass];
#pragma unroll
    for (int i = 0; i < kTilesPerPass; ++i) {
      acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      int nt = first + i * G;
      int e = nt * 16 + m;
      bok[i] = nt < n_tiles && e < E;
      brow[i] = wg + (size_t)(bok[i] ? e : 0) * H + kq;
    }
#pragma unroll 4
    for (int ks = ks0; ks < ks1; ++ks) {
      const int kk = ks * 32;
      bf16x8 a = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (row_ok) a = *(const bf16x8*)(xrow + kk);
#pragma unroll
      for (int i = 0; i < kTilesPerPass; ++i) {
        if (first + i * G < n_tiles) {  // wave-uniform
          bf16x8 b = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
          if (bok[i]) b = *(const bf16x8*)(brow[i] + kk);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kTilesPerPass; ++i) {
      int nt = first + i * G;
      if (nt >= n_tiles) continue;
      int e = nt * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = (lane >> 4) * 4 + r;
        if (e < E) part[row * Epad + e] = acc[i][r];
      }
    }
  }
  __syncthreads();
  // sum the R partial blocks into block 0 (fixed order), add the bias
  for (int i = threadIdx.x; i < kRouteTokens * E; i += blockDim.x) {
    int row = i / E, e = i % E;
    float v = lds[row * Epad + e];
    for (int r = 1; r < R; ++r) v += lds[((size_t)r * kRouteTokens + row) * Epad + e];
    v += bias ? bias[e] : 0.f;
    lds[row * Epad + e] = v;
    if (logits && t0 + row < T) logits[(size_t)(t0 + row) * E + e] = v;
  }
  __syncthreads();
  for (int row = wave; row < kRouteTokens; row += kRouteThreads / 64) {
    int t = t0 + row;
    if (t >= T) break;
    wave_topk(lds + row * Epad, E, k, ids + (size_t)t * k, w + (size_t)t * k);
  }
}

// ---- small T: the router's weight read is spread over many workgroups
//
// route_partial_kernel: workgroup (expert tile, K range, token tile) computes a 16 x 16 block of
// partial logits over its K range (its 4 waves split the range, summed in LDS in wave order)
// and stores it to part[range][t][e].  route_topk_kernel: one wave per token sums the ranges in
// order, adds the bias and selects the top k.  Both fixed-order: deterministic.
constexpr int kSplitMinSteps = 16;  // k-steps per K range (4 waves x 4)

__global__ __launch_bounds__(256) void route_partial_kernel(const unsigned short* __restrict__ x,
                                                            const unsigned short* __restrict__ wg, int T, int H,
                                                            int E, int KS, float* __restrict__ part) {
  __shared__ f32x4 red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int et = blockIdx.x, r = blockIdx.y, tt = blockIdx.z;
  const int nks = H / 32;
  const int ks0 = r * nks / KS, ks1 = (r + 1) * nks / KS;
  const int w0 = ks0 + wave * (ks1 - ks0) / 4, w1 = ks0 + (wave + 1) * (ks1 - ks0) / 4;
  const int m = lane & 15, kq = (lane >> 4) * 8;
  const int t = tt * 16 + m, e = et * 16 + m;
  const bool tok = t < T, exp = e < E;
  const unsigned short* xr = x + (size_t)(tok ? t : 0) * H + kq;
  const unsigned short* wr = wg + (size_t)(exp ? e : 0) * H + kq;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int ks = w0; ks < w1; ++ks) {
    bf16x8 a = bf16x8{0, 0, 0, 0, 0, 0, 0, 0}, b = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (tok) a = *(const bf16x8*)(xr + ks * 32);
    if (exp) b = *(const bf16x8*)(wr + ks * 32);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 v = red[0][lane];
    for (int w = 1; w < 4; ++w) {
      const f32x4 o = red[w][lane];
      v[0] += o[0], v[1] += o[1], v[2] += o[2], v[3] += o[3];
    }
    const int col = et * 16 + (lane & 15);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = tt * 16 + (lane >> 4) * 4 + q;
      if (row < T && col < E) part[((size_t)r * T + row) * E + col] = v[q];
    }
  }
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                         int T, int E, int KS, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w, float* __restrict__ logits) {
  extern __shared__ float lds[];  // [4][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave; no block barrier below
  float* lg = lds + (size_t)wave * E;
  for (int e = lane; e < E; e += 64) {
    const float v = split_logit(part, bias, T, E, KS, t, e);
    lg[e] = v;
    if (logits) logits[(size_t)t * E + e] = v;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  wave_topk(lg, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

int route_split_ranges(int T, int H, int E) {
  const int nks = H / 32;
  const int tiles = ((E + 15) / 16) * ((T + 15) / 16);
  int KS = 512 / (tiles > 0 ? tiles : 1);
  if (KS > nks / kSplitMinSteps) KS = nks / kSplitMinSteps;
  return KS < 1 ? 1 : KS;
}

__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x, const float* __restrict__ wg,
                                                        const float* __restrict__ bias, int T, int H, int E, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ w,
                                                        float* __restrict__ logits) {
  extern __shared__ float lds[];  // [E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * H;
  for (int e = wave; e < E; e += nw) {
    const float* wr = wg + (size_t)e * H;
    float acc = 0.f;
    for (int h = lane; h < H; h += 64) acc = fmaf(xr[h], wr[h], acc);
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) lds[e] = acc + (bias ? bias[e] : 0.f);
  }
  __syncthreads();
  if (logits)
    for (int e = threadIdx.x; e < E; e += blockDim.x) logits[(size_t)t * E + e] = lds[e];
  __syncthreads();
  if (wave == 0) wave_topk(lds, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

}  // namespace

// ---- large T: the logits are a dense [T x H] x [H x E] product, computed by the prefill MFMA
// tile kernel as a "down" projection of one expert whose package is the router matrix in the
// fragment layout; then the top-k kernel above with one range.

// Wg [E][H] bf16 row-major -> strips of 16 rows, 1 KiB per 32-wide k-step, lane l's 16 bytes =
// row 16s + l%16, k 32ks + 8(l/16)..+7 (the bf16 package layout); also writes offsets {0, T}.
__global__ __launch_bounds__(256) void route_pack_kernel(const unsigned short* __restrict__ wg, int H, int E, int T,
                                                         int rt, unsigned short* __restrict__ packed,
                                                         int32_t* __restrict__ offsets, int4* __restrict__ plan,
                                                         int* __restrict__ counters) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx == 0) offsets[0] = 0, offsets[1] = T;
  // The tile plan: the T rows in tiles of rt rows, each described as an "expert" of its own (one
  // tile, first row t*rt), so that the few columns (E) still give enough work items to fill the
  // GPU; and zeroed work counters.
  const int nt = (T + rt - 1) / rt;
  if (idx == 0) plan[0] = make_int4(nt, 0, 0, 0);
  if (idx < (size_t)nt) plan[1 + idx] = make_int4((int)idx, (int)idx * rt, min(rt, T - (int)idx * rt), 0);
  if (idx < 8) counters[idx] = 0;
  const size_t per_row = (size_t)H / 8;
  if (idx >= (size_t)E * per_row) return;
  const int r = (int)(idx / per_row), k = (int)(idx % per_row) * 8;
  const int st = r / 16, rr = r % 16, ks = k / 32, q = (k % 32) / 8, nks = H / 32;
  const uint4 v = *(const uint4*)(wg + (size_t)r * H + k);
  *(uint4*)(packed + ((size_t)st * nks + ks) * 512 + (rr + 16 * q) * 8) = v;
}

struct RouteTileWs {
  size_t packed_off, logits_off, offsets_off, plan_off, count_off, total;
};

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

bool route_split_path(int T, int H, int E, int xdt) {
  return xdt == MOE_BF16 && H % 32 == 0 && (long long)T * E <= kSplitMaxTE;
}

bool route_tile_path(int T, int H, int E, int xdt) {
  return xdt == MOE_BF16 && !route_split_path(T, H, E, xdt) && H % 32 == 0 && E % 16 == 0 &&
         (double)T * H < 2147483648.0;
}

RouteTileWs route_tile_ws(int T, int H, int E) {
  RouteTileWs L;
  L.packed_off = 0;
  L.logits_off = al256((size_t)E * H * 2);
  L.offsets_off = L.logits_off + al256((size_t)T * E * sizeof(float));
  L.plan_off = L.offsets_off + 256;
  L.count_off = L.plan_off + al256((size_t)(1 + (T + 15) / 16) * 16);  // tiles of >= 16 rows
  L.total = L.count_off + 256;
  return L;
}

size_t route_workspace(int T, int H, int E, int xdt) {
  if (route_tile_path(T, H, E, xdt)) return route_tile_ws(T, H, E).total;
  if (!route_split_path(T, H, E, xdt)) return 0;
  return (size_t)route_split_ranges(T, H, E) * T * E * sizeof(float);
}

int route_split_partials(const void* x, int T, int H, const void* wg, int E, float* part, int* ks_out, hipStream_t s) {
  const int KS = route_split_ranges(T, H, E);
  *ks_out = KS;
  hipLaunchKernelGGL(route_partial_kernel, dim3((E + 15) / 16, KS, (T + 15) / 16), dim3(256), 0, s,
                     (const unsigned short*)x, (const unsigned short*)wg, T, H, E, KS, part);
  MOE_CHECK_LAUNCH("moe_route launch");
  return MOE_OK;
}

int launch_route(const void* x, int xdt, int T, int H, const void* wg, const float* bias, int E, int k, int32_t* ids,
                 float* w, float* logits, void* ws, size_t ws_bytes, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (E > kMaxE) return fail(MOE_ERR_INVALID, "moe_route: E=%d exceeds %d", E, kMaxE);
  if (route_tile_path(T, H, E, xdt)) {
    const RouteTileWs L = route_tile_ws(T, H, E);
    if (!ws || ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu", ws_bytes, L.total);
    char* wsp = (char*)ws;
    unsigned short* packed = (unsigned short*)(wsp + L.packed_off);
    float* lg = (float*)(wsp + L.logits_off);
    int32_t* offs = (int32_t*)(wsp + L.offsets_off);
    int4* plan = (int4*)(wsp + L.plan_off);
    int* counters = (int*)(wsp + L.count_off);
    // row tile height: about one work item (row tile x 256 columns) per CU, 32 to kTileRows rows (every
    // row tile reads the whole router matrix again, from L2)
    const long long ncol = (E + 255) / 256;
    int rt = (int)((long long)T * ncol / cu_count()) / 16 * 16;
    rt = rt < 32 ? 32 : (rt > kTileRows ? kTileRows : rt);
    const size_t chunks = (size_t)E * H / 8, nt = (size_t)(T + rt - 1) / rt;
    const size_t threads = chunks > nt + 8 ? chunks : nt + 8;
    hipLaunchKernelGGL(route_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       (const unsigned short*)wg, H, E, T, rt, packed, offs, plan, counters);
    FfnArgs a{};
    a.packages = (const char*)packed;
    a.pkg_stride = (size_t)E * H * 2;
    a.slot_of_expert = nullptr;
    a.n_slots = 1;
    a.min_rows = 0, a.max_rows = 0x7FFFFFFF;
    a.offsets = offs;
    a.perm_src = nullptr;
    a.a = (const unsigned short*)x;
    a.out = lg;
    a.H = E;  // output columns of the "down" projection
    a.I = H;  // its contraction
    a.E = 1, a.k = 1;
    a.region_codes = 0, a.region_scales = 0;
    a.plan = plan;
    a.tcount = counters;
    // (the launch bounds the row tiles by "experts" = the nt chunks of at most rt rows)
    int rc = launch_ffn_tile_part(MOE_W_BF16, false, a, E, H, T, (int)nt, s);
    if (rc != MOE_OK) return rc;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), (size_t)4 * E * sizeof(float), s,
                       (const float*)lg, bias, T, E, 1, k, ids, w, logits);
    MOE_CHECK_LAUNCH("moe_route launch");
    return MOE_OK;
  }
  if (route_split_path(T, H, E, xdt)) {
    const size_t need = route_workspace(T, H, E, xdt);
    if (!ws || ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu", ws_bytes, need);
    int KS = 0;
    int rc = route_split_partials(x, T, H, wg, E, (float*)ws, &KS, s);
    if (rc != MOE_OK) return rc;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), (size_t)4 * E * sizeof(float), s,
                       (const float*)ws, bias, T, E, KS, k, ids, w, logits);
    MOE_CHECK_LAUNCH("moe_route launch");
    return MOE_OK;
  }
  if (xdt == MOE_BF16) {
    if (H % 32) return fail(MOE_ERR_UNSUPPORTED, "moe_route: bf16 path needs H %% 32 == 0 (H=%d)", H);
    const int Epad = ((E + 15) / 16) * 16 + 1;
    const int n_tiles = (E + 15) / 16;
    int G = 1;  // expert-tile groups; the other 8 / G waves split H
    while (G < 8 && (n_tiles + G - 1) / G > kTilesPerPass) G *= 2;
    const size_t lds = (size_t)(8 / G) * kRouteTokens * Epad * sizeof(float);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)route_bf16_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return hip_fail(e, "moe_route: LDS attribute");
    }
    hipLaunchKernelGGL(route_bf16_kernel, dim3((T + kRouteTokens - 1) / kRouteTokens), dim3(kRouteThreads), lds,
                       s, (const unsigned short*)x, (const unsigned short*)wg, bias, T, H, E, k, G, ids, w, logits);
  } else {
    hipLaunchKernelGGL(route_f32_kernel, dim3(T), dim3(256), (size_t)E * sizeof(float), s, (const float*)x,
                       (const float*)wg, bias, T, H, E, k, ids, w, logits);
  }
  MOE_CHECK_LAUNCH("moe_route launch");
  return MOE_OK;
}

}  // namespace moe
