// Device pieces shared by the expert-FFN kernels (streaming and tile variants): in-register
// decoders of the 4-bit formats, MFMA wrappers, the row-tile lookup and the argument block.
#pragma once

#include <math.h>

#include "common.hpp"

namespace moe {

// Read-only zeros (one copy per translation unit): the address of prefetches that fall past the
// last stage or block, so that the loads of a software pipeline stay unconditional.  1 KiB covers
// one lane-strided 16-byte fragment load and every scale or activation offset of a stage.
static __device__ __attribute__((aligned(1024))) unsigned char g_zero_page[1024];

// s_waitcnt that waits until at most n vector-memory loads are outstanding (expcnt and lgkmcnt
// left alone); n < 64
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier that leaves vector-memory loads in flight (__syncthreads' fence would wait
// for all of them, including direct-to-LDS loads of later pipeline stages).  The memory clobber
// keeps the compiler from moving memory accesses across it; LDS reads of this wave are complete.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ decoders

// The scaled conversions read only the exponent field of their fp32 scale operand, which is
// exactly an E8M0 byte placed at bit 23 (0 -> 2^-127, 0xFF -> NaN).
__device__ __forceinline__ float e8m0_to_f32(unsigned s) { return __uint_as_float(s << 23); }

// 8 MXFP4 elements (4 bytes, element 2b / 2b+1 in the low / high nibble of byte b) -> bf16
__device__ __forceinline__ bf16x8 dec_mxfp4(unsigned word, unsigned scale_byte) {
  float s = e8m0_to_f32(scale_byte);
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// A constant the compiler must keep in a VGPR: three-operand instructions (v_and_or_b32) take no
// literal operand, so constants in registers let (x & mask) | magic be one instruction.
__device__ __forceinline__ unsigned in_vgpr(unsigned c) {
  unsigned r;
  asm("; const in vgpr" : "=v"(r) : "0"(c));
  return r;
}

// 8 INT4 elements (nibble n < 4: element 2n, n >= 4: element 2(n-4)+1, stored as q + 8) -> fp16 q*s,
// by the usual "magic number" integer-to-float conversion: fp16 0x6400 is 1024, whose unit in the
// last place is 1, so OR-ing c = q + 8 into its low mantissa bits gives exactly 1024 + c in each
// half; minus 1032 gives q, times s.  The nibble pairs at bits 4-7 of each half need no shift:
// fp16 0x5400 is 64, whose unit in the last place is 1/16, so OR-ing c << 4 into it gives exactly
// 64 + c, minus 72 gives q.  Pairs 0 and 1 come from v, pairs 2 and 3 from v >> 8 (one shift for
// the eight elements).  Every step is exact in fp16 for s in binary16's normal range.
__device__ __forceinline__ f16x8 dec_int4(unsigned v, _Float16 s) {
  const f16x2 bias_lo = {(_Float16)1032.0f, (_Float16)1032.0f}, bias_hi = {(_Float16)72.0f, (_Float16)72.0f};
  const f16x2 ss = {s, s};
  const unsigned mask_lo = in_vgpr(0x000F000Fu), magic_lo = in_vgpr(0x64006400u);
  const unsigned mask_hi = in_vgpr(0x00F000F0u), magic_hi = in_vgpr(0x54005400u);
  const unsigned v8 = v >> 8;
  f16x2 r[4];
  r[0] = (__builtin_bit_cast(f16x2, (v & mask_lo) | magic_lo) - bias_lo) * ss;
  r[1] = (__builtin_bit_cast(f16x2, (v & mask_hi) | magic_hi) - bias_hi) * ss;
  r[2] = (__builtin_bit_cast(f16x2, (v8 & mask_lo) | magic_lo) - bias_lo) * ss;
  r[3] = (__builtin_bit_cast(f16x2, (v8 & mask_hi) | magic_hi) - bias_hi) * ss;
  return f16x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

template <int FMT>
struct Op;  // MFMA operand type per weight format
template <>
struct Op<MOE_W_BF16> {
  typedef bf16x8 T;
};
template <>
struct Op<MOE_W_MXFP4> {
  typedef bf16x8 T;
};
template <>
struct Op<MOE_W_INT4G32> {
  typedef f16x8 T;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ row tiles

// Row tile `slot` of the grouped rows: experts in id order (those with lo <= n_e <= hi), each cut
// into ceil(n_e / mr) tiles.
// Executed by wave 0; result in shared memory.  Returns false (all threads) when the slot is
// past the last tile.
struct RowTile {
  int e, p0, rows;  // expert, first grouped row, rows in this tile (<= mr)
};

__device__ inline bool find_row_tile(const int32_t* __restrict__ offsets, int E, int mr, int slot, RowTile* sh,
                                     int lo = 0, int hi = 0x7FFFFFFF) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int e_begin = lane * per, e_end = min(E, e_begin + per);
    int local = 0;
    for (int e = e_begin; e < e_end; ++e) {
      int c = offsets[e + 1] - offsets[e];
      if (c < lo || c > hi) c = 0;
      local += (c + mr - 1) / mr;
    }
    int incl = local;
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - local;
    bool mine = slot >= excl && slot < incl;
    if (lane == 63 && slot >= incl) sh->e = -1;
    if (mine) {
      int acc = excl;
      for (int e = e_begin; e < e_end; ++e) {
        int o0 = offsets[e], c = offsets[e + 1] - o0;
        if (c < lo || c > hi) c = 0;
        int nt = (c + mr - 1) / mr;
        if (slot < acc + nt) {
          int t = slot - acc;
          sh->e = e;
          sh->p0 = o0 + t * mr;
          sh->rows = min(mr, c - t * mr);
          break;
        }
        acc += nt;
      }
    }
  }
  __syncthreads();
  return sh->e >= 0;
}

struct FfnArgs {
  const char* packages;
  size_t pkg_stride;
  const int32_t* slot_of_expert;
  int n_slots;            // valid slots are [0, n_slots)
  int min_rows, max_rows;  // experts with a row count outside [min_rows, max_rows] are left to the other variant
  const int32_t* offsets;
  const int32_t* perm_src;
  const unsigned short* a;  // GU: activations [T][H] (operand type); down: h [T*k][I]
  void* out;                // GU: h [T*k][I] (operand type); down: y_perm [T*k][H] fp32
  int H, I, E, k;
  size_t region_codes, region_scales;  // byte offsets of this matrix's codes / scales in a package
  // row tiles (16 * mt rows for the streaming variant, 192 for the tile variant): plan[0].x =
  // tiles; plan[1 + t] = {first tile of the expert of tile t, the expert's first grouped row, its
  // rows, its slot}, written by the plan kernel from the offsets and the slot table (streaming
  // variant: null when the kernel finds its tile itself, see DirectTiles)
  const int4* plan;
  int* tcount;  // [8] work counters of the persistent kernels, one per XCD range, zeroed by the plan kernel
  // INT4 experts: the power of two each token's activations were divided by in the fp16 cast
  // (xscale[t] = s_t), or null when they were not scaled
  const float* xscale;
  // block-scaled MXFP4 path: the A operand as two MXFP8 terms, [rows][K] bytes each, and the E8M0
  // scales of every 32-element block [rows][K/32] (hi byte | lo byte << 8)
  const unsigned char* a_hi;
  const unsigned char* a_lo;
  const unsigned short* a_sc;
};

// INT4 experts multiply fp16 activations scaled per token: x' = x / s_t, with s_t a power of two
// chosen so that the token's largest magnitude lies in [4, 8) (any finite activation then fits
// binary16 with its bf16 precision).  Gate/up then yield g' = g / s and u' = u / s (exactly: scaling by a
// power of two commutes with every rounding); the stored intermediate is h' = SiLU(g) u / s^2 =
// g' u' / (1 + e^(-g' s)), and the down projection yields y' = y / s^2, multiplied back by s twice.
__device__ __forceinline__ float token_scale(const FfnArgs& a, int p) { return a.xscale[a.perm_src[p] / a.k]; }
__device__ __forceinline__ float swiglu_scaled(float g, float u, float s) { return g * u / (1.0f + __expf(-(g * s))); }


// The streaming kernels' row tiles without a plan kernel (launches with few routed rows): the tiles
// plan_kernel would write -- mr rows at a time over the experts in order, counting the experts whose
// row count lies in [min_rows, max_rows] and whose slot is resident -- found by each wave on its own
// from the offsets, so the results are wave-uniform and no LDS or barrier is involved.  Lane l
// covers experts [l * per, (l + 1) * per), per <= kDirectPer (E <= 512), and keeps their first row,
// row count and slot in registers; scan() gives its tiles' range [excl, incl) and the total.
constexpr int kDirectPer = 8;
struct DirectTiles {
  int per, excl, incl, total;
  int o0[kDirectPer], c[kDirectPer], slot[kDirectPer];

  __device__ void scan(const FfnArgs& a, int mr) {
    const int lane = threadIdx.x & 63;
    per = (a.E + 63) / 64;
    int local = 0;
#pragma unroll
    for (int i = 0; i < kDirectPer; ++i) {
      const int e = lane * per + i;
      o0[i] = 0, c[i] = 0, slot[i] = -1;
      if (i < per && e < a.E) {
        o0[i] = a.offsets[e];
        c[i] = a.offsets[e + 1] - o0[i];
        slot[i] = a.slot_of_expert ? a.slot_of_expert[e] : e;
        if (c[i] < a.min_rows || c[i] > a.max_rows || (unsigned)slot[i] >= (unsigned)a.n_slots) c[i] = 0;
      }
      local += (c[i] + mr - 1) / mr;
    }
    incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    excl = incl - local;
    total = __builtin_amdgcn_readlane(incl, 63);
  }
  // the plan entry of tile `tile` (uniform, < total): {first tile of its expert, the expert's first
  // grouped row, its rows, its slot}
  __device__ int4 entry(int mr, int tile) const {
    const unsigned long long b = __ballot(tile >= excl && tile < incl);
    const int owner = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(b));
    int4 r = make_int4(0, 0, 0, 0);
    int acc = excl;
    bool found = false;
#pragma unroll
    for (int i = 0; i < kDirectPer; ++i) {
      const int nt = (c[i] + mr - 1) / mr;
      if (!found && tile < acc + nt) {
        r = make_int4(acc, o0[i], c[i], slot[i]);
        found = true;
      }
      acc += nt;
    }
    return make_int4(__builtin_amdgcn_readlane(r.x, owner), __builtin_amdgcn_readlane(r.y, owner),
                     __builtin_amdgcn_readlane(r.z, owner), __builtin_amdgcn_readlane(r.w, owner));
  }
};

constexpr int kXcds = 8;  // XCDs of an MI355X; workgroup i is dispatched to XCD i % 8
// Rows of a tile of the prefill (MFMA tile) kernel at most: its plans cut an expert with n rows
// into ceil(n / kTileRows) tiles that split the rows evenly.
constexpr int kTileRows = 192;

// Dynamic work distribution over a persistent grid.  The work items are dealt in contiguous
// ranges of `per` to the 8 XCDs (workgroup i runs on XCD i % 8), so that consecutive items (the
// column tiles or unit groups of one row tile) run on one XCD and share its L2; each range has a
// counter (zeroed by the plan kernel), and a workgroup takes the next item of its own XCD's range,
// then of the others' once that is drained.  Only thread 0 holds the state; an atomic is issued
// one item ahead and resolved at the start of the next item, after it has long returned.
struct WorkSched {
  int* cnt;  // [kXcds] items taken from each range
  int per, total;
  int xs, tried, pend;  // range being drained, ranges tried, raw result of the last atomic
};
__device__ __forceinline__ int sched_resolve(WorkSched& s) {
  for (;;) {
    if (s.tried >= kXcds) return -1;
    if (s.pend < min(s.per, s.total - s.xs * s.per)) return s.xs * s.per + s.pend;
    if (++s.tried >= kXcds) return -1;  // every range drained
    s.xs = (s.xs + 1) % kXcds;
    s.pend = atomicAdd(&s.cnt[s.xs], 1);
  }
}
__device__ __forceinline__ void sched_issue(WorkSched& s) {
  if (s.tried < kXcds) s.pend = atomicAdd(&s.cnt[s.xs], 1);
}

// compute units of the current device (cached per device)
inline int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Prefill (tile) variant, one matrix: gate/up (with SwiGLU) or down, for the experts whose row
// count lies in [a.min_rows, a.max_rows].
int launch_ffn_tile_part(int fmt, bool gate_up, const FfnArgs& a, int H, int I, int n, int E, hipStream_t s);

// Block-scaled MXFP4 path: rows of x (bf16 / fp32) or h (bf16) -> two MXFP8 terms and their scales;
// then one matrix of the streaming FFN on v_mfma_scale_f32_16x16x128_f8f6f4 (a.plan: 16*mt-row tiles).
void launch_quant_mx8(const void* x, bool src_bf16, int rows, int K, unsigned char* hi, unsigned char* lo,
                      unsigned short* sc, hipStream_t s);
int launch_ffn_mx_part(int mt, bool gate_up, const FfnArgs& a, int H, int I, int S, hipStream_t s);

}  // namespace moe
