// Prefill variant of the grouped SwiGLU expert FFN: output-stationary MFMA tiles.
//
// When many tokens share an expert, one read of its weights serves many rows and the
// contraction becomes dense ("Understanding MoE Inference Costs on Galactus", section "Prompt
// processing is a different phase"), so the roofline is MFMA throughput rather than HBM.
//
// A workgroup (4 waves, one per SIMD) computes up to 192 rows x 256 columns of one expert:
//  - an expert with c rows gets ceil(c / 192) row tiles that split its rows evenly; a tile of
//    `rows` rows runs with NMT = ceil(rows / 16) MFMA row tiles (a template parameter), so the
//    matrix cores only compute rows that exist, to 16-row granularity;
//  - activation rows (gathered through perm_src for gate/up) are staged in LDS by direct
//    global->LDS loads, one K block (64 wide for 4-bit weights, 32 for bf16) per buffer, and
//    read back as MFMA A operands (16-byte chunks XOR-swizzled per row against bank conflicts);
//  - each wave owns all rows x 4 strips of 16 columns; its weight fragments come straight from
//    the package into registers (16 bytes per lane are one bf16 MFMA B operand; a 4-bit lane
//    word holds 4 k-steps, a block reads half of it) and are decoded in registers (MXFP4 ->
//    bf16, INT4 -> fp16, both exact);
//  - a kD-deep software pipeline: block kb+kD-1's activations and weights are issued while
//    block kb is computed, every load unconditional and issued in block order, so waiting for
//    one block never waits for a later one, and the barrier leaves later loads in flight;
//  - v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation in AGPRs, updated in place;
//  - one wave per SIMD issues every instruction itself, so the K loop is laid out by hand:
//    between consecutive MFMAs sits at most a step or two of other work (the decode of the next
//    strip's operand, an A-fragment read for the next k-step, one load of the block kD-1 ahead);
//  - the weights are the MFMA's first operand, so a lane's results are 4 consecutive output
//    features of one row; gate/up epilogue: SiLU(g) * u on the lane's own (gate, up) pairs,
//    rounded once to h, 8 bytes per store; down epilogue: fp32 y_perm, 16 bytes per store.
// The grid is persistent (one workgroup per CU) and work items are taken dynamically, XCD-aware:
// consecutive items (all column blocks of a row tile, then the next row tile of the same expert)
// belong to the same XCD's range, so one L2 holds the tile's activations and the expert's weights
// while they are reused; a workgroup moves on to other XCDs' ranges once its own is drained.  The
// next item's first blocks are loaded while the current item's results are written.
#pragma once

#include <utility>

#include "ffn_common.hpp"

namespace moe {
namespace {

constexpr int kTW = 4;    // waves per workgroup, one per SIMD; each owns 64 columns
constexpr int kTM = kTileRows;  // rows per workgroup tile (at most)
constexpr int kTN = 256;  // columns per workgroup tile
constexpr int kMT = kTM / 16;  // 16-row MFMA tiles of a full row tile
constexpr int kWGPerCU = kTM <= 96 ? 2 : 1;  // resident workgroups per CU (register file)
constexpr int kWNS = 4;   // 16-column strips per wave
#ifndef MOE_CFG_TILE_D_BF16
#define MOE_CFG_TILE_D_BF16 4
#endif
#ifndef MOE_CFG_TILE_D_Q4
#define MOE_CFG_TILE_D_Q4 4
#endif
template <int FMT>
struct TileCfg {
  static constexpr int BK = FMT == MOE_W_BF16 ? 32 : 64;  // K per block
  // pipeline depth kD: K blocks in flight (4 covers the load latency: 5 measured no faster for
  // 4-bit weights and costs 12 more registers, 3 measured 14% slower on the INT4 gate/up of the
  // Kimi-shaped layer); even kD * BK / 32 keeps the register buffers of A fragments in step
  // across loop iterations
  static constexpr int D = FMT == MOE_W_BF16 ? MOE_CFG_TILE_D_BF16 : MOE_CFG_TILE_D_Q4;
  static constexpr int CPR = BK / 8;    // 16-byte chunks per staged row
  static constexpr int RPI = 64 / CPR;  // rows per wave-wide direct-to-LDS load
  // activation loads per wave and block of a full tile: load i of wave w fills rows
  // (i*kTW + w)*RPI + [0, RPI)
  static constexpr int IPW_MAX = (kTM + kTW * RPI - 1) / (kTW * RPI);
  // rows of an LDS block buffer: every load of a full tile lands inside (rows past the tile's
  // own are filled too, and never read)
  static constexpr int ROWS = IPW_MAX * kTW * RPI;
  static constexpr size_t LDS = (size_t)D * ROWS * BK * 2;  // kD ring buffers
  static constexpr bool Q4 = FMT != MOE_W_BF16;
  static constexpr int KS = BK / 32;         // k-steps per block
  static constexpr int NBL = Q4 ? 2 : KS;    // weight loads per strip and block
  static constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;  // scale bytes
};

// weight registers of one K block.  bf16: KS fragments of 16 bytes per strip.  4-bit: half of
// the lane's 16-byte word of a 4-k-step chunk (8 bytes, 2 k-steps) and the 2 matching scales.
template <int FMT>
struct TileB {
  unsigned v[kWNS][TileCfg<FMT>::Q4 ? 2 : 4 * TileCfg<FMT>::KS];
  unsigned sc[kWNS];
};

// In-place MFMA on an accumulator held in AGPRs, written as inline assembly: with the compiler's
// own MFMA the register allocator moves accumulators between registers across the K loop, which
// costs a copy per accumulator and iteration.  The compiler sees no MFMA here, so the wait
// states it would insert are explicit: the first MFMA that reads a freshly decoded operand
// starts with s_nop 1 (two wait states after a vector-ALU write of a source); the others read
// operands written several instructions earlier or by loads (covered by s_waitcnt).
// acc_hazard_guard() covers the MFMA result latency; it ends every stretch of MFMA code, before
// the compiler may read or copy an accumulator.
// The weights are the first operand (the rows of the 16 x 16 result are output features) and the
// activations the second (its columns are grouped rows), so a lane's 4 results are 4 consecutive
// output features of one row: 16 contiguous bytes of y_perm (8 of h), stored as they are.
template <bool WAIT>
__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (WAIT)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %2, %1, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %1, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool WAIT>
__device__ __forceinline__ void mfma_acc(f32x4& acc, const f16x8& a, const f16x8& b) {
  if constexpr (WAIT)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %2, %1, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %2, %1, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void acc_hazard_guard() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// An empty volatile asm that takes a value: the arithmetic producing it stays before this point
// (the compiler would otherwise sink the decode next to the MFMA that reads it).
__device__ __forceinline__ unsigned pin(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, so that every index is
// a constant expression in the body (the K loop's schedule is decided while the code is written
// out, not left to the unroller, which gives up on bodies this large).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// n items spread over T slots, item i in slot i*T/n: the items of slot s are [spread_lo, spread_hi)
constexpr int spread_lo(int s, int n, int T) { return (s * n + T - 1) / T; }
constexpr int spread_hi(int s, int n, int T) { return ((s + 1) * n + T - 1) / T; }

typedef const __attribute__((address_space(1))) char* gptr;

// What every row-tile body needs: the work item and the matrix it multiplies.
struct TileCtx {
  int K, N, n_strips, nks, nkb, nfb;
  int lane, wave, p0, rows, col, slot;
};

// Weight bases of the wave's strips, computed per tile from c.slot and c.col (pointers carried
// across the persistent loop would be kept in vector registers).
struct TileBases {
  const char* cbase[kWNS];  // code base of each of the wave's strips
  const char* sbase[kWNS];  // scale base of each strip
};

// Work item w (row tile w / ncol, column tile w % ncol) from the tile plan: plan[1 + t] = {first
// tile of the expert, the expert's first grouped row, its rows, its slot}; an expert with n rows
// has ceil(n / 192) tiles, tile i covering rows [i*n/nt, (i+1)*n/nt).  w is uniform.
// Integer division has no scalar instruction: the quotients (and the plan entry, a vector load
// once the kernel has stored anything) are moved back to scalar registers, or everything derived
// from them would stay in vector registers across the persistent loop.
template <int FMT>
__device__ __forceinline__ void tile_set_item(const FfnArgs& args, TileCtx& c, int w, int ncol) {
  const int t = __builtin_amdgcn_readfirstlane(w / ncol);
  c.col = w - t * ncol;
  const int4 d = args.plan[1 + t];
  const int first = __builtin_amdgcn_readfirstlane(d.x), row0 = __builtin_amdgcn_readfirstlane(d.y);
  const int n = __builtin_amdgcn_readfirstlane(d.z), slot = __builtin_amdgcn_readfirstlane(d.w);
  const int nt = __builtin_amdgcn_readfirstlane((n + kTM - 1) / kTM), i = t - first;
  const int r0 = __builtin_amdgcn_readfirstlane((int)((long long)i * n / nt));
  const int r1 = __builtin_amdgcn_readfirstlane((int)((long long)(i + 1) * n / nt));
  c.p0 = row0 + r0;
  c.rows = r1 - r0;
  c.slot = slot;
}
template <int FMT>
__device__ __forceinline__ TileBases tile_bases(const FfnArgs& args, const TileCtx& c) {
  TileBases b;
  const char* pkg = args.packages + (size_t)c.slot * args.pkg_stride;
  // this wave's strips (clamped into range; results of strips past the end are dropped)
#pragma unroll
  for (int j = 0; j < kWNS; ++j) {
    const int s = min(c.col * 16 + c.wave * kWNS + j, c.n_strips - 1);
    b.cbase[j] = pkg + args.region_codes + (size_t)s * (TileCfg<FMT>::Q4 ? 8 : 32) * c.K;
    b.sbase[j] = pkg + args.region_scales + (size_t)s * 16 * c.nks * TileCfg<FMT>::SB;
  }
  return b;
}

// Activation staging: lane l writes slot l % CPR of row l / CPR of its load's rows, so it fetches
// chunk (l % CPR) ^ (row % CPR) of that row.  Rows past the tile's end repeat row 0 (their
// results are dropped).  Source row of the lane in activation load i:
template <int FMT, bool GU>
__device__ __forceinline__ int tile_a_row(const FfnArgs& args, const TileCtx& c, int i) {
  constexpr int CPR = TileCfg<FMT>::CPR, RPI = TileCfg<FMT>::RPI;
  const int r = (i * kTW + c.wave) * RPI + c.lane / CPR;
  const int rr = r < c.rows ? r : 0;
  return GU ? args.perm_src[c.p0 + rr] / args.k : c.p0 + rr;
}
template <int FMT>
__device__ __forceinline__ unsigned tile_a_chunk(const TileCtx& c, int i) {
  constexpr int CPR = TileCfg<FMT>::CPR, RPI = TileCfg<FMT>::RPI;
  return (unsigned)((c.lane % CPR) ^ (((i * kTW + c.wave) * RPI + c.lane / CPR) % CPR));
}

// Activation load i of block kb (kb < nfb) into LDS buffer buf: a uniform base plus the lane's
// 32-bit offset of block 0 (block kb adds kb * BK * 2 bytes).
template <int FMT>
__device__ __forceinline__ void tile_load_a(const FfnArgs& args, const TileCtx& c, unsigned short* lds_a,
                                            unsigned avoff, int i, int kb, int buf) {
  constexpr int BK = TileCfg<FMT>::BK, RPI = TileCfg<FMT>::RPI;
  const int r0 = (i * kTW + c.wave) * RPI;
  gptr g = (gptr)args.a + (size_t)kb * (BK * 2) + avoff;
  unsigned short* l = lds_a + ((size_t)buf * TileCfg<FMT>::ROWS + r0) * BK;
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// Weight load L (< kWNS * NBL) of block kb (kb < nfb): one instruction on a scalar base, the
// per-lane offsets shared by all strips.
template <int FMT>
__device__ __forceinline__ void tile_load_b(const TileCtx& c, const TileBases& tb, TileB<FMT>& B, int L, int kb) {
  constexpr int KS = TileCfg<FMT>::KS, SB = TileCfg<FMT>::SB;
  const unsigned lane = (unsigned)c.lane;
  if constexpr (!TileCfg<FMT>::Q4) {
    const int j = L / KS, q = L % KS;
    const unsigned off = (unsigned)(kb * KS + q) * 1024u + lane * 16u;
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)((gptr)tb.cbase[j] + off);
    B.v[j][4 * q] = v[0], B.v[j][4 * q + 1] = v[1], B.v[j][4 * q + 2] = v[2], B.v[j][4 * q + 3] = v[3];
  } else {
    const int j = L / 2, part = L % 2;
    const unsigned ch = (unsigned)kb >> 1, h = (unsigned)kb & 1;
    if (part == 0) {
      const unsigned off = ch * 1024u + h * 8u + lane * 16u;
      const u32x2 v = *(const __attribute__((address_space(1))) u32x2*)((gptr)tb.cbase[j] + off);
      B.v[j][0] = v[0], B.v[j][1] = v[1];
    } else {
      const unsigned off = (ch * 64u + 2u * h) * SB + (lane & 15) * 4u * SB;
      if constexpr (SB == 1)
        B.sc[j] = *(const __attribute__((address_space(1))) unsigned short*)((gptr)tb.sbase[j] + off);
      else
        B.sc[j] = *(const __attribute__((address_space(1))) unsigned*)((gptr)tb.sbase[j] + off);
    }
  }
}

// The prologue of tile c: its first kD-1 blocks (all of them when nfb < kD-1, the last one
// repeated), with the activation offsets of all IPW_MAX loads.  It is issued before the tile's own
// body runs: at the end of the previous tile of the workgroup, while that tile's results are
// written.  Part b (the source rows of the activation loads, through perm_src for gate/up, and
// the weights) needs only the ring registers free; part a (the activations, into LDS buffers
// 0 .. kD-2) needs every wave done with those buffers.
template <int FMT, bool GU>
__device__ __forceinline__ void tile_prologue_b(const FfnArgs& args, const TileCtx& c,
                                                TileB<FMT> (&ring)[TileCfg<FMT>::D],
                                                int (&rows)[TileCfg<FMT>::IPW_MAX]) {
  constexpr int kD = TileCfg<FMT>::D, IPW = TileCfg<FMT>::IPW_MAX, NB = kWNS * TileCfg<FMT>::NBL;
#pragma unroll
  for (int i = 0; i < IPW; ++i) rows[i] = tile_a_row<FMT, GU>(args, c, i);
  __builtin_amdgcn_sched_barrier(0);
  if (c.nfb > 0) {
    const TileBases tb = tile_bases<FMT>(args, c);
#pragma unroll
    for (int i = 0; i < kD - 1; ++i)
#pragma unroll
      for (int L = 0; L < NB; ++L) tile_load_b<FMT>(c, tb, ring[i], L, min(i, c.nfb - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
}
template <int FMT>
__device__ __forceinline__ void tile_prologue_a(const FfnArgs& args, const TileCtx& c, unsigned short* lds_a,
                                                unsigned (&avoff)[TileCfg<FMT>::IPW_MAX],
                                                const int (&rows)[TileCfg<FMT>::IPW_MAX]) {
  constexpr int kD = TileCfg<FMT>::D, IPW = TileCfg<FMT>::IPW_MAX;
#pragma unroll
  for (int i = 0; i < IPW; ++i) avoff[i] = ((unsigned)rows[i] * (unsigned)c.K + tile_a_chunk<FMT>(c, i) * 8) * 2;
  if (c.nfb > 0) {
#pragma unroll
    for (int i = 0; i < kD - 1; ++i)
#pragma unroll
      for (int L = 0; L < IPW; ++L) tile_load_a<FMT>(args, c, lds_a, avoff[L], L, min(i, c.nfb - 1), i);
  }
}


// One row tile of NMT 16-row MFMA tiles (rows <= 16 * NMT), whose first kD-1 blocks are in
// flight (tile_prologue_b and _a).  Before its results are written, the next work item of the workgroup
// is fetched and its prologue issued; c becomes that item (c.rows = 0: none).
template <int FMT, bool GU, int NMT>
__device__ __forceinline__ void tile_body(const FfnArgs& args, TileCtx& c, unsigned short* lds_a,
                                          TileB<FMT> (&ring)[TileCfg<FMT>::D],
                                          unsigned (&avoff)[TileCfg<FMT>::IPW_MAX], WorkSched& sch, int ncol,
                                          int* sh_item) {
  typedef typename Op<FMT>::T OpT;
  typedef TileB<FMT> BReg;
  constexpr int BK = TileCfg<FMT>::BK;
  constexpr int KS = BK / 32;                     // k-steps per block
  constexpr bool Q4 = FMT != MOE_W_BF16;
  constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;  // scale bytes
  constexpr int CPR = BK / 8;                     // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPR;                   // rows per wave-wide direct-to-LDS load
  // activation loads per wave and block: load i of wave w fills rows (i*kTW + w)*RPI + [0, RPI)
  constexpr int IPW = (16 * NMT + kTW * RPI - 1) / (kTW * RPI);
  constexpr int NBL = Q4 ? 2 : KS;                // weight loads per strip and block
  constexpr int kLoads = IPW + kWNS * NBL;        // vector loads per block and wave
  constexpr int R = NMT * kWNS;                   // MFMAs per k-step and wave
  constexpr int kD = TileCfg<FMT>::D;             // pipeline depth
  static_assert(!Q4 || KS == 2, "a 4-bit block is half of a 4-k-step package chunk");
  static_assert(IPW <= TileCfg<FMT>::IPW_MAX, "activation loads stay inside the tile buffer");
  const int K = c.K, lane = c.lane, wave = c.wave;
  const int nkb = c.nkb, nfb = c.nfb, nks = c.nks;

  const TileBases tb = tile_bases<FMT>(args, c);
  auto a_row = [&](int i) { return tile_a_row<FMT, GU>(args, c, i); };
  auto a_chunk = [&](int i) { return tile_a_chunk<FMT>(c, i); };
  // load L of block kb's load list (the IPW activation loads, then the weight loads), kb < nfb
  auto load_one = [&](int L, BReg& B, int kb, int buf) {
    if (L < IPW)
      tile_load_a<FMT>(args, c, lds_a, avoff[L], L, kb, buf);
    else
      tile_load_b<FMT>(c, tb, B, L - IPW, kb);
  };
  // a block of the partial last chunk: ns k-steps packed 4 * ns bytes per lane; k-steps past
  // the end get zero codes and zero scales
  auto load_b_partial = [&](BReg& B, int kb) {
    const int ch = kb >> 1, h = kb & 1, ns = nks - 4 * ch;
#pragma unroll
    for (int j = 0; j < kWNS; ++j) {
      // (scalar base plus 32-bit lane offset, as in the whole blocks: a vector use of the bases would
      // move them to vector registers for the whole kernel)
      const unsigned coff = (unsigned)ch * 1024u + (unsigned)lane * 4u * (unsigned)ns;
      const unsigned soff = ((unsigned)ch * 64u + (unsigned)(lane & 15) * (unsigned)ns) * SB;
      unsigned cw[2] = {0, 0}, sw[2] = {0, 0};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int qq = 2 * h + q;
        if (qq < ns) {
          cw[q] = *(const __attribute__((address_space(1))) unsigned*)((gptr)tb.cbase[j] + (coff + 4u * qq));
          if constexpr (SB == 1)
            sw[q] = *(const __attribute__((address_space(1))) unsigned char*)((gptr)tb.sbase[j] + (soff + qq));
          else
            sw[q] = *(const __attribute__((address_space(1))) unsigned short*)((gptr)tb.sbase[j] + (soff + 2u * qq));
        }
      }
      B.v[j][0] = cw[0], B.v[j][1] = cw[1];
      B.sc[j] = sw[0] | (sw[1] << (8 * SB));
    }
  };

  f32x4 acc[NMT][kWNS];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int j = 0; j < kWNS; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand of strip j, k-step q, whole
  auto decode = [&](const BReg& B, int j, int q) -> OpT {
    if constexpr (!Q4)
      return __builtin_bit_cast(OpT, u32x4{B.v[j][4 * q], B.v[j][4 * q + 1], B.v[j][4 * q + 2], B.v[j][4 * q + 3]});
    else if constexpr (FMT == MOE_W_MXFP4)
      return dec_mxfp4(B.v[j][q], (B.sc[j] >> (8 * q)) & 255);
    else
      return dec_int4(B.v[j][q], __builtin_bit_cast(_Float16, (unsigned short)(B.sc[j] >> (16 * q))));
  };
  // the same decode cut into 8 sub-steps of one or two instructions (4-bit formats), so that it
  // can be spread between MFMAs with no two dependent instructions adjacent; t: scratch words
  auto decode_sub = [&](const BReg& B, int j, int q, int st, u32x4& out, unsigned (&t)[4]) {
    if constexpr (FMT == MOE_W_MXFP4) {
      if (st % 2 == 0) {
        const float s = e8m0_to_f32((B.sc[j] >> (8 * q)) & 255);
        const unsigned w = B.v[j][q];
        bf16x2 r;
        if (st == 0) r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
        else if (st == 2) r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
        else if (st == 4) r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
        else r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
        out[st / 2] = pin(__builtin_bit_cast(unsigned, r));
      }
    } else if constexpr (FMT == MOE_W_INT4G32) {
      // the INT4 decode of dec_int4, one nibble pair at a time: pairs 0 and 2 (bits 0-3 of each
      // half of v and of v >> 8) as (w & 0x000F000F) | 0x6400 per half, minus 1032; pairs 1 and 3
      // (bits 4-7) as (w & 0x00F000F0) | 0x5400, minus 72; then times the scale
      const _Float16 sc = __builtin_bit_cast(_Float16, (unsigned short)(B.sc[j] >> (16 * q)));
      const f16x2 bias_lo = {(_Float16)1032.0f, (_Float16)1032.0f}, bias_hi = {(_Float16)72.0f, (_Float16)72.0f};
      const f16x2 ss = {sc, sc};
      const unsigned mask_lo = in_vgpr(0x000F000Fu), magic_lo = in_vgpr(0x64006400u);
      const unsigned mask_hi = in_vgpr(0x00F000F0u), magic_hi = in_vgpr(0x54005400u);
      const unsigned v = B.v[j][q];
      auto sub = [&](unsigned w, const f16x2& b) {
        return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, w) - b);
      };
      auto mul = [&](unsigned w) { return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, w) * ss); };
      // 13 instructions in 8 sub-steps, ordered so that no instruction reads the result of the
      // instruction right before it with only MFMA code in between (the compiler would insert a
      // wait state there: it cannot see that the assembly is not a vector op).
      switch (st) {
        case 0: t[1] = pin((v & mask_hi) | magic_hi); t[0] = pin((v & mask_lo) | magic_lo); break;
        case 1: t[1] = pin(sub(t[1], bias_hi)); t[0] = pin(sub(t[0], bias_lo)); break;
        case 2: out[1] = pin(mul(t[1])); t[2] = pin(v >> 8); break;
        case 3: out[0] = pin(mul(t[0])); break;
        case 4: t[3] = pin((t[2] & mask_hi) | magic_hi); t[2] = pin((t[2] & mask_lo) | magic_lo); break;
        case 5: t[3] = pin(sub(t[3], bias_hi)); t[2] = pin(sub(t[2], bias_lo)); break;
        case 6: out[3] = pin(mul(t[3])); out[2] = pin(mul(t[2])); break;
        default: break;
      }
    }
  };
  // A fragment of M tile mt, k-step q of buffer buf: row mt*16 + lane%16, chunk 4q + lane/16
  auto read_a_one = [&](OpT& dst, int buf, int q, int mt) {
    const unsigned short* abase = lds_a + ((size_t)buf * TileCfg<FMT>::ROWS + (lane & 15)) * BK;
    const int slot = (4 * q + (lane >> 4)) ^ (lane & (CPR - 1));
    dst = *(const OpT*)(abase + mt * 16 * BK + slot * 8);
  };
  auto read_a = [&](OpT (&a)[NMT], int buf, int q) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) read_a_one(a[mt], buf, q, mt);
  };
  // one k-step outside the main loop: strip j's MFMAs run while strip j+1 is decoded
  auto mfma_step = [&](const BReg& B, const OpT (&a)[NMT], int q) {
    OpT b = decode(B, 0, q), bn = b;
#pragma unroll
    for (int j = 0; j < kWNS; ++j) {
      if (j + 1 < kWNS) bn = decode(B, j + 1, q);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) mfma_acc<true>(acc[mt][j], a[mt], b);
      b = bn;
    }
  };

  // ---- K loop over the blocks of whole package chunks: kD blocks in flight.  At the start of
  // block kb a barrier publishes block kb+1's LDS buffer (every wave has waited for its own loads
  // of it) and retires block kb-1's buffer, into which block kb+kD-1 is then loaded.  The A
  // fragments of the next k-step are read from LDS while the current k-step's MFMAs run, across
  // block edges too (the next block is already published); so is the operand of the next strip,
  // the next k-step's first strip included.
  static_assert(kD >= 3 && (kD * KS) % 2 == 0, "pipeline depth");
  // The prologue's loads (and the previous tile's stores, and thread 0's work fetch) complete
  // before the loop: the loop's waits count its own loads only.  Thread 0 resolves the next work
  // item; the barrier publishes it with the first kD-1 blocks.
  __builtin_amdgcn_s_waitcnt(0);
  if (threadIdx.x == 0) *sh_item = sched_resolve(sch);
  barrier_keep_loads();
  const int next = __builtin_amdgcn_readfirstlane(*sh_item);
  int kb = 0;
  if (nfb > 0) {  // (uniform)
    OpT abuf[2][NMT];
    read_a(abuf[0], 0, 0);
    u32x4 b0 = __builtin_bit_cast(u32x4, decode(ring[0], 0, 0));  // operand of the next strip
    for (; kb + kD <= nfb; kb += kD) {
      static_for<kD>([&](auto ic) {
        constexpr int i = ic;
        // block kb+i+1 landed (own loads), then every wave: its buffer is published and block
        // kb+i-1's buffer is free
        MOE_WAIT_VMCNT((kD - 3) * kLoads);
        barrier_keep_loads();
        __builtin_amdgcn_sched_barrier(0);
        // block to issue, into the buffer of block kb+i-1; past the end, the last block again
        // (its buffer and registers are not read any more)
        const int nb = min(kb + i + kD - 1, nfb - 1);
        constexpr int lbuf = (i + kD - 1) % kD;
        BReg& lring = ring[(i + kD - 1) % kD];
        static_for<KS>([&](auto qc) {
          constexpr int q = qc;
          // A of the next k-step (the next block's first when q is the last); the register buffer
          // alternates per k-step, and kD * KS is even, so every block of the loop starts on 0
          constexpr int step = i * KS + q;
          constexpr int nbuf = q + 1 < KS ? i : (i + 1) % kD;
          constexpr int nq = (q + 1) % KS;
          OpT(&acur)[NMT] = abuf[step & 1];
          OpT(&anx)[NMT] = abuf[(step + 1) & 1];
          u32x4 b = b0, bn = b0;
          unsigned dt[4];
          static_for<kWNS>([&](auto jc) {
            constexpr int j = jc;
            if constexpr (!Q4) b = __builtin_bit_cast(u32x4, decode(ring[i], j, q));
            static_for<NMT>([&](auto mtc) {
              constexpr int mt = mtc;
              constexpr int r = j * NMT + mt;
              // the first MFMA of a strip reads the operand decoded during the previous strip; with
              // at least 10 M tiles the decode ends two MFMAs before the strip does (no wait states)
              mfma_acc<Q4 && mt == 0 && NMT < 10>(acc[mt][j], acur[mt], __builtin_bit_cast(OpT, b));
              // the next strip's operand: 8 sub-steps over this strip's MFMAs, done before its last
              if constexpr (Q4) {
                constexpr int T = NMT > 1 ? NMT - 1 : 1;
                constexpr int lo = spread_lo(mt, 8, T), hi = mt < T ? spread_hi(mt, 8, T) : lo;
                static_for<hi - lo>([&](auto sc) {
                  constexpr int st = lo + sc;
                  if constexpr (j + 1 < kWNS) decode_sub(ring[i], j + 1, q, st, bn, dt);
                  else decode_sub(ring[nbuf], 0, nq, st, bn, dt);
                });
              }
              // the next k-step's A fragments, over the first three quarters of this k-step
              {
                constexpr int T = 3 * R / 4 > 0 ? 3 * R / 4 : 1;
                constexpr int lo = spread_lo(r, NMT, T), hi = r < T ? spread_hi(r, NMT, T) : lo;
                static_for<hi - lo>([&](auto mc) {
                  constexpr int m = lo + mc;
                  read_a_one(anx[m], nbuf, nq, m);
                });
              }
              // block nb's loads, over the MFMAs of the whole block
              {
                constexpr int s0 = q * R + r;
                constexpr int lo = spread_lo(s0, kLoads, KS * R), hi = spread_hi(s0, kLoads, KS * R);
                static_for<hi - lo>([&](auto Lc) { load_one(lo + Lc, lring, nb, lbuf); });
              }
              __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (Q4) b = bn;
          });
          if constexpr (Q4) b0 = b;
        });
      });
      // leaving the MFMA code (the loop's exit may copy accumulators between registers)
      acc_hazard_guard();
    }
    // the last nfb - kb (< kD) blocks were issued kD-1 blocks ahead; the A fragments of block
    // kb's first k-step are in abuf[0]
    __builtin_amdgcn_s_waitcnt(0);
    barrier_keep_loads();
#pragma unroll
    for (int i = 0; i < kD - 1; ++i) {
      if (kb + i < nfb) {
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          const int step = i * KS + q;
          const int nbuf = q + 1 < KS ? i : (i + 1) % kD;
          read_a(abuf[(step + 1) & 1], nbuf, (q + 1) % KS);
          mfma_step(ring[i], abuf[step & 1], q);
        }
        acc_hazard_guard();
      }
    }
  }
  // ---- the blocks of a partial last chunk (4-bit weights, K/32 not a multiple of 4): staged
  // alone in buffer 0, chunks past K repeating the last chunk (their weights are zero)
  for (int pb = nfb; pb < nkb; ++pb) {
    __builtin_amdgcn_s_waitcnt(0);
    barrier_keep_loads();  // every wave is done with buffer 0
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r0 = (i * kTW + wave) * RPI;
      const unsigned ch = min((unsigned)(pb * CPR) + a_chunk(i), (unsigned)(K / 8 - 1));
      gptr g = (gptr)args.a + ((size_t)a_row(i) * K + ch * 8) * 2;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)(lds_a + (size_t)r0 * BK), 16, 0, 0);
    }
    BReg bp;
    load_b_partial(bp, pb);
    __builtin_amdgcn_s_waitcnt(0);
    barrier_keep_loads();
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      OpT a[NMT];
      read_a(a, 0, q);
      mfma_step(bp, a, q);
    }
    acc_hazard_guard();
  }

  // ---- the next work item: its first kD-1 blocks are issued now and land while this tile's
  // results are written; the weights at once (the ring registers are free), the activations once
  // every wave is done with the LDS buffers (the barrier)
  acc_hazard_guard();
  const int p0 = c.p0, rows = c.rows, col = c.col;
  // INT4: the token scale of each of the lane's result rows (row mt*16 + lane % 16), looked up before
  // the next item's loads are issued, so that waiting for it does not wait for them
  float tsc[NMT];
  const bool scaled = FMT == MOE_W_INT4G32 && args.xscale != nullptr;
  if (scaled) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) tsc[mt] = token_scale(args, p0 + min(mt * 16 + (lane & 15), rows - 1));
  }
  int nrows[TileCfg<FMT>::IPW_MAX];
  if (next >= 0) {
    tile_set_item<FMT>(args, c, next, ncol);
    tile_prologue_b<FMT, GU>(args, c, ring, nrows);
  }
  barrier_keep_loads();
  if (next >= 0) {
    tile_prologue_a<FMT>(args, c, lds_a, avoff, nrows);
    if (threadIdx.x == 0) sched_issue(sch);
  } else {
    c.rows = 0;
  }

  // ---- epilogue: the wait states of the last MFMAs' results, then every accumulator passes an
  // empty asm after them, so no read of it can be scheduled before the wait
  acc_hazard_guard();
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int j = 0; j < kWNS; ++j) asm volatile("" : "+a"(acc[mt][j]));
  // The lane holds 4 consecutive output features (columns) of row mt*16 + lane % 16 of each MFMA
  // tile: down stores them as 16 bytes, gate/up turns its (gate, up) strip pairs into 4 h values
  // (8 bytes) each.
  const int m_lane = lane & 15, q4 = (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int m = mt * 16 + m_lane;
    const bool row_ok = m < rows;
    if constexpr (GU) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int hc = (col * 8 + wave * 2 + p) * 16 + q4;  // h columns of strip pair col*8 + wave*2 + p
        unsigned short hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[mt][2 * p][r], u = acc[mt][2 * p + 1][r];
          if constexpr (FMT == MOE_W_INT4G32)
            hv[r] = __builtin_bit_cast(unsigned short, (_Float16)(scaled ? swiglu_scaled(g, u, tsc[mt]) : silu(g) * u));
          else
            hv[r] = f32_to_bf16_rne(silu(g) * u);
        }
        const u32x2 pk = {(unsigned)hv[0] | ((unsigned)hv[1] << 16), (unsigned)hv[2] | ((unsigned)hv[3] << 16)};
        if (row_ok && hc < args.I)
          *(__attribute__((address_space(1))) u32x2*)((unsigned short*)args.out + (size_t)(p0 + m) * args.I + hc) = pk;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kWNS; ++j) {
        const int n = col * (kWNS * kTW * 16) + wave * (kWNS * 16) + j * 16 + q4;
        f32x4 y = acc[mt][j];
        if (scaled) {
          const float s2 = tsc[mt];
          y = f32x4{y[0] * s2 * s2, y[1] * s2 * s2, y[2] * s2 * s2, y[3] * s2 * s2};
        }
        if (row_ok && n < c.N)
          *(__attribute__((address_space(1))) f32x4*)((float*)args.out + (size_t)(p0 + m) * args.H + n) = y;
      }
    }
  }
}

template <int FMT, bool GU>
// one wave per SIMD: the accumulators (up to 192 registers) live in the AGPR half of the file.
// Persistent: one workgroup per CU takes work items until every XCD's range is drained.
__global__ __launch_bounds__(kTW * 64, kWGPerCU) void ffn_tile_kernel(FfnArgs args) {
  extern __shared__ __align__(16) unsigned short lds_a[];
  __shared__ int sh_item;
  constexpr int kD = TileCfg<FMT>::D;

  TileCtx c;
  c.K = GU ? args.H : args.I;
  c.N = GU ? 2 * args.I : args.H;  // columns of this matrix (GU: interleaved gate/up rows)
  c.n_strips = c.N / 16;
  const int ncol = (c.N + kTN - 1) / kTN;
  c.nks = c.K / 32;
  constexpr int KS = TileCfg<FMT>::BK / 32;
  c.nkb = (c.nks + KS - 1) / KS;                        // K blocks
  c.nfb = FMT != MOE_W_BF16 ? (c.nks / 4) * 2 : c.nks;  // blocks in whole package chunks
  const int tid = threadIdx.x;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  WorkSched sch;
  sch.cnt = args.tcount;
  sch.total = args.plan[0].x * ncol;
  sch.per = (sch.total + kXcds - 1) / kXcds;
  sch.xs = (int)(blockIdx.x % kXcds), sch.tried = 0, sch.pend = 0;
  if (tid == 0) {
    sch.pend = atomicAdd(&sch.cnt[sch.xs], 1);
    sh_item = sched_resolve(sch);
    sched_issue(sch);
  }
  __syncthreads();
  const int first = __builtin_amdgcn_readfirstlane(sh_item);
  __syncthreads();  // every wave has read sh_item before thread 0 writes the next one
  if (first < 0) return;

  TileB<FMT> ring[kD];
  unsigned avoff[TileCfg<FMT>::IPW_MAX];
  tile_set_item<FMT>(args, c, first, ncol);
  {
    int rows[TileCfg<FMT>::IPW_MAX];
    tile_prologue_b<FMT, GU>(args, c, ring, rows);
    tile_prologue_a<FMT>(args, c, lds_a, avoff, rows);
  }
  do {
    // the variant with NMT = ceil(rows / 16) MFMA row tiles
    const int nmt = (c.rows + 15) / 16;
    static_for<kMT>([&](auto ic) {
      constexpr int m = ic + 1;
      if (nmt == m || (m == kMT && nmt > kMT)) tile_body<FMT, GU, m>(args, c, lds_a, ring, avoff, sch, ncol, &sh_item);
    });
  } while (c.rows > 0);
}

// Launch of one (format, matrix) kernel over the row tiles of a.plan (written on the stream by
// the plan kernel, which also zeroes the work counters a.tcount): at most S row tiles (each expert
// with n_e rows has ceil(n_e / 192) of them) times the column tiles of the matrix, taken by a
// persistent grid of one workgroup per CU (a multiple of 8, so every XCD has the same number).
template <int FMT, bool GU>
int tile_launch(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s) {
  static bool attr_set[64];  // per device
  const size_t lds = TileCfg<FMT>::LDS;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)ffn_tile_kernel<FMT, GU>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: LDS attribute of the prefill kernel");
    attr_set[dev] = true;
  }
  // activation offsets are 32-bit byte offsets: the A matrix (x for gate/up, h for down) must
  // stay under 4 GiB
  const long long a_rows = GU ? (a.k > 0 ? n / a.k : 0) : n;
  if (a_rows * (long long)(GU ? H : I) * 2 >= (1LL << 32))
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: prefill activations of %lld x %d elements exceed 4 GiB", a_rows,
                GU ? H : I);
  const long long nz = n < E ? n : E;
  const long long S = ((long long)n + nz * (kTM - 1)) / kTM;
  const int N = GU ? 2 * I : H;
  const int ncol = (N + kTN - 1) / kTN;
  const long long total = S * ncol;
  const long long per = (total + kXcds - 1) / kXcds;
  const long long resident = (long long)kWGPerCU * cu_count() / kXcds;  // resident workgroups per XCD
  const long long grid = kXcds * (per < resident ? per : (resident > 0 ? resident : 1));
  hipLaunchKernelGGL((ffn_tile_kernel<FMT, GU>), dim3((unsigned)grid), dim3(kTW * 64), lds, s, a);
  return MOE_OK;
}

}  // namespace
}  // namespace moe
