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
//  - gate/up epilogue: SiLU(g) * u on the lane's own (gate, up) pair, rounded once to h;
//    down epilogue: fp32 y_perm; both staged through LDS per 16-row tile, so that the stores
//    are 16 bytes of one row per lane rather than 4 bytes of a column.
// Work order is XCD-aware: consecutive work items (all column blocks of a row tile, then the
// next row tile of the same expert) go to the same XCD, so one L2 holds the tile's activations
// and the expert's weights while they are reused.
#pragma once

#include <utility>

#include "ffn_common.hpp"

namespace moe {
namespace {

constexpr int kTW = 4;    // waves per workgroup, one per SIMD; each owns 64 columns
constexpr int kTM = 192;  // rows per workgroup tile (at most)
constexpr int kTN = 256;  // columns per workgroup tile
constexpr int kMT = 12;   // 16-row MFMA tiles of a full row tile
constexpr int kWNS = 4;   // 16-column strips per wave
constexpr int kXCD = 8;   // XCDs of an MI355X; workgroup i is dispatched to XCD i % 8
#ifndef MOE_CFG_TILE_D_BF16
#define MOE_CFG_TILE_D_BF16 4
#endif
#ifndef MOE_CFG_TILE_D_Q4
#define MOE_CFG_TILE_D_Q4 4
#endif
// Epilogue staging, one area per wave: 16 rows x 64 fp32 (down) or 16 rows x 32 h values (gate/up),
// row pitches padded so that the column-wise writes of a wave hit distinct banks.
constexpr int kEpiPitchY = 68;  // floats
constexpr int kEpiPitchH = 40;  // 16-bit values
constexpr int kEpiBytes = 16 * kEpiPitchY * 4;
template <int FMT>
struct TileCfg {
  static constexpr int BK = FMT == MOE_W_BF16 ? 32 : 64;  // K per block
  // pipeline depth kD: K blocks in flight (4 covers the load latency: 5 measured no faster for
  // 4-bit weights and costs 12 more registers); even kD * BK / 32 keeps the register buffers of
  // A fragments in step across loop iterations
  static constexpr int D = FMT == MOE_W_BF16 ? MOE_CFG_TILE_D_BF16 : MOE_CFG_TILE_D_Q4;
  static constexpr size_t LDS = (size_t)D * kTM * BK * 2 + kTW * kEpiBytes;  // kD ring buffers, epilogue
};

// In-place MFMA on an accumulator held in AGPRs, written as inline assembly: with the compiler's
// own MFMA the register allocator moves accumulators between registers across the K loop, which
// costs a copy per accumulator and iteration.  The compiler sees no MFMA here, so the wait
// states it would insert are explicit: the first MFMA that reads a freshly decoded operand
// starts with s_nop 1 (two wait states after a vector-ALU write of a source); the others read
// operands written several instructions earlier or by loads (covered by s_waitcnt).
// acc_hazard_guard() covers the MFMA result latency; it ends every stretch of MFMA code, before
// the compiler may read or copy an accumulator.
template <bool WAIT>
__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (WAIT)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool WAIT>
__device__ __forceinline__ void mfma_acc(f32x4& acc, const f16x8& a, const f16x8& b) {
  if constexpr (WAIT)
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
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
  int lane, wave, p0, rows, col;
  const char* cbase[kWNS];  // code base of each of the wave's strips
  const char* sbase[kWNS];  // scale base of each strip
};

// One row tile of NMT 16-row MFMA tiles (rows <= 16 * NMT).
template <int FMT, bool GU, int NMT>
__device__ __forceinline__ void tile_body(const FfnArgs& args, const TileCtx& c, unsigned short* lds_a) {
  typedef typename Op<FMT>::T OpT;
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
  static_assert(IPW * kTW * RPI <= kTM, "activation loads stay inside the tile buffer");
  const int K = c.K, lane = c.lane, wave = c.wave;
  const int nkb = c.nkb, nfb = c.nfb, nks = c.nks;

  // ---- activation staging: lane l writes slot l % CPR of row l / CPR of its load's rows, so it
  // fetches chunk (l % CPR) ^ (row % CPR) of that row.  Rows past the tile's end repeat row 0
  // (their results are dropped).
  auto a_row = [&](int i) {  // source row of the lane in activation load i
    const int r = (i * kTW + wave) * RPI + lane / CPR;
    const int rr = r < c.rows ? r : 0;
    return GU ? args.perm_src[c.p0 + rr] / args.k : c.p0 + rr;
  };
  auto a_chunk = [&](int i) { return (unsigned)((lane % CPR) ^ (((i * kTW + wave) * RPI + lane / CPR) % CPR)); };
  unsigned avoff[IPW];  // byte offset of the lane's chunk of block 0 (block kb adds kb * BK * 2)
#pragma unroll
  for (int i = 0; i < IPW; ++i) avoff[i] = ((unsigned)a_row(i) * (unsigned)K + a_chunk(i) * 8) * 2;

  // weight registers of one K block.  bf16: KS fragments of 16 bytes per strip.  4-bit: half of
  // the lane's 16-byte word of a 4-k-step chunk (8 bytes, 2 k-steps) and the 2 matching scales.
  struct BReg {
    unsigned v[kWNS][Q4 ? 2 : 4 * KS];
    unsigned sc[kWNS];
  };
  // load L of block kb's load list (the IPW activation loads, then the weight loads), kb < nfb:
  // a uniform base plus a 32-bit per-lane offset, so every load is one instruction on a scalar
  // base, and the offsets of one block are shared by all strips
  auto load_one = [&](int L, BReg& B, int kb, int buf) {
    if (L < IPW) {
      const int i = L;
      const int r0 = (i * kTW + wave) * RPI;
      gptr g = (gptr)args.a + (size_t)kb * (BK * 2) + avoff[i];
      unsigned short* l = lds_a + ((size_t)buf * kTM + r0) * BK;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)l, 16, 0, 0);
    } else if constexpr (!Q4) {
      const int j = (L - IPW) / KS, q = (L - IPW) % KS;
      const unsigned off = (unsigned)(kb * KS + q) * 1024u + (unsigned)lane * 16u;
      const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)((gptr)c.cbase[j] + off);
      B.v[j][4 * q] = v[0], B.v[j][4 * q + 1] = v[1], B.v[j][4 * q + 2] = v[2], B.v[j][4 * q + 3] = v[3];
    } else {
      const int j = (L - IPW) / 2, part = (L - IPW) % 2;
      const unsigned ch = (unsigned)kb >> 1, h = (unsigned)kb & 1;
      if (part == 0) {
        const unsigned off = ch * 1024u + h * 8u + (unsigned)lane * 16u;
        const u32x2 v = *(const __attribute__((address_space(1))) u32x2*)((gptr)c.cbase[j] + off);
        B.v[j][0] = v[0], B.v[j][1] = v[1];
      } else {
        const unsigned off = (ch * 64u + 2u * h) * SB + ((unsigned)lane & 15) * 4u * SB;
        if constexpr (SB == 1)
          B.sc[j] = *(const __attribute__((address_space(1))) unsigned short*)((gptr)c.sbase[j] + off);
        else
          B.sc[j] = *(const __attribute__((address_space(1))) unsigned*)((gptr)c.sbase[j] + off);
      }
    }
  };
  auto load_block = [&](BReg& B, int kb, int buf) {
#pragma unroll
    for (int L = 0; L < kLoads; ++L) load_one(L, B, kb, buf);
  };
  // a block of the partial last chunk: ns k-steps packed 4 * ns bytes per lane; k-steps past
  // the end get zero codes and zero scales
  auto load_b_partial = [&](BReg& B, int kb) {
    const int ch = kb >> 1, h = kb & 1, ns = nks - 4 * ch;
#pragma unroll
    for (int j = 0; j < kWNS; ++j) {
      const char* cb = c.cbase[j] + (size_t)ch * 1024 + (size_t)lane * 4 * ns;
      const char* sp = c.sbase[j] + ((size_t)ch * 64 + (lane & 15) * ns) * SB;
      unsigned cw[2] = {0, 0}, sw[2] = {0, 0};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int qq = 2 * h + q;
        if (qq < ns) {
          cw[q] = *(const unsigned*)(cb + 4 * qq);
          sw[q] = SB == 1 ? (unsigned)*(const unsigned char*)(sp + qq) : (unsigned)*(const unsigned short*)(sp + 2 * qq);
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
      // the INT4 decode of dec_int4, one nibble pair p at a time: (v >> 4p) & mask | magic,
      // minus 1032, times the scale
      const _Float16 sc = __builtin_bit_cast(_Float16, (unsigned short)(B.sc[j] >> (16 * q)));
      const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
      const f16x2 ss = {sc, sc};
      const unsigned mask = in_vgpr(0x000F000Fu), magic = in_vgpr(0x64006400u);
      const unsigned v = B.v[j][q];
      auto sub = [&](unsigned w) { return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, w) - bias); };
      auto mul = [&](unsigned w) { return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, w) * ss); };
      // Two dependency chains, one instruction of each per sub-step, the longer chain first: an
      // instruction never follows its producer with only MFMA code in between (the compiler
      // would insert a wait state there: it cannot see that the assembly is not a vector op).
      //   chain a (pairs 1, 3): shift, and-or, subtract, multiply, then the same for pair 3
      //   chain b (pairs 0, 2): and-or, subtract, multiply, then shift, and-or, subtract, multiply
      switch (st) {
        case 0: t[1] = pin(v >> 4); t[0] = pin((v & mask) | magic); break;
        case 1: t[1] = pin((t[1] & mask) | magic); t[0] = pin(sub(t[0])); break;
        case 2: t[1] = pin(sub(t[1])); out[0] = pin(mul(t[0])); break;
        case 3: out[1] = pin(mul(t[1])); t[2] = pin(v >> 8); break;
        case 4: t[3] = pin(v >> 12); t[2] = pin((t[2] & mask) | magic); break;
        case 5: t[3] = pin((t[3] & mask) | magic); t[2] = pin(sub(t[2])); break;
        case 6: t[3] = pin(sub(t[3])); out[2] = pin(mul(t[2])); break;
        default: out[3] = pin(mul(t[3])); break;
      }
    }
  };
  // A fragment of M tile mt, k-step q of buffer buf: row mt*16 + lane%16, chunk 4q + lane/16
  auto read_a_one = [&](OpT& dst, int buf, int q, int mt) {
    const unsigned short* abase = lds_a + ((size_t)buf * kTM + (lane & 15)) * BK;
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
  int kb = 0;
  if (nfb > 0) {  // (uniform)
    BReg ring[kD];
    OpT abuf[2][NMT];
    // blocks in order (the waits count loads in issue order, so no load of a later block may be
    // scheduled before one of an earlier block)
#pragma unroll
    for (int i = 0; i < kD - 1; ++i) {
      load_block(ring[i], min(i, nfb - 1), i);
      __builtin_amdgcn_sched_barrier(0);
    }
    MOE_WAIT_VMCNT((kD - 2) * kLoads);  // block 0 has landed
    barrier_keep_loads();
    read_a(abuf[0], 0, 0);
    // The prologue's loads complete before the loop (once per row tile): otherwise the compiler,
    // merging the loop entry with the loop's back edge, waits for every outstanding load at the
    // first use of a weight register in each iteration.
    __builtin_amdgcn_s_waitcnt(0);
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

  // ---- epilogue: the wait states of the last MFMAs' results, then every accumulator passes an
  // empty asm after them, so no read of it can be scheduled before the wait
  acc_hazard_guard();
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int j = 0; j < kWNS; ++j) asm volatile("" : "+a"(acc[mt][j]));
  // The lane holds 4 consecutive rows of one column of each MFMA tile; every 16-row tile passes
  // through the wave's own LDS area (no barrier: a wave's LDS accesses complete in order), so
  // each lane stores 16 contiguous bytes of one row.  Down: 16 x 64 fp32, read back as 4 rows of
  // 256 bytes per store; gate/up: 16 x 32 h values, read back as 16 rows of 64 bytes.
  const int g = lane >> 4, cl = lane & 15;
  char* const ep = (char*)(lds_a + (size_t)kD * kTM * BK) + (size_t)wave * kEpiBytes;
  if constexpr (GU) {
    // h columns of the wave: strip pair u = (col*16 + wave*4 + 2p) / 2 -> columns 16u + [0, 16)
    const int hc = (c.col * 8 + wave * 2) * 16 + (lane & 3) * 8;  // this lane's 8 stored columns
    const bool col_ok = hc < args.I;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float hv = silu(acc[mt][2 * p][r]) * acc[mt][2 * p + 1][r];
          unsigned short hb;
          if constexpr (FMT == MOE_W_INT4G32)
            hb = __builtin_bit_cast(unsigned short, (_Float16)hv);
          else
            hb = f32_to_bf16_rne(hv);
          *(unsigned short*)(ep + ((4 * g + r) * kEpiPitchH + 16 * p + cl) * 2) = hb;
        }
      const int R = lane >> 2;
      const u32x4 v = *(const u32x4*)(ep + (R * kEpiPitchH + (lane & 3) * 8) * 2);
      __builtin_amdgcn_sched_barrier(0);
      if (col_ok && mt * 16 + R < c.rows)
        *(__attribute__((address_space(1))) u32x4*)((unsigned short*)args.out + (size_t)(c.p0 + mt * 16 + R) * args.I + hc) = v;
    }
  } else {
    const int yc = c.col * (kWNS * kTW * 16) + wave * (kWNS * 16) + cl * 4;  // this lane's 4 columns
    const bool col_ok = yc < c.N;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int j = 0; j < kWNS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) *(float*)(ep + ((4 * g + r) * kEpiPitchY + 16 * j + cl) * 4) = acc[mt][j][r];
      f32x4 v[4];  // all four reads in flight before the first store
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *(const f32x4*)(ep + ((4 * q + g) * kEpiPitchY + cl * 4) * 4);
      __builtin_amdgcn_sched_barrier(0);
      float* const yrow = (float*)args.out + (size_t)(c.p0 + mt * 16 + g) * args.H + yc;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (col_ok && mt * 16 + 4 * q + g < c.rows)
          *(__attribute__((address_space(1))) f32x4*)(yrow + (size_t)(4 * q) * args.H) = v[q];
    }
  }
}

template <int FMT, bool GU>
// one wave per SIMD: the accumulators (up to 192 registers) live in the AGPR half of the file
__global__ __launch_bounds__(kTW * 64, 1) void ffn_tile_kernel(FfnArgs args) {
  extern __shared__ __align__(16) unsigned short lds_a[];
  __shared__ RowTile tile;
  __shared__ int sh_total;

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

  // ---- row tiles of all experts (wave 0), XCD-aware work item, this workgroup's tile.  An
  // expert with n rows has ceil(n / 192) tiles; tile t covers rows [t*n/nt, (t+1)*n/nt).
  int excl = 0, incl = 0, e_begin = 0, e_end = 0;
  if (tid < 64) {
    const int per = (args.E + 63) / 64;
    e_begin = c.lane * per;
    e_end = min(args.E, e_begin + per);
    int local = 0;
    for (int e = e_begin; e < e_end; ++e) {
      int n = args.offsets[e + 1] - args.offsets[e];
      if (n < args.min_rows || n > args.max_rows) n = 0;
      local += (n + kTM - 1) / kTM;
    }
    incl = local;
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (c.lane >= off) incl += o;
    }
    excl = incl - local;
    if (c.lane == 63) sh_total = incl;
  }
  __syncthreads();
  const int total_work = sh_total * ncol;
  const int per_xcd = (total_work + kXCD - 1) / kXCD;
  const int w = (int)(blockIdx.x % kXCD) * per_xcd + (int)(blockIdx.x / kXCD);
  if (w >= total_work || (int)(blockIdx.x / kXCD) >= per_xcd) return;
  const int slot = w / ncol;
  c.col = w % ncol;
  if (tid < 64 && slot >= excl && slot < incl) {
    int acc_t = excl;
    for (int e = e_begin; e < e_end; ++e) {
      const int o0 = args.offsets[e];
      int n = args.offsets[e + 1] - o0;
      if (n < args.min_rows || n > args.max_rows) n = 0;
      const int nt = (n + kTM - 1) / kTM;
      if (slot < acc_t + nt) {
        const int t = slot - acc_t;
        const int r0 = (int)((long long)t * n / nt), r1 = (int)((long long)(t + 1) * n / nt);
        tile.e = e;
        tile.p0 = o0 + r0;
        tile.rows = r1 - r0;
        break;
      }
      acc_t += nt;
    }
  }
  __syncthreads();
  const int e = tile.e;
  c.p0 = tile.p0;
  c.rows = tile.rows;
  const int eslot = args.slot_of_expert ? args.slot_of_expert[e] : e;
  if ((unsigned)eslot >= (unsigned)args.n_slots) return;  // workgroup-uniform: not resident, skip
  const char* pkg = args.packages + (size_t)eslot * args.pkg_stride;

  // this wave's strips (clamped into range; results of strips past the end are dropped)
  constexpr bool Q4 = FMT != MOE_W_BF16;
  constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;
#pragma unroll
  for (int j = 0; j < kWNS; ++j) {
    const int s = min(c.col * 16 + c.wave * kWNS + j, c.n_strips - 1);
    c.cbase[j] = pkg + args.region_codes + (size_t)s * (Q4 ? 8 : 32) * c.K;
    c.sbase[j] = pkg + args.region_scales + (size_t)s * 16 * c.nks * SB;
  }

  switch ((c.rows + 15) / 16) {
    case 1: tile_body<FMT, GU, 1>(args, c, lds_a); break;
    case 2: tile_body<FMT, GU, 2>(args, c, lds_a); break;
    case 3: tile_body<FMT, GU, 3>(args, c, lds_a); break;
    case 4: tile_body<FMT, GU, 4>(args, c, lds_a); break;
    case 5: tile_body<FMT, GU, 5>(args, c, lds_a); break;
    case 6: tile_body<FMT, GU, 6>(args, c, lds_a); break;
    case 7: tile_body<FMT, GU, 7>(args, c, lds_a); break;
    case 8: tile_body<FMT, GU, 8>(args, c, lds_a); break;
    case 9: tile_body<FMT, GU, 9>(args, c, lds_a); break;
    case 10: tile_body<FMT, GU, 10>(args, c, lds_a); break;
    case 11: tile_body<FMT, GU, 11>(args, c, lds_a); break;
    default: tile_body<FMT, GU, kMT>(args, c, lds_a); break;
  }
}

// Launch of one (format, matrix) kernel over the routed rows: S row tiles at most (each expert
// with n_e rows has ceil(n_e / 192) of them), times the column tiles of the matrix.
template <int FMT, bool GU>
int tile_launch(const FfnArgs& a, int H, int I, int n, int E, hipStream_t s) {
  static bool attr_set = false;
  const size_t lds = TileCfg<FMT>::LDS;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)ffn_tile_kernel<FMT, GU>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: LDS attribute of the prefill kernel");
    attr_set = true;
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
  const long long per = (total + kXCD - 1) / kXCD;
  hipLaunchKernelGGL((ffn_tile_kernel<FMT, GU>), dim3((unsigned)(per * kXCD)), dim3(kTW * 64), lds, s, a);
  return MOE_OK;
}

}  // namespace
}  // namespace moe
