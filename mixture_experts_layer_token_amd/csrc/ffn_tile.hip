// Prefill variant of the grouped SwiGLU expert FFN: output-stationary MFMA tiles.
//
// When many tokens share an expert, one read of its weights serves many rows and the
// contraction becomes dense ("Understanding MoE Inference Costs on Galactus", section "Prompt
// processing is a different phase"), so the roofline is MFMA throughput rather than HBM.
//
// A workgroup (8 waves as 2 x 4) computes a 192-row x 256-column tile of one expert:
//  - activation rows (gathered through perm_src for gate/up) are staged in LDS by direct
//    global->LDS loads, one K block (64 wide for 4-bit weights, 32 for bf16) per buffer, and
//    read back as MFMA A operands (16-byte chunks XOR-swizzled per row against bank conflicts);
//  - each wave owns 96 rows x 4 strips of 16 columns; its weight fragments come straight from
//    the package into registers (16 bytes per lane are one bf16 MFMA B operand; a 4-bit lane
//    word holds 4 k-steps, a block reads half of it) and are decoded in registers (MXFP4 ->
//    bf16, INT4 -> fp16, both exact);
//  - a kD-deep software pipeline: block kb+kD-1's activations and weights are issued while
//    block kb is computed, every load unconditional and issued in block order, so waiting for
//    one block never waits for a later one, and the barrier leaves later loads in flight;
//  - v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation, 24 accumulator tiles per wave;
//  - gate/up epilogue: SiLU(g) * u on the lane's own (gate, up) pair, rounded once to h;
//    down epilogue: fp32 y_perm.
// Work order is XCD-aware: consecutive work items (all column blocks of a row tile, then the
// next row tile of the same expert) go to the same XCD, so one L2 holds the tile's activations
// and the expert's weights while they are reused.
#include "ffn_common.hpp"

namespace moe {
namespace {

constexpr int kTW = 4;       // waves per workgroup, one per SIMD; each owns 64 columns
constexpr int kTM = 192;     // rows per workgroup tile
constexpr int kTN = 256;     // columns per workgroup tile
constexpr int kWMT = 12;     // 16-row MFMA tiles per wave (all 192 rows)
constexpr int kWNS = 4;      // 16-column strips per wave
constexpr int kXCD = 8;      // XCDs of an MI355X; workgroup i is dispatched to XCD i % 8
constexpr int kD = 4;        // pipeline depth: K blocks in flight

template <int FMT>
struct TileCfg {
  static constexpr int BK = FMT == MOE_W_BF16 ? 32 : 64;  // K per block
  // kD ring buffers plus one that absorbs the loads of blocks past the end
  static constexpr size_t LDS = (size_t)(kD + 1) * kTM * BK * 2;
};

template <int FMT, bool GU>
// one wave per SIMD: the 96 accumulator tiles' 192 registers live in the AGPR half of the file
__global__ __launch_bounds__(kTW * 64, 1) void ffn_tile_kernel(FfnArgs args) {
  typedef typename Op<FMT>::T OpT;
  constexpr int BK = TileCfg<FMT>::BK;
  constexpr int KS = BK / 32;                     // k-steps per block
  constexpr bool Q4 = FMT != MOE_W_BF16;
  constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;  // scale bytes
  constexpr int CPR = BK / 8;                     // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPR;                   // rows per wave-wide direct-to-LDS load
  constexpr int IPW = (kTM + kTW * RPI - 1) / (kTW * RPI);  // such loads per wave per block
  static_assert(!Q4 || KS == 2, "a 4-bit block is half of a 4-k-step package chunk");
  // LDS: [kD + 1][kTM rows][CPR chunks of 16 B]; chunk c of row r sits in slot c ^ (r % CPR)
  extern __shared__ __align__(16) unsigned short lds_a[];
  __shared__ RowTile tile;
  __shared__ int sh_total;

  const int K = GU ? args.H : args.I;
  const int N = GU ? 2 * args.I : args.H;  // columns of this matrix (GU: interleaved gate/up rows)
  const int n_strips = N / 16;
  const int ncol = (N + kTN - 1) / kTN;
  const int nks = K / 32;
  const int nkb = (nks + KS - 1) / KS;                     // K blocks
  const int nfb = Q4 ? (nks / 4) * 2 : nks;                // blocks in whole package chunks
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- row tiles of all experts (wave 0), XCD-aware work item, this workgroup's tile
  int excl = 0, incl = 0, e_begin = 0, e_end = 0;
  if (tid < 64) {
    const int per = (args.E + 63) / 64;
    e_begin = lane * per;
    e_end = min(args.E, e_begin + per);
    int local = 0;
    for (int e = e_begin; e < e_end; ++e) {
      int c = args.offsets[e + 1] - args.offsets[e];
      if (c < args.min_rows || c > args.max_rows) c = 0;
      local += (c + kTM - 1) / kTM;
    }
    incl = local;
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    excl = incl - local;
    if (lane == 63) sh_total = incl;
  }
  __syncthreads();
  const int total_work = sh_total * ncol;
  const int per_xcd = (total_work + kXCD - 1) / kXCD;
  const int w = (int)(blockIdx.x % kXCD) * per_xcd + (int)(blockIdx.x / kXCD);
  if (w >= total_work || (int)(blockIdx.x / kXCD) >= per_xcd) return;
  const int slot = w / ncol, col = w % ncol;
  if (tid < 64 && slot >= excl && slot < incl) {
    int acc_t = excl;
    for (int e = e_begin; e < e_end; ++e) {
      const int o0 = args.offsets[e];
      int c = args.offsets[e + 1] - o0;
      if (c < args.min_rows || c > args.max_rows) c = 0;
      const int nt = (c + kTM - 1) / kTM;
      if (slot < acc_t + nt) {
        const int t = slot - acc_t;
        tile.e = e;
        tile.p0 = o0 + t * kTM;
        tile.rows = min(kTM, c - t * kTM);
        break;
      }
      acc_t += nt;
    }
  }
  __syncthreads();
  const int e = tile.e, p0 = tile.p0, rows = tile.rows;
  const int eslot = args.slot_of_expert ? args.slot_of_expert[e] : e;
  if ((unsigned)eslot >= (unsigned)args.n_slots) return;  // workgroup-uniform: not resident, skip
  const char* pkg = args.packages + (size_t)eslot * args.pkg_stride;

  // ---- this wave's strips (clamped into range; results of strips past the end are dropped)
  const char* cbase[kWNS];
  const char* sbase[kWNS];
#pragma unroll
  for (int j = 0; j < kWNS; ++j) {
    const int s = min(col * 16 + wave * kWNS + j, n_strips - 1);
    cbase[j] = pkg + args.region_codes + (size_t)s * (Q4 ? 8 : 32) * K;
    sbase[j] = pkg + args.region_scales + (size_t)s * 16 * nks * SB;
  }

  // ---- activation staging: direct global -> LDS loads (16 bytes per lane, lane-linear in LDS).
  // Load i of this wave fills tile rows (wave*IPW + i)*RPI + [0, RPI); lane l writes slot l % CPR
  // of row l / CPR, so it fetches chunk (l % CPR) ^ (row % CPR) of that row.  Rows past the tile's
  // end repeat a valid row (their results are dropped); chunks past K repeat the last chunk
  // (their weights are zero); loads whose rows lie past the 192-row tile, and loads of blocks
  // past the end, go to the spare buffer kD.
  unsigned aoff[IPW];  // element offset of the lane's source row in args.a
  unsigned achunk[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * RPI + lane / CPR;
    const int rr = r < rows ? r : 0;
    const int row = GU ? args.perm_src[p0 + rr] / args.k : p0 + rr;
    aoff[i] = (unsigned)row * (unsigned)K;
    achunk[i] = (unsigned)((lane % CPR) ^ (r % CPR));
  }
  auto load_a = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r0 = (wave * IPW + i) * RPI;
      const unsigned c = min((unsigned)(kb * CPR) + achunk[i], (unsigned)(K / 8 - 1));
      const unsigned short* g = args.a + aoff[i] + c * 8;
      const int b = r0 < kTM ? buf : kD;
      unsigned short* l = lds_a + ((size_t)b * kTM + (r0 < kTM ? r0 : 0)) * BK;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)l, 16, 0, 0);
    }
  };

  // ---- weight fragments of one K block for this wave's strips.  bf16: KS fragments of 16 bytes
  // per strip.  4-bit: half of the lane's 16-byte word of a 4-k-step chunk (8 bytes, 2 k-steps)
  // and the 2 matching scales.  Blocks past the whole chunks read the zero page (weights 0); the
  // blocks of a partial last chunk are recomputed after the loop from their packed layout.
  struct BReg {
    unsigned v[kWNS][Q4 ? 2 : 4 * KS];
    unsigned sc[kWNS];
  };
  auto load_b = [&](BReg& B, int kb, bool valid) {
#pragma unroll
    for (int j = 0; j < kWNS; ++j) {
      if constexpr (!Q4) {
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          const char* cp = valid ? cbase[j] + (size_t)(kb * KS + q) * 1024 : (const char*)g_zero_page;
          const u32x4 v = *(const u32x4*)(cp + lane * 16);
          B.v[j][4 * q] = v[0], B.v[j][4 * q + 1] = v[1], B.v[j][4 * q + 2] = v[2], B.v[j][4 * q + 3] = v[3];
        }
      } else {
        const int c = kb >> 1, h = kb & 1;
        const char* cp = valid ? cbase[j] + (size_t)c * 1024 + h * 8 : (const char*)g_zero_page;
        const uint2 v = *(const uint2*)(cp + lane * 16);
        B.v[j][0] = v.x, B.v[j][1] = v.y;
        const char* sp = valid ? sbase[j] + ((size_t)c * 64 + 2 * h) * SB : (const char*)g_zero_page;
        sp += (lane & 15) * 4 * SB;
        if constexpr (SB == 1)
          B.sc[j] = *(const unsigned short*)sp;
        else
          B.sc[j] = *(const unsigned*)sp;
      }
    }
  };
  // a block of the partial last chunk: ns k-steps packed 4 * ns bytes per lane; k-steps past
  // the end get zero codes and zero scales
  auto load_b_partial = [&](BReg& B, int kb) {
    const int c = kb >> 1, h = kb & 1, ns = nks - 4 * c;
#pragma unroll
    for (int j = 0; j < kWNS; ++j) {
      const char* cb = cbase[j] + (size_t)c * 1024 + (size_t)lane * 4 * ns;
      const char* sp = sbase[j] + ((size_t)c * 64 + (lane & 15) * ns) * SB;
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

  f32x4 acc[kWMT][kWNS];
#pragma unroll
  for (int mt = 0; mt < kWMT; ++mt)
#pragma unroll
    for (int j = 0; j < kWNS; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // An (empty) use of an accumulation register: without it the compiler keeps the function to
  // the 256 architectural VGPRs; with it the 192 accumulator registers go to the AGPRs.
  asm volatile("" ::: "a0");

  auto decode = [&](const BReg& B, int j, int q) -> OpT {
    if constexpr (!Q4)
      return __builtin_bit_cast(OpT, u32x4{B.v[j][4 * q], B.v[j][4 * q + 1], B.v[j][4 * q + 2], B.v[j][4 * q + 3]});
    else if constexpr (FMT == MOE_W_MXFP4)
      return dec_mxfp4(B.v[j][q], (B.sc[j] >> (8 * q)) & 255);
    else
      return dec_int4(B.v[j][q], __builtin_bit_cast(_Float16, (unsigned short)(B.sc[j] >> (16 * q))));
  };
  // A fragment of M tile mt, k-step q of buffer buf: row mt*16 + lane%16, chunk 4q + lane/16
  auto read_a = [&](OpT (&a)[kWMT], int buf, int q) {
    const unsigned short* abase = lds_a + ((size_t)buf * kTM + (lane & 15)) * BK;
    const int slot = (4 * q + (lane >> 4)) ^ (lane & (CPR - 1));
#pragma unroll
    for (int mt = 0; mt < kWMT; ++mt) a[mt] = *(const OpT*)(abase + mt * 16 * BK + slot * 8);
  };
  // one k-step: strip j's 12 MFMAs run while strip j+1 is decoded
  auto mfma_step = [&](const BReg& B, const OpT (&a)[kWMT], int q) {
    OpT b = decode(B, 0, q), bn = b;
#pragma unroll
    for (int j = 0; j < kWNS; ++j) {
      if (j + 1 < kWNS) bn = decode(B, j + 1, q);
#pragma unroll
      for (int mt = 0; mt < kWMT; ++mt) acc[mt][j] = mfma(a[mt], b, acc[mt][j]);
      b = bn;
    }
  };

  // ---- K loop: kD blocks in flight.  At the start of block kb a barrier publishes block kb+1's
  // LDS buffer (every wave has waited for its own loads of it) and retires block kb-1's buffer,
  // into which block kb+kD-1 is then loaded (activations, then weights).  The A fragments of the
  // next k-step are read from LDS while the current k-step's MFMAs run, across block edges too
  // (the next block is already published), so the matrix cores never wait for LDS.
  static_assert(kD == 4 && (kD * KS) % 2 == 0, "the loop below is unrolled for four blocks");
  constexpr int kLoads = IPW + kWNS * (Q4 ? 2 : KS);  // vector loads per block and wave
  BReg ring[kD];
  OpT abuf[2][kWMT];
#pragma unroll
  for (int i = 0; i < kD - 1; ++i) {
    load_a(i, i < nkb ? i : kD);
    load_b(ring[i], i, i < nfb);
  }
  MOE_WAIT_VMCNT((kD - 2) * kLoads);  // block 0 has landed
  barrier_keep_loads();
  read_a(abuf[0], 0, 0);
  // The prologue's loads complete before the loop (once per workgroup): otherwise the compiler,
  // merging the loop entry with the loop's back edge, waits for every outstanding load at the
  // first use of a weight register in each iteration.
  __builtin_amdgcn_s_waitcnt(0);
  int kb = 0;
  for (; kb + kD <= nkb; kb += kD) {
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      // block kb+i+1 landed (own loads), then every wave: its buffer is published and block
      // kb+i-1's buffer is free
      MOE_WAIT_VMCNT((kD - 3) * kLoads);
      barrier_keep_loads();
      const int nb = kb + i + kD - 1;  // block to issue, into the buffer of block kb+i-1
      load_a(nb, nb < nkb ? (i + kD - 1) % kD : kD);
      load_b(ring[(i + kD - 1) % kD], nb, nb < nfb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        // A of the next k-step (the next block's first when q is the last); the register buffer
        // alternates per k-step, and kD * KS is even, so every block of the loop starts on 0
        const int step = i * KS + q;
        const int nbuf = q + 1 < KS ? i : (i + 1) % kD;
        read_a(abuf[(step + 1) & 1], nbuf, (q + 1) % KS);
        mfma_step(ring[i], abuf[step & 1], q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the last nkb - kb (< kD) blocks were issued kD-1 blocks ahead; the A fragments of block
  // kb's first k-step are in abuf[0]
  __builtin_amdgcn_s_waitcnt(0);
  barrier_keep_loads();
#pragma unroll
  for (int i = 0; i < kD - 1; ++i) {
    if (kb + i < nkb) {
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        const int step = i * KS + q;
        const int nbuf = q + 1 < KS ? i : (i + 1) % kD;
        read_a(abuf[(step + 1) & 1], nbuf, (q + 1) % KS);
        mfma_step(ring[i], abuf[step & 1], q);
      }
    }
  }
  // the blocks of a partial last chunk computed above with zero weights: again with their own
  for (int pb = nfb; pb < nkb; ++pb) {
    BReg bp;
    load_b_partial(bp, pb);
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      OpT a[kWMT];
      read_a(a, pb % kD, q);
      mfma_step(bp, a, q);
    }
  }

  // ---- epilogue
#pragma unroll
  for (int mt = 0; mt < kWMT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + (lane >> 4) * 4 + r;
      if (row >= rows) continue;
      const size_t pr = (size_t)(p0 + row);
      if constexpr (GU) {
#pragma unroll
        for (int j = 0; j < kWNS; j += 2) {
          const int gs = col * 16 + wave * kWNS + j;  // gate strip 2u, up strip 2u + 1
          if (gs + 1 >= n_strips) continue;
          const int f = (gs >> 1) * 16 + (lane & 15);
          const float hv = silu(acc[mt][j][r]) * acc[mt][j + 1][r];
          unsigned short hb;
          if constexpr (FMT == MOE_W_INT4G32)
            hb = __builtin_bit_cast(unsigned short, (_Float16)hv);
          else
            hb = f32_to_bf16_rne(hv);
          ((unsigned short*)args.out)[pr * args.I + f] = hb;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kWNS; ++j) {
          const int s = col * 16 + wave * kWNS + j;
          if (s >= n_strips) continue;
          ((float*)args.out)[pr * args.H + s * 16 + (lane & 15)] = acc[mt][j][r];
        }
      }
    }
  }
}

template <int FMT, bool GU>
int launch_one(const FfnArgs& a, int S, int N, hipStream_t s) {
  static bool attr_set = false;
  const size_t lds = TileCfg<FMT>::LDS;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)ffn_tile_kernel<FMT, GU>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: LDS attribute of the prefill kernel");
    attr_set = true;
  }
  const int ncol = (N + kTN - 1) / kTN;
  const long long total = (long long)S * ncol;
  const long long per = (total + kXCD - 1) / kXCD;
  hipLaunchKernelGGL((ffn_tile_kernel<FMT, GU>), dim3((unsigned)(per * kXCD)), dim3(kTW * 64), lds, s, a);
  return MOE_OK;
}

}  // namespace

int launch_ffn_tile_part(int fmt, bool gate_up, const FfnArgs& a, int H, int I, int n, int E, hipStream_t s) {
  const long long nz = n < E ? n : E;
  const int S = (int)(((long long)n + nz * (kTM - 1)) / kTM);
  if (gate_up) {
    switch (fmt) {
      case MOE_W_BF16: return launch_one<MOE_W_BF16, true>(a, S, 2 * I, s);
      case MOE_W_MXFP4: return launch_one<MOE_W_MXFP4, true>(a, S, 2 * I, s);
      case MOE_W_INT4G32: return launch_one<MOE_W_INT4G32, true>(a, S, 2 * I, s);
    }
  } else {
    switch (fmt) {
      case MOE_W_BF16: return launch_one<MOE_W_BF16, false>(a, S, H, s);
      case MOE_W_MXFP4: return launch_one<MOE_W_MXFP4, false>(a, S, H, s);
      case MOE_W_INT4G32: return launch_one<MOE_W_INT4G32, false>(a, S, H, s);
    }
  }
  return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: no prefill kernel for format %d", fmt);
}

}  // namespace moe
