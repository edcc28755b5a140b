// Grouped SwiGLU expert FFN: for every expert e and its n_e grouped rows,
//   h = SiLU(X_e W_gate^T) * (X_e W_up^T),   y = h W_down^T
// (pith.science verdict on FloE, arXiv 2505.05950: experts are gate/up/down projections with a
// SiLU gate), over bf16, MXFP4 or INT4-group-32 weights decoded in registers (4-bit experts are
// computed at higher precision: "Mixture of experts VRAM: total vs active parameters", section
// "How current MoE models route each token").
//
// Weight-streaming kernel ("decode" variant).  Decode reads every touched expert's bytes once
// per step ("Understanding MoE Inference Costs on Galactus", section "Turning throughput into a
// cost estimate": time is bytes over bandwidth), so the kernel is built around HBM streaming:
//  - a workgroup owns (one row tile of one expert) x (one 16-row strip of W_down, or one
//    gate strip + its matching up strip of the interleaved GU matrix);
//  - its NW waves split the contraction dimension into contiguous ranges, so every wave reads
//    one contiguous run of whole 1 KiB fragments: each 16-byte load of a lane is directly its
//    MFMA B operand (package layout in common.hpp); 4-bit fragments are decoded in registers
//    (MXFP4: v_cvt_scalef32_pk_bf16_fp4, exact; INT4: nibble|0x6400 magic, exact in fp16);
//  - v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation; the NW partial tiles are summed in
//    LDS in fixed wave order (deterministic), then the epilogue applies SiLU(g)*u (GU) or
//    stores fp32 (down).
// A workgroup finds its (expert, first row) from the per-expert counts on the device, so the
// host never reads the routing back.
#include <math.h>

#include <mutex>

#include "ffn_common.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ streaming kernel


// Weight loads of one pipeline stage, held in registers until consumed PF stages later.
// bf16: a stage is one k-step: NSTR fragments of 16 bytes per lane.
// 4-bit: a stage is one chunk of up to 4 k-steps: NSTR 16-byte code words + their scales.
// Each stage also carries its activation fragments (KPS k-steps x MT row tiles).
template <int FMT, int NSTR, int KPS, int MT, typename OpT>
struct Stage {
  u32x4 code[NSTR];
  unsigned scale[NSTR][FMT == MOE_W_INT4G32 ? 2 : 1];
  OpT a[KPS][MT];
};

// GU = true: a unit is the strip pair (2u, 2u+1) of the GU matrix (gate rows, up rows; K = H),
//            epilogue SiLU(g)*u -> h.
// GU = false: a unit is strip u of the down matrix (K = I), epilogue -> y_perm.
// A workgroup owns NP units of one row tile; its NW waves split K.  Work items (row tile, unit
// group) are ordered expert by expert, unit group by unit group, the row tiles of one expert
// consecutive, and dealt to the XCDs in contiguous ranges (workgroup i runs on XCD i % 8): the row
// tiles of an expert read the same weights at the same time on one XCD, one HBM read and L2 hits.
template <int FMT, int MT, int NW, int NP, int PF, bool GU>
// (second bound: minimum waves per SIMD, i.e. the register budget: 3 -> 168 VGPRs, 2 -> 256)
__global__ __launch_bounds__(NW * 64, FMT == MOE_W_BF16 ? 3 : 2) void ffn_stream_kernel(FfnArgs args) {
  static_assert(NW >= 1 && NW <= 8, "waves per workgroup");
  typedef typename Op<FMT>::T OpT;
  constexpr int SPU = GU ? 2 : 1;  // strips per unit
  constexpr int NSTR = NP * SPU;   // strips per workgroup (every wave covers all of them)
  constexpr int MR = 16 * MT;
  constexpr bool Q4 = FMT != MOE_W_BF16;
  constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;  // scale bytes
  constexpr int KPS = Q4 ? 4 : 1;                 // k-steps per stage
  __shared__ f32x4 red[NW > 1 ? NW * NSTR * 64 : 1];

  const int K = GU ? args.H : args.I;
  const int N = GU ? args.I : args.H;  // output features of this matrix
  const int n_units = N / 16;
  const int gx = (n_units + NP - 1) / NP;  // unit groups
  // work item (uniform: scalar loads).  plan[0].x = row tiles; plan[1 + t] = {first tile of the
  // expert, its first grouped row, its rows, its slot} for every tile t of that expert
  DirectTiles dt;
  if (!args.plan) dt.scan(args, MR);
  const int n_items = (args.plan ? args.plan[0].x : dt.total) * gx;
  const int per_xcd = (n_items + 7) / 8;
  const int j = (int)blockIdx.x / 8, item = (int)(blockIdx.x % 8) * per_xcd + j;
  if (j >= per_xcd || item >= n_items) return;
  const int4 td = args.plan ? args.plan[1 + item / gx] : dt.entry(MR, item / gx);
  const int nt = (td.z + MR - 1) / MR;
  const int local = item - gx * td.x;
  const int t = local % nt;
  const int p0 = td.y + t * MR, rows = min(MR, td.z - t * MR), slot = td.w;
  const int u0 = (local / nt) * NP;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
  const int nks = K / 32;

  const char* pkg = args.packages + (size_t)slot * args.pkg_stride;

  // strip bases (workgroup-uniform); units past the end repeat the last unit, results dropped
  const char* cbase[NSTR];
  const char* sbase[NSTR];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int u = min(u0 + p, n_units - 1);
#pragma unroll
    for (int t = 0; t < SPU; ++t) {
      const int strip = GU ? 2 * u + t : u;
      cbase[p * SPU + t] = pkg + args.region_codes + (size_t)strip * (Q4 ? 8 : 32) * K;
      sbase[p * SPU + t] = pkg + args.region_scales + (size_t)strip * 16 * nks * SB;
    }
  }
  const unsigned lane16 = (unsigned)lane * 16, lrow = (unsigned)(lane & 15);

  f32x4 acc[MT][NSTR];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < NSTR; ++s) acc[mt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // This wave's contiguous range of stages (k-steps for bf16, chunks of 4 k-steps for 4-bit).
  // A 4-bit matrix whose K is not a multiple of 128 ends in a partial chunk; the wave holding
  // it computes the nfull whole stages in the pipelined loop and the partial one after it.
  const int n_stages = Q4 ? (nks + 3) / 4 : nks;
  const int st0 = wave * n_stages / NW, st1 = (wave + 1) * n_stages / NW;
  const int count = st1 - st0;
  const bool part = Q4 && (nks & 3) != 0 && st1 == n_stages && count > 0;
  const int nfull = count - (part ? 1 : 0);

  // Every load of the pipelined loop is unconditional (a load skipped on one path would make
  // the compiler wait for all outstanding loads where the paths join), and a stage's weights and
  // activations are issued together, PF stages before use, so waiting for one stage never waits
  // for a younger one.  Prefetches past the last stage read the zero page; activation rows past
  // the tile repeat the tile's last row (their output rows are never stored).
  typedef Stage<FMT, NSTR, KPS, MT, OpT> StageT;
  // gate/up rows are gathered through perm_src: its load is issued first, so that its latency
  // overlaps the first stage's weight loads
  int srow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(mt * 16 + (lane & 15), rows - 1);
    srow[mt] = GU ? args.perm_src[p0 + r] : p0 + r;
  }
  const unsigned short* arow[MT];
  // weights are read once per call: non-temporal loads stream them without displacing cached data
  auto load_w = [&](StageT& S, int st, bool valid) {
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      const char* cb = valid ? cbase[s] + (size_t)st * 1024 : (const char*)g_zero_page;
      S.code[s] = __builtin_nontemporal_load((const u32x4*)(cb + lane16));
      if constexpr (Q4) {
        const char* sc = valid ? sbase[s] + (size_t)st * 64 * SB : (const char*)g_zero_page;
        sc += lrow * 4 * SB;
        if constexpr (SB == 1) {
          S.scale[s][0] = __builtin_nontemporal_load((const unsigned*)sc);
        } else {
          typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
          const u32x2 v = __builtin_nontemporal_load((const u32x2*)sc);
          S.scale[s][0] = v[0], S.scale[s][SB - 1] = v[1];
        }
      }
    }
  };
  auto load_a = [&](StageT& S, int st, bool valid) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const unsigned short* ar = valid ? arow[mt] + KPS * st * 32 : (const unsigned short*)g_zero_page;
#pragma unroll
      for (int q = 0; q < KPS; ++q) S.a[q][mt] = *(const OpT*)(ar + q * 32);
    }
  };
  auto load = [&](StageT& S, int st, bool valid) {
    load_w(S, st, valid);
    load_a(S, st, valid);
  };
  auto compute = [&](const StageT& S) {
    if constexpr (!Q4) {
#pragma unroll
      for (int s = 0; s < NSTR; ++s) {
        const OpT b = __builtin_bit_cast(OpT, S.code[s]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][s] = mfma(S.a[0][mt], b, acc[mt][s]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int s = 0; s < NSTR; ++s) {
          OpT b;
          if constexpr (FMT == MOE_W_MXFP4) {
            b = dec_mxfp4(S.code[s][q], (S.scale[s][0] >> (8 * q)) & 255);
          } else {
            const unsigned sw = S.scale[s][q >> 1];
            b = dec_int4(S.code[s][q], __builtin_bit_cast(_Float16, (unsigned short)(sw >> (16 * (q & 1)))));
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][s] = mfma(S.a[q][mt], b, acc[mt][s]);
        }
      }
    }
  };

  // software pipeline: a ring of PF stages in registers (the scheduling barriers keep each
  // refill right after the compute that frees its registers)
  StageT ring[PF];
  load_w(ring[0], st0, 0 < nfull);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    arow[mt] = args.a + (size_t)(GU ? srow[mt] / args.k : srow[mt]) * K + (lane >> 4) * 8;
  load_a(ring[0], st0, 0 < nfull);
#pragma unroll
  for (int i = 1; i < PF; ++i) load(ring[i], st0 + i, i < nfull);
  __builtin_amdgcn_sched_barrier(0);
  int base = 0;
  for (; base + PF <= nfull; base += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      compute(ring[i]);
      load(ring[i], st0 + base + i + PF, base + i + PF < nfull);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the last nfull - base (< PF) stages are already in the ring
#pragma unroll
  for (int i = 0; i < PF - 1; ++i)
    if (base + i < nfull) compute(ring[i]);
  // the partial last chunk: ns k-steps packed 4 * ns bytes per lane; the missing k-steps get
  // zero codes, zero scales and zero activations, so all 4 k-steps are computed
  if (part) {
    const int st = st1 - 1, ns = nks - 4 * st;
    StageT S;
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      const char* cb = cbase[s] + (size_t)st * 1024 + (size_t)lane * 4 * ns;
      const char* sb = sbase[s] + ((size_t)st * 64 + lrow * ns) * SB;
      unsigned c[4] = {0, 0, 0, 0}, sc[4] = {0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < ns) {
          c[q] = *(const unsigned*)(cb + 4 * q);
          sc[q] = SB == 1 ? (unsigned)*(const unsigned char*)(sb + q) : (unsigned)*(const unsigned short*)(sb + 2 * q);
        }
      }
      S.code[s] = u32x4{c[0], c[1], c[2], c[3]};
      if constexpr (SB == 1) {
        S.scale[s][0] = sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24);
      } else {
        S.scale[s][0] = sc[0] | (sc[1] << 16);
        S.scale[s][SB - 1] = sc[2] | (sc[3] << 16);
      }
    }
#pragma unroll
    for (int q = 0; q < KPS; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        OpT v = OpT{0, 0, 0, 0, 0, 0, 0, 0};
        if (q < ns) v = *(const OpT*)(arow[mt] + (KPS * st + q) * 32);
        S.a[q][mt] = v;
      }
    compute(S);
  }
  // ---- sum the NW partial tiles (fixed wave order) one M tile at a time, then the epilogue
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt * 16 >= rows) break;  // block-uniform
    if constexpr (NW > 1) {
      if (mt) __syncthreads();
#pragma unroll
      for (int s = 0; s < NSTR; ++s) red[(wave * NSTR + s) * 64 + lane] = acc[mt][s];
      __syncthreads();
    }
    for (int idx = threadIdx.x; idx < NP * 64; idx += NW * 64) {
      const int p = idx >> 6, ln = idx & 63;
      const int u = u0 + p;
      if (u >= n_units) continue;
      f32x4 v[SPU];
#pragma unroll
      for (int t = 0; t < SPU; ++t) {
        const int s = p * SPU + t;
        if constexpr (NW > 1) {
          v[t] = red[s * 64 + ln];
          for (int w = 1; w < NW; ++w) {
            const f32x4 o = red[(w * NSTR + s) * 64 + ln];
            v[t][0] += o[0], v[t][1] += o[1], v[t][2] += o[2], v[t][3] += o[3];
          }
        } else {
          v[t] = acc[mt][s];
        }
      }
      const int col = u * 16 + (ln & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + (ln >> 4) * 4 + r;
        if (row >= rows) continue;
        const size_t pr = (size_t)(p0 + row);
        if constexpr (GU) {
          unsigned short hb;
          if constexpr (FMT == MOE_W_INT4G32) {
            const float h = args.xscale ? swiglu_scaled(v[0][r], v[1][r], token_scale(args, (int)pr))
                                        : silu(v[0][r]) * v[1][r];
            hb = __builtin_bit_cast(unsigned short, (_Float16)h);
          } else {
            hb = f32_to_bf16_rne(silu(v[0][r]) * v[1][r]);
          }
          ((unsigned short*)args.out)[pr * N + col] = hb;
        } else {
          float y = v[0][r];
          if constexpr (FMT == MOE_W_INT4G32)
            if (args.xscale) {
              const float sc = token_scale(args, (int)pr);
              y = y * sc * sc;
            }
          ((float*)args.out)[pr * N + col] = y;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 4-bit streaming, shared activations

// KiB of LDS that hold one wave's scales in the shared-activation kernel: nstr strips of nks k-steps,
// 16 rows and sb bytes per scale
__host__ __device__ constexpr int sl_kib(int nks, int nstr, int sb) { return (nstr * 16 * nks * sb + 1023) / 1024; }
// The scales go to LDS while they take at most this much of it per workgroup (measured on the
// gpt-oss-shaped MXFP4 layer: at one M tile, gate/up 12 KiB and down 24 KiB leave 4 workgroups per CU;
// at two M tiles they leave 3 instead of 4, and the step still gained 4%, T = 512: 329.8 -> 315.5 us;
// INT4 gate/up at H = 5120, 40 KiB, is left to the per-stage loads)
#ifndef MOE_CFG_SL_MAX_KIB
#define MOE_CFG_SL_MAX_KIB 24
#endif
constexpr size_t kSlMaxLds = MOE_CFG_SL_MAX_KIB * 1024;

// 4-bit weights carry as many activation bytes per stage as weight bytes (16 rows x 2 B per k
// against 4 strips x 16 rows x 0.5 B per k), and every unit group of a row tile loads them again.
// This variant shares them: a workgroup's NW waves each own NPW units over the whole
// contraction (no cross-wave sum), and a stage's activation fragments (4 k-steps x MT row tiles,
// 1 KiB each in lane order) are loaded once per workgroup straight into LDS, NA / NW fragments by
// each wave, and read back by every wave.  Stage st lives in LDS buffer st % (PF + 1): the loads
// of stage st + PF, issued after stage st's barrier, go to the buffer of stage st - 1, which every
// wave has finished reading once it reached that barrier.
// SL: the block scales of a wave's strips are copied into LDS once, with direct-to-LDS loads issued
// ahead of the first stage (one contiguous run per strip), and every stage reads its scales from
// there; otherwise each stage loads its 64 (MXFP4) or 128 (INT4) scale bytes per strip from HBM
// beside its codes.  The launch passes NW * sl_kib(K) KiB of dynamic LDS for them.
template <int FMT, int MT, int NW, int NPW, int PF, bool GU, bool SL>
__global__ __launch_bounds__(NW * 64, 2) void ffn_stream_sa_kernel(FfnArgs args) {
  typedef typename Op<FMT>::T OpT;
  constexpr int SPU = GU ? 2 : 1;  // strips per unit
  constexpr int NSTR = NPW * SPU;  // strips per wave
  constexpr int MR = 16 * MT;
  constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;  // scale bytes
  constexpr int KPS = 4;                          // k-steps per stage
  constexpr int NA = KPS * MT;                    // activation fragments per stage
  static_assert(FMT != MOE_W_BF16 && NW == KPS, "4-bit weights; wave q loads k-step q's fragments");
  constexpr int NAW = MT;        // activation loads per wave and stage
  constexpr int NBUF = PF + 1;   // LDS stage buffers
  constexpr int L = (SL ? 1 : 2) * NSTR + NAW;  // vector loads per wave and stage
  __shared__ __align__(16) unsigned char a_lds[NBUF * NA * 1024];
  extern __shared__ __align__(16) unsigned char s_lds[];  // SL: the scales, sl_kib KiB per wave

  const int K = GU ? args.H : args.I;
  const int N = GU ? args.I : args.H;  // output features of this matrix
  const int n_units = N / 16;
  constexpr int UPW = NW * NPW;        // units per workgroup
  const int gx = (n_units + UPW - 1) / UPW;
  // work item, as in ffn_stream_kernel
  DirectTiles dt;
  if (!args.plan) dt.scan(args, MR);
  const int n_items = (args.plan ? args.plan[0].x : dt.total) * gx;
  const int per_xcd = (n_items + 7) / 8;
  const int j = (int)blockIdx.x / 8, item = (int)(blockIdx.x % 8) * per_xcd + j;
  if (j >= per_xcd || item >= n_items) return;
  const int4 td = args.plan ? args.plan[1 + item / gx] : dt.entry(MR, item / gx);
  const int nt = (td.z + MR - 1) / MR;
  const int local = item - gx * td.x;
  const int t = local % nt;
  const int p0 = td.y + t * MR, rows = min(MR, td.z - t * MR), slot = td.w;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u0 = (local / nt) * UPW + wave * NPW;
  const int nks = K / 32;
  const char* pkg = args.packages + (size_t)slot * args.pkg_stride;

  const char* cbase[NSTR];
  const char* sbase[NSTR];
#pragma unroll
  for (int p = 0; p < NPW; ++p) {
    const int u = min(u0 + p, n_units - 1);
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
      const int strip = GU ? 2 * u + s : u;
      cbase[p * SPU + s] = pkg + args.region_codes + (size_t)strip * 8 * K;
      sbase[p * SPU + s] = pkg + args.region_scales + (size_t)strip * 16 * nks * SB;
    }
  }
  const unsigned lane16 = (unsigned)lane * 16, lrow = (unsigned)(lane & 15);
  // the zero page's address, computed once (rematerialised inside the loop it costs a scalar
  // load there, whose wait also waits for the LDS reads)
  typedef const __attribute__((address_space(1))) char* gptr;
  gptr zpage = (gptr)g_zero_page;
  asm volatile("" : "+s"(zpage));
  // SL: the wave's NSTR scale runs of R bytes each, back to back from sl (R is a multiple of 16);
  // KiB i of that copy is one direct-to-LDS load, lanes past the end read the zero page
  const int R = 16 * nks * SB;
  unsigned char* const sl = s_lds + (size_t)wave * sl_kib(nks, NSTR, SB) * 1024;
  if constexpr (SL) {
    const int nkib = sl_kib(nks, NSTR, SB);
    for (int i = 0; i < nkib; ++i) {
      const int o = i * 1024 + (int)lane16;
      gptr g = zpage + lane16;
#pragma unroll
      for (int s = 0; s < NSTR; ++s)
        if (o >= s * R && o < (s + 1) * R) g = (gptr)(sbase[s] + (o - s * R));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)(sl + i * 1024), 16, 0, 0);
    }
  }
  // this lane's activation row of every M tile (rows past the tile repeat its last row)
  const unsigned short* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(mt * 16 + (lane & 15), rows - 1);
    const int srow = GU ? args.perm_src[p0 + r] / args.k : p0 + r;
    arow[mt] = args.a + (size_t)srow * K + (lane >> 4) * 8;
  }

  f32x4 acc[MT][NSTR];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < NSTR; ++s) acc[mt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nfull = nks / 4;                // whole stages
  const bool part = (nks & 3) != 0;         // one partial stage after them
  struct WStage {
    u32x4 code[NSTR];
    unsigned scale[NSTR][SB];
  };
  // every load unconditional: past the whole stages they read the zero page
  auto load_w = [&](WStage& S, int st, bool valid) {
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      gptr cb = valid ? (gptr)(cbase[s] + (size_t)st * 1024) : zpage;
      // one M tile (few rows per expert: most experts have one row tile) streams the weights past
      // the cache; at two M tiles hot experts have several row tiles on one XCD, and ordinary loads
      // let the later ones find the weights in L2 (gpt-oss-shaped MXFP4: T = 64, 111.4 against 113.5
      // us per step with ordinary loads; T = 512, 317.5 against 304.7 us)
      typedef const __attribute__((address_space(1))) u32x4* gv4;
      if constexpr (MT == 1)
        S.code[s] = __builtin_nontemporal_load((gv4)(cb + lane16));
      else
        S.code[s] = *(gv4)(cb + lane16);
      if constexpr (SL) continue;
      gptr sc = valid ? (gptr)(sbase[s] + (size_t)st * 64 * SB) : zpage;
      sc += lrow * 4 * SB;
      if constexpr (SB == 1) {
        S.scale[s][0] = __builtin_nontemporal_load((const __attribute__((address_space(1))) unsigned*)sc);
      } else {
        const u32x2 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x2*)sc);
        S.scale[s][0] = v[0], S.scale[s][1] = v[1];
      }
    }
  };
  // this wave's share of stage st's activation fragments: wave q loads fragments f = q * MT + mt
  // (k-step q of every M tile), 16 bytes per lane in lane order, straight into the stage's LDS
  // buffer
  auto load_a = [&](int st, bool valid) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int q = wave, f = q * MT + mt;
      gptr g = valid ? (gptr)(arow[mt] + (KPS * st + q) * 32) : zpage + lane16;
      unsigned char* l = a_lds + ((size_t)(st % NBUF) * NA + f) * 1024;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)l, 16, 0, 0);
    }
  };
  auto compute = [&](const WStage& S, const unsigned (&scale)[NSTR][SB], const OpT (&a)[KPS][MT]) {
#pragma unroll
    for (int q = 0; q < KPS; ++q) {
#pragma unroll
      for (int s = 0; s < NSTR; ++s) {
        OpT b;
        if constexpr (FMT == MOE_W_MXFP4) {
          b = dec_mxfp4(S.code[s][q], (scale[s][0] >> (8 * q)) & 255);
        } else {
          const unsigned sw = scale[s][q >> 1];
          b = dec_int4(S.code[s][q], __builtin_bit_cast(_Float16, (unsigned short)(sw >> (16 * (q & 1)))));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][s] = mfma(a[q][mt], b, acc[mt][s]);
      }
    }
  };
  // SL: stage st's scales of every strip (the stage-st copy of a full chunk: 4 * SB bytes of row lrow)
  auto read_s = [&](unsigned (&scale)[NSTR][SB], int st) {
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      const unsigned char* p = sl + s * R + (st * 64 + (int)lrow * 4) * SB;
      if constexpr (SB == 1) {
        scale[s][0] = *(const unsigned*)p;
      } else {
        const u32x2 v = *(const u32x2*)p;
        scale[s][0] = v[0], scale[s][1] = v[1];
      }
    }
  };
  auto read_a = [&](OpT (&a)[KPS][MT], int st) {
    const unsigned char* l = a_lds + (size_t)(st % NBUF) * NA * 1024 + lane16;
#pragma unroll
    for (int q = 0; q < KPS; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[q][mt] = *(const OpT*)(l + (q * MT + mt) * 1024);
  };

  WStage ring[PF];
  // stages in order (the waits count this wave's loads in issue order)
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    load_w(ring[i], i, i < nfull);
    load_a(i, i < nfull);
    __builtin_amdgcn_sched_barrier(0);
  }
  // SL: the scales of the next stage to compute, read from LDS one stage ahead of their use (the
  // copy was issued before every stage, so once it has landed it stays valid for the whole call)
  unsigned scn[NSTR][SB];
  if constexpr (SL) {
    MOE_WAIT_VMCNT(PF * L);  // the scale copy has landed (the stages' loads may not have)
    read_s(scn, 0);
  }
  auto next_scales = [&](unsigned (&sc)[NSTR][SB], int st) {
#pragma unroll
    for (int s = 0; s < NSTR; ++s)
#pragma unroll
      for (int b = 0; b < SB; ++b) sc[s][b] = scn[s][b];
    read_s(scn, st + 1 < nfull ? st + 1 : st);
  };
  int base = 0;
  for (; base + PF <= nfull; base += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int st = base + i;
      MOE_WAIT_VMCNT((PF - 1) * L);  // this wave's loads of stage st have landed
      barrier_keep_loads();          // every wave's: stage st is in LDS, stage st - 1 is read
      __builtin_amdgcn_sched_barrier(0);
      OpT a[KPS][MT];
      read_a(a, st);
      if constexpr (SL) {
        unsigned sc[NSTR][SB];
        next_scales(sc, st);
        compute(ring[i], sc, a);
      } else {
        compute(ring[i], ring[i].scale, a);
      }
      load_w(ring[i], st + PF, st + PF < nfull);
      load_a(st + PF, st + PF < nfull);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the last nfull - base (< PF) stages are already loaded
  __builtin_amdgcn_s_waitcnt(0);
  barrier_keep_loads();
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) {
    if (base + i < nfull) {
      OpT a[KPS][MT];
      read_a(a, base + i);
      if constexpr (SL) {
        unsigned sc[NSTR][SB];
        next_scales(sc, base + i);
        compute(ring[i], sc, a);
      } else {
        compute(ring[i], ring[i].scale, a);
      }
    }
  }
  // the partial last chunk: ns k-steps packed 4 * ns bytes per lane; the missing k-steps get
  // zero codes, zero scales and zero activations
  if (part) {
    const int st = nfull, ns = nks - 4 * st;
    WStage S;
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      const char* cb = cbase[s] + (size_t)st * 1024 + (size_t)lane * 4 * ns;
      const char* sb = (SL ? (const char*)sl + s * R : sbase[s]) + ((size_t)st * 64 + lrow * ns) * SB;
      unsigned c[4] = {0, 0, 0, 0}, sc[4] = {0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < ns) {
          c[q] = *(const unsigned*)(cb + 4 * q);
          sc[q] = SB == 1 ? (unsigned)*(const unsigned char*)(sb + q) : (unsigned)*(const unsigned short*)(sb + 2 * q);
        }
      }
      S.code[s] = u32x4{c[0], c[1], c[2], c[3]};
      if constexpr (SB == 1) {
        S.scale[s][0] = sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24);
      } else {
        S.scale[s][0] = sc[0] | (sc[1] << 16);
        S.scale[s][1] = sc[2] | (sc[3] << 16);
      }
    }
    OpT a[KPS][MT];
#pragma unroll
    for (int q = 0; q < KPS; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        OpT v = OpT{0, 0, 0, 0, 0, 0, 0, 0};
        if (q < ns) v = *(const OpT*)(arow[mt] + (KPS * st + q) * 32);
        a[q][mt] = v;
      }
    compute(S, S.scale, a);
  }
  // ---- epilogue: this wave's strips
#pragma unroll
  for (int p = 0; p < NPW; ++p) {
    const int u = u0 + p;
    if (u >= n_units) continue;
    const int col = u * 16 + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + (lane >> 4) * 4 + r;
        if (row >= rows) continue;
        const size_t pr = (size_t)(p0 + row);
        if constexpr (GU) {
          const float g = acc[mt][p * 2][r], u = acc[mt][p * 2 + 1][r];
          unsigned short hb;
          if constexpr (FMT == MOE_W_INT4G32) {
            const float h = args.xscale ? swiglu_scaled(g, u, token_scale(args, (int)pr)) : silu(g) * u;
            hb = __builtin_bit_cast(unsigned short, (_Float16)h);
          } else {
            hb = f32_to_bf16_rne(silu(g) * u);
          }
          ((unsigned short*)args.out)[pr * N + col] = hb;
        } else {
          float y = acc[mt][p][r];
          if constexpr (FMT == MOE_W_INT4G32)
            if (args.xscale) {
              const float sc = token_scale(args, (int)pr);
              y = y * sc * sc;
            }
          ((float*)args.out)[pr * N + col] = y;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ row-tile plan

// One workgroup of 1024 threads, thread e for expert e (E <= 1024): experts whose row count lies
// in [lo, hi] and whose slot is resident are cut into ceil(rows / mr) tiles, in expert order;
// plan[0] = {number of tiles}, plan[1 + i] = {first tile of its expert, the expert's first grouped
// row, the expert's rows, its slot} for every tile i.  Also zeroes zero[0, nzero) (the work
// counters of the tile kernels that read this plan).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, int mr, int lo,
                                                    int hi, const int32_t* __restrict__ slot_of_expert,
                                                    int n_slots, int4* __restrict__ plan, int* __restrict__ zero,
                                                    int nzero) {
  __shared__ int wsum[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  if (e < nzero) zero[e] = 0;
  int c = 0, o0 = 0, slot = -1;
  if (e < E) {
    o0 = offsets[e];
    c = offsets[e + 1] - o0;
    slot = slot_of_expert ? slot_of_expert[e] : e;
    if (c < lo || c > hi || (unsigned)slot >= (unsigned)n_slots) c = 0;
  }
  const int nt = (c + mr - 1) / mr;
  int incl = nt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    base += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  const int excl = base + incl - nt;
  for (int t = 0; t < nt; ++t) plan[1 + excl + t] = make_int4(excl, o0, c, slot);
  if (e == 0) plan[0] = make_int4(total, 0, 0, 0);
}

// ------------------------------------------------------------------ fp32 experts (VALU)

// Lanes own rows (64 per tile), each wave one output feature at a time; fp32 FMA in
// contraction order.  XT: element type of the activations (float or bf16 bits).
template <typename XT, bool GU>
__global__ __launch_bounds__(256) void ffn_f32_kernel(FfnArgs args) {
  __shared__ RowTile tile;
  if (!find_row_tile(args.offsets, args.E, 64, blockIdx.y, &tile)) return;
  const int e = tile.e, p0 = tile.p0, rows = tile.rows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = args.slot_of_expert ? args.slot_of_expert[e] : e;
  if ((unsigned)slot >= (unsigned)args.n_slots) return;  // workgroup-uniform: not resident, skip
  const float* pkg = (const float*)(args.packages + (size_t)slot * args.pkg_stride);
  const int H = args.H, I = args.I;
  const bool ok = lane < rows;
  const int p = p0 + (ok ? lane : 0);
  if constexpr (GU) {
    const int f = blockIdx.x * 4 + wave;
    if (f >= I) return;
    const int t = args.perm_src[p] / args.k;
    const XT* xr = (const XT*)args.a + (size_t)t * H;
    const float* wgr = pkg + (size_t)f * H;
    const float* wur = pkg + (size_t)I * H + (size_t)f * H;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < H; ++c) {
      float xv;
      if constexpr (sizeof(XT) == 4)
        xv = (float)xr[c];
      else
        xv = bf16_to_f32((unsigned short)xr[c]);
      g = fmaf(wgr[c], xv, g);
      u = fmaf(wur[c], xv, u);
    }
    if (ok) ((float*)args.out)[(size_t)p * I + f] = silu(g) * u;
  } else {
    const int o = blockIdx.x * 4 + wave;
    if (o >= H) return;
    const float* hr = (const float*)args.a + (size_t)p * I;
    const float* wdr = pkg + (size_t)2 * I * H + (size_t)o * I;
    float acc = 0.f;
    for (int c = 0; c < I; ++c) acc = fmaf(wdr[c], hr[c], acc);
    if (ok) ((float*)args.out)[(size_t)p * H + o] = acc;
  }
}

// ------------------------------------------------------------------ activation cast

// x [n] of type xdt -> operand type (fp16 for INT4 experts, bf16 otherwise)
template <bool TO_F16>
__device__ __forceinline__ unsigned short cast_one(float v) {
  return TO_F16 ? __builtin_bit_cast(unsigned short, (_Float16)v) : f32_to_bf16_rne(v);
}
template <bool TO_F16>
__global__ void cast_act_kernel(const void* __restrict__ x, int xdt, size_t n, unsigned short* __restrict__ y) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    float v = xdt == MOE_BF16 ? bf16_to_f32(((const unsigned short*)x)[i]) : ((const float*)x)[i];
    y[i] = cast_one<TO_F16>(v);
  }
}
// The same, 8 elements per thread and step (n8 = n / 8; x and y 16-byte aligned)
template <bool TO_F16, bool SRC_BF16>
__global__ __launch_bounds__(256) void cast_act8_kernel(const void* __restrict__ x, size_t n8,
                                                        unsigned short* __restrict__ y) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    float v[8];
    if constexpr (SRC_BF16) {
      const u32x4 w = ((const u32x4*)x)[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[2 * q] = __uint_as_float(w[q] << 16), v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    } else {
      const f32x4 a = ((const f32x4*)x)[2 * i], b = ((const f32x4*)x)[2 * i + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = a[q], v[4 + q] = b[q];
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (unsigned)cast_one<TO_F16>(v[2 * q]) | ((unsigned)cast_one<TO_F16>(v[2 * q + 1]) << 16);
    ((u32x4*)y)[i] = o;
  }
}

// INT4 experts: each token row of x -> fp16, divided by the power of two s_t that puts the row's
// largest finite magnitude in [4, 8) (s_t = 1 for a row of zeros or with an infinite largest
// magnitude); s_t goes to xscale[t] for the epilogues.  One wave per row, 8 elements per lane and
// step (H a multiple of 8, rows 16-byte aligned); the second pass re-reads the row from cache.
template <bool SRC_BF16>
__device__ __forceinline__ void load8(const void* x, size_t i8, float (&v)[8]) {
  if constexpr (SRC_BF16) {
    const u32x4 w = ((const u32x4*)x)[i8];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[2 * q] = __uint_as_float(w[q] << 16), v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  } else {
    const f32x4 a = ((const f32x4*)x)[2 * i8], b = ((const f32x4*)x)[2 * i8 + 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = a[q], v[4 + q] = b[q];
  }
}
template <bool SRC_BF16>
__global__ __launch_bounds__(256) void cast_rows_scaled_kernel(const void* __restrict__ x, int T, int H,
                                                               unsigned short* __restrict__ y,
                                                               float* __restrict__ xscale) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const int n8 = H / 8;
  const size_t base = (size_t)t * n8;
  float m = 0.f;
  for (int c = lane; c < n8; c += 64) {
    float v[8];
    load8<SRC_BF16>(x, base + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));  // (NaN elements ignored)
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  int e = 0;
  if (m > 0.f && m <= 3.4028235e38f) e = min(max(ilogbf(m) - 2, -126), 127);
  const float inv = ldexpf(1.f, -e);
  if (lane == 0) xscale[t] = ldexpf(1.f, e);
  for (int c = lane; c < n8; c += 64) {
    float v[8];
    load8<SRC_BF16>(x, base + c, v);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (unsigned)__builtin_bit_cast(unsigned short, (_Float16)(v[2 * q] * inv)) |
             ((unsigned)__builtin_bit_cast(unsigned short, (_Float16)(v[2 * q + 1] * inv)) << 16);
    ((u32x4*)y)[base + c] = o;
  }
}

// ------------------------------------------------------------------ dequant hook

__global__ void dequant_kernel(const char* __restrict__ pkg, int H, int I, int fmt, float* __restrict__ out) {
  // one thread per (matrix row, k-step): 8 x 4 elements... simpler: one thread per 8 elements
  PackGeom g = pack_geom(H, I, fmt);
  const size_t n_gu = (size_t)2 * I * H / 8, n_d = (size_t)H * I / 8;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_gu + n_d) return;
  const bool gu = i < n_gu;
  const size_t li = gu ? i : i - n_gu;
  const int K = gu ? H : I;
  const int nks = K / 32;
  const size_t octets_per_row = K / 8;
  const int prow = (int)(li / octets_per_row);  // row of the (interleaved for GU) packed matrix
  const int k8 = (int)(li % octets_per_row) * 8;
  const int strip = prow / 16, rr = prow % 16;
  const int ks = k8 / 32, q = (k8 % 32) / 8, lane = rr + 16 * q;
  // logical destination
  int mat, lrow;
  if (gu) {
    mat = strip & 1;  // 0 gate, 1 up
    lrow = (strip >> 1) * 16 + rr;
  } else {
    mat = 2;
    lrow = prow;
  }
  float* dst = out + (size_t)mat * I * H + (size_t)lrow * K + k8;
  const size_t codes = gu ? g.gu_codes : g.d_codes;
  if (fmt == MOE_W_BF16) {
    const unsigned short* src = (const unsigned short*)(pkg + codes) + (size_t)strip * 16 * K + (size_t)ks * 512 + lane * 8;
    for (int t = 0; t < 8; ++t) dst[t] = bf16_to_f32(src[t]);
    return;
  }
  const int c = ks / 4, j = ks % 4, ns = min(4, nks - 4 * c);
  const char* cbase = pkg + codes + (size_t)strip * 8 * K + (size_t)c * 1024 + (size_t)lane * 4 * ns + 4 * j;
  unsigned word = *(const unsigned*)cbase;
  const size_t sreg = gu ? g.gu_scales : g.d_scales;
  const size_t sidx = (size_t)strip * 16 * nks + (size_t)64 * c + (size_t)rr * ns + j;
  if (fmt == MOE_W_MXFP4) {
    unsigned sb = (unsigned char)pkg[sreg + sidx];
    bf16x8 v = dec_mxfp4(word, sb);
    for (int t = 0; t < 8; ++t) dst[t] = bf16_to_f32((unsigned short)v[t]);
  } else {
    unsigned short sh = *(const unsigned short*)(pkg + sreg + 2 * sidx);
    f16x8 v = dec_int4(word, __builtin_bit_cast(_Float16, sh));
    for (int t = 0; t < 8; ++t) dst[t] = (float)v[t];
  }
}

__global__ void dequant_f32_kernel(const float* __restrict__ pkg, size_t n, float* __restrict__ out) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = pkg[i];
}

// ------------------------------------------------------------------ host side

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t cast_off, cast_bytes, xs_off, xs_bytes, h_off, h_bytes, plan_off, plan_bytes, tplan_off, tplan_bytes;
  size_t mx_off, mx_bytes;  // block-scaled mode: x and h as two MXFP8 terms with their scales
  size_t total;
};

WsLayout ws_layout(const moe_experts* w, int T, int k, int xdt, int mode = MOE_FFN_AUTO) {
  WsLayout L{};
  const size_t n = (size_t)T * k;
  const bool f32w = w->fmt == MOE_W_F32;
  // activations are cast when the MFMA operand type differs from xdt
  bool cast = !f32w && (w->fmt == MOE_W_INT4G32 || xdt == MOE_F32);
  L.cast_off = 0;
  L.cast_bytes = cast ? align256((size_t)T * w->H * 2) : 0;
  // INT4: the power-of-two scale of every token's fp16 activations
  L.xs_off = L.cast_off + L.cast_bytes;
  L.xs_bytes = w->fmt == MOE_W_INT4G32 ? align256((size_t)T * sizeof(float)) : 0;
  L.h_off = L.xs_off + L.xs_bytes;
  L.h_bytes = align256(n * w->I * (f32w ? 4 : 2));
  // row-tile plan of the streaming kernels: at most n / 16 + min(n, E) tiles
  L.plan_off = L.h_off + L.h_bytes;
  L.plan_bytes = f32w ? 0 : align256((1 + n / 16 + (n < (size_t)w->E ? n : (size_t)w->E)) * sizeof(int4));
  // row-tile plan of the tile kernels (at most n / kTileRows + min(n, E) tiles), then their work
  // counters (8 for gate/up, 8 for down)
  L.tplan_off = L.plan_off + L.plan_bytes;
  L.tplan_bytes = f32w ? 0 : align256((1 + n / kTileRows + (n < (size_t)w->E ? n : (size_t)w->E)) * sizeof(int4)) + 256;
  // block-scaled mode: x hi, x lo [T][H], x scales [T][H/32] u16; h hi, h lo [n][I], h scales [n][I/32]
  L.mx_off = L.tplan_off + L.tplan_bytes;
  L.mx_bytes = mode == MOE_FFN_DECODE_MX
                   ? 2 * align256((size_t)T * w->H) + align256((size_t)T * w->H / 16) + 2 * align256(n * w->I) +
                         align256(n * w->I / 16)
                   : 0;
  L.total = L.mx_off + L.mx_bytes;
  return L;
}

// M tiles per streaming row tile, from the average rows per expert (the counts are on the device):
// bf16 from 4 rows (Mixtral T = 16 / 32: 428 -> 423, 459 -> 440 us per step; T = 8 the same), 4-bit
// only from about 11 (two M tiles measured slower for the 4-bit kernels at gpt-oss T = 32 .. 128)
// routed rows up to which the streaming kernels find their row tiles themselves (no plan kernel)
#ifndef MOE_CFG_DIRECT_ROWS
#define MOE_CFG_DIRECT_ROWS 64
#endif
constexpr size_t kDirectRows = MOE_CFG_DIRECT_ROWS;

int pick_mt(int T, int k, int E, int fmt) {
  const double avg = (double)T * k / E;
  if (fmt == MOE_W_BF16) return avg >= 4.0 ? 2 : 1;
  return 1.5 * avg > 16.0 ? 2 : 1;
}

void trace(int i, hipStream_t s) {
  void* const* ev = trace_events();
  if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], s);
}

// Tile shapes per format and M-tile count: (units per workgroup, waves, pipeline depth) for
// gate/up and down, chosen by measurement on MI355X.  bf16 fragments are 1 KiB per strip and
// k-step, so a few strips already keep enough bytes in flight; at two M tiles a workgroup covers
// two units, so one activation fragment feeds twice the weight bytes (L2 traffic of the
// activations stays half the weight traffic).  4-bit fragments are 4x smaller; the 4-bit shapes
// stay within 256 VGPRs (2 waves per SIMD).
// NARROW: few experts can be touched (small batches), so the workgroups cover fewer strips and
// there are enough of them to occupy every CU.
// (MOE_CFG_* macros override the defaults when tuning.)
#ifndef MOE_CFG_HYBRID_4BIT_MIN_AVG
#define MOE_CFG_HYBRID_4BIT_MIN_AVG 24.0  // AUTO, 4-bit: average rows per expert from which hot experts go to
                                          // the tile kernel
#endif
#ifndef MOE_CFG_Q4_GU_NP
#define MOE_CFG_Q4_GU_NP 2  // 4-bit gate/up units per workgroup at one M tile (wide)
#endif
#ifndef MOE_CFG_Q4_D_NP
#define MOE_CFG_Q4_D_NP 4
#endif
#ifndef MOE_CFG_Q4_NW
#define MOE_CFG_Q4_NW 2
#endif
#ifndef MOE_CFG_Q4_PF
#define MOE_CFG_Q4_PF 4  // narrow 4-bit shapes (few experts): 4 stages in flight (gpt-oss T = 1: 39.4 -> 38.3 us)
#endif
#ifndef MOE_CFG_BF16_GU_PF
#define MOE_CFG_BF16_GU_PF 2
#endif
#ifndef MOE_CFG_BF16_GU_PF1
#define MOE_CFG_BF16_GU_PF1 MOE_CFG_BF16_GU_PF  // bf16 gate/up pipeline depth at one M tile
#endif
#ifndef MOE_CFG_BF16_D_PF1
#define MOE_CFG_BF16_D_PF1 MOE_CFG_BF16_D_PF  // bf16 down pipeline depth at one M tile
#endif
#ifndef MOE_CFG_BF16_D_PF
#define MOE_CFG_BF16_D_PF 4
#endif
#ifndef MOE_CFG_BF16_GU_NW
#define MOE_CFG_BF16_GU_NW 4
#endif
#ifndef MOE_CFG_BF16_D_NW
#define MOE_CFG_BF16_D_NW 8
#endif
#ifndef MOE_CFG_BF16_GU_NP2
#define MOE_CFG_BF16_GU_NP2 2  // bf16 gate/up units per workgroup at two M tiles
#endif
#ifndef MOE_CFG_Q4S_GU_NPW
#define MOE_CFG_Q4S_GU_NPW 1  // shared-activation 4-bit kernel: gate/up units per wave
#endif
#ifndef MOE_CFG_Q4S_D_NPW
#define MOE_CFG_Q4S_D_NPW 4  // down strips per wave
#endif
#ifndef MOE_CFG_Q4S_PF
#define MOE_CFG_Q4S_PF 3
#endif
template <int FMT, int MT, bool NARROW>
struct Cfg {
  static constexpr bool Q4 = FMT != MOE_W_BF16;
  static constexpr int GU_NP = Q4 ? (NARROW ? 1 : (MT == 1 ? MOE_CFG_Q4_GU_NP : 2)) : (MT == 1 ? 1 : MOE_CFG_BF16_GU_NP2);
  static constexpr int GU_NW = Q4 ? MOE_CFG_Q4_NW : MOE_CFG_BF16_GU_NW;
  static constexpr int GU_PF = Q4 ? MOE_CFG_Q4_PF : (MT == 1 ? MOE_CFG_BF16_GU_PF1 : MOE_CFG_BF16_GU_PF);
  static constexpr int D_NP = Q4 ? (NARROW ? 2 : (MT == 1 ? MOE_CFG_Q4_D_NP : 4)) : 2 * MT;
  static constexpr int D_NW = Q4 ? MOE_CFG_Q4_NW : MOE_CFG_BF16_D_NW;
  static constexpr int D_PF = Q4 ? MOE_CFG_Q4_PF : (MT == 1 ? MOE_CFG_BF16_D_PF1 : MOE_CFG_BF16_D_PF);
};

template <int FMT, int MT, bool NARROW>
void launch_stream_cfg(bool gate_up, const FfnArgs& a, int H, int I, int S, hipStream_t s) {
  // one workgroup per (unit group, row tile) at most, rounded up to whole rounds of the 8 XCDs
  auto grid8 = [](int g, int S) { return (unsigned)(((long long)g * S + 7) / 8 * 8); };
  typedef Cfg<FMT, MT, NARROW> C;
  if constexpr (FMT != MOE_W_BF16 && !NARROW) {
    // 4-bit weights, many experts touched: shared activations (4 waves, each with its gate/up
    // units or down strips over the whole contraction)
    constexpr int NW = 4, GU_NPW = MOE_CFG_Q4S_GU_NPW, D_NPW = MOE_CFG_Q4S_D_NPW, PF = MOE_CFG_Q4S_PF;
    constexpr int SB = FMT == MOE_W_MXFP4 ? 1 : 2;
    if (gate_up) {
      const int gx = (I / 16 + NW * GU_NPW - 1) / (NW * GU_NPW);
      const size_t dyn = (size_t)NW * sl_kib(H / 32, 2 * GU_NPW, SB) * 1024;
      if (dyn <= kSlMaxLds)
        hipLaunchKernelGGL((ffn_stream_sa_kernel<FMT, MT, NW, GU_NPW, PF, true, true>), dim3(grid8(gx, S)),
                           dim3(64 * NW), dyn, s, a);
      else
        hipLaunchKernelGGL((ffn_stream_sa_kernel<FMT, MT, NW, GU_NPW, PF, true, false>), dim3(grid8(gx, S)),
                           dim3(64 * NW), 0, s, a);
    } else {
      const int dx = (H / 16 + NW * D_NPW - 1) / (NW * D_NPW);
      const size_t dyn = (size_t)NW * sl_kib(I / 32, D_NPW, SB) * 1024;
      if (dyn <= kSlMaxLds)
        hipLaunchKernelGGL((ffn_stream_sa_kernel<FMT, MT, NW, D_NPW, PF, false, true>), dim3(grid8(dx, S)),
                           dim3(64 * NW), dyn, s, a);
      else
        hipLaunchKernelGGL((ffn_stream_sa_kernel<FMT, MT, NW, D_NPW, PF, false, false>), dim3(grid8(dx, S)),
                           dim3(64 * NW), 0, s, a);
    }
  } else {  // (an else, so that no wide 4-bit shape of this kernel is instantiated)
    if (gate_up) {
      const int gx = (I / 16 + C::GU_NP - 1) / C::GU_NP;
      hipLaunchKernelGGL((ffn_stream_kernel<FMT, MT, C::GU_NW, C::GU_NP, C::GU_PF, true>), dim3(grid8(gx, S)),
                         dim3(64 * C::GU_NW), 0, s, a);
    } else {
      const int dx = (H / 16 + C::D_NP - 1) / C::D_NP;
      hipLaunchKernelGGL((ffn_stream_kernel<FMT, MT, C::D_NW, C::D_NP, C::D_PF, false>), dim3(grid8(dx, S)),
                         dim3(64 * C::D_NW), 0, s, a);
    }
  }
}

template <int FMT>
void launch_stream(int mt, bool narrow, bool gate_up, const FfnArgs& a, int H, int I, int S, hipStream_t s) {
  if (mt == 1) {
    if (narrow)
      launch_stream_cfg<FMT, 1, true>(gate_up, a, H, I, S, s);
    else
      launch_stream_cfg<FMT, 1, false>(gate_up, a, H, I, S, s);
  } else {
    if (narrow)
      launch_stream_cfg<FMT, 2, true>(gate_up, a, H, I, S, s);
    else
      launch_stream_cfg<FMT, 2, false>(gate_up, a, H, I, S, s);
  }
}

int launch_stream_fmt(int fmt, int mt, bool narrow, bool gate_up, const FfnArgs& a, int H, int I, int S,
                      hipStream_t s) {
  switch (fmt) {
    case MOE_W_BF16: launch_stream<MOE_W_BF16>(mt, false, gate_up, a, H, I, S, s); break;
    case MOE_W_MXFP4: launch_stream<MOE_W_MXFP4>(mt, narrow, gate_up, a, H, I, S, s); break;
    case MOE_W_INT4G32: launch_stream<MOE_W_INT4G32>(mt, narrow, gate_up, a, H, I, S, s); break;
    default: return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: format %d", fmt);
  }
  return MOE_OK;
}

}  // namespace

size_t ffn_workspace(const moe_experts* w, int T, int k, int mode) {
  // the cast buffer is sized for the worst case (any xdt)
  WsLayout a = ws_layout(w, T, k, MOE_F32, mode), b = ws_layout(w, T, k, MOE_BF16, mode);
  return a.total > b.total ? a.total : b.total;
}

// The helper stream of a device (default priority, non-blocking) and the two events that fork it
// from the caller's stream and join it back; created on first use, kept until the process ends.
// The mutex also covers each fork / launch / join sequence, so host threads do not interleave theirs.
struct Helper {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_helper_mu;
Helper g_helper[64];

int helper_for_current_device(Helper** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: device %d", dev);
  Helper& h = g_helper[dev];
  if (!h.s) {
    if ((e = hipStreamCreateWithFlags(&h.s, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h.fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h.join, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "moe_expert_ffn: helper stream");
  }
  *out = &h;
  return MOE_OK;
}

int launch_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
               const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes, hipStream_t s,
               bool helper_stream) {
  if (T == 0) return MOE_OK;
  const int H = w->H, I = w->I, E = w->E;
  WsLayout L = ws_layout(w, T, k, xdt, mode);
  if (!ws || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace %zu bytes < %zu", ws_bytes, L.total);
  char* wsp = (char*)ws;
  const size_t n = (size_t)T * k;
  PackGeom g = pack_geom(H, I, w->fmt);

  FfnArgs gu{};
  gu.packages = (const char*)w->packages;
  gu.pkg_stride = w->pkg_stride;
  gu.slot_of_expert = w->slot_of_expert;
  gu.n_slots = w->slot_of_expert ? w->n_slots : E;
  gu.offsets = offsets;
  gu.perm_src = perm_src;
  gu.H = H, gu.I = I, gu.E = E, gu.k = k;
  FfnArgs dn = gu;
  void* h = wsp + L.h_off;

  if (w->fmt == MOE_W_F32) {
    trace(0, s);
    const int S = (int)((n + (size_t)(n < (size_t)E ? n : E) * 63) / 64);
    gu.a = (const unsigned short*)x;
    gu.out = h;
    dn.a = (const unsigned short*)h;
    dn.out = y_perm;
    if (xdt == MOE_F32)
      hipLaunchKernelGGL((ffn_f32_kernel<float, true>), dim3((I + 3) / 4, S), dim3(256), 0, s, gu);
    else
      hipLaunchKernelGGL((ffn_f32_kernel<unsigned short, true>), dim3((I + 3) / 4, S), dim3(256), 0, s, gu);
    trace(1, s);
    hipLaunchKernelGGL((ffn_f32_kernel<float, false>), dim3((H + 3) / 4, S), dim3(256), 0, s, dn);
    trace(2, s);
    MOE_CHECK_LAUNCH("moe_expert_ffn f32 launch");
    return MOE_OK;
  }

  if (mode == MOE_FFN_DECODE_MX) {
    // every expert streamed on the block-scaled MFMA: x -> MXFP8 terms, gate/up, h -> MXFP8 terms, down
    const int mt = pick_mt(T, k, E, w->fmt), mr = 16 * mt;
    const size_t nz = n < (size_t)E ? n : (size_t)E;
    const int S = (int)((n + nz * (mr - 1)) / mr);
    unsigned char* mx = (unsigned char*)(wsp + L.mx_off);
    unsigned char* xh = mx;
    unsigned char* xl = xh + align256((size_t)T * H);
    unsigned short* xsc = (unsigned short*)(xl + align256((size_t)T * H));
    unsigned char* hh = (unsigned char*)xsc + align256((size_t)T * H / 16);
    unsigned char* hl = hh + align256(n * I);
    unsigned short* hsc = (unsigned short*)(hl + align256(n * I));
    if ((uintptr_t)x % 16) return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: the block-scaled mode needs 16-byte aligned x");
    launch_quant_mx8(x, xdt == MOE_BF16, T, H, xh, xl, xsc, s);
    int4* plan = (int4*)(wsp + L.plan_off);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, E, mr, 1, 0x7FFFFFFF, w->slot_of_expert,
                       gu.n_slots, plan, (int*)nullptr, 0);
    gu.plan = plan;
    gu.out = h;
    gu.region_codes = g.gu_codes, gu.region_scales = g.gu_scales;
    gu.a_hi = xh, gu.a_lo = xl, gu.a_sc = xsc;
    gu.min_rows = 1, gu.max_rows = 0x7FFFFFFF;
    FfnArgs dm = gu;
    dm.out = y_perm;
    dm.region_codes = g.d_codes, dm.region_scales = g.d_scales;
    dm.a_hi = hh, dm.a_lo = hl, dm.a_sc = hsc;
    trace(0, s);
    int rc = launch_ffn_mx_part(mt, true, gu, H, I, S, s);
    if (rc != MOE_OK) return rc;
    trace(1, s);
    launch_quant_mx8(h, true, (int)n, I, hh, hl, hsc, s);
    rc = launch_ffn_mx_part(mt, false, dm, H, I, S, s);
    if (rc != MOE_OK) return rc;
    trace(2, s);
    MOE_CHECK_LAUNCH("moe_expert_ffn block-scaled launch");
    return MOE_OK;
  }

  const unsigned short* a = (const unsigned short*)x;
  const float* xscale = nullptr;
  if (w->fmt == MOE_W_INT4G32) {
    // fp16 operands: every token row scaled by its own power of two (any finite magnitude fits)
    unsigned short* xc = (unsigned short*)(wsp + L.cast_off);
    float* xs = (float*)(wsp + L.xs_off);
    if ((uintptr_t)x % 16)
      return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: INT4 experts need 16-byte aligned activations");
    if (xdt == MOE_BF16)
      hipLaunchKernelGGL((cast_rows_scaled_kernel<true>), dim3((T + 3) / 4), dim3(256), 0, s, x, T, H, xc, xs);
    else
      hipLaunchKernelGGL((cast_rows_scaled_kernel<false>), dim3((T + 3) / 4), dim3(256), 0, s, x, T, H, xc, xs);
    a = xc;
    xscale = xs;
  } else if (L.cast_bytes) {
    // fp32 activations for bf16 operands: rounded to bf16 (nearest-even)
    unsigned short* xc = (unsigned short*)(wsp + L.cast_off);
    size_t ne = (size_t)T * H;
    int blocks = (int)((ne + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (ne % 8 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)xc % 16 == 0) {
      const size_t n8 = ne / 8;
      const unsigned b8 = (unsigned)((n8 + 255) / 256 < 4096 ? (n8 + 255) / 256 : 4096);
      if (xdt == MOE_BF16)
        hipLaunchKernelGGL((cast_act8_kernel<false, true>), dim3(b8), dim3(256), 0, s, x, n8, xc);
      else
        hipLaunchKernelGGL((cast_act8_kernel<false, false>), dim3(b8), dim3(256), 0, s, x, n8, xc);
    } else {
      hipLaunchKernelGGL(cast_act_kernel<false>, dim3(blocks), dim3(256), 0, s, x, xdt, ne, xc);
    }
    a = xc;
  }
  // Variant per expert, decided on the device from its row count: experts with at most kHot rows
  // go to the weight-streaming kernel, the others to the MFMA tile kernel (one weight read per kTileRows
  // rows instead of one per 16 * mt rows).  AUTO launches only the variants that can have work; DECODE
  // and PREFILL force one variant for every expert.
  const int kHot = 4 * 16 * pick_mt(T, k, E, w->fmt);  // at most 4 streaming row tiles per expert
  // (the tile kernel addresses activation rows with 32-bit element offsets)
  const bool tile_ok = (double)((size_t)T > n ? T : n) * (H > I ? H : I) < 2147483648.0;
  bool use_stream = true, use_tile = false;
  int split = 0x7FFFFFFF;  // streaming kernel: rows <= split; tile kernel: rows > split
  if (mode == MOE_FFN_PREFILL && tile_ok) {
    use_stream = false, use_tile = true, split = 0;
  } else if (mode == MOE_FFN_AUTO && tile_ok) {
    // 4-bit weights below 24 rows per expert on average: streaming every expert measured faster
    // than sending the hot ones to the tile kernel, which runs after the streaming kernel with too
    // few tiles to fill the GPU (gpt-oss-shaped MXFP4, 128 experts, top-4: T = 256 / 512 / 1024,
    // 223 vs 294, 317 vs 368, 488 vs 469 us per layer step)
    const double min_avg_rows = w->fmt == MOE_W_BF16 ? 0.0 : MOE_CFG_HYBRID_4BIT_MIN_AVG;
    // bf16 experts from 28 rows per expert on average: the tile kernel for every expert (a second
    // streaming row tile re-reads a whole expert from HBM; Mixtral-shaped, 8 experts, top-2:
    // T = 96 / 128, streaming 531 / 693 us, tile kernel 568 / 576 us per layer step)
    const double tile_all_rows = w->fmt == MOE_W_BF16 ? 28.0 : 64.0;
    if ((double)n >= tile_all_rows * E) {
      use_stream = false, use_tile = true, split = 0;
    } else if (T > kHot && (double)n >= min_avg_rows * E) {  // (no expert has more than T rows)
      use_tile = true, split = kHot;
    }
  }
  const int mt = pick_mt(T, k, E, w->fmt);
  const int mr = 16 * mt;
  const size_t nz = n < (size_t)E ? n : (size_t)E;
  const int S = (int)((n + nz * (mr - 1)) / mr);
  gu.a = a;
  gu.xscale = xscale;
  gu.out = h;
  gu.region_codes = g.gu_codes;
  gu.region_scales = g.gu_scales;
  dn.a = (const unsigned short*)h;
  dn.xscale = xscale;
  dn.out = y_perm;
  dn.region_codes = g.d_codes;
  dn.region_scales = g.d_scales;
  FfnArgs gu_s = gu, dn_s = dn, gu_t = gu, dn_t = dn;
  gu_s.min_rows = dn_s.min_rows = 1, gu_s.max_rows = dn_s.max_rows = split;
  gu_t.min_rows = dn_t.min_rows = split == 0x7FFFFFFF ? split : split + 1;
  gu_t.max_rows = dn_t.max_rows = 0x7FFFFFFF;
  // at most min(E, n) experts are touched: with the wide 4-bit shapes that could leave CUs idle
  const long long wide_wgs = (long long)nz * ((I / 16 + Cfg<MOE_W_MXFP4, 1, false>::GU_NP - 1) /
                                              Cfg<MOE_W_MXFP4, 1, false>::GU_NP);
  const bool narrow = wide_wgs < 1024;
  if (use_stream && n <= kDirectRows && E <= 64 * kDirectPer) {
    // few routed rows, so few row tiles: each streaming workgroup finds its own from the offsets
    // (DirectTiles), one dependent launch less (gpt-oss T = 1: the plan kernel took 3.1 us)
    gu_s.plan = dn_s.plan = nullptr;
  } else if (use_stream) {
    int4* plan = (int4*)(wsp + L.plan_off);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, E, mr, 1, split, w->slot_of_expert,
                       gu.n_slots, plan, (int*)nullptr, 0);
    gu_s.plan = dn_s.plan = plan;
  }
  // the hybrid's two shares touch disjoint experts (their h and y_perm rows too): the tile share
  // runs on the helper stream beside the streaming share, forked after the activation cast
  const bool concurrent = use_stream && use_tile && helper_stream;
  Helper* hp = nullptr;
  std::unique_lock<std::mutex> lock(g_helper_mu, std::defer_lock);
  hipStream_t ts = s;
  if (concurrent) {
    lock.lock();
    int rc = helper_for_current_device(&hp);
    if (rc != MOE_OK) return rc;
    hipError_t e;
    if ((e = hipEventRecord(hp->fork, s)) != hipSuccess || (e = hipStreamWaitEvent(hp->s, hp->fork, 0)) != hipSuccess)
      return hip_fail(e, "moe_expert_ffn: fork to the helper stream");
    ts = hp->s;
  }
  if (use_tile) {
    int4* tplan = (int4*)(wsp + L.tplan_off);
    int* counters = (int*)(wsp + L.tplan_off + L.tplan_bytes - 256);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, ts, offsets, E, kTileRows, gu_t.min_rows, 0x7FFFFFFF,
                       w->slot_of_expert, gu.n_slots, tplan, counters, 16);
    gu_t.plan = dn_t.plan = tplan;
    gu_t.tcount = counters;
    dn_t.tcount = counters + 8;
  }
  int rc = MOE_OK;
  if (concurrent) {
    rc = launch_ffn_tile_part(w->fmt, true, gu_t, H, I, (int)n, E, ts);
    if (rc == MOE_OK) rc = launch_ffn_tile_part(w->fmt, false, dn_t, H, I, (int)n, E, ts);
    hipError_t e = hipEventRecord(hp->join, ts);
    trace(0, s);
    if (rc == MOE_OK) rc = launch_stream_fmt(w->fmt, mt, narrow, true, gu_s, H, I, S, s);
    trace(1, s);
    if (rc == MOE_OK) rc = launch_stream_fmt(w->fmt, mt, narrow, false, dn_s, H, I, S, s);
    // the caller's stream waits for the helper's share whatever happened above
    if (e == hipSuccess) e = hipStreamWaitEvent(s, hp->join, 0);
    if (rc != MOE_OK) return rc;
    if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn: join from the helper stream");
    trace(2, s);
    MOE_CHECK_LAUNCH("moe_expert_ffn launch");
    return MOE_OK;
  }
  trace(0, s);
  if (use_stream) rc = launch_stream_fmt(w->fmt, mt, narrow, true, gu_s, H, I, S, s);
  if (rc == MOE_OK && use_tile) rc = launch_ffn_tile_part(w->fmt, true, gu_t, H, I, (int)n, E, s);
  if (rc != MOE_OK) return rc;
  trace(1, s);
  if (use_stream) rc = launch_stream_fmt(w->fmt, mt, narrow, false, dn_s, H, I, S, s);
  if (rc == MOE_OK && use_tile) rc = launch_ffn_tile_part(w->fmt, false, dn_t, H, I, (int)n, E, s);
  if (rc != MOE_OK) return rc;
  trace(2, s);
  MOE_CHECK_LAUNCH("moe_expert_ffn launch");
  return MOE_OK;
}

int launch_dequant(const void* pkg, int H, int I, int fmt, float* out, hipStream_t s) {
  if (fmt == MOE_W_F32) {
    size_t n = (size_t)3 * H * I;
    hipLaunchKernelGGL(dequant_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)pkg, n,
                       out);
  } else {
    size_t n = (size_t)3 * H * I / 8;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const char*)pkg, H, I,
                       fmt, out);
  }
  MOE_CHECK_LAUNCH("moe_dequant_expert launch");
  return MOE_OK;
}

}  // namespace moe
