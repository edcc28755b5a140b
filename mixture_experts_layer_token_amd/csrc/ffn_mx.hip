// MXFP4 experts computed on the block-scaled matrix cores: the FP4 weights go into
// v_mfma_scale_f32_16x16x128_f8f6f4 as stored, with their E8M0 block scales, instead of being decoded
// to bf16 on the vector ALU first (chips that compute FP4 directly, "Mixture of experts VRAM: total vs
// active parameters", section "How current MoE models route each token", last paragraph).
//
// The activations (x for gate/up, h for down) must then be block-scaled too.  Each 32-element block
// along K becomes two MXFP8 (OCP E4M3) terms with their own E8M0 scales,
//     x = 2^eh * hi + 2^el * lo,   el = eh - 4,
// hi the nearest E4M3 value of s = x / 2^eh (eh puts the block's largest magnitude at most at 448),
// lo the nearest E4M3 value of 16 (s - hi): the remainder is at most 2^-4 |s| <= 28, so 16 times it
// stays within E4M3's range, and lo holds it to 2^-4 of itself: each element is held to within 2^-8
// of its magnitude (bf16 rounding is 2^-9).  The product is two MFMAs, one per term.
//
// Operand layout of the 16x16x128 instruction (measured on gfx950): lane l holds row l % 16; an FP4
// operand lane holds the 32 elements of K block g = l / 16 in order (16 bytes, element i in nibble i),
// an FP8 operand lane holds K [16g, 16g + 16) in its bytes 0-15 and K [64 + 16g, 64 + 16g + 16) in bytes
// 16-31; the scale byte of lane group b applies to K block b of its row, whichever lanes hold that
// block's elements.  The package keeps the bf16-decode layout (lane l of a 4-k-step chunk holds 8
// elements of each k-step, sub-range l / 16), so a chunk's four 32-bit words are transposed across the
// four 16-lane groups (two permlane32 and two permlane16 swaps): lane group g then holds block (k-step)
// g, in order.  The activation rows are quantised in K order, so a lane reads its two 16-byte pieces
// directly.
//
// The streaming kernel follows the shared-activation 4-bit kernel (a workgroup's four waves each own
// whole units over the full contraction; a stage's activation fragments go to LDS once per workgroup):
// per stage (one 128-wide chunk) and M tile, wave q loads fragment q = (hi piece 0, hi piece 1,
// lo piece 0, lo piece 1) of the lane layout.
#include <float.h>

#include "ffn_common.hpp"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short i16x2;

constexpr float kE4M3Max = 448.f;  // largest finite OCP E4M3 value

// ------------------------------------------------------------------ activation quantisation

// One lane per 32-element block of a row (rows x K, K a multiple of 32).
template <bool SRC_BF16>
__global__ __launch_bounds__(256) void quant_mx8_kernel(const void* __restrict__ x, int rows, int K,
                                                        unsigned char* __restrict__ hi,
                                                        unsigned char* __restrict__ lo,
                                                        unsigned short* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nb = K / 32;
  for (int b = lane; b < nb; b += 64) {
    const size_t base = (size_t)r * K + (size_t)b * 32;
    float v[32];
    if constexpr (SRC_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 w = *(const u32x4*)((const unsigned short*)x + base + 8 * i);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[8 * i + 2 * q] = __uint_as_float(w[q] << 16), v[8 * i + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 w = *(const f32x4*)((const float*)x + base + 4 * i);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[4 * i + q] = w[q];
      }
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    int eh = 0;  // (an all-zero block keeps scale 1)
    if (m > 0.f && m <= FLT_MAX) {
      eh = ilogbf(m) - 8;  // m / 2^eh in [256, 512)
      if (ldexpf(m, -eh) > kE4M3Max) eh += 1;
      eh = min(max(eh, -127), 127);
    }
    const int el = max(eh - 4, -127);
    const float inv_h = ldexpf(1.f, -eh), to_l = ldexpf(1.f, eh - el);
    unsigned wh[8], wl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s[4], rr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] = v[4 * i + q] * inv_h;
      i16x2 ph = {0, 0};
      ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ph, s[0], s[1], 1.0f, false);
      ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ph, s[2], s[3], 1.0f, true);
      const unsigned uh = __builtin_bit_cast(unsigned, ph);
      rr[0] = (s[0] - __builtin_amdgcn_cvt_scalef32_f32_fp8(uh, 1.0f, 0)) * to_l;
      rr[1] = (s[1] - __builtin_amdgcn_cvt_scalef32_f32_fp8(uh, 1.0f, 1)) * to_l;
      rr[2] = (s[2] - __builtin_amdgcn_cvt_scalef32_f32_fp8(uh, 1.0f, 2)) * to_l;
      rr[3] = (s[3] - __builtin_amdgcn_cvt_scalef32_f32_fp8(uh, 1.0f, 3)) * to_l;
      i16x2 pl = {0, 0};
      pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, rr[0], rr[1], 1.0f, false);
      pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, rr[2], rr[3], 1.0f, true);
      wh[i] = uh;
      wl[i] = __builtin_bit_cast(unsigned, pl);
    }
    *(u32x4*)(hi + base) = u32x4{wh[0], wh[1], wh[2], wh[3]};
    *(u32x4*)(hi + base + 16) = u32x4{wh[4], wh[5], wh[6], wh[7]};
    *(u32x4*)(lo + base) = u32x4{wl[0], wl[1], wl[2], wl[3]};
    *(u32x4*)(lo + base + 16) = u32x4{wl[4], wl[5], wl[6], wl[7]};
    sc[(size_t)r * nb + b] = (unsigned short)((eh + 127) | ((el + 127) << 8));
  }
}

// ------------------------------------------------------------------ weights: lane words -> K blocks

// Lane (row r, group g) holds word j = 8 elements of k-step j, sub-range g.  Afterwards it holds word j =
// sub-range j of k-step g: the 32 elements of K block g in order.  With half index h = g / 2, i = g % 2
// and word index j = 2p + q: the 32-lane swaps exchange h with p, the 16-lane swaps i with q.
__device__ __forceinline__ u32x4 blocks_of_chunk(u32x4 w) {
  const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return u32x4{(unsigned)c[0], (unsigned)c[1], (unsigned)d[0], (unsigned)d[1]};
}

// acc += (activations hi term) x weights + (lo term) x weights, K = 128; the activation scales are
// the bytes 0 (hi) and 1 (lo) of asc, the weight scale is wsc (byte 0)
__device__ __forceinline__ f32x4 mfma_mx(const u32x4& ah0, const u32x4& ah1, const u32x4& al0, const u32x4& al1,
                                         const u32x4& wq, unsigned asc, unsigned wsc, f32x4 acc) {
  const i32x8 b = {(int)wq[0], (int)wq[1], (int)wq[2], (int)wq[3], 0, 0, 0, 0};
  const i32x8 hi = {(int)ah0[0], (int)ah0[1], (int)ah0[2], (int)ah0[3], (int)ah1[0], (int)ah1[1], (int)ah1[2], (int)ah1[3]};
  const i32x8 lo = {(int)al0[0], (int)al0[1], (int)al0[2], (int)al0[3], (int)al1[0], (int)al1[1], (int)al1[2], (int)al1[3]};
  // A: E4M3 (format 0), B: E2M1 (format 4)
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(hi, b, acc, 0, 4, 0, (int)asc, 0, (int)wsc);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lo, b, acc, 0, 4, 1, (int)asc, 0, (int)wsc);
  return acc;
}

// ------------------------------------------------------------------ streaming kernel

template <int MT, int NPW, int PF, bool GU>
__global__ __launch_bounds__(256, 2) void ffn_mx_kernel(FfnArgs args) {
  constexpr int NW = 4;            // waves; wave q loads activation fragment q of every M tile
  constexpr int SPU = GU ? 2 : 1;  // strips per unit
  constexpr int NSTR = NPW * SPU;  // strips per wave
  constexpr int MR = 16 * MT;
  constexpr int NA = 4 * MT;       // activation fragments per stage
  constexpr int NBUF = PF + 1;     // LDS stage buffers
  __shared__ __align__(16) unsigned char a_lds[NBUF * NA * 1024];

  const int K = GU ? args.H : args.I;
  const int N = GU ? args.I : args.H;
  const int n_units = N / 16;
  constexpr int UPW = NW * NPW;
  const int gx = (n_units + UPW - 1) / UPW;
  const int n_items = args.plan[0].x * gx;
  const int per_xcd = (n_items + 7) / 8;
  const int j = (int)blockIdx.x / 8, item = (int)(blockIdx.x % 8) * per_xcd + j;
  if (j >= per_xcd || item >= n_items) return;
  const int4 td = args.plan[1 + item / gx];
  const int nt = (td.z + MR - 1) / MR;
  const int local = item - gx * td.x;
  const int t = local % nt;
  const int p0 = td.y + t * MR, rows = min(MR, td.z - t * MR), slot = td.w;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u0 = (local / nt) * UPW + wave * NPW;
  const int nks = K / 32;
  const char* pkg = args.packages + (size_t)slot * args.pkg_stride;
  const int g = lane >> 4;

  const char* cbase[NSTR];
  const char* sbase[NSTR];
#pragma unroll
  for (int p = 0; p < NPW; ++p) {
    const int u = min(u0 + p, n_units - 1);
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
      const int strip = GU ? 2 * u + s : u;
      cbase[p * SPU + s] = pkg + args.region_codes + (size_t)strip * 8 * K;
      sbase[p * SPU + s] = pkg + args.region_scales + (size_t)strip * 16 * nks;
    }
  }
  const unsigned lane16 = (unsigned)lane * 16, lrow = (unsigned)(lane & 15);
  typedef const __attribute__((address_space(1))) char* gptr;
  gptr zpage = (gptr)g_zero_page;
  asm volatile("" : "+s"(zpage));
  // this lane's activation row of every M tile (rows past the tile repeat its last row): its two pieces
  // of chunk st start at row * K + 128 st + 16 g (+ 64); its scale (block g) at row * K / 32 + 4 st + g
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(mt * 16 + (lane & 15), rows - 1);
    arow[mt] = GU ? args.perm_src[p0 + r] / args.k : p0 + r;
  }

  f32x4 acc[MT][NSTR];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < NSTR; ++s) acc[mt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nfull = nks / 4;
  const bool part = (nks & 3) != 0;
  struct Stage {
    u32x4 code[NSTR];
    unsigned wsc[NSTR];
    unsigned asc[MT];
  };
  auto load_w = [&](Stage& S, int st, bool valid) {
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      gptr cb = valid ? (gptr)(cbase[s] + (size_t)st * 1024) : zpage;
      S.code[s] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(cb + lane16));
      gptr sp = valid ? (gptr)(sbase[s] + (size_t)st * 64) : zpage;
      S.wsc[s] = __builtin_nontemporal_load((const __attribute__((address_space(1))) unsigned*)(sp + lrow * 4));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      gptr sp = valid ? (gptr)(args.a_sc + (size_t)arow[mt] * nks + 4 * st + g) : zpage;
      S.asc[mt] = *(const __attribute__((address_space(1))) unsigned short*)sp;
    }
  };
  auto load_a = [&](int st, bool valid) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int q = wave, f = q * MT + mt;
      const unsigned char* src = (q < 2 ? args.a_hi : args.a_lo) + (size_t)arow[mt] * K + 128 * st + 16 * g + 64 * (q & 1);
      gptr gsrc = valid ? (gptr)src : zpage + lane16;
      unsigned char* l = a_lds + ((size_t)(st % NBUF) * NA + f) * 1024;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                       (__attribute__((address_space(3))) void*)l, 16, 0, 0);
    }
  };
  // per strip: the chunk's words transposed to K blocks, the lane's own block scale; then both terms
  // for every M tile
  auto compute = [&](const Stage& S, const u32x4 (&a)[4][MT]) {
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      const u32x4 wq = blocks_of_chunk(S.code[s]);
      const unsigned wsc = (S.wsc[s] >> (8 * g)) & 255u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][s] = mfma_mx(a[0][mt], a[1][mt], a[2][mt], a[3][mt], wq, S.asc[mt], wsc, acc[mt][s]);
    }
  };
  auto read_a = [&](u32x4 (&a)[4][MT], int st) {
    const unsigned char* l = a_lds + (size_t)(st % NBUF) * NA * 1024 + lane16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[q][mt] = *(const u32x4*)(l + (q * MT + mt) * 1024);
  };

  constexpr int L = 2 * NSTR + MT + MT;  // vector loads per wave and stage (codes, scales, act scales, act)
  Stage ring[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    load_w(ring[i], i, i < nfull);
    load_a(i, i < nfull);
    __builtin_amdgcn_sched_barrier(0);
  }
  int base = 0;
  for (; base + PF <= nfull; base += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int st = base + i;
      MOE_WAIT_VMCNT((PF - 1) * L);  // this wave's loads of stage st have landed
      barrier_keep_loads();          // every wave's: stage st is in LDS, stage st - 1 is read
      __builtin_amdgcn_sched_barrier(0);
      u32x4 a[4][MT];
      read_a(a, st);
      compute(ring[i], a);
      load_w(ring[i], st + PF, st + PF < nfull);
      load_a(st + PF, st + PF < nfull);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  barrier_keep_loads();
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) {
    if (base + i < nfull) {
      u32x4 a[4][MT];
      read_a(a, base + i);
      compute(ring[i], a);
    }
  }
  // the partial last chunk (ns < 4 K blocks): codes, scales and activation bytes of the missing blocks
  // are zero (0 x 2^-127 adds nothing)
  if (part) {
    const int st = nfull, ns = nks - 4 * st;
    Stage S;
#pragma unroll
    for (int s = 0; s < NSTR; ++s) {
      const char* cb = cbase[s] + (size_t)st * 1024 + (size_t)lane * 4 * ns;
      const unsigned char* sb = (const unsigned char*)sbase[s] + (size_t)st * 64 + lrow * ns;
      unsigned c[4] = {0, 0, 0, 0}, sc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < ns) c[q] = *(const unsigned*)(cb + 4 * q), sc |= (unsigned)sb[q] << (8 * q);
      S.code[s] = u32x4{c[0], c[1], c[2], c[3]};
      S.wsc[s] = sc;
    }
    u32x4 a[4][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      S.asc[mt] = g < ns ? args.a_sc[(size_t)arow[mt] * nks + 4 * st + g] : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // piece q & 1 holds K block g / 2 + 2 (q & 1) of the chunk
        const bool ok = g / 2 + 2 * (q & 1) < ns;
        const unsigned char* src = (q < 2 ? args.a_hi : args.a_lo) + (size_t)arow[mt] * K + 128 * st + 16 * g + 64 * (q & 1);
        a[q][mt] = ok ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
      }
    }
    compute(S, a);
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
        if constexpr (GU)
          ((unsigned short*)args.out)[pr * N + col] = f32_to_bf16_rne(silu(acc[mt][p * 2][r]) * acc[mt][p * 2 + 1][r]);
        else
          ((float*)args.out)[pr * N + col] = acc[mt][p][r];
      }
    }
  }
}

}  // namespace

void launch_quant_mx8(const void* x, bool src_bf16, int rows, int K, unsigned char* hi, unsigned char* lo,
                      unsigned short* sc, hipStream_t s) {
  if (rows <= 0) return;
  if (src_bf16)
    hipLaunchKernelGGL((quant_mx8_kernel<true>), dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, hi, lo, sc);
  else
    hipLaunchKernelGGL((quant_mx8_kernel<false>), dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, hi, lo, sc);
}

#ifndef MOE_CFG_MX_PF
#define MOE_CFG_MX_PF 3
#endif

int launch_ffn_mx_part(int mt, bool gate_up, const FfnArgs& a, int H, int I, int S, hipStream_t s) {
  auto grid8 = [](int g, int S) { return (unsigned)(((long long)g * S + 7) / 8 * 8); };
  // units per wave: gate/up 1 (a gate and an up strip), down 4 strips (2 at two M tiles, within 256 VGPRs)
  constexpr int PF = MOE_CFG_MX_PF, GU_NPW = 1;
  const int npw = gate_up ? GU_NPW : (mt == 1 ? 4 : 2);
  const int gx = ((gate_up ? I : H) / 16 + 4 * npw - 1) / (4 * npw);
  if (mt == 1) {
    if (gate_up)
      hipLaunchKernelGGL((ffn_mx_kernel<1, GU_NPW, PF, true>), dim3(grid8(gx, S)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_mx_kernel<1, 4, PF, false>), dim3(grid8(gx, S)), dim3(256), 0, s, a);
  } else {
    if (gate_up)
      hipLaunchKernelGGL((ffn_mx_kernel<2, GU_NPW, PF, true>), dim3(grid8(gx, S)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_mx_kernel<2, 2, PF, false>), dim3(grid8(gx, S)), dim3(256), 0, s, a);
  }
  return MOE_OK;
}

}  // namespace moe
