// GPU decoder of the lossless exponent-window code (format in moe.h, moe_compress_package): a
// list of (compressed slot, decoded slot) pairs, each a whole package, in one launch.  Memory
// bound: about 0.75 byte read and 1 byte written per package byte.
//
// One wave decodes kChunksPerWave consecutive 1024-byte chunks, lane l the 8 values 8l .. 8l+7 of
// each.  All of the wave's loads are issued first, one 16-byte load per lane and chunk whatever
// the chunk's form (lanes past a short chunk re-read its last 16 bytes), so they are all in flight
// together.  A chunk's size says how it is stored, the same for the whole wave: 1024 bytes is raw
// (the lane's 16 bytes are its output), less is coded: the wave copies the chunk to its own 1 KiB
// of LDS and each lane reads back its 8 sign/mantissa bytes and its 32-bit word of codes; escapes,
// which are rare, take a wave prefix sum of per-lane escape counts to find each lane's escape bytes.
#include "common.hpp"
#include "xw4.hpp"

namespace moe {
namespace {

constexpr int kDecThreads = 256;
constexpr int kChunksPerWave = 4;

__device__ __forceinline__ unsigned zero_nibbles(unsigned w) {
  const unsigned nz = w | (w >> 1) | (w >> 2) | (w >> 3);
  return __builtin_popcount(~nz & 0x11111111u);
}

// value of one element: sign/mantissa byte, exponent
__device__ __forceinline__ unsigned bf16_of(unsigned smb, unsigned e) {
  return ((smb & 0x80u) << 8) | (e << 7) | (smb & 0x7Fu);
}

__global__ __launch_bounds__(kDecThreads) void xw4_decode_kernel(const uint8_t* __restrict__ src_base,
                                                                 size_t src_stride, uint8_t* __restrict__ dst_base,
                                                                 size_t dst_stride, const int32_t* __restrict__ pairs,
                                                                 int n_chunks) {
  __shared__ __align__(16) uint8_t lds[kDecThreads / 64][kXw4Chunk];
  const int p = blockIdx.y;
  const int ss = __builtin_amdgcn_readfirstlane(pairs[2 * p]);
  const int ds = __builtin_amdgcn_readfirstlane(pairs[2 * p + 1]);
  if (ss < 0 || ds < 0) return;
  const uint8_t* blob = src_base + (size_t)ss * src_stride;
  uint8_t* out = dst_base + (size_t)ds * dst_stride;
  const uint32_t* offs = (const uint32_t*)(blob + xw4_offsets_at());
  const uint8_t* bases = blob + xw4_bases_at(n_chunks);
  const uint8_t* data = blob + xw4_data_offset(n_chunks);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = (blockIdx.x * (kDecThreads / 64) + wave) * kChunksPerWave;
  const int nc = min(kChunksPerWave, n_chunks - c0);  // chunks of this wave (>= 1: the grid is exact per pair)
  if (nc <= 0) return;
  uint32_t o[kChunksPerWave + 1];
#pragma unroll
  for (int i = 0; i <= kChunksPerWave; ++i) o[i] = __builtin_amdgcn_readfirstlane(offs[c0 + min(i, nc)]);
  // the chunks' window bases, read as the two aligned words around them (scalar loads, before the
  // vector loads: waiting for a vector load issued after the chunks' would wait for all of them)
  const uintptr_t ba = (uintptr_t)(bases + c0);
  const uint32_t* bw = (const uint32_t*)(ba & ~(uintptr_t)3);
  const uint64_t bq = ((uint64_t)__builtin_amdgcn_readfirstlane(bw[1]) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane(bw[0]);
  const uint32_t b4 = (uint32_t)(bq >> (8 * (ba & 3)));  // bases of chunks c0 .. c0+3, one byte each
  const u32x4* src[kChunksPerWave];
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    // chunks past the wave's last re-read it (their results are not stored)
    const uint32_t a = o[min(i, nc - 1)], size = o[min(i, nc - 1) + 1] - a;
    src[i] = (const u32x4*)(data + a + min((uint32_t)lane * 16u, size - 16u));
  }
  // issued in chunk order, so waiting for chunk i never waits for a later one
  u32x4 v[kChunksPerWave];
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    v[i] = __builtin_nontemporal_load(src[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint8_t* buf = lds[wave];
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    if (i >= nc) break;
    const uint32_t size = o[i + 1] - o[i];
    u32x4 r = v[i];
    if (size != (uint32_t)kXw4Chunk) {
      const unsigned b1 = ((b4 >> (8 * i)) & 0xFFu) - 1u;  // e = base - 1 + code
      *(u32x4*)(buf + lane * 16) = v[i];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const u32x2 sm = *(const u32x2*)(buf + lane * 8);
      const unsigned cw = *(const unsigned*)(buf + 512 + lane * 4);
      unsigned e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = b1 + ((cw >> (4 * j)) & 15u);
      if (size > (uint32_t)kXw4CodedMin) {
        // escapes: this lane's first escape byte is the number of escapes in lanes below it
        const unsigned mine = zero_nibbles(cw);
        unsigned incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const unsigned t = __shfl_up(incl, off, 64);
          if (lane >= off) incl += t;
        }
        const uint8_t* esc = buf + kXw4CodedMin + (incl - mine);
        int k = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (((cw >> (4 * j)) & 15u) == 0) e[j] = esc[k++];
      }
      unsigned w[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const unsigned s2 = h < 2 ? sm[0] >> (16 * h) : sm[1] >> (16 * (h - 2));
        w[h] = bf16_of(s2 & 0xFFu, e[2 * h]) | (bf16_of((s2 >> 8) & 0xFFu, e[2 * h + 1]) << 16);
      }
      r = u32x4{w[0], w[1], w[2], w[3]};
      __builtin_amdgcn_wave_barrier();  // every lane has read this chunk from LDS before the next one lands
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    *((u32x4*)(out + (size_t)(c0 + i) * kXw4Chunk) + lane) = r;
  }
}


// ---------------------------------------------------------------- order-0 rANS decoder
//
// One wave per group of 64 streams: the lanes decode their streams in step (one symbol each per
// step), then the lanes whose state fell below 2^16 take the next words of the group's sequence in
// lane order (ballot and bit count).  A symbol costs one LDS lookup: a 4096-entry table from the low
// 12 bits of the state to (symbol, f - 1, slot - c), built per workgroup from the region's model.
// The words go through a 512-word ring in LDS, refilled 256 at a time from registers loaded one
// refill ahead; the decoded bytes collect in LDS, 16 steps of 64 streams per wave, and leave as one
// 16-byte store per lane every 16 steps.  The step itself waits on no global memory access, so even
// a lone package (1024 waves, one per SIMD) steps at LDS latency.

constexpr int kRnsThreads = 256;
constexpr int kRnsWaves = kRnsThreads / 64;
constexpr int kRnsRing = 512;   // words per wave
constexpr int kRnsChunk = 256;  // words per refill (4 per lane)
constexpr int kRnsRows = 16;    // steps per output flush

__global__ __launch_bounds__(kRnsThreads) void rns_decode_kernel(const uint8_t* __restrict__ src_base,
                                                                 size_t src_stride, uint8_t* __restrict__ dst_base,
                                                                 size_t dst_stride, const int32_t* __restrict__ pairs,
                                                                 long long raw_bytes) {
  __shared__ uint32_t tab[4096];  // slot -> symbol | (f - 1) << 8 | (slot - c) << 20
  __shared__ uint32_t fc[256];    // f | c << 16
  __shared__ uint16_t ring[kRnsWaves][kRnsRing];
  __shared__ __align__(16) uint8_t ob[kRnsWaves][kRnsRows * 64];
  __shared__ uint32_t wsum[kRnsWaves];
  // (pairs == nullptr: one package, the blob at src_base decoded to dst_base)
  const int ss = pairs ? __builtin_amdgcn_readfirstlane(pairs[2 * blockIdx.y]) : 0;
  const int ds = pairs ? __builtin_amdgcn_readfirstlane(pairs[2 * blockIdx.y + 1]) : 0;
  if (ss < 0 || ds < 0) return;
  const uint8_t* blob = src_base + (size_t)ss * src_stride;
  uint8_t* out = dst_base + (size_t)ds * dst_stride;
  const long long n = (long long)*(const uint64_t*)(blob + 8), q = (long long)*(const uint64_t*)(blob + 16);
  if (n != raw_bytes || q > n) return;  // not a blob of this package size: nothing is written
  constexpr int kWgPerRegion = kRnsGroups / kRnsWaves;
  const int region = blockIdx.x / kWgPerRegion;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = (blockIdx.x % kWgPerRegion) * kRnsWaves + wave;
  size_t sec_off = 64;
  if (region == 1) {
    const uint32_t w0 = *(const uint32_t*)(blob + 64 + 512 + 4 * (size_t)kRnsStreams + 4 * (size_t)kRnsGroups);
    sec_off += (rns_section_head() + 2 * (size_t)w0 + 15) & ~(size_t)15;
  }
  const uint8_t* sec = blob + sec_off;
  const long long m = region ? n - q : q;
  uint8_t* dst = out + (region ? q : 0);
  if (m == 0) return;  // (whole workgroup: no barrier below is skipped by part of it)

  // this wave's group: its states and word range, loaded ahead of the model's barriers
  const long long i = 64LL * g + lane;
  uint32_t x = *(const uint32_t*)(sec + 512 + 4 * (size_t)i);
  const uint32_t* offs = (const uint32_t*)(sec + 512 + 4 * (size_t)kRnsStreams);
  const uint32_t w_begin = __builtin_amdgcn_readfirstlane(offs[g]);
  const uint32_t n_words = __builtin_amdgcn_readfirstlane(offs[g + 1]) - w_begin;
  const uint16_t* words = (const uint16_t*)(sec + rns_section_head()) + w_begin;

  // model: cumulative counts by a scan over the 256 frequencies
  const uint32_t f = *(const uint16_t*)(sec + 2 * tid);
  uint32_t incl = f;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const uint32_t c = base + incl - f;
  fc[tid] = f | (c << 16);
#pragma unroll
  for (int k = 0; k < 4096 / kRnsThreads; ++k) tab[tid + k * kRnsThreads] = 0;
  __syncthreads();
  // slot -> symbol: the first slot of each present symbol names it, and a running maximum over the
  // slots gives every slot the largest present symbol starting at or before it (present symbols
  // start at increasing slots)
  if (f && c < 4096) tab[c] = tid;
  __syncthreads();
  constexpr int kPer = 4096 / kRnsThreads;  // 16 slots per thread
  uint32_t v[kPer], run = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    run = max(run, tab[kPer * tid + k]);
    v[k] = run;
  }
  uint32_t mx = run;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(mx, off, 64);
    if (lane >= off) mx = max(mx, t);
  }
  if (lane == 63) wsum[wave] = mx;  // (its sums were read before the previous barrier)
  __syncthreads();
  uint32_t before = __shfl_up(mx, 1, 64);
  if (lane == 0) before = 0;
  for (int w = 0; w < wave; ++w) before = max(before, wsum[w]);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t slot = kPer * tid + k, sym = max(before, v[k]), e = fc[sym];
    tab[slot] = sym | (((e & 0xFFFFu) - 1u) & 0xFFFu) << 8 | ((slot - (e >> 16)) & 0xFFFu) << 20;
  }
  __syncthreads();

  // the state's load completes here, once: inside the loop the compiler could no longer tell it
  // apart from the ring's prefetches and the flushes, and would wait for all of them every step
  asm volatile("" : "+v"(x));
  const long long cnt = rns_count(m, i);
  const int steps = (int)__builtin_amdgcn_readfirstlane((int)rns_count(m, 64LL * g));
  uint16_t* rw = ring[wave];
  uint8_t* ow = ob[wave];
  const bool aligned = ((uintptr_t)dst & 15) == 0;
  // words [fetched, fetched + 256) of the sequence, 4 per lane (lanes past the end load nothing)
  uint16_t pre[4];
  auto prefetch = [&](uint32_t fetched) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t wi = fetched + (uint32_t)(k * 64 + lane);
      pre[k] = wi < n_words ? words[wi] : (uint16_t)0;
    }
  };
  uint32_t loaded = 0, consumed = 0;  // words in the ring so far; words taken
  prefetch(0);
  for (int j = 0; j < steps; ++j) {
    if (loaded - consumed < 64 && loaded < n_words) {  // (wave-uniform) a step takes at most 64 words
#pragma unroll
      for (int k = 0; k < 4; ++k) rw[(loaded + k * 64 + lane) & (kRnsRing - 1)] = pre[k];
      loaded += kRnsChunk;
      if (loaded < n_words) prefetch(loaded);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    const bool act = j < cnt;
    if (act) {
      const uint32_t e = tab[x & 4095u];
      x = (((e >> 8) & 0xFFFu) + 1u) * (x >> 12) + (e >> 20);
      ow[(j & (kRnsRows - 1)) * 64 + lane] = (uint8_t)e;
    }
    const bool need = act && x < kRnsLow;
    const unsigned long long b = __ballot(need);
    if (need) {
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
      x = (x << 16) | rw[(consumed + rank) & (kRnsRing - 1)];
    }
    consumed += (uint32_t)__popcll(b);
    if ((j & (kRnsRows - 1)) == kRnsRows - 1 || j == steps - 1) {
      // flush: lane l stores bytes 16 (l % 4) .. +15 of row l / 4 (16 streams at one step)
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const int rows = (j & (kRnsRows - 1)) + 1, r = lane >> 2, part = lane & 3;
      if (r < rows) {
        const long long pos = 64LL * g + 16 * part + (long long)((j & ~(kRnsRows - 1)) + r) * kRnsStreams;
        const uint8_t* src = ow + r * 64 + 16 * part;
        if (aligned && pos + 16 <= m) {
          *(uint4*)(dst + pos) = *(const uint4*)src;
        } else {
          for (int k = 0; k < 16; ++k)
            if (pos + k < m) dst[pos + k] = src[k];
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    // (LDS accesses of one wave complete in order: a ring word is read before a later refill
    // rewrites it)
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

int launch_rns_decode_one(const void* blob, void* dst, size_t raw_bytes, hipStream_t s) {
  if (raw_bytes == 0) return MOE_OK;
  hipLaunchKernelGGL(rns_decode_kernel, dim3(2 * kRnsGroups / kRnsWaves, 1), dim3(kRnsThreads), 0, s,
                     (const uint8_t*)blob, (size_t)0, (uint8_t*)dst, (size_t)0, (const int32_t*)nullptr,
                     (long long)raw_bytes);
  MOE_CHECK_LAUNCH("rANS decode launch");
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_decompress_packages(const void* src_base, size_t src_stride, void* dst_base, size_t dst_stride,
                                       const int32_t* pairs, int n, size_t raw_bytes, void* stream) {
  if (n < 0) return fail(MOE_ERR_INVALID, "moe_decompress_packages: n=%d", n);
  if (raw_bytes % kXw4Chunk || raw_bytes / kXw4Chunk > 0x7FFFFFFFu)
    return fail(MOE_ERR_INVALID, "moe_decompress_packages: %zu bytes is not a multiple of 1024", raw_bytes);
  if (src_stride % 256 || dst_stride % 16)
    return fail(MOE_ERR_INVALID, "moe_decompress_packages: strides %zu / %zu (need multiples of 256 / 16)",
                src_stride, dst_stride);
  if (dst_stride < raw_bytes)
    return fail(MOE_ERR_INVALID, "moe_decompress_packages: dst_stride %zu < %zu", dst_stride, raw_bytes);
  if (n == 0 || raw_bytes == 0) return MOE_OK;
  if (!src_base || !dst_base || !pairs) return fail(MOE_ERR_INVALID, "moe_decompress_packages: null pointer");
  const int n_chunks = (int)(raw_bytes / kXw4Chunk);
  const int per_block = (kDecThreads / 64) * kChunksPerWave;
  if (n > 65535) return fail(MOE_ERR_INVALID, "moe_decompress_packages: n=%d exceeds 65535", n);
  hipLaunchKernelGGL(xw4_decode_kernel, dim3((n_chunks + per_block - 1) / per_block, n), dim3(kDecThreads), 0,
                     (hipStream_t)stream, (const uint8_t*)src_base, src_stride, (uint8_t*)dst_base, dst_stride, pairs,
                     n_chunks);
  MOE_CHECK_LAUNCH("moe_decompress_packages launch");
  return MOE_OK;
}

extern "C" int moe_decompress_rans(const void* src_base, size_t src_stride, void* dst_base, size_t dst_stride,
                                   const int32_t* pairs, int n, size_t raw_bytes, void* stream) {
  if (n < 0 || n > 65535) return fail(MOE_ERR_INVALID, "moe_decompress_rans: n=%d out of 0..65535", n);
  if (src_stride % 256 || dst_stride < raw_bytes)
    return fail(MOE_ERR_INVALID, "moe_decompress_rans: strides %zu / %zu for %zu bytes (source a multiple of 256)",
                src_stride, dst_stride, raw_bytes);
  if (n == 0 || raw_bytes == 0) return MOE_OK;
  if (!src_base || !dst_base || !pairs) return fail(MOE_ERR_INVALID, "moe_decompress_rans: null pointer");
  hipLaunchKernelGGL(rns_decode_kernel, dim3(2 * kRnsGroups / kRnsWaves, n), dim3(kRnsThreads), 0,
                     (hipStream_t)stream, (const uint8_t*)src_base, src_stride, (uint8_t*)dst_base, dst_stride, pairs,
                     (long long)raw_bytes);
  MOE_CHECK_LAUNCH("moe_decompress_rans launch");
  return MOE_OK;
}
