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

}  // namespace
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
