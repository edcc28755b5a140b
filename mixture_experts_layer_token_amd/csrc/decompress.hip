// GPU decoder of the lossless exponent-window code (format in moe.h, moe_compress_package): a
// list of (compressed slot, decoded slot) pairs, each a whole package, in one launch.  Memory
// bound: about 0.75 byte read and 1 byte written per package byte.
//
// One wave decodes one 1024-byte chunk at a time, lane l the 8 values 8l .. 8l+7: 8 sign/mantissa
// bytes and one 32-bit word of codes, 16 bytes out.  A chunk's size says how it is stored (1024:
// raw, 768: no escapes, more: escapes), the same for the whole wave; escapes, which are rare,
// take a wave prefix sum of per-lane escape counts to find each lane's escape bytes.
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
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    const int c = c0 + i;
    if (c >= n_chunks) break;
    const uint32_t o0 = __builtin_amdgcn_readfirstlane(offs[c]);
    const uint32_t size = __builtin_amdgcn_readfirstlane(offs[c + 1]) - o0;
    const uint8_t* ch = data + o0;
    u32x4 r;
    if (size == kXw4Chunk) {
      r = __builtin_nontemporal_load((const u32x4*)ch + lane);
    } else {
      const unsigned b1 = (unsigned)__builtin_amdgcn_readfirstlane(bases[c]) - 1u;  // e = base - 1 + code
      const u32x2 sm = __builtin_nontemporal_load((const u32x2*)ch + lane);
      const unsigned cw = __builtin_nontemporal_load((const unsigned*)(ch + 512) + lane);
      unsigned e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = b1 + ((cw >> (4 * j)) & 15u);
      if (size > (uint32_t)kXw4CodedMin) {
        // escapes: this lane's first escape byte is the number of escapes in lanes below it
        const unsigned mine = zero_nibbles(cw);
        unsigned incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const unsigned o = __shfl_up(incl, off, 64);
          if (lane >= off) incl += o;
        }
        const uint8_t* esc = ch + kXw4CodedMin + (incl - mine);
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
    }
    *((u32x4*)(out + (size_t)c * kXw4Chunk) + lane) = r;
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
