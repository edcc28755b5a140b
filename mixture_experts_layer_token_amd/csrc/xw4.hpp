// Blob layout of the lossless exponent-window code of bf16 packages (encoder: compress.cpp,
// decoder kernel: decompress.hip).  The format itself is specified in moe.h beside
// moe_compress_package.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr uint32_t kXw4Magic = 0x31345758u;
constexpr int kXw4Chunk = 1024;       // raw bytes per chunk (512 bf16 values)
constexpr int kXw4CodedMin = 768;     // sign/mantissa bytes + code nibbles
constexpr int kXw4HeaderBytes = 64;

// byte offset of the chunk data: past the header, the n + 1 u32 offsets and the n u8 bases
__host__ __device__ inline size_t xw4_data_offset(size_t n_chunks) {
  return (kXw4HeaderBytes + 4 * (n_chunks + 1) + n_chunks + 255) / 256 * 256;
}
__host__ __device__ inline size_t xw4_offsets_at() { return kXw4HeaderBytes; }
__host__ __device__ inline size_t xw4_bases_at(size_t n_chunks) { return kXw4HeaderBytes + 4 * (n_chunks + 1); }

}  // namespace moe
