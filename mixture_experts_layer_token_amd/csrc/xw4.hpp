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

namespace moe {

// Blob layout of the order-0 rANS code (encoder: compress.cpp, decoder kernel: decompress.hip);
// the format is specified in moe.h beside moe_compress_rans.
constexpr uint32_t kRnsMagic = 0x31534E52u;
constexpr int kRnsStreams = 32768;             // per region
constexpr int kRnsGroups = kRnsStreams / 64;   // streams of a group share one word sequence
constexpr int kRnsProb = 12;                   // frequencies sum to 2^12
constexpr uint32_t kRnsLow = 1u << 16;         // state interval [2^16, 2^32)

// bytes of a region section before its words: frequencies, states, group word offsets
__host__ __device__ inline size_t rns_section_head() { return 512 + 4 * (size_t)kRnsStreams + 4 * (size_t)(kRnsGroups + 1); }
// symbols of stream i in a region of m bytes
__host__ __device__ inline long long rns_count(long long m, long long i) {
  return i < m ? (m - i + kRnsStreams - 1) / kRnsStreams : 0;
}

}  // namespace moe
