// Host encoder of the lossless exponent-window code (format in moe.h, moe_compress_package).
// Offline work, like the packer: a bank of compressed packages is built once; the GPU decodes.
//
// bf16 weights drawn around zero use few exponents: within a chunk of 512 values, the largest
// exponent and the 14 below it hold all but a handful, so 4 bits name the exponent and the sign and
// mantissa keep their own byte: 12 bits per value instead of 16, the rare value outside the window
// carries its exponent in an escape byte.
#include <string.h>

#include <algorithm>
#include <vector>

#include "common.hpp"
#include "xw4.hpp"

namespace moe {
namespace {

inline void st32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
inline void st64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }

// One chunk -> dst; returns the bytes written (a coded size below 1024, or 1024 for a raw chunk)
// and the window base through *base.
size_t encode_chunk(const uint16_t* v, uint8_t* dst, uint8_t* base) {
  unsigned top = 0;
  for (int j = 0; j < 512; ++j) {
    const unsigned e = (v[j] >> 7) & 0xFFu;
    top = e > top ? e : top;
  }
  const unsigned b = top >= 14 ? top - 14 : 0;
  // values outside [b, b + 14]: since b >= top - 14, only those below b
  int n_esc = 0;
  for (int j = 0; j < 512; ++j) n_esc += ((v[j] >> 7) & 0xFFu) < b;
  const size_t coded = kXw4CodedMin + (size_t)((n_esc + 15) & ~15);
  if (coded >= (size_t)kXw4Chunk) {
    memcpy(dst, v, kXw4Chunk);
    *base = 0;
    return kXw4Chunk;
  }
  uint8_t* sm = dst;
  uint8_t* codes = dst + 512;
  uint8_t* esc = dst + kXw4CodedMin;
  memset(esc, 0, coded - kXw4CodedMin);
  for (int j = 0; j < 512; j += 2) {
    unsigned c[2];
    for (int h = 0; h < 2; ++h) {
      const uint16_t x = v[j + h];
      const unsigned e = (x >> 7) & 0xFFu;
      sm[j + h] = (uint8_t)(((x >> 8) & 0x80u) | (x & 0x7Fu));
      if (e >= b) {
        c[h] = e - b + 1;
      } else {
        c[h] = 0;
        *esc++ = (uint8_t)e;
      }
    }
    codes[j >> 1] = (uint8_t)(c[0] | (c[1] << 4));
  }
  *base = (uint8_t)b;
  return coded;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_compress_bound(size_t raw_bytes) {
  if (raw_bytes % kXw4Chunk) return 0;
  return xw4_data_offset(raw_bytes / kXw4Chunk) + raw_bytes;
}

extern "C" int moe_compress_package(const void* raw, size_t raw_bytes, void* blob, size_t cap, size_t* blob_bytes) {
  if (raw_bytes % kXw4Chunk || raw_bytes >= ((size_t)1 << 32))
    return fail(MOE_ERR_INVALID, "moe_compress_package: %zu bytes is not a multiple of 1024 below 4 GiB", raw_bytes);
  if ((raw_bytes && !raw) || !blob || !blob_bytes) return fail(MOE_ERR_INVALID, "moe_compress_package: null pointer");
  if (cap < moe_compress_bound(raw_bytes))
    return fail(MOE_ERR_INVALID, "moe_compress_package: capacity %zu < bound %zu", cap, moe_compress_bound(raw_bytes));
  const size_t n = raw_bytes / kXw4Chunk, data = xw4_data_offset(n);
  uint8_t* out = (uint8_t*)blob;
  memset(out, 0, data);
  uint8_t* offs = out + xw4_offsets_at();
  uint8_t* bases = out + xw4_bases_at(n);
  // (raw bytes are read as bf16 values through memcpy: the caller's buffer need not be aligned)
  uint16_t v[512];
  size_t pos = 0;
  for (size_t i = 0; i < n; ++i) {
    memcpy(v, (const uint8_t*)raw + i * kXw4Chunk, kXw4Chunk);
    pos += encode_chunk(v, out + data + pos, bases + i);
    st32(offs + 4 * (i + 1), (uint32_t)pos);
  }
  st32(out, kXw4Magic);
  st32(out + 4, (uint32_t)n);
  st64(out + 8, raw_bytes);
  st64(out + 16, data);
  st64(out + 24, data + pos);
  *blob_bytes = data + pos;
  return MOE_OK;
}

// ---------------------------------------------------------------- order-0 rANS code

namespace moe {
namespace {

// byte model of a region: frequencies summing to 2^12, every present byte at least 1
void rns_freqs(const uint8_t* r, size_t m, uint32_t f[256]) {
  uint64_t h[256] = {};
  for (size_t j = 0; j < m; ++j) ++h[r[j]];
  long long total = 0;
  for (int s = 0; s < 256; ++s) {
    f[s] = h[s] ? (uint32_t)std::max<uint64_t>(1, h[s] * 4096 / m) : 0;
    total += f[s];
  }
  if (!m) return;
  while (total != 4096) {
    const int top = (int)(std::max_element(f, f + 256) - f);  // (the first of equal maxima)
    if (total > 4096) {
      --f[top];
      --total;
    } else {
      f[top] += (uint32_t)(4096 - total);
      total = 4096;
    }
  }
}

// one region into out; returns the section's bytes
size_t rns_region(const uint8_t* r, size_t m, uint8_t* out) {
  uint32_t f[256], c[256];
  rns_freqs(r, m, f);
  for (int s = 0, acc = 0; s < 256; ++s) c[s] = (uint32_t)acc, acc += (int)f[s];
  for (int s = 0; s < 256; ++s) {
    const uint16_t v = (uint16_t)f[s];
    memcpy(out + 2 * s, &v, 2);
  }
  uint8_t* states = out + 512;
  uint8_t* offs = states + 4 * (size_t)kRnsStreams;
  uint8_t* words = out + rns_section_head();
  std::vector<uint16_t> emitted;
  uint32_t total_words = 0;
  for (int g = 0; g < kRnsGroups; ++g) {
    st32(offs + 4 * (size_t)g, total_words);
    uint32_t x[64];
    std::fill(x, x + 64, kRnsLow);
    emitted.clear();
    const long long steps = rns_count((long long)m, 64LL * g);
    // the group in step, last symbol first and streams in descending order: the decoder reads the
    // words of a step in ascending stream order after the step's symbols
    for (long long j = steps - 1; j >= 0; --j)
      for (int l = 63; l >= 0; --l) {
        const long long i = 64LL * g + l;
        if (j >= rns_count((long long)m, i)) continue;
        const uint8_t sym = r[i + j * kRnsStreams];
        // largest state before the symbol that stays below 2^32 after it: (2^16 / 2^12) 2^16 f = 2^20 f
        const uint64_t limit = (uint64_t)f[sym] << 20;
        uint64_t v = x[l];
        if (v >= limit) {
          emitted.push_back((uint16_t)(v & 0xFFFF));
          v >>= 16;
        }
        x[l] = (uint32_t)(((v / f[sym]) << kRnsProb) + v % f[sym] + c[sym]);
      }
    for (int l = 0; l < 64; ++l) st32(states + 4 * (64 * (size_t)g + l), x[l]);
    for (size_t k = 0; k < emitted.size(); ++k) {
      const uint16_t w = emitted[emitted.size() - 1 - k];
      memcpy(words + 2 * ((size_t)total_words + k), &w, 2);
    }
    total_words += (uint32_t)emitted.size();
  }
  st32(offs + 4 * (size_t)kRnsGroups, total_words);
  const size_t bytes = rns_section_head() + 2 * (size_t)total_words, padded = (bytes + 15) & ~(size_t)15;
  memset(out + bytes, 0, padded - bytes);
  return padded;
}

size_t rns_region_bound(size_t m) { return rns_section_head() + 2 * (m + 2 * (size_t)kRnsStreams) + 16; }

}  // namespace
}  // namespace moe

extern "C" size_t moe_compress_rans_bound(size_t raw_bytes) {
  return 64 + rns_region_bound(raw_bytes) * 2;
}

extern "C" int moe_compress_rans(const void* raw, size_t raw_bytes, size_t split, void* blob, size_t cap,
                                 size_t* blob_bytes) {
  if (split > raw_bytes) return fail(MOE_ERR_INVALID, "moe_compress_rans: split %zu > %zu bytes", split, raw_bytes);
  if (raw_bytes >= ((size_t)1 << 32)) return fail(MOE_ERR_INVALID, "moe_compress_rans: %zu bytes (4 GiB at most)", raw_bytes);
  if ((raw_bytes && !raw) || !blob || !blob_bytes) return fail(MOE_ERR_INVALID, "moe_compress_rans: null pointer");
  if (cap < moe_compress_rans_bound(raw_bytes))
    return fail(MOE_ERR_INVALID, "moe_compress_rans: capacity %zu < bound %zu", cap, moe_compress_rans_bound(raw_bytes));
  uint8_t* out = (uint8_t*)blob;
  memset(out, 0, 64);
  const uint8_t* r = (const uint8_t*)raw;
  size_t pos = 64;
  pos += rns_region(r, split, out + pos);
  pos += rns_region(r + split, raw_bytes - split, out + pos);
  st32(out, kRnsMagic);
  st32(out + 4, (uint32_t)kRnsStreams);
  st64(out + 8, raw_bytes);
  st64(out + 16, split);
  st64(out + 24, pos);
  *blob_bytes = pos;
  return MOE_OK;
}
