// Host-side repacking of one expert from the logical layout into the device package the
// kernels stream (layout described in common.hpp).  Offline work: runs once per expert when a
// weight bank is built, never on the forward path.
#include <math.h>
#include <string.h>

#include "common.hpp"

namespace moe {
namespace {

// binary16 bits of an INT4 group scale the kernels can use, or -1: the scale must be a normal
// binary16 number (bf16 has fewer significand bits, so only the range matters) and every product
// q * s, q in [-8, 7], must stay finite in binary16 (|s| <= 65504 / 8)
int exact_f16_bits(uint16_t bf16) {
  uint32_t u = (uint32_t)bf16 << 16;
  float f;
  memcpy(&f, &u, 4);
  if (f == 0.0f) return (bf16 & 0x8000) ? 0x8000 : 0;
  float a = fabsf(f);
  if (!(a >= 0x1.0p-14f && a <= 65504.0f / 8.0f)) return -1;
  int e;
  float m = frexpf(a, &e);  // a = m * 2^e, m in [0.5, 1)
  // 11 significant bits available; bf16 has 8, so only the range matters
  uint32_t mant = (uint32_t)ldexpf(m, 11) - 1024;  // 10 explicit bits
  uint32_t exp = (uint32_t)(e - 1 + 15);
  return (int)(((bf16 & 0x8000) ? 0x8000u : 0u) | (exp << 10) | mant);
}

// copy one [rows][K] bf16 matrix into strips starting at strip index s0 with strip step `step`
void pack_bf16_matrix(const uint16_t* src, int rows, int K, uint16_t* dst_region, int s0, int step) {
  const int nks = K / 32;
  for (int r = 0; r < rows; ++r) {
    int strip = s0 + step * (r / 16), rr = r % 16;
    uint16_t* sb = dst_region + (size_t)strip * 16 * K;
    for (int ks = 0; ks < nks; ++ks)
      for (int q = 0; q < 4; ++q) {
        int lane = rr + 16 * q;
        memcpy(sb + (size_t)ks * 512 + lane * 8, src + (size_t)r * K + ks * 32 + q * 8, 16);
      }
  }
}

inline unsigned src_nibble(const uint8_t* codes, int K, int r, int k) {
  uint8_t b = codes[(size_t)r * (K / 2) + k / 2];
  return (k & 1) ? (b >> 4) : (b & 15);
}

// 4-bit matrix -> strip chunks; scales -> per-strip [chunk][16 rows][ns]
int pack_4bit_matrix(int fmt, const uint8_t* codes, const void* scales, int rows, int K, uint8_t* code_region,
                     uint8_t* scale_region, int s0, int step) {
  const int nks = K / 32, nch = (nks + 3) / 4;
  const size_t sb = scale_bytes(fmt);
  for (int r = 0; r < rows; ++r) {
    int strip = s0 + step * (r / 16), rr = r % 16;
    uint8_t* cs = code_region + (size_t)strip * 8 * K;  // 16 rows * K/2 bytes
    uint8_t* ss = scale_region + (size_t)strip * 16 * nks * sb;
    for (int c = 0; c < nch; ++c) {
      int ns = nks - 4 * c < 4 ? nks - 4 * c : 4;
      uint8_t* chunk = cs + (size_t)c * 1024;
      for (int j = 0; j < ns; ++j) {
        int ks = 4 * c + j;
        for (int q = 0; q < 4; ++q) {
          int lane = rr + 16 * q;
          uint8_t* word = chunk + (size_t)lane * 4 * ns + 4 * j;
          uint32_t v = 0;
          for (int t = 0; t < 8; ++t) {
            unsigned nib = src_nibble(codes, K, r, ks * 32 + q * 8 + t);
            if (fmt == MOE_W_MXFP4) {
              v |= (uint32_t)nib << (4 * t);  // byte t/2, low nibble first
            } else {
              unsigned ob = (nib + 8) & 15;          // two's complement -> q + 8
              int pos = (t & 1) ? 4 + t / 2 : t / 2;  // element 2n -> nibble n, 2n+1 -> nibble n+4
              v |= (uint32_t)ob << (4 * pos);
            }
          }
          memcpy(word, &v, 4);
        }
        // scale of (row r, k-step ks)
        uint8_t* sdst = ss + ((size_t)16 * 4 * c + (size_t)rr * ns + j) * sb;
        if (fmt == MOE_W_MXFP4) {
          sdst[0] = ((const uint8_t*)scales)[(size_t)r * nks + ks];
        } else {
          int h = exact_f16_bits(((const uint16_t*)scales)[(size_t)r * nks + ks]);
          if (h < 0)
            return fail(MOE_ERR_UNSUPPORTED,
                        "moe_pack_expert: INT4 scale (row %d, group %d) outside [2^-14, 65504/8] (binary16 operands)", r, ks);
          uint16_t hb = (uint16_t)h;
          memcpy(sdst, &hb, 2);
        }
      }
    }
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_package_bytes(int H, int I, int fmt) {
  if (H <= 0 || I <= 0 || H % 32 || I % 32 || !fmt_valid(fmt)) return 0;
  return pack_geom(H, I, fmt).bytes;
}

extern "C" int moe_pack_expert(int H, int I, int fmt, const void* gate, const void* gate_scales, const void* up,
                               const void* up_scales, const void* down, const void* down_scales, void* package,
                               size_t package_bytes) {
  if (!fmt_valid(fmt)) return fail(MOE_ERR_INVALID, "moe_pack_expert: bad format %d", fmt);
  if (H <= 0 || I <= 0) return fail(MOE_ERR_INVALID, "moe_pack_expert: H=%d I=%d", H, I);
  if (H % 32 || I % 32) return fail(MOE_ERR_UNSUPPORTED, "moe_pack_expert: H=%d, I=%d must be multiples of 32", H, I);
  if (!gate || !up || !down || !package) return fail(MOE_ERR_INVALID, "moe_pack_expert: null pointer");
  const bool q4 = fmt == MOE_W_MXFP4 || fmt == MOE_W_INT4G32;
  if (q4 && (!gate_scales || !up_scales || !down_scales))
    return fail(MOE_ERR_INVALID, "moe_pack_expert: 4-bit format needs scales");
  PackGeom g = pack_geom(H, I, fmt);
  if (package_bytes < g.bytes)
    return fail(MOE_ERR_INVALID, "moe_pack_expert: package_bytes %zu < %zu", package_bytes, g.bytes);
  uint8_t* pkg = (uint8_t*)package;
  if (fmt == MOE_W_F32) {
    size_t m = (size_t)H * I * 4;
    memcpy(pkg, gate, m);
    memcpy(pkg + m, up, m);
    memcpy(pkg + 2 * m, down, m);
    return MOE_OK;
  }
  if (fmt == MOE_W_BF16) {
    uint16_t* gu = (uint16_t*)(pkg + g.gu_codes);
    pack_bf16_matrix((const uint16_t*)gate, I, H, gu, 0, 2);
    pack_bf16_matrix((const uint16_t*)up, I, H, gu, 1, 2);
    pack_bf16_matrix((const uint16_t*)down, H, I, (uint16_t*)(pkg + g.d_codes), 0, 1);
    return MOE_OK;
  }
  int rc = pack_4bit_matrix(fmt, (const uint8_t*)gate, gate_scales, I, H, pkg + g.gu_codes, pkg + g.gu_scales, 0, 2);
  if (rc == MOE_OK)
    rc = pack_4bit_matrix(fmt, (const uint8_t*)up, up_scales, I, H, pkg + g.gu_codes, pkg + g.gu_scales, 1, 2);
  if (rc == MOE_OK)
    rc = pack_4bit_matrix(fmt, (const uint8_t*)down, down_scales, H, I, pkg + g.d_codes, pkg + g.d_scales, 0, 1);
  return rc;
}
