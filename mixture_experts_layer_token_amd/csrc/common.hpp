// Internal definitions shared by the HIP kernels and the C-ABI glue of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------ vector types
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr int kWave = 64;

// ------------------------------------------------------------ error state
int fail(int code, const char* fmt, ...);
int hip_fail(hipError_t e, const char* what);

#define MOE_CHECK_LAUNCH(what)                              \
  do {                                                      \
    hipError_t e_ = hipGetLastError();                      \
    if (e_ != hipSuccess) return ::moe::hip_fail(e_, what); \
  } while (0)

// ------------------------------------------------------------ scalar conversions
__device__ __forceinline__ float bf16_to_f32(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

// nearest-even rounding of an fp32 value to bf16 (NaN kept quiet)
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (unsigned short)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ------------------------------------------------------------ package layout
//
// A package holds one expert.  Matrices:
//   GU: the gate and up projections, 2I rows of K = H, interleaved by 16-row strips
//       (strip 2s = gate rows 16s..16s+15, strip 2s+1 = up rows 16s..16s+15);
//   D : the down projection, H rows of K = I.
// f32 packages are plain row-major gate [I][H], up [I][H], down [H][I].
// bf16: each strip of 16 rows is a run of K/32 fragments of 1 KiB; fragment g holds, for
//   lane l (0..63), the 8 elements of row (l % 16), k = 32 g + 8 (l / 16) .. + 7 (16 bytes at 16 l).
//   That is exactly the B operand of v_mfma_f32_16x16x32_{bf16,f16} for lane l.
// 4-bit: each strip is a run of chunks of up to 4 k-steps (ns = min(4, K/32 - 4c)); chunk c
//   occupies 256 * ns bytes; lane l owns 4 * ns bytes at 4 * ns * l: for k-step j, 4 bytes
//   holding the 8 elements of row (l % 16), k = 32 (4c + j) + 8 (l / 16) .. + 7.
//   MXFP4 byte b of those 4 holds elements (2b, 2b+1), low nibble first.
//   INT4 nibble n of the 32-bit word holds element (n < 4 ? 2n : 2(n-4)+1), stored as q + 8.
//   Scales of a strip: chunk c at 16 * 4c entries: [16 rows][ns] (E8M0 bytes; INT4: binary16).
// Region order: GU codes, D codes, GU scales, D scales.
struct PackGeom {
  int H, I, fmt;
  size_t gu_codes, d_codes, gu_scales, d_scales;  // byte offsets
  size_t bytes;
};

__host__ __device__ inline size_t elem_bits(int fmt) { return fmt == MOE_W_F32 ? 32 : fmt == MOE_W_BF16 ? 16 : 4; }
__host__ __device__ inline size_t scale_bytes(int fmt) { return fmt == MOE_W_MXFP4 ? 1 : fmt == MOE_W_INT4G32 ? 2 : 0; }

__host__ __device__ inline PackGeom pack_geom(int H, int I, int fmt) {
  PackGeom g;
  g.H = H;
  g.I = I;
  g.fmt = fmt;
  size_t n_gu = (size_t)2 * I * H, n_d = (size_t)H * I;
  size_t eb = elem_bits(fmt), sb = scale_bytes(fmt);
  g.gu_codes = 0;
  g.d_codes = n_gu * eb / 8;
  g.gu_scales = g.d_codes + n_d * eb / 8;
  g.d_scales = g.gu_scales + n_gu / 32 * sb;
  g.bytes = g.d_scales + n_d / 32 * sb;
  return g;
}

bool fmt_valid(int fmt);
void* const* trace_events();  // moe_ffn_trace_events setting of this thread (or nullptr)
bool dtype_valid(int dt);

// ------------------------------------------------------------ launch helpers (internal)
size_t route_workspace(int T, int H, int E, int xdt);
int launch_route(const void* x, int xdt, int T, int H, const void* wg, const float* bias, int E, int k, int32_t* ids,
                 float* w, float* logits, void* ws, size_t ws_bytes, hipStream_t s);
bool route_split_path(int T, int H, int E, int xdt);
int route_split_partials(const void* x, int T, int H, const void* wg, int E, float* part, int* ks_out, hipStream_t s);
size_t route_permute_workspace(int T, int H, int E, int k, int xdt);
int launch_route_permute(const void* x, int xdt, int T, int H, const void* wg, const float* bias, int E, int k,
                         int32_t* ids, float* w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* inv, void* ws, size_t ws_bytes, hipStream_t s);
size_t permute_workspace(int T, int k, int E);
int launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                   int32_t* inv, void* ws, size_t ws_bytes, hipStream_t s);
int launch_combine(const float* y, const float* w, const int32_t* inv, int T, int k, int H, const float* shared,
                   void* out, int odt, hipStream_t s);
int launch_dequant(const void* pkg, int H, int I, int fmt, float* out, hipStream_t s);
// one rANS blob (moe_compress_rans) of a raw_bytes package decoded into dst
int launch_rns_decode_one(const void* blob, void* dst, size_t raw_bytes, hipStream_t s);
size_t ffn_workspace(const moe_experts* w, int T, int k, int mode);
// helper_stream: the AUTO hybrid may run its tile-kernel share on a library-owned helper stream
// (created once per device), beside the streaming kernels
int launch_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
               const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes, hipStream_t s,
               bool helper_stream);
// moe_expert_ffn's validation, then launch_ffn
int expert_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
               const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes, void* stream,
               bool helper_stream);

}  // namespace moe
