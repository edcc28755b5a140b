/*
 * Seeded synthetic input generator for the routed-expert MoE layer.
 *
 * This module produces inputs only: activations, router weights and expert
 * weights (plain or block-quantized), drawn from a counter-based generator so
 * that any element of any tensor can be produced on its own, in any order, on
 * any number of threads, with identical bytes.  It holds none of the layer's
 * arithmetic (no routing, no permutation, no FFN, no combine, no decoding of
 * the packed formats); both the HIP path and the CPU oracle consume what it
 * writes.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Element i of stream (seed, stream) is
 * mix64(key + (i + 1) * GAMMA) with key = mix64(seed ^ mix64(stream)), i.e. the
 * i-th output of a SplitMix64 sequence started at key.  Normal variates use the
 * Box-Muller transform on the pair (2p, 2p+1): element 2p takes the cosine
 * branch, element 2p+1 the sine branch.
 *
 * Block quantizers (produce the input weights of the 4-bit formats):
 *  - MXFP4: OCP Microscaling Formats v1.0.  Blocks of 32 along K, one E8M0
 *    scale X per block with X = floor(log2(amax)) - 2 (2 = largest exponent
 *    of E2M1), elements rounded to nearest-even E2M1 of w / 2^X, saturating
 *    at +-6.  Element 2i of a row sits in the low nibble of byte i.
 *  - INT4 group-32 (symmetric): s = bf16_rne(amax / 7); q = clamp(rne(w / s),
 *    -7, 7) (q = 0 when s = 0); two's-complement nibbles, element 2i in the
 *    low nibble; one bf16 scale per (row, group of 32 along K).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed ^ mix64(stream + GAMMA));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* uniform on the open interval (0, 1): 53 random bits, centred in their cell */
static inline double unit_open(uint64_t u) { return ((double)(u >> 11) + 0.5) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = unit_open(draw(key, 2 * p));
  double u2 = unit_open(draw(key, 2 * p + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* round-to-nearest-even of a double to bfloat16 (8 significant bits), as bits */
static uint16_t bf16_rne_bits(double d) {
  if (d == 0.0) return signbit(d) ? 0x8000 : 0x0000;
  if (isnan(d)) return 0x7FC0;
  int e;
  double m = frexp(fabs(d), &e); /* |d| = m * 2^e, m in [0.5, 1) */
  double r;
  if (e - 1 < -126) {
    /* subnormal bf16: quantum 2^-133 */
    r = nearbyint(ldexp(fabs(d), 133)) * 0x1.0p-133;
  } else {
    r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
  }
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t h = (uint16_t)(u >> 16);
  if (isinf(f) || (u & 0xFFFF)) h = 0x7F80; /* overflow to inf */
  return (uint16_t)(h | (d < 0 ? 0x8000 : 0));
}

static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) { return stream_key(seed, stream); }

uint64_t synth_raw_u64(uint64_t seed, uint64_t stream, uint64_t i) { return draw(stream_key(seed, stream), i); }

/* i-th output of a SplitMix64 sequence whose state starts at key */
uint64_t synth_draw_key(uint64_t key, uint64_t i) { return draw(key, i); }

void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unit_open(draw(key, offset + (uint64_t)i));
}

void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma, double* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sigma * normal_at(key, offset + (uint64_t)i);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_at(key, offset + (uint64_t)i));
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne_bits(sigma * normal_at(key, offset + (uint64_t)i));
}

/* E2M1 magnitudes by code 0..7 (sign is bit 3) */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* nearest E2M1 code to |v| with ties to the even code (mantissa bit 0), saturating at 6 */
static int e2m1_rne_code(double a) {
  if (a >= 6.0) return 7;
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(a - kE2M1[c]), db = fabs(a - kE2M1[best]);
    if (dc < db || (dc == db && (c & 1) == 0 && (best & 1) == 1)) best = c;
  }
  return best;
}

/*
 * rows x K weights ~ N(0, sigma) from stream (seed, stream), row-major, quantized
 * to MXFP4.  codes: [rows][K/2] bytes; scales: [rows][K/32] E8M0 bytes.
 */
void synth_quant_mxfp4(uint64_t seed, uint64_t stream, int64_t rows, int64_t K, double sigma, uint8_t* codes,
                       uint8_t* scales) {
  uint64_t key = stream_key(seed, stream);
  int64_t nblk = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t rb = 0; rb < rows * nblk; ++rb) {
    int64_t r = rb / nblk, b = rb % nblk;
    double w[32], amax = 0.0;
    for (int j = 0; j < 32; ++j) {
      w[j] = sigma * normal_at(key, (uint64_t)(r * K + b * 32 + j));
      if (fabs(w[j]) > amax) amax = fabs(w[j]);
    }
    int X;
    if (amax == 0.0) {
      X = -127;
    } else {
      int e;
      frexp(amax, &e); /* amax = m * 2^e, m in [0.5,1) -> floor(log2 amax) = e - 1 */
      X = (e - 1) - 2;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    scales[r * nblk + b] = (uint8_t)(X + 127);
    for (int j = 0; j < 32; j += 2) {
      int c[2];
      for (int t = 0; t < 2; ++t) {
        double v = ldexp(w[j + t], -X);
        int code = e2m1_rne_code(fabs(v));
        if (v < 0 && code != 0) code |= 8;
        c[t] = code;
      }
      codes[r * (K / 2) + (b * 32 + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));
    }
  }
}

/*
 * rows x K weights ~ N(0, sigma), row-major, quantized to symmetric INT4 with
 * one bf16 scale per group of 32 along K.  codes: [rows][K/2]; scales: [rows][K/32] bf16 bits.
 */
void synth_quant_int4g32(uint64_t seed, uint64_t stream, int64_t rows, int64_t K, double sigma, uint8_t* codes,
                         uint16_t* scales) {
  uint64_t key = stream_key(seed, stream);
  int64_t nblk = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t rb = 0; rb < rows * nblk; ++rb) {
    int64_t r = rb / nblk, b = rb % nblk;
    double w[32], amax = 0.0;
    for (int j = 0; j < 32; ++j) {
      w[j] = sigma * normal_at(key, (uint64_t)(r * K + b * 32 + j));
      if (fabs(w[j]) > amax) amax = fabs(w[j]);
    }
    uint16_t sb = bf16_rne_bits(amax / 7.0);
    double s = bf16_bits_to_double(sb);
    scales[r * nblk + b] = sb;
    for (int j = 0; j < 32; j += 2) {
      int c[2];
      for (int t = 0; t < 2; ++t) {
        int q = 0;
        if (s != 0.0) {
          double qq = nearbyint(w[j + t] / s);
          if (qq > 7) qq = 7;
          if (qq < -7) qq = -7;
          q = (int)qq;
        }
        c[t] = q & 15;
      }
      codes[r * (K / 2) + (b * 32 + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));
    }
  }
}
