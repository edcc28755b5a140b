/* Runs every function of the oracle and of the input generator once on small inputs, for builds
 * with AddressSanitizer and UndefinedBehaviorSanitizer (any report ends the process with an error). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int fmt;
  const void* w[3];
  const void* s[3];
} oracle_expert;

void synth_normal_f32(uint64_t, uint64_t, uint64_t, int64_t, double, float*);
void synth_normal_bf16(uint64_t, uint64_t, uint64_t, int64_t, double, uint16_t*);
void synth_uniform_f64(uint64_t, uint64_t, uint64_t, int64_t, double*);
void synth_quant_mxfp4(uint64_t, uint64_t, int64_t, int64_t, double, uint8_t*, uint8_t*);
void synth_quant_int4g32(uint64_t, uint64_t, int64_t, int64_t, double, uint8_t*, uint16_t*);
void oracle_decode(int, const void*, const void*, int64_t, int64_t, double*);
void oracle_decode_act(int, const void*, int64_t, double*);
void oracle_router_logits(int, const void*, const void*, const float*, int64_t, int64_t, int64_t, double*);
void oracle_topk_gates(const double*, int64_t, int64_t, int, int32_t*, double*);
void oracle_permute(const int32_t*, int64_t, int, int64_t, int32_t*, int32_t*, int32_t*, int32_t*);
void oracle_ffn(const oracle_expert*, int64_t, int64_t, const double*, int64_t, double*);
int oracle_moe_layer(int, const void*, int64_t, int64_t, const void*, const float*, int64_t, int, int64_t,
                     const oracle_expert*, const oracle_expert*, int64_t, const int64_t*, int64_t, double*, int32_t*,
                     double*);
int oracle_lru(int64_t, int64_t, const int64_t*, const int64_t*, int64_t*, int64_t*, int64_t*, int64_t*);
int oracle_lfu_decay(int64_t, int64_t, int64_t, const int64_t*, const int64_t*, int64_t*, int64_t*, int64_t*,
                     int64_t*);
int oracle_belady(int64_t, int64_t, const int64_t*, const int64_t*, int64_t*, int64_t*);
int oracle_cache_sim(int64_t, int, int64_t, int64_t, const int64_t*, const int64_t*, const int32_t*, int64_t*,
                     int64_t*, int64_t*, int64_t*, int64_t*);

enum { H = 64, I = 96, E = 6, K = 2, T = 5 };

static void* xmalloc(size_t n) {
  void* p = malloc(n);
  if (!p) abort();
  return p;
}

int64_t oracle_xw4_bound(int64_t);
int64_t oracle_xw4_encode(const uint8_t*, int64_t, uint8_t*, int64_t);
int oracle_xw4_decode(const uint8_t*, int64_t, uint8_t*, int64_t);

/* the lossless code on gaussian, random and escape-heavy chunks, round trip and malformed blobs */
static int xw4_checks(void) {
  enum { N = 1024 * 24 };
  uint16_t* v = xmalloc(N);
  uint8_t* back = xmalloc(N);
  synth_normal_bf16(7, 1, 0, N / 2, 0.02, v);
  for (int i = 0; i < 512; ++i) v[4 * 512 + i] = (uint16_t)(i * 2654435761u >> 16); /* a random-bits chunk */
  for (int i = 0; i < 300; ++i) v[6 * 512 + i] = 0x0080;                         /* many escapes: raw */
  for (int i = 0; i < 40; ++i) v[8 * 512 + 3 * i] = 0;                           /* a few escapes */
  const int64_t cap = oracle_xw4_bound(N);
  uint8_t* blob = xmalloc((size_t)cap);
  const int64_t n = oracle_xw4_encode((const uint8_t*)v, N, blob, cap);
  if (n <= 0 || n > cap) return 1;
  if (oracle_xw4_decode(blob, n, back, N) != 0 || memcmp(back, v, N) != 0) return 2;
  if (oracle_xw4_decode(blob, 100, back, N) == 0) return 3; /* truncated */
  blob[64 + 4] ^= 0x40;                                      /* a corrupt chunk offset */
  (void)oracle_xw4_decode(blob, n, back, N);
  if (oracle_xw4_encode((const uint8_t*)v, 1000, blob, cap) != -1) return 4;
  free(v);
  free(back);
  free(blob);
  return 0;
}

int main(void) {
  /* experts in all four formats */
  oracle_expert ex[4];
  void* keep[32];
  int nk = 0;
  for (int f = 0; f < 4; ++f) {
    ex[f].fmt = f;
    for (int m = 0; m < 3; ++m) {
      const int64_t rows = m < 2 ? I : H, k = m < 2 ? H : I;
      if (f == 0) {
        float* w = xmalloc(sizeof(float) * rows * k);
        synth_normal_f32(1, 10 + m, 0, rows * k, 0.02, w);
        ex[f].w[m] = keep[nk++] = w, ex[f].s[m] = NULL;
      } else if (f == 1) {
        uint16_t* w = xmalloc(2 * rows * k);
        synth_normal_bf16(1, 20 + m, 0, rows * k, 0.02, w);
        ex[f].w[m] = keep[nk++] = w, ex[f].s[m] = NULL;
      } else {
        uint8_t* c = xmalloc(rows * k / 2);
        void* s = xmalloc(2 * rows * k / 32);
        if (f == 2) synth_quant_mxfp4(1, 30 + m, rows, k, 0.02, c, s);
        else synth_quant_int4g32(1, 40 + m, rows, k, 0.02, c, s);
        ex[f].w[m] = keep[nk++] = c, ex[f].s[m] = keep[nk++] = s;
      }
      double* d = xmalloc(sizeof(double) * rows * k);
      oracle_decode(f, ex[f].w[m], ex[f].s[m], rows, k, d);
      free(d);
    }
  }
  double u[16];
  synth_uniform_f64(3, 3, 0, 16, u);
  uint16_t* x = xmalloc(2 * T * H);
  uint16_t* wg = xmalloc(2 * E * H);
  float bias[E];
  synth_normal_bf16(2, 1, 0, T * H, 1.0, x);
  synth_normal_bf16(2, 2, 0, E * H, 0.02, wg);
  for (int e = 0; e < E; ++e) bias[e] = (float)(-0.1 * e);
  double* xd = xmalloc(sizeof(double) * T * H);
  oracle_decode_act(1, x, T * H, xd);
  double lg[T * E], w[T * K], y[T * H], out[T * H], wo[T * K];
  int32_t ids[T * K], ids2[T * K], counts[E], offsets[E + 1], perm[T * K], inv[T * K];
  oracle_router_logits(1, x, wg, bias, T, H, E, lg);
  oracle_topk_gates(lg, T, E, K, ids, w);
  oracle_permute(ids, T, K, E, counts, offsets, perm, inv);
  for (int f = 0; f < 4; ++f) oracle_ffn(&ex[f], H, I, xd, T, y);
  oracle_expert bank[E];
  for (int e = 0; e < E; ++e) bank[e] = ex[1 + e % 3];
  int64_t sample[3] = {0, 2, 4};
  if (oracle_moe_layer(1, x, T, H, wg, bias, E, K, I, bank, &ex[1], I, sample, 3, out, ids2, wo) != 0) return 2;
  /* cache simulations */
  enum { G = 60, PER = 3 };
  int64_t off[G + 1], keys[G * PER], hits[G], misses[G], victims[G * PER], nv[G], ph;
  int32_t kinds[G];
  for (int g = 0; g <= G; ++g) off[g] = (int64_t)g * PER;
  for (int i = 0; i < G * PER; ++i) keys[i] = (i * 7 + i / 5) % 13;
  for (int g = 0; g < G; ++g) kinds[g] = g % 5 == 1 ? 1 : (g == 3 ? 2 : 0);
  if (oracle_lru(4, G, off, keys, hits, misses, victims, nv) != 0) return 3;
  if (oracle_lfu_decay(4, 3, G, off, keys, hits, misses, victims, nv) != 0) return 4;
  if (oracle_belady(4, G, off, keys, hits, misses) != 0) return 5;
  /* (group 3 pins three keys: 8 slots leave room for every demand group of three) */
  if (oracle_cache_sim(8, 0, 0, G, off, keys, kinds, hits, misses, victims, nv, &ph) != 0) return 6;
  if (oracle_cache_sim(8, 1, 4, G, off, keys, kinds, hits, misses, victims, nv, &ph) != 0) return 7;
  if (xw4_checks() != 0) return 8;
  for (int i = 0; i < nk; ++i) free(keep[i]);
  free(x);
  free(wg);
  free(xd);
  puts("oracle and generator: ok");
  return 0;
}
