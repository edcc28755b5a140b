/*
 * CPU oracle for the routed-expert MoE layer forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 C.  Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header, table or helper with the HIP library: it
 * has its own decoders for every weight format and its own LRU.
 *
 * What the layer computes, and where the pages say so:
 *  - A router scores every expert for every token and picks a few of them
 *    (Mixture of experts VRAM: total vs active parameters, section "How current
 *    MoE models route each token").  The pages name no scoring function; the
 *    reading taken here is softmax over the router logits (x . Wg_e + b_e),
 *    restricted to the top k and renormalised.
 *  - An expert is a gated FFN with gate, up and down projections whose gate
 *    branch goes through SiLU (pith.science verdict on FloE, arXiv 2505.05950:
 *    referee_report.summary and pith_extraction.core_discovery).  Reading:
 *    y = W_down (SiLU(W_gate x) * (W_up x)), SiLU(z) = z / (1 + e^-z), no biases.
 *  - Experts are stored at 4 bits (FP4 / INT4) but computed at higher precision
 *    (Mixture of experts VRAM..., "How current MoE models route each token",
 *    last paragraph).  Formats: OCP MXFP4 (E2M1 elements, E8M0 block scale, 32
 *    per block) and symmetric INT4 with one bf16 scale per 32 weights along K.
 *  - Tokens choosing the same expert are grouped so one weight read serves them
 *    all (Understanding MoE Inference Costs on Galactus, "Prompt processing is a
 *    different phase").  Reading: a stable grouping by expert id, tokens in
 *    ascending flat index t*k+j inside each expert.
 *  - Results are collected back per token (Mixture of experts VRAM..., "Expert
 *    parallelism on RTX PRO 6000 and H200 NVL", dispatch and combine).  Reading:
 *    out[t] = sum_j w[t,j] * y[t,j], plus the always-on shared expert with
 *    weight 1 where the model has one (same page, routing section).
 *  - A least-recently-used expert cache can serve most lookups (theflow.svmpsp.dev
 *    related-abstracts list, the router-locality study of Qwen3-235B); weights
 *    are addressed through stable logical slots while physical residency moves
 *    (What expert offloading actually costs, "Inside expert paging").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* activation / plain-weight element types */
enum { ODT_F32 = 0, ODT_BF16 = 1 };
/* expert weight formats */
enum { OFMT_F32 = 0, OFMT_BF16 = 1, OFMT_MXFP4 = 2, OFMT_INT4G32 = 3 };

typedef struct {
  int fmt;
  const void* w[3]; /* gate [I][H], up [I][H], down [H][I]; row-major, K contiguous */
  const void* s[3]; /* block scales [rows][K/32]; NULL for plain formats */
} oracle_expert;

/* ---------------------------------------------------------------- decoders */

static double f32_val(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* bfloat16 is the top half of an IEEE binary32 */
static double bf16_val(uint16_t h) { return f32_val((uint32_t)h << 16); }

/* OCP MXFP4 element: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit */
static double e2m1_val(unsigned code) {
  unsigned s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return s ? -mag : mag;
}

/* OCP E8M0 scale: 2^(x - 127); 0xFF is NaN */
static double e8m0_val(uint8_t x) { return x == 0xFF ? NAN : ldexp(1.0, (int)x - 127); }

/* two's-complement nibble */
static int int4_val(unsigned nib) { return (nib & 8) ? (int)nib - 16 : (int)nib; }

static unsigned nibble(const uint8_t* codes, int64_t K, int64_t r, int64_t k) {
  uint8_t b = codes[r * (K / 2) + k / 2];
  return (k & 1) ? (b >> 4) : (b & 15);
}

/* element (r, k) of a [rows][K] matrix stored in format fmt */
static double weight_at(int fmt, const void* w, const void* s, int64_t K, int64_t r, int64_t k) {
  switch (fmt) {
    case OFMT_F32: return f32_val(((const uint32_t*)w)[r * K + k]);
    case OFMT_BF16: return bf16_val(((const uint16_t*)w)[r * K + k]);
    case OFMT_MXFP4:
      return e2m1_val(nibble((const uint8_t*)w, K, r, k)) * e8m0_val(((const uint8_t*)s)[r * (K / 32) + k / 32]);
    case OFMT_INT4G32:
      return int4_val(nibble((const uint8_t*)w, K, r, k)) * bf16_val(((const uint16_t*)s)[r * (K / 32) + k / 32]);
  }
  return NAN;
}

static void decode_row(int fmt, const void* w, const void* s, int64_t K, int64_t r, double* out) {
  for (int64_t k = 0; k < K; ++k) out[k] = weight_at(fmt, w, s, K, r, k);
}

static double act_at(int dt, const void* x, int64_t i) {
  return dt == ODT_F32 ? f32_val(((const uint32_t*)x)[i]) : bf16_val(((const uint16_t*)x)[i]);
}

/* Decode a whole [rows][K] weight matrix to fp64 (the exact value of every weight). */
void oracle_decode(int fmt, const void* w, const void* s, int64_t rows, int64_t K, double* out) {
  for (int64_t r = 0; r < rows; ++r) decode_row(fmt, w, s, K, r, out + r * K);
}

void oracle_decode_act(int dt, const void* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = act_at(dt, x, i);
}

/* ------------------------------------------------------------------ router */

/* logits[t][e] = sum_h x[t][h] * Wg[e][h] + b[e], summed in order of h */
void oracle_router_logits(int dt, const void* x, const void* wg, const float* bias, int64_t T, int64_t H, int64_t E,
                          double* logits) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += act_at(dt, x, t * H + h) * act_at(dt, wg, e * H + h);
      logits[t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
    }
  }
}

typedef struct {
  double v;
  int32_t e;
} scored;

/* larger logit first; equal logits: lower expert id first */
static int by_score(const void* a, const void* b) {
  const scored *x = (const scored*)a, *y = (const scored*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->e > y->e) - (x->e < y->e);
}

/*
 * Top-k by a full sort of the E experts, then the gate weights: softmax over the
 * k chosen logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), which equals the
 * softmax over all E logits renormalised over the chosen k.
 */
void oracle_topk_gates(const double* logits, int64_t T, int64_t E, int k, int32_t* ids, double* w) {
#pragma omp parallel
  {
    scored* s = (scored*)malloc(sizeof(scored) * (size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t e = 0; e < E; ++e) {
        s[e].v = logits[t * E + e];
        s[e].e = (int32_t)e;
      }
      qsort(s, (size_t)E, sizeof(scored), by_score);
      double z = 0.0;
      for (int j = 0; j < k; ++j) z += exp(s[j].v - s[0].v);
      for (int j = 0; j < k; ++j) {
        ids[t * k + j] = s[j].e;
        w[t * k + j] = exp(s[j].v - s[0].v) / z;
      }
    }
    free(s);
  }
}

/* ------------------------------------------------------------- permutation */

typedef struct {
  int32_t e, i;
} tagged;

static int by_expert_then_index(const void* a, const void* b) {
  const tagged *x = (const tagged*)a, *y = (const tagged*)b;
  if (x->e != y->e) return (x->e > y->e) - (x->e < y->e);
  return (x->i > y->i) - (x->i < y->i);
}

/*
 * Group the T*k (token, slot) pairs by expert: perm_src lists the flat indices
 * t*k+j sorted by (expert id, flat index) -- a stable sort by expert --
 * counts[e] is the group size, offsets its exclusive prefix sum (E+1 entries),
 * inv_perm the position of each flat index in perm_src.
 */
void oracle_permute(const int32_t* ids, int64_t T, int k, int64_t E, int32_t* counts, int32_t* offsets,
                    int32_t* perm_src, int32_t* inv_perm) {
  int64_t n = T * k;
  tagged* a = (tagged*)malloc(sizeof(tagged) * (size_t)(n ? n : 1));
  for (int64_t i = 0; i < n; ++i) {
    a[i].e = ids[i];
    a[i].i = (int32_t)i;
  }
  qsort(a, (size_t)n, sizeof(tagged), by_expert_then_index);
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n; ++i) counts[ids[i]]++;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int64_t p = 0; p < n; ++p) {
    perm_src[p] = a[p].i;
    inv_perm[a[p].i] = (int32_t)p;
  }
  free(a);
}

/* ---------------------------------------------------------------- expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * y[r] = W_down (SiLU(W_gate x[r]) * (W_up x[r])) for n rows x[r] of length H,
 * one expert with intermediate size I.  Every dot product is a sequential fp64
 * sum over the contraction index.
 */
void oracle_ffn(const oracle_expert* ex, int64_t H, int64_t I, const double* x, int64_t n, double* y) {
  double* h = (double*)malloc(sizeof(double) * (size_t)(n * I + 1));
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)H);
    double* u = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
      decode_row(ex->fmt, ex->w[0], ex->s[0], H, i, g);
      decode_row(ex->fmt, ex->w[1], ex->s[1], H, i, u);
      for (int64_t r = 0; r < n; ++r) {
        double ag = 0.0, au = 0.0;
        for (int64_t c = 0; c < H; ++c) {
          ag += g[c] * x[r * H + c];
          au += u[c] * x[r * H + c];
        }
        h[r * I + i] = silu(ag) * au;
      }
    }
    free(g);
    free(u);
    double* d = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(static)
    for (int64_t o = 0; o < H; ++o) {
      decode_row(ex->fmt, ex->w[2], ex->s[2], I, o, d);
      for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i) acc += d[i] * h[r * I + i];
        y[r * H + o] = acc;
      }
    }
    free(d);
  }
  free(h);
}

/* ------------------------------------------------------------- whole layer */

/*
 * Layer output for the tokens listed in sample[0..n_sample):
 *   out[s] = sum_{j<k} w[t,j] * FFN_{ids[t,j]}(x[t]) (+ FFN_shared(x[t])),   t = sample[s]
 * with routing from oracle_router_logits + oracle_topk_gates.  Routing is per
 * token, so a sample of tokens gives exactly those tokens' outputs.  Expert
 * outputs are summed in slot order j = 0..k-1, then the shared expert.
 * ids_out [n_sample][k] and w_out [n_sample][k] receive the routing.
 * experts: E descriptors (any format); shared: NULL or one descriptor, inter I_sh.
 */
int oracle_moe_layer(int dt, const void* x, int64_t T, int64_t H, const void* wg, const float* bias, int64_t E, int k,
                     int64_t I, const oracle_expert* experts, const oracle_expert* shared, int64_t I_sh,
                     const int64_t* sample, int64_t n_sample, double* out, int32_t* ids_out, double* w_out) {
  (void)T;
  double* xs = (double*)malloc(sizeof(double) * (size_t)(n_sample * H + 1));
  double* lg = (double*)malloc(sizeof(double) * (size_t)(n_sample * E + 1));
  for (int64_t s = 0; s < n_sample; ++s)
    for (int64_t c = 0; c < H; ++c) xs[s * H + c] = act_at(dt, x, sample[s] * H + c);
  /* router on the sampled rows: same sum as oracle_router_logits */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < n_sample; ++s) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t c = 0; c < H; ++c) acc += xs[s * H + c] * act_at(dt, wg, e * H + c);
      lg[s * E + e] = acc + (bias ? (double)bias[e] : 0.0);
    }
  }
  oracle_topk_gates(lg, n_sample, E, k, ids_out, w_out);

  /* y[s][j] = FFN of expert ids[s][j] at x[sample[s]]; each expert evaluated once on its rows */
  double* y = (double*)malloc(sizeof(double) * (size_t)(n_sample * k * H + 1));
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_sample * k + 1));
  double* xin = (double*)malloc(sizeof(double) * (size_t)(n_sample * k * H + 1));
  double* yout = (double*)malloc(sizeof(double) * (size_t)(n_sample * k * H + 1));
  for (int64_t e = 0; e < E; ++e) {
    int64_t n = 0;
    for (int64_t q = 0; q < n_sample * k; ++q)
      if (ids_out[q] == e) rows[n++] = q;
    if (!n) continue;
    for (int64_t r = 0; r < n; ++r) memcpy(xin + r * H, xs + (rows[r] / k) * H, sizeof(double) * (size_t)H);
    oracle_ffn(&experts[e], H, I, xin, n, yout);
    for (int64_t r = 0; r < n; ++r) memcpy(y + rows[r] * H, yout + r * H, sizeof(double) * (size_t)H);
  }
  double* ysh = NULL;
  if (shared) {
    ysh = (double*)malloc(sizeof(double) * (size_t)(n_sample * H + 1));
    oracle_ffn(shared, H, I_sh, xs, n_sample, ysh);
  }
  for (int64_t s = 0; s < n_sample; ++s) {
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += w_out[s * k + j] * y[(s * k + j) * H + c];
      if (ysh) acc += ysh[s * H + c];
      out[s * H + c] = acc;
    }
  }
  free(xs);
  free(lg);
  free(y);
  free(rows);
  free(xin);
  free(yout);
  free(ysh);
  return 0;
}

/* -------------------------------------------------------------- expert cache */

/*
 * Least-recently-used cache over keys (layer * E + expert) with `capacity`
 * slots, starting empty.  Lookups come in groups (one group = one layer of one
 * decode step); inside a group duplicate keys count once.  A distinct key found
 * resident is a hit, otherwise a miss that takes a free slot or evicts.  Every
 * key touched by a group gets that group's index as its recency tick; the
 * victim is the resident key, not in the current group, with the smallest
 * (tick, key).  A group with more distinct keys than the capacity is an error
 * (returns -1).
 * group_off[g]..group_off[g+1] delimit the raw keys of group g.
 * Outputs per group: hits[g], misses[g]; victims (in eviction order) go to
 * victims[], their count per group to n_victims[g].
 */
int oracle_lru(int64_t capacity, int64_t n_groups, const int64_t* group_off, const int64_t* keys, int64_t* hits,
               int64_t* misses, int64_t* victims, int64_t* n_victims) {
  int64_t max_key = 0;
  for (int64_t i = 0; i < group_off[n_groups]; ++i)
    if (keys[i] > max_key) max_key = keys[i];
  int64_t nk = max_key + 1;
  int64_t* tick = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk); /* -1 = not resident */
  int64_t* in_group = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  for (int64_t i = 0; i < nk; ++i) tick[i] = -1, in_group[i] = -1;
  int64_t resident = 0, nv = 0, rc = 0;
  for (int64_t g = 0; g < n_groups && rc == 0; ++g) {
    int64_t distinct = 0;
    for (int64_t i = group_off[g]; i < group_off[g + 1]; ++i)
      if (in_group[keys[i]] != g) in_group[keys[i]] = g, distinct++;
    if (distinct > capacity) {
      rc = -1;
      break;
    }
    hits[g] = misses[g] = n_victims[g] = 0;
    /* visit the group's distinct keys in ascending order */
    for (int64_t key = 0; key < nk; ++key) {
      if (in_group[key] != g) continue;
      if (tick[key] >= 0) {
        hits[g]++;
      } else {
        misses[g]++;
        if (resident == capacity) {
          int64_t best = -1;
          for (int64_t c = 0; c < nk; ++c) {
            if (tick[c] < 0 || in_group[c] == g) continue;
            if (best < 0 || tick[c] < tick[best] || (tick[c] == tick[best] && c < best)) best = c;
          }
          tick[best] = -1;
          resident--;
          victims[nv++] = best;
          n_victims[g]++;
        }
        resident++;
      }
      tick[key] = g;
    }
  }
  free(tick);
  free(in_group);
  return (int)rc;
}

/*
 * Frequency with decay, over the same groups: every key carries a use count.  At the start
 * of group g (g > 0, period > 0, g multiple of period) every count is halved (integer
 * shift); then each distinct key of the group gains 1024.  A miss with a full cache evicts
 * the resident key not in the current group with the smallest count, then the oldest last
 * use, then the smallest key.  Keys of a group are visited in ascending order; a key's last
 * use becomes g when it is visited.  Outputs as oracle_lru.
 */
int oracle_lfu_decay(int64_t capacity, int64_t period, int64_t n_groups, const int64_t* group_off,
                     const int64_t* keys, int64_t* hits, int64_t* misses, int64_t* victims, int64_t* n_victims) {
  int64_t max_key = 0;
  for (int64_t i = 0; i < group_off[n_groups]; ++i)
    if (keys[i] > max_key) max_key = keys[i];
  int64_t nk = max_key + 1;
  int64_t* last = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);     /* last use, -1 = never */
  int64_t* count = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  char* res = (char*)malloc((size_t)nk);                                 /* resident? */
  int64_t* in_group = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  for (int64_t i = 0; i < nk; ++i) last[i] = -1, count[i] = 0, res[i] = 0, in_group[i] = -1;
  int64_t resident = 0, nv = 0, rc = 0;
  for (int64_t g = 0; g < n_groups && rc == 0; ++g) {
    int64_t distinct = 0;
    for (int64_t i = group_off[g]; i < group_off[g + 1]; ++i)
      if (in_group[keys[i]] != g) in_group[keys[i]] = g, distinct++;
    if (distinct > capacity) {
      rc = -1;
      break;
    }
    if (period > 0 && g > 0 && g % period == 0)
      for (int64_t k = 0; k < nk; ++k) count[k] /= 2; /* counts are non-negative: a shift */
    for (int64_t k = 0; k < nk; ++k)
      if (in_group[k] == g) count[k] += 1024;
    hits[g] = misses[g] = n_victims[g] = 0;
    for (int64_t key = 0; key < nk; ++key) {
      if (in_group[key] != g) continue;
      if (res[key]) {
        hits[g]++;
      } else {
        misses[g]++;
        if (resident == capacity) {
          int64_t best = -1;
          for (int64_t c = 0; c < nk; ++c) {
            if (!res[c] || in_group[c] == g) continue;
            if (best < 0 || count[c] < count[best] || (count[c] == count[best] && last[c] < last[best]) ||
                (count[c] == count[best] && last[c] == last[best] && c < best))
              best = c;
          }
          res[best] = 0;
          resident--;
          victims[nv++] = best;
          n_victims[g]++;
        }
        res[key] = 1;
        resident++;
      }
      last[key] = g;
    }
  }
  free(last);
  free(count);
  free(res);
  free(in_group);
  return (int)rc;
}

/*
 * Belady's MIN on the same groups: on a miss with a full cache, evict the
 * resident key (not in the current group) whose next use lies farthest ahead
 * (never = infinitely far; ties: smallest key).  Gives the largest hit count
 * any policy can reach; used only as a bound.
 */
int oracle_belady(int64_t capacity, int64_t n_groups, const int64_t* group_off, const int64_t* keys, int64_t* hits,
                  int64_t* misses) {
  int64_t n = group_off[n_groups], max_key = 0;
  for (int64_t i = 0; i < n; ++i)
    if (keys[i] > max_key) max_key = keys[i];
  int64_t nk = max_key + 1;
  /* nu[i]: index of the first group after the one holding position i that uses keys[i] */
  int64_t* nu = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int64_t* last = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  for (int64_t c = 0; c < nk; ++c) last[c] = INT64_MAX;
  for (int64_t g = n_groups - 1; g >= 0; --g) {
    for (int64_t i = group_off[g]; i < group_off[g + 1]; ++i) nu[i] = last[keys[i]];
    for (int64_t i = group_off[g]; i < group_off[g + 1]; ++i) last[keys[i]] = g;
  }
  char* res = (char*)calloc((size_t)nk, 1);
  int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  int64_t* in_group = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  for (int64_t c = 0; c < nk; ++c) in_group[c] = -1, next[c] = INT64_MAX;
  int64_t resident = 0, rc = 0;
  for (int64_t g = 0; g < n_groups; ++g) {
    int64_t distinct = 0;
    for (int64_t i = group_off[g]; i < group_off[g + 1]; ++i)
      if (in_group[keys[i]] != g) in_group[keys[i]] = g, pos[keys[i]] = i, distinct++;
    if (distinct > capacity) {
      rc = -1;
      break;
    }
    hits[g] = misses[g] = 0;
    for (int64_t key = 0; key < nk; ++key) {
      if (in_group[key] != g) continue;
      if (res[key]) {
        hits[g]++;
      } else {
        misses[g]++;
        if (resident == capacity) {
          int64_t best = -1;
          for (int64_t c = 0; c < nk; ++c) {
            if (!res[c] || in_group[c] == g) continue;
            if (best < 0 || next[c] > next[best]) best = c;
          }
          res[best] = 0;
          resident--;
        }
        res[key] = 1;
        resident++;
      }
      next[key] = nu[pos[key]];
    }
  }
  free(nu);
  free(last);
  free(res);
  free(next);
  free(in_group);
  free(pos);
  return (int)rc;
}

/*
 * The cache with fetching ahead and pinning (the planner's moe_cache_prefetch and
 * moe_cache_pin), groups of three kinds over the same keys:
 *  kind 0, a demand lookup: as oracle_lru (policy 0) or oracle_lfu_decay (policy 1, counts halved
 *    every `period` demand groups), counting demand groups only for ticks and decay, and pinned
 *    keys are never victims.  A group whose absent keys outnumber the free slots plus the
 *    evictable keys outside the group is an error.
 *  kind 1, a prefetch: the group's absent keys, ascending, each take a free slot or evict the
 *    policy's first victim among the keys that are neither pinned, nor in this group, nor in the
 *    latest demand group; when none is left the rest of the group is skipped.  A key brought in
 *    this way has last use -1 (its count unchanged) until a demand group uses it.
 *  kind 2, a pin: as a prefetch, but every key of the group is pinned from then on, and a group
 *    that does not fit is an error.
 * Outputs per group: hits (keys already resident), misses (keys fetched), victims as oracle_lru;
 * *prefetch_hits counts demand hits on keys a prefetch brought in and no demand group used since.
 * Returns -1 on an error (the group that does not fit), else 0.
 */
int oracle_cache_sim(int64_t capacity, int policy, int64_t period, int64_t n_groups, const int64_t* group_off,
                     const int64_t* keys, const int32_t* kinds, int64_t* hits, int64_t* misses, int64_t* victims,
                     int64_t* n_victims, int64_t* prefetch_hits) {
  int64_t max_key = 0;
  for (int64_t i = 0; i < group_off[n_groups]; ++i)
    if (keys[i] > max_key) max_key = keys[i];
  const int64_t nk = max_key + 1;
  char* res = (char*)calloc((size_t)nk, 1);
  char* pin = (char*)calloc((size_t)nk, 1);
  char* fresh = (char*)calloc((size_t)nk, 1);
  int64_t* last = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  int64_t* count = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);
  int64_t* mark = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);    /* group index of the latest group naming the key */
  int64_t* dmark = (int64_t*)malloc(sizeof(int64_t) * (size_t)nk);   /* demand tick + 1 of the latest demand group naming it */
  for (int64_t i = 0; i < nk; ++i) last[i] = -1, count[i] = 0, mark[i] = -1, dmark[i] = 0;
  int64_t resident = 0, nv = 0, tick = 0, cur_dmark = 0, rc = 0;
  *prefetch_hits = 0;
  for (int64_t g = 0; g < n_groups && rc == 0; ++g) {
    for (int64_t i = group_off[g]; i < group_off[g + 1]; ++i) mark[keys[i]] = g;
    const int kind = kinds[g];
    hits[g] = misses[g] = n_victims[g] = 0;
    /* may key c be evicted by group g? */
#define EVICTABLE(c) (res[c] && !pin[c] && mark[c] != g && (kind == 0 || dmark[c] != cur_dmark || cur_dmark == 0))
    if (kind != 1) { /* demand and pin groups must fit */
      int64_t absent = 0, evictable = 0;
      for (int64_t c = 0; c < nk; ++c) {
        if (mark[c] == g && !res[c]) absent++;
        if (EVICTABLE(c)) evictable++;
      }
      if (absent > capacity - resident + evictable) {
        rc = -1;
        break;
      }
    }
    if (kind == 0 && policy == 1) {
      if (period > 0 && tick > 0 && tick % period == 0)
        for (int64_t c = 0; c < nk; ++c) count[c] /= 2;
      for (int64_t c = 0; c < nk; ++c)
        if (mark[c] == g) count[c] += 1024;
    }
    for (int64_t key = 0; key < nk; ++key) {
      if (mark[key] != g) continue;
      if (res[key]) {
        hits[g]++;
        if (kind == 0 && fresh[key]) (*prefetch_hits)++, fresh[key] = 0;
      } else {
        if (resident == capacity) {
          int64_t best = -1;
          for (int64_t c = 0; c < nk; ++c) {
            if (!EVICTABLE(c)) continue;
            const int64_t pc = policy == 1 ? count[c] : 0, pb = best < 0 ? 0 : (policy == 1 ? count[best] : 0);
            if (best < 0 || pc < pb || (pc == pb && last[c] < last[best]) || (pc == pb && last[c] == last[best] && c < best))
              best = c;
          }
          if (best < 0) break; /* only a prefetch gets here: skip the rest of the group */
          res[best] = 0, fresh[best] = 0;
          resident--;
          victims[nv++] = best;
          n_victims[g]++;
        }
        res[key] = 1;
        resident++;
        misses[g]++;
        if (kind == 1) last[key] = -1, fresh[key] = 1;
      }
      if (kind == 0) last[key] = tick, fresh[key] = 0;
      if (kind == 2) pin[key] = 1, fresh[key] = 0;
    }
#undef EVICTABLE
    if (kind == 0) {
      for (int64_t c = 0; c < nk; ++c)
        if (mark[c] == g) dmark[c] = tick + 1;
      cur_dmark = tick + 1;
      tick++;
    }
  }
  free(res);
  free(pin);
  free(fresh);
  free(last);
  free(count);
  free(mark);
  free(dmark);
  return (int)rc;
}

/* ------------------------------------------------------------------------------------------
 * Lossless compression of bf16 expert packages.  The pages place a tier of losslessly
 * compressed experts in GPU memory beside the host tier, lossless so that no output bit
 * changes (What expert offloading actually costs, "Inside expert paging"); they name no codec.
 * Reading: an exponent-window code, from this definition:
 *
 *  - The package is read as little-endian bf16 values in chunks of 512 (1024 bytes; the package
 *    size must be a multiple of 1024).  Value v has sign s = v >> 15, exponent field
 *    e = (v >> 7) & 255 and mantissa m = v & 127.
 *  - Chunk window: M = the largest e in the chunk, base b = M - 14 (0 if M < 14); e is in the
 *    window when b <= e <= b + 14, with code c = e - b + 1 (1..15); any other e is an escape,
 *    code 0.
 *  - Coded chunk: 512 bytes s << 7 | m (value order), 256 bytes of codes (byte t holds value
 *    2t's code in its low nibble, value 2t+1's in its high nibble), then the e of each escaped
 *    value in value order, zero-padded to a multiple of 16.  Its size is 768 + 16 ceil(n_esc/16).
 *    A chunk whose coded size would be 1024 or more is stored raw (its 1024 bytes as they are).
 *  - Blob: a 64-byte header (u32 magic 0x31345758, u32 chunk count n, u64 package bytes, u64
 *    data offset, u64 blob bytes, zeros), u32 chunk offsets off[0..n] (relative to the data
 *    offset, off[0] = 0), u8 window bases (0 for raw chunks), zeros up to the data offset (the
 *    smallest multiple of 256 past the tables), then the chunks back to back.  A chunk of
 *    off[i+1] - off[i] = 1024 bytes is raw.
 * ------------------------------------------------------------------------------------------ */
#define XW4_MAGIC 0x31345758u

static void le_put(uint8_t* p, uint64_t v, int bytes) {
  for (int i = 0; i < bytes; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
static uint64_t le_get(const uint8_t* p, int bytes) {
  uint64_t v = 0;
  for (int i = 0; i < bytes; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}
static int64_t xw4_data_offset(int64_t n) { return (64 + 4 * (n + 1) + n + 255) / 256 * 256; }

int64_t oracle_xw4_bound(int64_t raw_bytes) {
  if (raw_bytes < 0 || raw_bytes % 1024) return -1;
  return xw4_data_offset(raw_bytes / 1024) + raw_bytes;
}

/* Returns the blob's size, or -1 (size not a multiple of 1024, or cap too small). */
int64_t oracle_xw4_encode(const uint8_t* raw, int64_t raw_bytes, uint8_t* out, int64_t cap) {
  if (raw_bytes < 0 || raw_bytes % 1024 || cap < oracle_xw4_bound(raw_bytes)) return -1;
  const int64_t n = raw_bytes / 1024, data = xw4_data_offset(n);
  memset(out, 0, (size_t)data);
  int64_t pos = 0;
  for (int64_t i = 0; i < n; ++i) {
    const uint8_t* src = raw + 1024 * i;
    uint8_t* dst = out + data + pos;
    int e[512], M = 0, n_esc = 0;
    for (int j = 0; j < 512; ++j) {
      const unsigned v = (unsigned)le_get(src + 2 * j, 2);
      e[j] = (int)((v >> 7) & 255);
      if (e[j] > M) M = e[j];
    }
    const int b = M < 14 ? 0 : M - 14;
    for (int j = 0; j < 512; ++j)
      if (e[j] < b || e[j] > b + 14) n_esc++;
    const int coded = 768 + 16 * ((n_esc + 15) / 16);
    if (coded >= 1024) {
      memcpy(dst, src, 1024);
      out[64 + 4 * (n + 1) + i] = 0;
      pos += 1024;
    } else {
      memset(dst, 0, (size_t)coded);
      int k = 0;
      for (int j = 0; j < 512; ++j) {
        const unsigned v = (unsigned)le_get(src + 2 * j, 2);
        dst[j] = (uint8_t)(((v >> 15) << 7) | (v & 127));
        const int in = e[j] >= b && e[j] <= b + 14;
        const unsigned c = in ? (unsigned)(e[j] - b + 1) : 0u;
        dst[512 + j / 2] |= (uint8_t)(c << (4 * (j % 2)));
        if (!in) dst[768 + k++] = (uint8_t)e[j];
      }
      out[64 + 4 * (n + 1) + i] = (uint8_t)b;
      pos += coded;
    }
    le_put(out + 64 + 4 * (i + 1), (uint64_t)pos, 4);
  }
  le_put(out, XW4_MAGIC, 4);
  le_put(out + 4, (uint64_t)n, 4);
  le_put(out + 8, (uint64_t)raw_bytes, 8);
  le_put(out + 16, (uint64_t)data, 8);
  le_put(out + 24, (uint64_t)(data + pos), 8);
  return data + pos;
}

/* Decodes a blob into raw_bytes bytes; returns 0, or -1 if the blob is not a well-formed
 * encoding of a package of that size. */
int oracle_xw4_decode(const uint8_t* blob, int64_t blob_bytes, uint8_t* raw, int64_t raw_bytes) {
  if (blob_bytes < 64 || raw_bytes < 0 || raw_bytes % 1024) return -1;
  const int64_t n = raw_bytes / 1024, data = xw4_data_offset(n);
  if (le_get(blob, 4) != XW4_MAGIC || (int64_t)le_get(blob + 4, 4) != n || (int64_t)le_get(blob + 8, 8) != raw_bytes ||
      (int64_t)le_get(blob + 16, 8) != data || blob_bytes < data)
    return -1;
  const int64_t total = (int64_t)le_get(blob + 24, 8);
  if (total > blob_bytes || le_get(blob + 64, 4) != 0 || data + (int64_t)le_get(blob + 64 + 4 * n, 4) != total) return -1;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t o0 = (int64_t)le_get(blob + 64 + 4 * i, 4), o1 = (int64_t)le_get(blob + 64 + 4 * (i + 1), 4);
    if (o1 < o0 || data + o1 > total) return -1; /* chunks lie in order inside the blob */
    const int64_t size = o1 - o0;
    const uint8_t* src = blob + data + o0;
    uint8_t* dst = raw + 1024 * i;
    if (size == 1024) {
      memcpy(dst, src, 1024);
      continue;
    }
    if (size < 768 || size > 1008 || size % 16) return -1;
    const int b = blob[64 + 4 * (n + 1) + i];
    int k = 0;
    for (int j = 0; j < 512; ++j) {
      const unsigned c = (src[512 + j / 2] >> (4 * (j % 2))) & 15u;
      unsigned ex;
      if (c) {
        ex = (unsigned)(b + (int)c - 1);
      } else {
        if (768 + k >= size) return -1;
        ex = src[768 + k++];
      }
      if (ex > 255) return -1;
      const unsigned v = ((unsigned)(src[j] >> 7) << 15) | (ex << 7) | (src[j] & 127u);
      le_put(dst + 2 * j, v, 2);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Lossless compression of any package (4-bit ones included): an order-0 range-asymmetric-numeral-
 * system (rANS) code of its bytes, from this definition (the pages name no codec; see the
 * exponent-window code above for the lossless tier they describe):
 *
 *  - The package of n bytes is cut at byte q into two regions (the codes, then the scales); each
 *    region is coded on its own.
 *  - Region model: h[s] = occurrences of byte s; f[s] = max(1, floor(4096 h[s] / m)) for every
 *    present s (m the region's length), 0 otherwise; while the f sum to more than 4096 the largest
 *    f (smallest s among equals) loses one, while they sum to less the largest gains the rest.
 *    c[s] = f[0] + ... + f[s-1].
 *  - Streams: region byte j belongs to stream j mod S (S = 32768), as its (j div S)-th symbol.  A
 *    stream is coded from x = 2^16, last symbol first: before a symbol s, if x >= 2^20 f[s] a word
 *    (the low 16 bits of x) is emitted and x shifts right by 16; then
 *    x = 4096 (x div f[s]) + (x mod f[s]) + c[s].  The final x is the stream's state.  Decoding: the
 *    symbol is the s with c[s] <= x mod 4096 < c[s] + f[s], then x = f[s] (x div 4096) +
 *    (x mod 4096) - c[s], and if x < 2^16, x = 2^16 x + the next word.  Decoding a whole stream
 *    returns x to 2^16.
 *  - Words: streams 64g .. 64g+63 form group g and share one word sequence, in decoding order: for
 *    each symbol index j ascending, the words the group's streams read after their j-th symbol, in
 *    stream order.  (So the coder runs the group's streams in step, j descending and streams in
 *    descending order, and stores the emitted words reversed.)
 *  - Blob: a 64-byte header (u32 magic 0x31534E52, u32 S, u64 n, u64 q, u64 blob bytes, zeros),
 *    then per region (region 0 first): u16 f[256], u32 states[S], u32 word offsets off[0..S/64]
 *    (group g's words are words off[g] .. off[g+1]-1 of the region), the u16 words, zeros up to a
 *    multiple of 16 bytes.
 * ------------------------------------------------------------------------------------------ */
#define RNS_MAGIC 0x31534E52u
#define RNS_S 32768

static void rns_model(const uint8_t* r, int64_t m, uint32_t* f) {
  int64_t h[256] = {0};
  for (int64_t j = 0; j < m; ++j) h[r[j]]++;
  int64_t sum = 0;
  for (int s = 0; s < 256; ++s) {
    f[s] = 0;
    if (h[s]) {
      const int64_t v = (int64_t)(h[s] * 4096 / m);
      f[s] = (uint32_t)(v < 1 ? 1 : v);
    }
    sum += f[s];
  }
  while (m > 0 && sum != 4096) {
    int best = 0;
    for (int s = 1; s < 256; ++s)
      if (f[s] > f[best]) best = s;
    if (sum > 4096) {
      f[best] -= 1;
      sum -= 1;
    } else {
      f[best] += (uint32_t)(4096 - sum);
      sum = 4096;
    }
  }
}

#define RNS_G (RNS_S / 64)
static int64_t rns_region_bound(int64_t m) { return 512 + 4 * RNS_S + 4 * (RNS_G + 1) + 2 * (m + 2 * RNS_S) + 16; }

int64_t oracle_rns_bound(int64_t n) { return 64 + rns_region_bound(n) * 2; }

static int64_t rns_count(int64_t m, int64_t i) { return i < m ? (m - i + RNS_S - 1) / RNS_S : 0; }

/* codes region r (m bytes) at out; returns its bytes (a multiple of 16) */
static int64_t rns_encode_region(const uint8_t* r, int64_t m, uint8_t* out) {
  uint32_t f[256], c[256];
  rns_model(r, m, f);
  c[0] = 0;
  for (int s = 1; s < 256; ++s) c[s] = c[s - 1] + f[s - 1];
  for (int s = 0; s < 256; ++s) le_put(out + 2 * s, f[s], 2);
  uint8_t* states = out + 512;
  uint8_t* offs = states + 4 * RNS_S;
  uint8_t* words = offs + 4 * (RNS_G + 1);
  uint16_t* tmp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(64 * (m / RNS_S + 2)));
  int64_t w = 0;
  for (int g = 0; g < RNS_G; ++g) {
    le_put(offs + 4 * g, (uint64_t)w, 4);
    uint64_t x[64];
    for (int l = 0; l < 64; ++l) x[l] = 1u << 16;
    int64_t nw = 0;
    for (int64_t j = rns_count(m, 64 * g) - 1; j >= 0; --j) {
      for (int l = 63; l >= 0; --l) {
        const int64_t i = 64 * g + l;
        if (j >= rns_count(m, i)) continue;
        const uint8_t s = r[i + j * RNS_S];
        if (x[l] >= ((uint64_t)f[s] << 20)) {
          tmp[nw++] = (uint16_t)(x[l] & 0xFFFF);
          x[l] >>= 16;
        }
        x[l] = (x[l] / f[s]) * 4096 + (x[l] % f[s]) + c[s];
      }
    }
    for (int l = 0; l < 64; ++l) le_put(states + 4 * (64 * g + l), x[l], 4);
    for (int64_t k = 0; k < nw; ++k) le_put(words + 2 * (w + k), tmp[nw - 1 - k], 2);
    w += nw;
  }
  le_put(offs + 4 * RNS_G, (uint64_t)w, 4);
  free(tmp);
  int64_t bytes = 512 + 4 * RNS_S + 4 * (RNS_G + 1) + 2 * w;
  const int64_t padded = (bytes + 15) / 16 * 16;
  memset(out + bytes, 0, (size_t)(padded - bytes));
  return padded;
}

/* Returns the blob's size, or -1 (q > n, or cap too small). */
int64_t oracle_rns_encode(const uint8_t* raw, int64_t n, int64_t q, uint8_t* out, int64_t cap) {
  if (n < 0 || q < 0 || q > n || cap < oracle_rns_bound(n)) return -1;
  memset(out, 0, 64);
  int64_t pos = 64;
  pos += rns_encode_region(raw, q, out + pos);
  pos += rns_encode_region(raw + q, n - q, out + pos);
  le_put(out, RNS_MAGIC, 4);
  le_put(out + 4, RNS_S, 4);
  le_put(out + 8, (uint64_t)n, 8);
  le_put(out + 16, (uint64_t)q, 8);
  le_put(out + 24, (uint64_t)pos, 8);
  return pos;
}

/* decodes region r (m bytes) from its section at in (avail bytes); returns the section's bytes or -1 */
static int64_t rns_decode_region(const uint8_t* in, int64_t avail, uint8_t* r, int64_t m) {
  const int64_t head = 512 + 4 * RNS_S + 4 * (RNS_G + 1);
  if (avail < head) return -1;
  uint32_t f[256], c[256];
  int64_t sum = 0;
  for (int s = 0; s < 256; ++s) f[s] = (uint32_t)le_get(in + 2 * s, 2), sum += f[s];
  if (m > 0 && sum != 4096) return -1;
  c[0] = 0;
  for (int s = 1; s < 256; ++s) c[s] = c[s - 1] + f[s - 1];
  const uint8_t* states = in + 512;
  const uint8_t* offs = states + 4 * RNS_S;
  const uint8_t* words = offs + 4 * (RNS_G + 1);
  const int64_t total_w = (int64_t)le_get(offs + 4 * RNS_G, 4);
  if (head + 2 * total_w > avail) return -1;
  for (int g = 0; g < RNS_G; ++g) {
    int64_t k = (int64_t)le_get(offs + 4 * g, 4);
    const int64_t kend = (int64_t)le_get(offs + 4 * (g + 1), 4);
    if (k > kend || kend > total_w) return -1;
    uint64_t x[64];
    for (int l = 0; l < 64; ++l) x[l] = le_get(states + 4 * (64 * g + l), 4);
    for (int64_t j = 0; j < rns_count(m, 64 * g); ++j) {
      for (int l = 0; l < 64; ++l) {
        const int64_t i = 64 * g + l;
        if (j >= rns_count(m, i)) continue;
        const uint32_t slot = (uint32_t)(x[l] & 4095);
        int s = 0;
        while (s < 255 && !(c[s] <= slot && slot < c[s] + f[s])) ++s;
        if (!(c[s] <= slot && slot < c[s] + f[s])) return -1;
        r[i + j * RNS_S] = (uint8_t)s;
        x[l] = (uint64_t)f[s] * (x[l] >> 12) + slot - c[s];
      }
      for (int l = 0; l < 64; ++l) {
        if (j >= rns_count(m, 64 * g + l) || x[l] >= (1u << 16)) continue;
        if (k >= kend) return -1;
        x[l] = (x[l] << 16) | le_get(words + 2 * k, 2);
        ++k;
      }
    }
    for (int l = 0; l < 64; ++l)
      if (x[l] != (1u << 16)) return -1;
    if (k != kend) return -1;
  }
  return (head + 2 * total_w + 15) / 16 * 16;
}

/* Decodes a blob into n bytes; 0, or -1 if the blob is not a well-formed encoding of n bytes. */
int oracle_rns_decode(const uint8_t* blob, int64_t blob_bytes, uint8_t* raw, int64_t n) {
  if (blob_bytes < 64 || le_get(blob, 4) != RNS_MAGIC || le_get(blob + 4, 4) != RNS_S ||
      (int64_t)le_get(blob + 8, 8) != n)
    return -1;
  const int64_t q = (int64_t)le_get(blob + 16, 8), total = (int64_t)le_get(blob + 24, 8);
  if (q < 0 || q > n || total > blob_bytes) return -1;
  const int64_t a = rns_decode_region(blob + 64, total - 64, raw, q);
  if (a < 0) return -1;
  const int64_t b = rns_decode_region(blob + 64 + a, total - 64 - a, raw + q, n - q);
  if (b < 0 || 64 + a + b != total) return -1;
  return 0;
}
