/*
 * oracle.c -- plain CPU oracle of the IndexPool sparse-attention path.
 * TEST INFRASTRUCTURE ONLY (see oracle.h for the sources and the rules).
 *
 * Each step is the definition written out, in the pages' order: pool, quantise,
 * score, select, attend.  No blocking, fusion or reordering beyond that.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Pooled value of group g, channel d ([WIKI] IndexPool: k_pool = sum_i w_i k_i,
 * the w_i summing to 1).  A last group with r < 4 tokens uses its r weights
 * divided by their sum, so that its weights also sum to 1. */
static double pooled_value(const uint16_t* keys, int64_t L, const double* w, int64_t g, int d) {
  int64_t first = g * OR_GROUP;
  int64_t r = L - first;
  if (r > OR_GROUP) r = OR_GROUP;
  double acc = 0.0;
  for (int64_t i = 0; i < r; ++i) acc += w[i] * bf16_value(keys[(first + i) * OR_IDX_DIM + d]);
  if (r == OR_GROUP) return acc;
  double wsum = 0.0;
  for (int64_t i = 0; i < r; ++i) wsum += w[i];
  return acc / wsum;
}

static int8_t quantise(double x, double scale) {
  double v = nearbyint(x / scale); /* default rounding mode: to nearest, ties to even */
  if (v > 127.0) v = 127.0;
  if (v < -127.0) v = -127.0;
  return (int8_t)v;
}

int oracle_pool(const uint16_t* keys, int64_t L, const float* w4, double* pooled, int8_t* k8, float* scale,
                double* amax_out) {
  if (L < 1) return -1;
  double w[OR_GROUP];
  for (int i = 0; i < OR_GROUP; ++i) w[i] = (double)w4[i];
  int64_t G = (L + OR_GROUP - 1) / OR_GROUP;
  double* kp = pooled ? pooled : (double*)malloc(sizeof(double) * (size_t)G * OR_IDX_DIM);
  if (!kp) return -2;
  double amax = 0.0;
  for (int64_t g = 0; g < G; ++g)
    for (int d = 0; d < OR_IDX_DIM; ++d) {
      double v = pooled_value(keys, L, w, g, d);
      kp[g * OR_IDX_DIM + d] = v;
      if (fabs(v) > amax) amax = fabs(v);
    }
  /* symmetric per-sequence scale: the largest magnitude maps to 127 */
  double s = amax > 0.0 ? amax / 127.0 : 1.0;
  for (int64_t e = 0; e < G * OR_IDX_DIM; ++e) k8[e] = quantise(kp[e], s);
  *scale = (float)s;
  if (amax_out) *amax_out = amax;
  if (!pooled) free(kp);
  return 0;
}

int oracle_pool_given_scale(const uint16_t* keys, int64_t L, const float* w4, float scale, int8_t* k8) {
  if (L < 1 || !(scale > 0.0f)) return -1;
  double w[OR_GROUP];
  for (int i = 0; i < OR_GROUP; ++i) w[i] = (double)w4[i];
  int64_t G = (L + OR_GROUP - 1) / OR_GROUP;
  for (int64_t g = 0; g < G; ++g)
    for (int d = 0; d < OR_IDX_DIM; ++d)
      k8[g * OR_IDX_DIM + d] = quantise(pooled_value(keys, L, w, g, d), (double)scale);
  return 0;
}

static int64_t score_one(const int8_t* q, const int8_t* w, const int8_t* key) {
  int64_t s = 0;
  for (int h = 0; h < OR_IDX_HEADS; ++h) {
    int64_t dot = 0;
    for (int d = 0; d < OR_IDX_DIM; ++d) dot += (int64_t)q[h * OR_IDX_DIM + d] * (int64_t)key[d];
    if (dot > 0) s += (int64_t)w[h] * dot; /* ReLU, then the head weight */
  }
  return s;
}

void oracle_scores(const int8_t* q, const int8_t* w, const int8_t* k8, int64_t G, int64_t* S) {
  for (int64_t g = 0; g < G; ++g) S[g] = score_one(q, w, k8 + g * OR_IDX_DIM);
}

void oracle_prefill_scores(const int8_t* q, const int8_t* w, int64_t pos, const int8_t* k8, int64_t G,
                           int64_t* S) {
  int64_t last = pos / OR_GROUP; /* the query's own group is visible (block-causal) */
  for (int64_t g = 0; g < G; ++g) S[g] = g <= last ? score_one(q, w, k8 + g * OR_IDX_DIM) : -1;
}

typedef struct {
  int64_t score;
  int64_t group;
} ranked;

/* higher score first, then lower group index */
static int by_rank(const void* a, const void* b) {
  const ranked* x = (const ranked*)a;
  const ranked* y = (const ranked*)b;
  if (x->score != y->score) return x->score > y->score ? -1 : 1;
  return (x->group > y->group) - (x->group < y->group);
}

static int by_index(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int oracle_topk(const int64_t* S, int64_t G, int32_t K, int32_t* idx, int32_t* count) {
  if (K < 1) return -1;
  ranked* v = (ranked*)malloc(sizeof(ranked) * (size_t)(G > 0 ? G : 1));
  if (!v) return -2;
  int64_t n = 0;
  for (int64_t g = 0; g < G; ++g)
    if (S[g] >= 0) {
      v[n].score = S[g];
      v[n].group = g;
      ++n;
    }
  int64_t take = n;
  if (n > K) { /* sparse: the K best under the order; otherwise dense fallback */
    qsort(v, (size_t)n, sizeof(ranked), by_rank);
    take = K;
  }
  for (int64_t i = 0; i < take; ++i) idx[i] = (int32_t)v[i].group;
  qsort(idx, (size_t)take, sizeof(int32_t), by_index);
  for (int64_t i = take; i < K; ++i) idx[i] = -1;
  *count = (int32_t)take;
  free(v);
  return 0;
}

/* Latent value of token t, channel d, from one of the two cache formats. */
typedef struct {
  const uint16_t* bf16; /* [L,512] bf16 bits, or NULL */
  const uint8_t* codes; /* [L,512] fp8 E4M3 codes (when bf16 is NULL) */
  const float* scales;  /* [L] per-row scales of the codes */
} latent_rows;

static double latent_value(const latent_rows* c, int64_t t, int d) {
  if (c->bf16) return bf16_value(c->bf16[t * OR_LAT_DIM + d]);
  return (double)c->scales[t] * oracle_fp8_decode(c->codes[t * OR_LAT_DIM + d]);
}

static int attention_rows(const uint16_t* q, const latent_rows* lat, int64_t L, int64_t pos, const int32_t* sel,
                          int32_t count, double scale, double* out, double* lse) {
  if (L < 1 || count < 0) return -1;
  /* the visible tokens of the selected groups */
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(count > 0 ? count : 1) * OR_GROUP);
  double* s = (double*)malloc(sizeof(double) * (size_t)(count > 0 ? count : 1) * OR_GROUP);
  if (!tok || !s) {
    free(tok);
    free(s);
    return -2;
  }
  int64_t T = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (sel[i] < 0) continue;
    for (int j = 0; j < OR_GROUP; ++j) {
      int64_t t = (int64_t)sel[i] * OR_GROUP + j;
      if (t < L && t <= pos) tok[T++] = t;
    }
  }
  for (int h = 0; h < OR_ATT_HEADS; ++h) {
    double* o = out + (size_t)h * OR_LAT_DIM;
    for (int d = 0; d < OR_LAT_DIM; ++d) o[d] = 0.0;
    if (T == 0) {
      lse[h] = -INFINITY;
      continue;
    }
    double m = -INFINITY;
    for (int64_t i = 0; i < T; ++i) {
      double dot = 0.0;
      for (int d = 0; d < OR_LAT_DIM; ++d)
        dot += bf16_value(q[h * OR_LAT_DIM + d]) * latent_value(lat, tok[i], d);
      s[i] = dot * scale;
      if (s[i] > m) m = s[i];
    }
    double l = 0.0;
    for (int64_t i = 0; i < T; ++i) {
      double e = exp(s[i] - m);
      l += e;
      for (int d = 0; d < OR_LAT_DIM; ++d) o[d] += e * latent_value(lat, tok[i], d);
    }
    for (int d = 0; d < OR_LAT_DIM; ++d) o[d] /= l;
    lse[h] = m + log(l);
  }
  free(tok);
  free(s);
  return 0;
}

int oracle_attention(const uint16_t* q, const uint16_t* lat, int64_t L, int64_t pos, const int32_t* sel,
                     int32_t count, double scale, double* out, double* lse) {
  latent_rows c = {lat, NULL, NULL};
  return attention_rows(q, &c, L, pos, sel, count, scale, out, lse);
}

/* ---- FP8 latent cache ([WIKI] quantisation section: the recent cache in FP8) ----
 * OCP 8-bit E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
 * holds subnormals m/8 * 2^-6; S.1111.111 is NaN and there are no infinities, so
 * the largest value is 1.75 * 2^8 = 448. */
double oracle_fp8_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^-6 */
  else
    v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

uint8_t oracle_fp8_encode(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a > 464.0) return sign | 0x7F;  /* rounds past the largest value: NaN (no saturation) */
  if (a >= 448.0) return sign | 0x7E; /* [448, 464] -> 448 (464 is a tie: to the even mantissa) */
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): the leading bit is 2^(e-1) */
  int ub = e - 1;
  if (ub < -6) ub = -6; /* below the smallest normal the spacing stays 2^-9 */
  double q = nearbyint(ldexp(a, 3 - ub)); /* units of the spacing 2^(ub-3); ties to even */
  if (q >= 16.0) { /* rounded up into the next binade */
    ub += 1;
    q = 8.0;
  }
  if (ub == -6 && q < 8.0) return sign | (uint8_t)q; /* subnormal (or zero) */
  return sign | (uint8_t)(((ub + 7) << 3) | ((int)q - 8));
}

int oracle_latent_fp8(const uint16_t* lat, int64_t n, uint8_t* codes, float* scales) {
  for (int64_t t = 0; t < n; ++t) {
    float amax = 0.f;
    for (int d = 0; d < OR_LAT_DIM; ++d) {
      float v = (float)bf16_value(lat[t * OR_LAT_DIM + d]);
      if (isnan(v) || isinf(v)) return -1;
      if (fabsf(v) > amax) amax = fabsf(v);
    }
    float s = amax > 0.f ? amax / 448.f : 1.f;
    scales[t] = s;
    for (int d = 0; d < OR_LAT_DIM; ++d) {
      float v = (float)bf16_value(lat[t * OR_LAT_DIM + d]);
      codes[t * OR_LAT_DIM + d] = oracle_fp8_encode(v / s);
    }
  }
  return 0;
}

int oracle_attention_fp8(const uint16_t* q, const uint8_t* codes, const float* scales, int64_t L, int64_t pos,
                         const int32_t* sel, int32_t count, double scale, double* out, double* lse) {
  latent_rows c = {NULL, codes, scales};
  return attention_rows(q, &c, L, pos, sel, count, scale, out, lse);
}


/* ---- linear-attention layers: one KDA decode step ----
 * [WIKI] linear attention section: the state matrix takes the delta update
 * S_t = S_{t-1} - beta k (k^T S_{t-1}) + beta k v^T; [TREND] section on why the
 * linear layers are the majority: KDA gates the decay channel by channel.
 * Reading (the pages give no more): the decay alpha multiplies the key-channel
 * rows of the state before the delta update, the output is o = S_t^T q, and
 * the state is stored in bf16 ([WIKI] quantisation section: the shared state
 * matrix stays BF16), rounded to nearest even after the step. */
static uint16_t bf16_round(double x) {
  /* nearest bf16 value of x (8 significant bits), ties to even, straight from
   * the double (no intermediate fp32 rounding) */
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  int e;
  frexp(x, &e);                       /* |x| = f 2^e, f in [0.5, 1) */
  if (e < -125) e = -125;             /* bf16 subnormals: fixed spacing 2^-133 */
  double m = nearbyint(ldexp(x, 8 - e)); /* 8 significant bits */
  double r = ldexp(m, e - 8);
  float f = (float)r;                 /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

int oracle_kda_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha, float beta,
                    uint16_t* S, double* o) {
  enum { D = OR_KDA_DIM };
  double* Sp = (double*)malloc(sizeof(double) * D * D);
  if (!Sp) return -2;
  /* decay, channel by channel over the key dimension */
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) Sp[i * D + j] = (double)alpha[i] * bf16_value(S[i * D + j]);
  /* delta update: erase what the key retrieves (u = S'^T k), write the value */
  for (int j = 0; j < D; ++j) {
    double u = 0.0;
    for (int i = 0; i < D; ++i) u += bf16_value(k[i]) * Sp[i * D + j];
    for (int i = 0; i < D; ++i) Sp[i * D + j] += (double)beta * bf16_value(k[i]) * (bf16_value(v[j]) - u);
  }
  /* read-out and the stored state */
  for (int j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += bf16_value(q[i]) * Sp[i * D + j];
    o[j] = acc;
  }
  int bad = 0;
  for (int i = 0; i < D * D; ++i) {
    if (!isfinite(Sp[i])) bad = 1;
    S[i] = bf16_round(Sp[i]);
  }
  free(Sp);
  return bad ? -1 : 0;
}

uint16_t oracle_bf16_round(double x) { return bf16_round(x); }
