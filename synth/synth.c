/*
 * synth.c -- seeded, counter-based generator for the synthetic inputs of the
 * sparse-attention path.  It is shared by the CPU oracle's tests and by the
 * GPU path's tests and benchmark, so that both consume identical bytes.  It
 * holds none of the method's arithmetic: it only draws numbers.
 *
 * Definition (every function below is a pure function of its arguments, so any
 * index range can be generated independently, in any order, on any thread):
 *
 *   mix(x)     = the SplitMix64 output finaliser (Steele, Lea, Flood,
 *                "Fast splittable pseudorandom number generators", 2014):
 *                z = x; z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;
 *                z = (z ^ z>>27) * 0x94D049BB133111EB; z ^ z>>31
 *   G          = 0x9E3779B97F4A7C15 (the SplitMix64 increment)
 *   key(s, t)  = mix(mix(s + G) ^ (t * 0xD1B54A32D192ED03))   seed s, tensor id t
 *   draw(k, i) = mix(k + (i + 1) * G)       element i: the (i+1)-th SplitMix64
 *                                           output from state k
 *   u01(x)     = (x >> 11) * 2^-53           uniform double in [0, 1)
 *   normal i   : pair p = i >> 1, a = 1 - u01(draw(k, 2p)), b = u01(draw(k, 2p+1)),
 *                r = sqrt(-2 ln a); element 2p = r cos(2 pi b), 2p+1 = r sin(2 pi b)
 *                (Box-Muller, computed in double)
 *   bf16       : round-to-nearest-even of the double to 8 significant bits
 *   int in [lo, hi] : Lemire's multiply-shift on the high 32 bits of draw(k, i)
 *                with his rejection step; rejected draws are re-drawn from
 *                key mix(k + j) for attempt j = 1, 2, ...
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_G 0x9E3779B97F4A7C15ull

static inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tensor) {
  return mix(mix(seed + SYNTH_G) ^ (tensor * 0xD1B54A32D192ED03ull));
}

static inline uint64_t draw(uint64_t k, uint64_t i) { return mix(k + (i + 1) * SYNTH_G); }

static inline double u01(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

static double normal_at(uint64_t k, uint64_t i) {
  uint64_t p = i >> 1;
  double a = 1.0 - u01(draw(k, 2 * p));
  double b = u01(draw(k, 2 * p + 1));
  double r = sqrt(-2.0 * log(a));
  double th = 6.283185307179586476925286766559 * b;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* Round a double to bfloat16 (round to nearest, ties to even) and return its bits. */
static uint16_t bf16_rne(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
  int e = ilogb(x);            /* x = m * 2^e with 1 <= |m| < 2 */
  if (e < -126) e = -126;      /* bf16 subnormals share the minimum exponent */
  double y = nearbyint(ldexp(x, 7 - e)); /* 8 significant bits, default mode is RNE */
  float f = (float)ldexp(y, e - 7);       /* exact: fits float */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t n, uint16_t* out) {
  uint64_t k = synth_key(seed, tensor);
  for (uint64_t j = 0; j < n; ++j) out[j] = bf16_rne(normal_at(k, start + j));
}

void synth_normal_f64(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t n, double* out) {
  uint64_t k = synth_key(seed, tensor);
  for (uint64_t j = 0; j < n; ++j) out[j] = normal_at(k, start + j);
}

void synth_uniform_f64(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t n, double* out) {
  uint64_t k = synth_key(seed, tensor);
  for (uint64_t j = 0; j < n; ++j) out[j] = u01(draw(k, start + j));
}

static int64_t int_at(uint64_t k, uint64_t i, int64_t lo, uint64_t range) {
  /* range = hi - lo + 1, 1 <= range <= 2^32 */
  if (range == (1ull << 32)) return lo + (int64_t)(draw(k, i) >> 32);
  uint64_t kk = k;
  for (uint64_t attempt = 1;; ++attempt) {
    uint32_t x = (uint32_t)(draw(kk, i) >> 32);
    uint64_t m = (uint64_t)x * range;
    uint32_t l = (uint32_t)m;
    if (l >= (uint32_t)range) return lo + (int64_t)(m >> 32);
    uint32_t t = (uint32_t)((0x100000000ull - range) % range);
    if (l >= t) return lo + (int64_t)(m >> 32);
    kk = mix(k + attempt);
  }
}

void synth_uniform_i8(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t n, int32_t lo, int32_t hi,
                      int8_t* out) {
  uint64_t k = synth_key(seed, tensor);
  uint64_t range = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
  for (uint64_t j = 0; j < n; ++j) out[j] = (int8_t)int_at(k, start + j, lo, range);
}

void synth_uniform_i64(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t n, int64_t lo, int64_t hi,
                       int64_t* out) {
  uint64_t k = synth_key(seed, tensor);
  uint64_t range = (uint64_t)(hi - lo + 1);
  for (uint64_t j = 0; j < n; ++j) out[j] = int_at(k, start + j, lo, range);
}

void synth_u64(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t n, uint64_t* out) {
  uint64_t k = synth_key(seed, tensor);
  for (uint64_t j = 0; j < n; ++j) out[j] = draw(k, start + j);
}
