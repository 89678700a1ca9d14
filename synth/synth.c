/*
 * Seeded synthetic inputs for the attention forward path.
 *
 * This module holds no attention arithmetic.  It turns (seed, tensor id,
 * element index) into bf16 bit patterns, and both the GPU path and the CPU
 * oracle consume the same bytes.  The pages fix only "iid N(0,1) values from
 * a seed" for the workloads, so the generator is defined here:
 *
 *   stream key  K_t = mix64(seed * 0x9E3779B97F4A7C15 + t + 1)
 *   uniform n   U_t(n) = (mix64(K_t + (n + 1) * 0x9E3779B97F4A7C15) >> 11) * 2^-53
 *
 * where mix64 is the SplitMix64 finaliser (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), so U is a
 * counter-based stream.  Element pair p (elements 2p and 2p+1) takes
 * u1 = U(2p), u2 = U(2p+1) and applies the Box-Muller transform
 * (Box and Muller, 1958):
 *   r = sqrt(-2 ln(1 - u1)),  z0 = r cos(2 pi u2),  z1 = r sin(2 pi u2)
 * in double precision; each value is multiplied by `mult` and rounded to
 * bfloat16 with round-to-nearest-even from the double directly (no double
 * rounding through float).  Magnitudes below 2^-120 become signed zero.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double uniform01(uint64_t key, uint64_t n) {
  return (double)(mix64(key + (n + 1) * GOLDEN) >> 11) * 0x1p-53;
}

/* Round a double to bf16 bits, round-to-nearest-even on the 8-bit significand. */
uint16_t synth_bf16_from_double(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x);
  if (a < 0x1p-120) return sign;
  if (isinf(a) || isnan(a)) return (uint16_t)(sign | (isnan(a) ? 0x7FC0u : 0x7F80u));
  int e;
  double m = frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) */
  double r = rint(ldexp(m, 8));         /* 8 significant bits, ties to even */
  float f = (float)ldexp(r, e - 8);     /* exact in float */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tensor_id) {
  return mix64(seed * GOLDEN + tensor_id + 1);
}

/* Fill out[0..n) with bf16 bits of mult * N(0,1) for stream (seed, tensor_id). */
void synth_normal_bf16(uint64_t seed, uint64_t tensor_id, double mult,
                       uint16_t* out, int64_t n) {
  const uint64_t key = synth_stream_key(seed, tensor_id);
  const int64_t npairs = (n + 1) / 2;
  #pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npairs; ++p) {
    double u1 = uniform01(key, (uint64_t)(2 * p));
    double u2 = uniform01(key, (uint64_t)(2 * p + 1));
    double r = sqrt(-2.0 * log(1.0 - u1));
    double t = 6.283185307179586476925286766559 * u2;
    out[2 * p] = synth_bf16_from_double(mult * r * cos(t));
    if (2 * p + 1 < n) out[2 * p + 1] = synth_bf16_from_double(mult * r * sin(t));
  }
}

/* Raw uniforms, exposed so tests can check the stream definition. */
void synth_uniforms(uint64_t seed, uint64_t tensor_id, double* out, int64_t n) {
  const uint64_t key = synth_stream_key(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = uniform01(key, (uint64_t)i);
}
