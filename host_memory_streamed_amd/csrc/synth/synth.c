/*
 * Seeded synthetic inputs: a counter-based generator shared by the CPU oracle's
 * tests and the benchmark harness. It holds none of the training step's
 * arithmetic; it only produces weights and token ids.
 *
 * Generator (counter-based SplitMix64, Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014):
 *   gamma      = 0x9E3779B97F4A7C15
 *   mix(z)     = SplitMix64 output function (xor-shift-multiply, 30/27/31)
 *   key(s, k)  = mix(mix(s) ^ (k * 0xD1B54A32D192ED03))
 *   word(K, i) = mix(K + (i + 1) * gamma)          (i = 0, 1, 2, ...)
 *
 * Normals (Box-Muller, pair j of stream k): w = word(key(seed, k), j),
 *   u1 = ((w >> 32) + 0.5) / 2^32,  u2 = ((w & 0xffffffff) + 0.5) / 2^32,
 *   r = sqrt(-2 ln u1),  x[2j] = r cos(2 pi u2),  x[2j+1] = r sin(2 pi u2),
 * computed in double, scaled by std, rounded once to float.
 *
 * Uniform integers in [0, n): w = word(key(seed, k), i), value = ((w >> 32) * n) >> 32.
 *
 * Every element depends only on (seed, stream, index), so any slice can be
 * produced independently and in parallel with identical results.
 */
#include <math.h>
#include <stdint.h>
#include <omp.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t sm_key(uint64_t seed, uint64_t stream) {
  return sm_mix(sm_mix(seed) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t sm_word(uint64_t key, uint64_t i) {
  return sm_mix(key + (i + 1) * SM_GAMMA);
}

static inline void sm_pair(uint64_t key, uint64_t j, double *a, double *b) {
  const uint64_t w = sm_word(key, j);
  const double u1 = ((double)(w >> 32) + 0.5) * (1.0 / 4294967296.0);
  const double u2 = ((double)(w & 0xffffffffULL) + 0.5) * (1.0 / 4294967296.0);
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  *a = r * cos(th);
  *b = r * sin(th);
}

/* out[i] = std * normal(seed, stream, offset + i), i in [0, n). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                      double std, float *out, int threads) {
  const uint64_t key = sm_key(seed, stream);
  if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static, 65536)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t g = offset + (uint64_t)i;
    double a, b;
    sm_pair(key, g >> 1, &a, &b);
    out[i] = (float)(std * ((g & 1) ? b : a));
  }
}

/* out[i] = uniform integer in [0, n_values) for element offset + i. */
void synth_uniform_i32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       int64_t n_values, int32_t *out, int threads) {
  const uint64_t key = sm_key(seed, stream);
  if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static, 65536)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t w = sm_word(key, offset + (uint64_t)i);
    out[i] = (int32_t)(((w >> 32) * (uint64_t)n_values) >> 32);
  }
}

/* Raw 64-bit words, for tests of the generator against its definition. */
void synth_words(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, uint64_t *out) {
  const uint64_t key = sm_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = sm_word(key, offset + (uint64_t)i);
}
