/* Host implementation of the seeded streams defined in synth.h (C11 + OpenMP). */
#include "synth.h"
#include <math.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_at(uint64_t key, uint64_t i) { return mix(key + (i + 1u) * GAMMA); }
uint64_t synth_key(uint64_t seed, uint64_t stream) { return synth_at(seed, stream); }

static inline double unif(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

static inline float normal_f32(uint64_t key, uint64_t i, double std) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unif(synth_at(key, 2u * i));
  double u2 = unif(synth_at(key, 2u * i + 1u));
  double z = sqrt(-2.0 * log(1.0 - u1)) * cos(two_pi * u2);
  return (float)(std * z);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, double std, uint64_t first, size_t n, float* out) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) out[i] = normal_f32(key, first + (uint64_t)i, std);
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, double std, uint64_t first, size_t n, uint16_t* out) {
  const uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i)
    out[i] = f32_to_bf16_rne(normal_f32(key, first + (uint64_t)i, std));
}

void synth_tokens(uint64_t seed, uint64_t stream, int32_t vocab, uint64_t first, size_t n, int32_t* out) {
  const uint64_t key = synth_key(seed, stream);
  for (size_t i = 0; i < n; ++i) out[i] = (int32_t)(synth_at(key, first + i) % (uint64_t)vocab);
}

void synth_uniforms(uint64_t seed, uint64_t stream, uint64_t first, size_t n, double* out) {
  const uint64_t key = synth_key(seed, stream);
  for (size_t i = 0; i < n; ++i) out[i] = unif(synth_at(key, first + i));
}
