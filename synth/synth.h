/*
 * Seeded synthetic inputs: the one module that both the CPU oracle and the GPU
 * path draw their inputs from.  It holds none of the decoding method's
 * arithmetic, only counter-based random streams.
 *
 * Definition (the same on the host, in synth.c, and on the device, in
 * synth_dev.hip):
 *   mix(z)      SplitMix64 output finaliser (Steele, Lea & Flood, "Fast
 *               splittable pseudorandom number generators", OOPSLA 2014):
 *               z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *               z *= 0x94D049BB133111EB; z ^= z>>31.
 *   at(key, i)  output number i (0-based) of a SplitMix64 generator whose
 *               state starts at key:  mix(key + (i+1) * 0x9E3779B97F4A7C15).
 *   key(seed, stream) = at(seed, stream).
 *   uniform(x)  = (x >> 11) * 2^-53, in [0, 1).
 *   normal element i of a stream: u1 = uniform(at(key, 2i)),
 *               u2 = uniform(at(key, 2i+1)),
 *               z = sqrt(-2 ln(1 - u1)) * cos(2 pi u2)   (Box-Muller, fp64),
 *               value = (float)(std * z); the bf16 form rounds that fp32
 *               value to nearest-even on its upper 16 bits.
 *   token element i = at(key, i) mod vocab.
 *
 * Streams used by the tests and the benchmark:
 *   weights  (tensor t, layer l): SYNTH_STREAM_WEIGHT(t, l)
 *   prompts  (request r):         SYNTH_STREAM_PROMPT(r)
 *   uniforms (request r, round n): SYNTH_STREAM_UNIFORM(r, n)
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>
#include <stddef.h>

#define SYNTH_STREAM_WEIGHT(t, l) (((uint64_t)(t) + 1u) * 0x10000ull + (uint64_t)(l))
#define SYNTH_STREAM_PROMPT(r) (0x20000000ull + (uint64_t)(r))
#define SYNTH_STREAM_UNIFORM(r, n) (0x40000000ull + (uint64_t)(r) * 0x10000ull + (uint64_t)(n))

#ifdef __cplusplus
extern "C" {
#endif
uint64_t synth_at(uint64_t key, uint64_t i);
uint64_t synth_key(uint64_t seed, uint64_t stream);
/* n elements starting at element index `first` of the stream. */
void synth_normal_f32(uint64_t seed, uint64_t stream, double std, uint64_t first, size_t n, float* out);
void synth_normal_bf16(uint64_t seed, uint64_t stream, double std, uint64_t first, size_t n, uint16_t* out);
void synth_tokens(uint64_t seed, uint64_t stream, int32_t vocab, uint64_t first, size_t n, int32_t* out);
void synth_uniforms(uint64_t seed, uint64_t stream, uint64_t first, size_t n, double* out);
#ifdef __cplusplus
}
#endif
#endif
