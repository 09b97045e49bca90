/*
 * Seeded synthetic-input generator, host implementation.
 *
 * This module produces the inputs that both the oracle and the GPU path
 * consume (expert weights, activations, router logits, biases).  It holds
 * none of the method's arithmetic: no quantisation, routing or dot products.
 *
 * Definition (shared with the device implementation in synth_device.hip,
 * which must produce bit-identical values):
 *
 *   mix64(z)       : the SplitMix64 output function of Steele, Lea and Flood,
 *                    "Fast splittable pseudorandom number generators"
 *                    (OOPSLA 2014): two xor-shift-multiply rounds and a final
 *                    xor-shift, with the published multipliers.
 *   base(seed, id) : mix64(mix64(seed + GAMMA) ^ (id * ID_MUL))
 *   draw(base, n)  : mix64(base + (n + 1) * GAMMA)           (counter based)
 *   normal(i)      : Irwin-Hall sum of twelve 16-bit uniforms taken from
 *                    draws 3i, 3i+1, 3i+2; S - 393210 is an exact integer,
 *                    scaled by 2^-16 (exact) to unit variance, then one
 *                    IEEE fp32 multiply by sigma.  Only integer arithmetic,
 *                    exact conversions and one rounded multiply are used,
 *                    so every IEEE-conforming host and device agree bit for
 *                    bit.  The distribution is the classic Irwin-Hall(12)
 *                    approximation of N(0, sigma^2), bounded at 6 sigma.
 *   uniform(i)     : ((draw(base, i) >> 11) + 0.5) * 2^-53, in (0, 1).
 */
#include <stdint.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
#define SYNTH_ID_MUL 0xD1B54A32D192ED03ULL

static inline uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_base(uint64_t seed, uint64_t stream_id) {
  return synth_mix64(synth_mix64(seed + SYNTH_GAMMA) ^ (stream_id * SYNTH_ID_MUL));
}

static inline uint64_t synth_draw(uint64_t base, uint64_t n) {
  return synth_mix64(base + (n + 1) * SYNTH_GAMMA);
}

static inline float synth_normal_at(uint64_t base, uint64_t i, float sigma) {
  uint32_t s = 0;
  for (uint64_t j = 0; j < 3; ++j) {
    uint64_t z = synth_draw(base, 3 * i + j);
    s += (uint32_t)(z & 0xFFFF) + (uint32_t)((z >> 16) & 0xFFFF) +
         (uint32_t)((z >> 32) & 0xFFFF) + (uint32_t)(z >> 48);
  }
  float zf = (float)((int32_t)s - 393210) * (1.0f / 65536.0f);
  return zf * sigma;
}

/* out[j] = normal(offset + j) of stream (seed, stream_id), j < n. */
void synth_normal(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n,
                  float sigma, float* out) {
  const uint64_t base = synth_stream_base(seed, stream_id);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = synth_normal_at(base, offset + (uint64_t)j, sigma);
}

/* out[j] = uniform(offset + j) in (0, 1), as doubles, j < n. */
void synth_uniform(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n,
                   double* out) {
  const uint64_t base = synth_stream_base(seed, stream_id);
  for (int64_t j = 0; j < n; ++j) {
    uint64_t z = synth_draw(base, offset + (uint64_t)j);
    out[j] = ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  }
}
