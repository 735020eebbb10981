/* CPU implementation of the seeded generator defined in synth.h.
 * Built with -ffp-contract=off so that mu + sigma*z is never fused. */
#include "synth.h"
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
/* sqrt(3/2) / 2^17 */
#define SYNTH_C 0x1.3988e1409212ep-17

uint64_t synth_mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

uint64_t synth_stream_key(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t index) {
  uint64_t k = synth_mix64(seed ^ SYNTH_GAMMA);
  k = synth_mix64(k ^ (uint64_t)tag);
  k = synth_mix64(k ^ (((uint64_t)layer << 32) | (uint64_t)index));
  return k;
}

static double synth_z(uint64_t key, uint64_t i) {
  uint64_t h1 = synth_mix64(key + (2 * i + 1) * SYNTH_GAMMA);
  uint64_t h2 = synth_mix64(key + (2 * i + 2) * SYNTH_GAMMA);
  int64_t s = 0;
  for (int f = 0; f < 4; ++f) {
    s += (int64_t)((h1 >> (16 * f)) & 0xFFFF);
    s += (int64_t)((h2 >> (16 * f)) & 0xFFFF);
  }
  return (double)(2 * s - 524280) * SYNTH_C;
}

static float synth_value(uint64_t key, uint64_t i, double mu, double sigma) {
  double t = sigma * synth_z(key, i);
  double v = mu + t;
  return (float)v;
}

void synth_normal_f32(uint64_t key, uint64_t first, uint64_t n, double mu, double sigma,
                      float* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 20))
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = synth_value(key, first + (uint64_t)j, mu, sigma);
}

static uint16_t synth_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

void synth_normal_bf16(uint64_t key, uint64_t first, uint64_t n, double mu, double sigma,
                       uint16_t* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 20))
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = synth_bf16_bits(synth_value(key, first + (uint64_t)j, mu, sigma));
}
