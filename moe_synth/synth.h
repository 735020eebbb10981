/* Seeded synthetic input generator shared by the CPU reference and the GPU
 * library's tests and benchmark.  It holds none of the MoE arithmetic: it only
 * turns (seed, tensor tag, layer, index, element) into numbers.
 *
 * Definition (identical on CPU and GPU, bit for bit):
 *   mix64(z)   : the splitmix64 output finalizer (Steele, Lea & Flood,
 *                "Fast splittable pseudorandom number generators", OOPSLA 2014):
 *                z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *                z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key        = mix64(mix64(mix64(seed ^ G) ^ tag) ^ (layer<<32 | index)),
 *                G = 0x9E3779B97F4A7C15 (the splitmix64 increment).
 *   element i  : h1 = mix64(key + (2i+1)G), h2 = mix64(key + (2i+2)G);
 *                s  = sum of the eight 16-bit fields of h1 and h2;
 *                z  = (double)(2s - 524280) * C,  C = sqrt(3/2)/2^17,
 *                which is an 8-term Irwin-Hall sum standardised to mean 0 and
 *                variance 1 (support +-4.9).
 *   N(mu,sigma): v = mu + sigma*z in fp64 (two correctly rounded operations,
 *                never fused), then rounded to fp32 (nearest even).
 *   bf16       : the fp32 value rounded to bf16 (nearest even) on its bits.
 * Only integer operations and correctly rounded IEEE multiplies and adds are
 * used, so any conforming CPU or GPU produces the same bits. */
#ifndef MOE_SYNTH_H
#define MOE_SYNTH_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor tags. */
enum { SYNTH_TAG_W13 = 1, SYNTH_TAG_W2 = 2, SYNTH_TAG_WR = 3, SYNTH_TAG_BIAS = 4,
       SYNTH_TAG_GAMMA = 5, SYNTH_TAG_X = 6 };

uint64_t synth_mix64(uint64_t z);
uint64_t synth_stream_key(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t index);
/* out[j] = N(mu, sigma) element (first + j) of stream `key`, j < n. */
void synth_normal_f32(uint64_t key, uint64_t first, uint64_t n, double mu, double sigma,
                      float* out);
/* Same values rounded to bf16 (returned as raw uint16 bits). */
void synth_normal_bf16(uint64_t key, uint64_t first, uint64_t n, double mu, double sigma,
                       uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
