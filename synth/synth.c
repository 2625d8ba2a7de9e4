/*
 * Seeded synthetic inputs: weights and prompt token ids.
 *
 * This module is input generation only. It holds none of the decoding
 * method's arithmetic and is the one piece shared by the CPU oracle and by
 * the harness that loads the GPU library.
 *
 * Generator (counter based, reproducible bit for bit on any IEEE machine):
 *   mix(x)   = SplitMix64 finaliser of x + 0x9E3779B97F4A7C15 (Vigna).
 *   key      = mix(seed ^ (stream_id * 0x9E3779B97F4A7C15))
 *   element i of a weight tensor:
 *     h1 = mix(key + 2i), h2 = mix(key + 2i + 1)
 *     S  = sum of the eight 16-bit lanes of h1 and h2        (integer)
 *     w  = (float)((double)(S - 262140) * C),  C = 0.02*sqrt(1.5)/65536
 *   S/65536 is an Irwin-Hall(8) sum of midpoint uniforms, mean 4, variance
 *   2/3, so w has mean 0 and standard deviation 0.02 (an approximately
 *   normal law with tails cut at 4.9 sigma). The only floating-point step is
 *   one correctly rounded multiply and one round-to-nearest conversion, so
 *   every IEEE implementation gives the same bits.
 *   bf16 = round-to-nearest-even of the fp32 value.
 *   token i of a prompt: mix(key + i) mod vocab.
 */
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
static const double SYNTH_C = 0x1.91530bd7c536ep-22; /* 0.02*sqrt(1.5)/65536 */

static inline uint64_t mix(uint64_t x) {
  uint64_t z = x + GOLDEN;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_mix(uint64_t x) { return mix(x); }

uint64_t synth_key(uint64_t seed, uint64_t stream_id) {
  return mix(seed ^ (stream_id * GOLDEN));
}

static inline uint32_t lanesum(uint64_t h) {
  return (uint32_t)(h & 0xFFFF) + (uint32_t)((h >> 16) & 0xFFFF) +
         (uint32_t)((h >> 32) & 0xFFFF) + (uint32_t)(h >> 48);
}

static inline float elem(uint64_t key, uint64_t i) {
  uint32_t s = lanesum(mix(key + 2 * i)) + lanesum(mix(key + 2 * i + 1));
  double z = (double)((int64_t)s - 262140) * SYNTH_C;
  return (float)z;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Elements [offset, offset+n) of tensor (seed, stream_id) as fp32. */
void synth_normal_f32(uint64_t seed, uint64_t stream_id, uint64_t offset,
                      uint64_t n, float *out) {
  uint64_t key = synth_key(seed, stream_id);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) out[i] = elem(key, offset + (uint64_t)i);
}

/* Same elements rounded to bf16 (raw 16-bit patterns). */
void synth_normal_bf16(uint64_t seed, uint64_t stream_id, uint64_t offset,
                       uint64_t n, uint16_t *out) {
  uint64_t key = synth_key(seed, stream_id);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i)
    out[i] = f32_to_bf16_rne(elem(key, offset + (uint64_t)i));
}

/* Same bf16 values widened back to fp32 (exactly representable), in one pass. */
void synth_normal_bf16_f32(uint64_t seed, uint64_t stream_id, uint64_t offset,
                           uint64_t n, float *out) {
  uint64_t key = synth_key(seed, stream_id);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    uint32_t u = (uint32_t)f32_to_bf16_rne(elem(key, offset + (uint64_t)i)) << 16;
    memcpy(&out[i], &u, 4);
  }
}

/* n token ids uniform in [0, vocab). */
void synth_tokens(uint64_t seed, uint64_t stream_id, uint64_t n, uint32_t vocab,
                  int32_t *out) {
  uint64_t key = synth_key(seed, stream_id);
  for (uint64_t i = 0; i < n; ++i) out[i] = (int32_t)(mix(key + i) % vocab);
}
