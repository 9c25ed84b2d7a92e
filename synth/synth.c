/*
 * Seeded synthetic inputs for the ternary linear layer: trits, uniform and
 * normal draws.  Shared by the CPU oracle's tests and the GPU path's tests and
 * benchmark; it holds none of the layer's arithmetic (no packing, no
 * transform, no products), only random numbers.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; finaliser constants as published by Vigna)
 * used as a counter-based hash: draw i of a stream is mix(key ^ i), so any
 * element can be regenerated on its own and the result does not depend on
 * the thread count.
 *
 * key = seed ^ (tag << 56) ^ (matrix_id << 40); index < 2^40.
 */
#include <math.h>
#include <stdint.h>

static inline uint64_t splitmix64_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag, uint64_t id) {
  return seed ^ (tag << 56) ^ (id << 40);
}

enum { TAG_TRIT = 1, TAG_UNIFORM = 2, TAG_NORMAL_A = 3, TAG_NORMAL_B = 4 };

/* Thresholds on the top 32 bits: P(-1) = P(+1) = 0.31, P(0) = 0.38. */
#define T_NEG 1331439862u  /* round(0.31 * 2^32) */
#define T_ZERO 2963527434u /* round(0.69 * 2^32) */

uint64_t synth_hash(uint64_t seed, uint64_t tag, uint64_t id, uint64_t index) {
  return splitmix64_mix(stream_key(seed, tag, id) ^ index);
}

/* count trits in {-1,0,+1}, element i = draw (first + i) of the stream. */
void synth_trits(uint64_t seed, uint64_t id, int64_t first, int64_t count, int8_t* out) {
  const uint64_t key = stream_key(seed, TAG_TRIT, id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint32_t u = (uint32_t)(splitmix64_mix(key ^ (uint64_t)(first + i)) >> 32);
    out[i] = (int8_t)(u < T_NEG ? -1 : (u < T_ZERO ? 0 : 1));
  }
}

/* count doubles uniform in [0,1): 53 high bits of the hash times 2^-53. */
void synth_uniform(uint64_t seed, uint64_t id, int64_t first, int64_t count, double* out) {
  const uint64_t key = stream_key(seed, TAG_UNIFORM, id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = (double)(splitmix64_mix(key ^ (uint64_t)(first + i)) >> 11) * 0x1.0p-53;
}

/* count standard normals by Box-Muller (cosine branch) from two streams. */
void synth_normal(uint64_t seed, uint64_t id, int64_t first, int64_t count, double* out) {
  const uint64_t ka = stream_key(seed, TAG_NORMAL_A, id);
  const uint64_t kb = stream_key(seed, TAG_NORMAL_B, id);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint64_t j = (uint64_t)(first + i);
    double u1 = (double)((splitmix64_mix(ka ^ j) >> 11) + 1) * 0x1.0p-53; /* (0,1] */
    double u2 = (double)(splitmix64_mix(kb ^ j) >> 11) * 0x1.0p-53;       /* [0,1) */
    out[i] = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
  }
}
