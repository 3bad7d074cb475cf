/*
 * synth.c -- seeded, counter-based normal draws for synthetic layer inputs.
 *
 * This module holds none of the layer's arithmetic: it only turns
 * (seed, stream, element index) into an N(mean, std) sample, so that any
 * slice of any tensor can be drawn independently and in parallel.
 *
 *   key   = splitmix64(seed ^ splitmix64(stream))
 *   u1    = (hi24(splitmix64(key + 2p))     + 1) / 2^24     in (0, 1]
 *   u2    =  hi24(splitmix64(key + 2p + 1))      / 2^24     in [0, 1)
 *   z     = sqrt(-2 ln u1) * (cos 2 pi u2  for even i,  sin 2 pi u2 for odd i)
 *   out_i = (float)(mean + std * z),  p = i / 2
 *
 * The transform runs in single precision (the draws only need to be the same
 * on both sides of a comparison, which read one host array).
 *
 * splitmix64 is the mixer of Steele, Lea and Flood (OOPSLA 2014) with the
 * constants of Vigna's public-domain reference; the pair transform is the
 * Box-Muller transform (Box and Muller, 1958).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>

static uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start,
                      int64_t n, double mean, double std, float* out) {
  const float two_pi = 6.28318530717958647692f;
  const float inv24 = 1.0f / 16777216.0f; /* 2^-24 */
  uint64_t key = splitmix64(seed ^ splitmix64(stream));
  uint64_t end = start + (uint64_t)n;
  for (uint64_t p = start >> 1; 2 * p < end; ++p) {
    float u1 = ((float)(splitmix64(key + 2 * p) >> 40) + 1.0f) * inv24;
    float u2 = (float)(splitmix64(key + 2 * p + 1) >> 40) * inv24;
    float r = sqrtf(-2.0f * logf(u1));
    float s, c;
    sincosf(two_pi * u2, &s, &c);
    uint64_t i0 = 2 * p, i1 = 2 * p + 1;
    if (i0 >= start) out[i0 - start] = (float)(mean + std * (double)(r * c));
    if (i1 >= start && i1 < end) out[i1 - start] = (float)(mean + std * (double)(r * s));
  }
}
