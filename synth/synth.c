/*
 * synth.c -- seeded, counter-based synthetic input generator.
 *
 * Serves both the HIP path and the CPU oracle with identical bf16 inputs.  It
 * holds none of the normalisation arithmetic: it only draws numbers.
 *
 * Definition.  Every tensor of every workload has its own stream key
 *     key = mix(seed ^ mix((workload << 32) | tensor))
 * and element i of that tensor uses the SplitMix64 outputs n = 2i+1 and
 * n = 2i+2 of the generator seeded with key, i.e. mix(key + n * GAMMA), where
 * GAMMA = 0x9E3779B97F4A7C15 and mix() is the SplitMix64 finaliser (Steele,
 * Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA
 * 2014; constants as in Vigna's public-domain splitmix64.c).  Each output is
 * turned into a uniform in [0, 1) from its top 53 bits.
 *   uniform(a, b):  a + (b - a) * u1
 *   normal(m, s):   m + s * sqrt(-2 ln(1 - u1)) * cos(2 pi u2)   (Box-Muller)
 * Optional row stress: activation row r is stressed when
 * mix(stress_key + (r+1) * GAMMA) < p * 2^64, with stress_key derived from the
 * seed and workload only (so x and residual stress the same rows); the drawn
 * value of a stressed row is multiplied by the stress factor.
 * The double is then converted to binary32 and that to bf16, each with
 * round-to-nearest-even (the second step on the integer bit pattern); -0 is
 * stored as +0.  No NaN or Inf is made (all drawn values are finite and far
 * below the bf16 overflow threshold).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint32_t workload, uint32_t tensor) {
  return mix(seed ^ mix(((uint64_t)workload << 32) | tensor));
}

static double unit(uint64_t v) { return (double)(v >> 11) * 0x1.0p-53; }

static uint16_t to_bf16(double v) {
  float f = (float)v;
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  bits += 0x7FFFu + ((bits >> 16) & 1u);
  uint16_t h = (uint16_t)(bits >> 16);
  return h == 0x8000 ? 0 : h;
}

enum { SYNTH_NORMAL = 0, SYNTH_UNIFORM = 1 };

/*
 * Fill out[0..n) with elements idx0 .. idx0+n-1 of tensor `tensor` of
 * workload `workload`.  dist: SYNTH_NORMAL (a = mean, b = std) or
 * SYNTH_UNIFORM on [a, b).  If stress_p > 0, element i belongs to row
 * i / row_len and stressed rows are multiplied by stress_mul.
 */
void synth_fill(uint16_t* out, int64_t n, int64_t idx0, uint64_t seed, uint32_t workload,
                uint32_t tensor, int dist, double a, double b, int64_t row_len,
                double stress_p, double stress_mul) {
  const uint64_t key = synth_key(seed, workload, tensor);
  const uint64_t skey = synth_key(seed, workload, 0xFFFFFFFFu);
  const double two_pi = 6.283185307179586476925286766559;
  const double thresh = stress_p * 0x1.0p64;
  for (int64_t j = 0; j < n; ++j) {
    uint64_t i = (uint64_t)(idx0 + j);
    double u1 = unit(mix(key + (2 * i + 1) * GAMMA));
    double v;
    if (dist == SYNTH_UNIFORM) {
      v = a + (b - a) * u1;
    } else {
      double u2 = unit(mix(key + (2 * i + 2) * GAMMA));
      v = a + b * sqrt(-2.0 * log(1.0 - u1)) * cos(two_pi * u2);
    }
    if (stress_p > 0.0 && row_len > 0) {
      uint64_t row = i / (uint64_t)row_len;
      if ((double)mix(skey + (row + 1) * GAMMA) < thresh) v *= stress_mul;
    }
    out[j] = to_bf16(v);
  }
}

/* Stressed-row predicate, for tests of the generator itself. */
int synth_row_stressed(uint64_t seed, uint32_t workload, int64_t row, double stress_p) {
  const uint64_t skey = synth_key(seed, workload, 0xFFFFFFFFu);
  return (double)mix(skey + ((uint64_t)row + 1) * GAMMA) < stress_p * 0x1.0p64;
}
