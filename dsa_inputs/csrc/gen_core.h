/*
 * Seeded, counter-based synthetic input generator (shared by the CPU oracle
 * harness and the GPU harness).  It holds no arithmetic of the attention
 * method: it only produces input tensors.
 *
 * Every value is a pure function of (seed, tensor id, logical flat index), so
 * any slice of any tensor can be regenerated on its own, on the host or on the
 * GPU, and both produce the same bits:
 *   - mixing is SplitMix64's output function (Steele, Lea, Flood, "Fast
 *     splittable pseudorandom number generators", OOPSLA 2014), applied to a
 *     counter advanced by the golden-ratio increment;
 *   - a normal draw is the Irwin-Hall sum of twelve 16-bit uniforms, centred
 *     and divided by 2^16.  All of it is integer arithmetic plus an exact
 *     int->float conversion and a power-of-two scaling, so host and device
 *     agree bit for bit (no libm calls anywhere);
 *   - bf16 values are taken from fp32 with one round-to-nearest-even.
 *
 * Compiled by gcc for the host library and by hipcc for the device library;
 * GEN_FN marks the functions for both.
 */
#ifndef DSA_INPUTS_GEN_CORE_H
#define DSA_INPUTS_GEN_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define GEN_FN __host__ __device__ static inline
#else
#define GEN_FN static inline
#endif

#define GEN_GAMMA 0x9E3779B97F4A7C15ULL
/* P(bernoulli) = 0.02 as a 32-bit threshold: ceil(0.02 * 2^32). */
#define GEN_P002_THRESH 85899346u

GEN_FN uint64_t gen_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* One independent stream per (seed, tensor id). */
GEN_FN uint64_t gen_stream_key(uint64_t seed, uint32_t tid) {
  return gen_mix64(seed + GEN_GAMMA * ((uint64_t)tid + 1u));
}

/* Word j (0..3) of element i of a stream. */
GEN_FN uint64_t gen_word(uint64_t key, uint64_t i, uint32_t j) {
  return gen_mix64(key + GEN_GAMMA * (4u * i + j + 1u));
}

GEN_FN uint32_t gen_sum4x16(uint64_t w) {
  return (uint32_t)(w & 0xFFFFu) + (uint32_t)((w >> 16) & 0xFFFFu) +
         (uint32_t)((w >> 32) & 0xFFFFu) + (uint32_t)(w >> 48);
}

/* Approximately N(0,1): (sum of 12 uniforms on [0,65535]) - 6*65535, / 2^16.
 * Variance is (65536^2-1)/65536^2, tails are cut at +-6. Exact in fp32. */
GEN_FN float gen_normal(uint64_t key, uint64_t i) {
  uint32_t s = gen_sum4x16(gen_word(key, i, 0)) + gen_sum4x16(gen_word(key, i, 1)) +
               gen_sum4x16(gen_word(key, i, 2));
  int32_t c = (int32_t)s - 393210;
  return (float)c * (1.0f / 65536.0f);
}

/* U[0,1) on a 2^-24 grid. */
GEN_FN float gen_uniform(uint64_t key, uint64_t i) {
  return (float)(uint32_t)(gen_word(key, i, 0) >> 40) * (1.0f / 16777216.0f);
}

GEN_FN int gen_bernoulli(uint64_t key, uint64_t i, uint32_t thresh32) {
  return (uint32_t)(gen_word(key, i, 0) >> 32) < thresh32;
}

GEN_FN uint32_t gen_f32_bits(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  return v.u;
}

/* fp32 -> bf16, round to nearest even (NaN stays NaN). */
GEN_FN uint16_t gen_bf16_rne(float f) {
  uint32_t u = gen_f32_bits(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Entry (row, col) of the 256x256 Sylvester-Hadamard matrix divided by 16:
 * its rows are orthonormal, and every entry is exactly +-1/16. */
GEN_FN float gen_hadamard16(uint32_t row, uint32_t col) {
  uint32_t x = row & col;
  x ^= x >> 4;
  x ^= x >> 2;
  x ^= x >> 1;
  return (x & 1u) ? -0.0625f : 0.0625f;
}

/* Planted low-rank bias for the 1M-context workload: region r of sequence b
 * is planted with probability 0.02 (same regions for every group).  For a
 * planted (b, r, g) the bias is beta = U_g c with U_g four orthonormal
 * Hadamard rows (rows 1+4g .. 4+4g) and c ~ N(0, 0.25 I_4), so |beta| ~ 1.
 * The same beta is added to each of the region's 8 index_k rows before the
 * single bf16 rounding.  Products c_k * (+-1/16) are exact, so the fixed
 * summation order gives identical fp32 on host and device. */
GEN_FN float gen_planted_beta(uint64_t key_coef, uint64_t breg, uint32_t g, uint32_t n_groups,
                              uint32_t d) {
  uint64_t base = (breg * n_groups + g) * 4u;
  float beta = (0.5f * gen_normal(key_coef, base + 0)) * gen_hadamard16(1u + 4u * g, d);
  beta = beta + (0.5f * gen_normal(key_coef, base + 1)) * gen_hadamard16(2u + 4u * g, d);
  beta = beta + (0.5f * gen_normal(key_coef, base + 2)) * gen_hadamard16(3u + 4u * g, d);
  beta = beta + (0.5f * gen_normal(key_coef, base + 3)) * gen_hadamard16(4u + 4u * g, d);
  return beta;
}

#endif
