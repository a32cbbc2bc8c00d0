/*
 * Host side of the synthetic input generator: fills host buffers in the
 * logical (token-major) layouts used by the CPU oracle harness.
 * See gen_core.h for the definition of every draw.
 */
#include <stdint.h>
#include "gen_core.h"

/* out[i] = bf16(normal(seed, tid, start + i) * scale), scale a power of two. */
void dsagen_normal_bf16(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float scale,
                        uint16_t* out) {
  uint64_t key = gen_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = gen_bf16_rne(gen_normal(key, start + (uint64_t)i) * scale);
}

/* out[i] = normal(seed, tid, start + i) * scale as fp32. */
void dsagen_normal_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float scale,
                       float* out) {
  uint64_t key = gen_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = gen_normal(key, start + (uint64_t)i) * scale;
}

void dsagen_uniform_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float* out) {
  uint64_t key = gen_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = gen_uniform(key, start + (uint64_t)i);
}

void dsagen_bernoulli_u8(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, uint32_t thresh,
                         uint8_t* out) {
  uint64_t key = gen_stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = (uint8_t)gen_bernoulli(key, start + (uint64_t)i, thresh);
}

/*
 * Slice of a 4-d logical tensor [B][T][G][C] of N(0,1)*scale bf16 values:
 * tokens [t0, t0+nt) of sequence b, written to out[nt][G][C].
 * Logical flat index = ((b*T + t)*G + g)*C + c.
 */
void dsagen_tokens_bf16(uint64_t seed, uint32_t tid, int64_t T, int32_t G, int32_t C, int32_t b,
                        int64_t t0, int64_t nt, float scale, uint16_t* out) {
  uint64_t key = gen_stream_key(seed, tid);
  uint64_t row = (uint64_t)G * (uint64_t)C;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < nt; ++t) {
    uint64_t base = ((uint64_t)b * (uint64_t)T + (uint64_t)(t0 + t)) * row;
    for (uint64_t e = 0; e < row; ++e)
      out[(uint64_t)t * row + e] = gen_bf16_rne(gen_normal(key, base + e) * scale);
  }
}

/*
 * Slice of index_k [B][T][G][P] (N(0,1)/16, tensor id tid): tokens [t0, t0+nt)
 * of sequence b, to out[nt][G][P].  With planted != 0 the low-rank bias of
 * gen_planted_beta is added to every row of each planted region (mask stream
 * tid_mask, coefficient stream tid_coef, regions of 8 tokens).
 */
void dsagen_index_k(uint64_t seed, uint32_t tid, uint32_t tid_mask, uint32_t tid_coef, int planted,
                    int64_t T, int32_t G, int32_t P, int32_t b, int64_t t0, int64_t nt,
                    uint16_t* out) {
  uint64_t key = gen_stream_key(seed, tid);
  uint64_t kmask = gen_stream_key(seed, tid_mask);
  uint64_t kcoef = gen_stream_key(seed, tid_coef);
  int64_t R = T / 8;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < nt; ++t) {
    int64_t tok = t0 + t;
    uint64_t breg = (uint64_t)b * (uint64_t)R + (uint64_t)(tok / 8);
    int is_planted = planted && gen_bernoulli(kmask, breg, GEN_P002_THRESH);
    for (int32_t g = 0; g < G; ++g) {
      uint64_t base = (((uint64_t)b * (uint64_t)T + (uint64_t)tok) * (uint64_t)G + (uint64_t)g) *
                      (uint64_t)P;
      for (int32_t d = 0; d < P; ++d) {
        float x = gen_normal(key, base + (uint64_t)d) * 0.0625f;
        if (is_planted) x = x + gen_planted_beta(kcoef, breg, (uint32_t)g, (uint32_t)G, (uint32_t)d);
        out[((uint64_t)t * (uint64_t)G + (uint64_t)g) * (uint64_t)P + (uint64_t)d] = gen_bf16_rne(x);
      }
    }
  }
}
