/*
 * Test driver (not product code): runs every function of the CPU oracle
 * (oracle/dsa_oracle.c) on small inputs held in exactly sized heap buffers,
 * so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * reports any out-of-bounds access, use of freed memory or undefined
 * arithmetic in the oracle.  Edge cases: position 0, a partial current
 * region, k above and below the candidate count, k = 1, all-zero summaries,
 * a window wider than the history.  Prints "ok" and returns 0 when every
 * invariant below holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double or_e4m3_value(uint8_t code);
uint8_t or_e4m3_encode(float x);
void or_compress_regions(const uint16_t* ik, int64_t T, int G, int P, int64_t r0, int64_t r1,
                         uint8_t* codes, float* scales);
void or_scores(const uint16_t* iq, const float* z, const uint8_t* codes, const float* scales,
               int G, int P, int heads_per_group, int64_t n_regions, double* out);
int or_select(const double* scores, int64_t c, int k, int32_t* sel);
void or_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int G, int D, int Hq,
               int64_t p, const int32_t* sel, const int32_t* nsel, int k, double tau, double* out);
void or_quantize_rows(const uint16_t* X, int64_t n_rows, int C, uint8_t* codes, float* scales);
void or_attend_fp8(const uint16_t* q, const uint8_t* Kc, const float* Ks, const uint8_t* Vc, const float* Vs,
                   int G, int D, int Hq, int64_t p, const int32_t* sel, const int32_t* nsel, int k, double tau,
                   double* out);
void or_swa(const uint16_t* q, const uint16_t* K, const uint16_t* V, int G, int D, int Hq,
            int64_t p, int64_t W, double tau, double* out);
void or_dsa_query(const uint16_t* iq, const float* z, const uint8_t* codes, const float* scales,
                  const uint16_t* q, const uint16_t* K, const uint16_t* V, int G, int P, int Hi,
                  int D, int Hq, int k, double tau, int64_t p, int32_t* sel, int32_t* nsel,
                  double* out, double* scores_out);

enum { G = 4, P = 256, HI = 16, HQ = 64, D = 192 };

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) { /* xorshift64*, test inputs only */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static uint16_t rand_bf16(float scale) {
  float x = ((float)next_u32() / 4294967296.0f - 0.5f) * 4.0f * scale;
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}
static int failures = 0;
#define CHECK(cond, what)                              \
  do {                                                 \
    if (!(cond)) {                                     \
      fprintf(stderr, "invariant failed: %s\n", what); \
      ++failures;                                      \
    }                                                  \
  } while (0)

static void run_query(int64_t T, int64_t p, int k, int zero_index_k) {
  const int64_t R = T / 8, c = p / 8;
  uint16_t* ik = xmalloc(sizeof(uint16_t) * (size_t)(T * G * P));
  uint16_t* K = xmalloc(sizeof(uint16_t) * (size_t)(T * G * D));
  uint16_t* V = xmalloc(sizeof(uint16_t) * (size_t)(T * G * D));
  uint16_t* iq = xmalloc(sizeof(uint16_t) * HI * P);
  uint16_t* q = xmalloc(sizeof(uint16_t) * HQ * D);
  float* z = xmalloc(sizeof(float) * HI);
  for (int64_t i = 0; i < T * G * P; ++i) ik[i] = zero_index_k ? 0 : rand_bf16(1.0f / 16);
  for (int64_t i = 0; i < T * G * D; ++i) {
    K[i] = rand_bf16(1.0f);
    V[i] = rand_bf16(1.0f);
  }
  for (int i = 0; i < HI * P; ++i) iq[i] = rand_bf16(1.0f / 16);
  for (int i = 0; i < HQ * D; ++i) q[i] = rand_bf16(1.0f);
  for (int i = 0; i < HI; ++i) z[i] = (float)next_u32() / 4294967296.0f;

  /* summaries of the complete regions only */
  uint8_t* codes = xmalloc((size_t)(R * G * P));
  float* scales = xmalloc(sizeof(float) * (size_t)(R * G));
  or_compress_regions(ik, T, G, P, 0, R, codes, scales);
  for (int64_t i = 0; i < R * G; ++i) CHECK(scales[i] >= 0.0f, "scale >= 0");

  /* scores of the candidates 0..c-1, exactly c per group */
  double* sc = xmalloc(sizeof(double) * (size_t)(G * (c > 0 ? c : 0)));
  if (c > 0) or_scores(iq, z, codes, scales, G, P, HI / G, c, sc);
  for (int64_t i = 0; i < G * c; ++i) CHECK(sc[i] >= 0.0, "score >= 0");

  /* selection, the end-to-end query and the attention on its selection */
  int32_t* sel = xmalloc(sizeof(int32_t) * (size_t)(G * k));
  int32_t* nsel = xmalloc(sizeof(int32_t) * G);
  double* out = xmalloc(sizeof(double) * HQ * D);
  double* sc2 = xmalloc(sizeof(double) * (size_t)(G * (c > 0 ? c : 1)));
  for (int i = 0; i < G * k; ++i) sel[i] = -1;
  or_dsa_query(iq, z, codes, scales, q, K, V, G, P, HI, D, HQ, k, 1.0 / sqrt((double)D), p, sel, nsel, out, sc2);
  for (int g = 0; g < G; ++g) {
    int32_t* one = xmalloc(sizeof(int32_t) * (size_t)k);
    int n = or_select(sc + (int64_t)g * c, c, k, one);
    CHECK(n == nsel[g], "select count matches the end-to-end query");
    CHECK(n == (c + 1 < k ? c + 1 : k), "count = min(k, c + 1)");
    int has_c = 0;
    for (int i = 0; i < n; ++i) {
      CHECK(one[i] == sel[(int64_t)g * k + i], "same selection");
      CHECK(i == 0 || one[i] > one[i - 1], "ascending");
      has_c |= one[i] == c;
    }
    CHECK(has_c, "current region selected");
    free(one);
  }
  double* out2 = xmalloc(sizeof(double) * HQ * D);
  or_attend(q, K, V, G, D, HQ, p, sel, nsel, k, 1.0 / sqrt((double)D), out2);
  for (int i = 0; i < HQ * D; ++i) CHECK(out[i] == out2[i] && isfinite(out[i]), "attention repeatable, finite");

  /* FP8 rows of the same K/V and attention over them */
  uint8_t* kc = xmalloc((size_t)(T * G * D));
  uint8_t* vc = xmalloc((size_t)(T * G * D));
  float* ks = xmalloc(sizeof(float) * (size_t)(T * G));
  float* vs = xmalloc(sizeof(float) * (size_t)(T * G));
  or_quantize_rows(K, T * G, D, kc, ks);
  or_quantize_rows(V, T * G, D, vc, vs);
  or_attend_fp8(q, kc, ks, vc, vs, G, D, HQ, p, sel, nsel, k, 1.0 / sqrt((double)D), out2);
  for (int i = 0; i < HQ * D; ++i) CHECK(isfinite(out2[i]), "fp8 attention finite");

  /* sliding window over the history 0..p (window wider and narrower than it) */
  or_swa(q, K, V, G, D, HQ, p, 512, 1.0 / sqrt((double)D), out2);
  or_swa(q, K, V, G, D, HQ, p, 3, 1.0 / sqrt((double)D), out2);
  for (int i = 0; i < HQ * D; ++i) CHECK(isfinite(out2[i]), "window attention finite");

  free(ik); free(K); free(V); free(iq); free(q); free(z); free(codes); free(scales); free(sc);
  free(sel); free(nsel); free(out); free(sc2); free(out2); free(kc); free(vc); free(ks); free(vs);
}

int main(void) {
  for (int c = 0; c < 256; ++c) {
    const double v = or_e4m3_value((uint8_t)c);
    if ((c & 0x7F) != 0x7F) CHECK(or_e4m3_encode((float)v) == (uint8_t)c || v == 0.0, "code round trip");
  }
  const float specials[] = {0.0f, -0.0f, 448.0f, 464.0f, -1e30f, 1e30f, 0x1p-9f, 0x1p-10f, 0x1.8p-10f};
  for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) (void)or_e4m3_encode(specials[i]);
  run_query(8, 0, 512, 0);     /* position 0: only region 0, nothing to score */
  run_query(40, 37, 3, 0);     /* partial current region, k below the candidates */
  run_query(40, 39, 512, 0);   /* k above the candidates */
  run_query(64, 63, 1, 0);     /* k = 1: only the current region */
  run_query(64, 50, 4, 1);     /* all-zero summaries: every score 0, ties to the lowest */
  run_query(720, 700, 16, 0);  /* history longer than the window */
  if (failures) {
    fprintf(stderr, "%d invariant(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
