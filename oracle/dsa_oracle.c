/*
 * ORACLE -- test infrastructure, not product code.
 *
 * A plain, slow CPU statement of what the DSA sparse-attention layer of
 * Step-5-Preview's full-attention layers computes, used only by tests/, by the
 * smoke check and by the benchmark's CPU-baseline leg.  It shares no code,
 * header, table or constant generator with the HIP library, and nothing in
 * the product may call it.
 *
 * Pages cited (title, address):
 *  [P1] Step-5-Preview long-context explainer (no title in the extract),
 *       kwkr.cn/news/601179
 *  [P2] "Step-5-Preview 如何实现1M长上下文？滑窗+DSA稀疏注意力混合机制完整揭秘",
 *       yfxerp.com/news/376439
 *  [P3] "100 万 token 上下文实测：Step 5 Preview 一次能吞下多大的工程",
 *       kwkr.cn/news/593658
 *
 * Layouts here are the plain logical ones, one sequence at a time:
 *   index_k, K, V : [T][G][C] (token-major), bf16 bits
 *   index_q       : [Hi][P] bf16 bits, z : [Hi] fp32
 *   q             : [Hq][D] bf16 bits
 *   codes         : [R][G][P] e4m3fn bytes, scales : [R][G] fp32
 *
 * Precision: fp64 everywhere except region compression, whose result is a
 * set of integer codes; that decision is taken in fp32, the precision of the
 * GPU kernel, in the fixed order written below.
 *
 * Pins (tests/test_oracle_*.py): e4m3 against brute-force nearest-code search;
 * compression against closed forms; scores against one-hot closed forms and a
 * brute-force numpy evaluation; selection against exhaustive subset search;
 * attention against torch's scaled_dot_product_attention in fp64 when every
 * region is selected (dense causal GQA) and against a banded mask (window).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops below use (reported with CPU timings). */
int or_num_threads(void) { return omp_get_max_threads(); }

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static float bf16_value_f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ---------------------------------------------------------------------------
 * OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7),
 * 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448,
 * subnormals m * 2^-9.  Region summaries are kept in 8-bit floating point
 * ([P1] section DSA 稀疏注意力, four-step list, step ②; [P2] section 区域压缩（CSA）).
 * ------------------------------------------------------------------------- */
double or_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -mag : mag;
}

/* Round to the nearest representable E4M3 value, ties to the even code,
 * values beyond the range saturate to +-448 (never NaN). */
uint8_t or_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  /* spacing of representable values around a */
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int lo_exp = e - 1;
  if (a < ldexp(1.0, -6)) lo_exp = -6; /* subnormal range shares the spacing of [2^-6, 2^-5) */
  double quantum = ldexp(1.0, lo_exp - 3);
  double v = nearbyint(a / quantum) * quantum; /* default mode: nearest, ties to even */
  if (v == 0.0) return sign;
  if (v < ldexp(1.0, -6)) return sign | (uint8_t)(v / ldexp(1.0, -9));
  int e2;
  double f = frexp(v, &e2); /* v = f * 2^e2, f in [0.5, 1) */
  int biased = e2 - 1 + 7;
  int mant = (int)((2.0 * f - 1.0) * 8.0);
  return sign | (uint8_t)(biased << 3) | (uint8_t)mant;
}

/* ---------------------------------------------------------------------------
 * Region compression ([P1] section DSA 稀疏注意力, four-step list, steps ① and ②: 8-token
 * regions, one 256-d summary each; [P2] section 区域压缩（CSA）: a summary is
 * made only once a region holds all 8 tokens).  The pages do not give the summary's maths; the stand-in
 * rule is: summary = mean of the region's 8 index_k rows of the group,
 * quantised to E4M3 with one fp32 scale per (region, group) equal to
 * amax / 448.  Mean: fp32 sum in token order, then * 0.125.  Codes: fp32
 * division m/scale, one rounding to E4M3.  scale == 0 gives all-zero codes.
 * ------------------------------------------------------------------------- */
void or_compress_region(const uint16_t* ik, int64_t T, int G, int P, int64_t r, int g,
                        uint8_t* codes, float* scale) {
  float* m = (float*)malloc(sizeof(float) * (size_t)P);
  (void)T;
  float amax = 0.0f;
  for (int d = 0; d < P; ++d) {
    float s = bf16_value_f(ik[((8 * r + 0) * G + g) * (int64_t)P + d]);
    for (int t = 1; t < 8; ++t) s = s + bf16_value_f(ik[((8 * r + t) * G + g) * (int64_t)P + d]);
    m[d] = s * 0.125f;
    if (fabsf(m[d]) > amax) amax = fabsf(m[d]);
  }
  float sc = amax / 448.0f;
  *scale = sc;
  for (int d = 0; d < P; ++d) codes[d] = (sc == 0.0f) ? 0x00 : or_e4m3_encode(m[d] / sc);
  free(m);
}

/* All complete regions r in [r0, r1) of one sequence, every group. */
void or_compress_regions(const uint16_t* ik, int64_t T, int G, int P, int64_t r0, int64_t r1,
                         uint8_t* codes, float* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = r0; r < r1; ++r)
    for (int g = 0; g < G; ++g)
      or_compress_region(ik, T, G, P, r, g, codes + (r * G + g) * (int64_t)P, scales + r * G + g);
}

/* ---------------------------------------------------------------------------
 * Indexer score of one region for one query and group ([P2] section
 * 索引器打分 + Top-K 选择: score_regions rates every region summary of the
 * request against the query).  The 16 indexer heads map 4 per KV group ([P2]
 * same section, closing note: regions are tied one-to-one to the 4 GQA groups).  Stand-in maths: s_g(r) = sum over heads h of group g
 * of z_h * ReLU(q_h . S_g[r]), with S = dequantised summary (code value * scale).
 * ------------------------------------------------------------------------- */
double or_region_score(const uint16_t* iq, const float* z, const uint8_t* codes, float scale,
                       int P, int g, int heads_per_group) {
  double s = 0.0;
  for (int h = g * heads_per_group; h < (g + 1) * heads_per_group; ++h) {
    double dot = 0.0;
    for (int d = 0; d < P; ++d)
      dot += bf16_value(iq[(int64_t)h * P + d]) * (or_e4m3_value(codes[d]) * (double)scale);
    s += (double)z[h] * (dot > 0.0 ? dot : 0.0);
  }
  return s;
}

/* Scores of regions [0, n_regions) for every group: out[g][r]. */
void or_scores(const uint16_t* iq, const float* z, const uint8_t* codes, const float* scales,
               int G, int P, int heads_per_group, int64_t n_regions, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_regions; ++r)
    for (int g = 0; g < G; ++g)
      out[(int64_t)g * n_regions + r] = or_region_score(
          iq, z, codes + (r * G + g) * (int64_t)P, scales[r * G + g], P, g, heads_per_group);
}

/* ---------------------------------------------------------------------------
 * Top-k region selection ([P1] section DSA 稀疏注意力, four-step list, step ③: keep the 512
 * best-scoring regions; [P2] section 索引器打分 + Top-K 选择: the region holding
 * the query is always kept).  Candidates are the complete
 * regions 0..c-1 before the query's current region c; c itself is always
 * taken (reading: within the k, not on top of it).  Order: score descending,
 * lower region index first on equal scores.  Output ascending, count
 * min(k, c+1).
 * ------------------------------------------------------------------------- */
typedef struct {
  double score;
  int64_t idx;
} or_ranked;

static int cmp_rank(const void* a, const void* b) {
  const or_ranked* x = (const or_ranked*)a;
  const or_ranked* y = (const or_ranked*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}
static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int or_select(const double* scores, int64_t c, int k, int32_t* sel) {
  if (k <= 0) return 0;
  or_ranked* cand = (or_ranked*)malloc(sizeof(or_ranked) * (size_t)(c > 0 ? c : 1));
  for (int64_t i = 0; i < c; ++i) {
    cand[i].score = scores[i];
    cand[i].idx = i;
  }
  qsort(cand, (size_t)c, sizeof(or_ranked), cmp_rank);
  int64_t take = (c < (int64_t)(k - 1)) ? c : (int64_t)(k - 1);
  int n = 0;
  sel[n++] = (int32_t)c;
  for (int64_t i = 0; i < take; ++i) sel[n++] = (int32_t)cand[i].idx;
  qsort(sel, (size_t)n, sizeof(int32_t), cmp_i32);
  free(cand);
  return n;
}

/* ---------------------------------------------------------------------------
 * Sparse GQA ([P1] section DSA 稀疏注意力, four-step list, step ④: attention runs over the real
 * K/V of the selected regions only; [P3] section 一, config table: 64 Q heads
 * in 4 KV groups): head h uses KV group g = h / (Hq/G) and attends to the real
 * K/V of the tokens 8r..min(8r+7, p) of every region r selected for group g.
 * o_h = sum_j softmax_j(tau * q_h . K_j) V_j, fp64, max-subtracted.
 * ------------------------------------------------------------------------- */
void or_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int G, int D, int Hq,
               int64_t p, const int32_t* sel, const int32_t* nsel, int k, double tau, double* out) {
  int hpg = Hq / G;
  int64_t cap = (int64_t)k * 8;
  double* s = (double*)malloc(sizeof(double) * (size_t)cap);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
  for (int h = 0; h < Hq; ++h) {
    int g = h / hpg;
    int64_t n = 0;
    for (int i = 0; i < nsel[g]; ++i) {
      int64_t r = sel[(int64_t)g * k + i];
      for (int64_t j = 8 * r; j <= 8 * r + 7 && j <= p; ++j) tok[n++] = j;
    }
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += bf16_value(q[(int64_t)h * D + d]) * bf16_value(K[(tok[t] * G + g) * (int64_t)D + d]);
      s[t] = tau * dot;
      if (s[t] > mx) mx = s[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      s[t] = exp(s[t] - mx);
      den += s[t];
    }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; ++t) acc += s[t] * bf16_value(V[(tok[t] * G + g) * (int64_t)D + d]);
      out[(int64_t)h * D + d] = n ? acc / den : 0.0;
    }
  }
  free(s);
  free(tok);
}

/* ---------------------------------------------------------------------------
 * FP8 K/V cache ([P3] section 一: keeping the KV cache in FP8 halves its size).
 * The pages give no quantisation rule for it; the stand-in is the summary
 * rule applied to every cached row: one fp32 scale per (token, group) row of
 * K or V equal to amax / 448 over the row's bf16 values, each value divided
 * by the scale in fp32 and rounded once to E4M3; scale 0 gives zero codes.
 * X is [n_rows][C] bf16 bits; codes [n_rows][C], scales [n_rows].
 * ------------------------------------------------------------------------- */
void or_quantize_rows(const uint16_t* X, int64_t n_rows, int C, uint8_t* codes, float* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    float amax = 0.0f;
    for (int d = 0; d < C; ++d) {
      float a = fabsf(bf16_value_f(X[i * C + d]));
      if (a > amax) amax = a;
    }
    float sc = amax / 448.0f;
    scales[i] = sc;
    for (int d = 0; d < C; ++d)
      codes[i * C + d] = (sc == 0.0f) ? 0x00 : or_e4m3_encode(bf16_value_f(X[i * C + d]) / sc);
  }
}

/* Sparse GQA over an FP8 cache: the sum of or_attend with every K and V value
 * taken as the E4M3 value of its code times its row's scale (fp64).
 * Kc, Vc [T][G][D] codes; Ks, Vs [T][G] scales. */
void or_attend_fp8(const uint16_t* q, const uint8_t* Kc, const float* Ks, const uint8_t* Vc, const float* Vs,
                   int G, int D, int Hq, int64_t p, const int32_t* sel, const int32_t* nsel, int k, double tau,
                   double* out) {
  int hpg = Hq / G;
  int64_t cap = (int64_t)k * 8;
  double* s = (double*)malloc(sizeof(double) * (size_t)cap);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
  for (int h = 0; h < Hq; ++h) {
    int g = h / hpg;
    int64_t n = 0;
    for (int i = 0; i < nsel[g]; ++i) {
      int64_t r = sel[(int64_t)g * k + i];
      for (int64_t j = 8 * r; j <= 8 * r + 7 && j <= p; ++j) tok[n++] = j;
    }
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      int64_t row = tok[t] * G + g;
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += bf16_value(q[(int64_t)h * D + d]) * (or_e4m3_value(Kc[row * D + d]) * (double)Ks[row]);
      s[t] = tau * dot;
      if (s[t] > mx) mx = s[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      s[t] = exp(s[t] - mx);
      den += s[t];
    }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        int64_t row = tok[t] * G + g;
        acc += s[t] * (or_e4m3_value(Vc[row * D + d]) * (double)Vs[row]);
      }
      out[(int64_t)h * D + d] = n ? acc / den : 0.0;
    }
  }
  free(s);
  free(tok);
}

/* ---------------------------------------------------------------------------
 * Sliding-window attention ([P1] section 滑窗注意力只读最近 512 个 token:
 * a 512-token window; [P2] section 512 Token 的环形缓冲区): the query at position p attends to positions
 * max(0, p-W+1) .. p (W keys including itself), read here from the full K/V
 * history rather than a ring so that the ring logic of the GPU path is
 * checked independently.
 * ------------------------------------------------------------------------- */
void or_swa(const uint16_t* q, const uint16_t* K, const uint16_t* V, int G, int D, int Hq,
            int64_t p, int64_t W, double tau, double* out) {
  int hpg = Hq / G;
  int64_t lo = p - W + 1 < 0 ? 0 : p - W + 1;
  int64_t n = p - lo + 1;
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  for (int h = 0; h < Hq; ++h) {
    int g = h / hpg;
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += bf16_value(q[(int64_t)h * D + d]) * bf16_value(K[((lo + t) * G + g) * (int64_t)D + d]);
      s[t] = tau * dot;
      if (s[t] > mx) mx = s[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      s[t] = exp(s[t] - mx);
      den += s[t];
    }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < n; ++t) acc += s[t] * bf16_value(V[((lo + t) * G + g) * (int64_t)D + d]);
      out[(int64_t)h * D + d] = acc / den;
    }
  }
  free(s);
}

/* ---------------------------------------------------------------------------
 * One query of the DSA layer end to end, given the summaries of the regions
 * before it: scores of the complete candidate regions, top-k per group with
 * the current region forced, sparse GQA.  scores_out (nullable) gets
 * [G][c] scores.  Returns nothing; sel [G][k], nsel [G], out [Hq][D].
 * ------------------------------------------------------------------------- */
void or_dsa_query(const uint16_t* iq, const float* z, const uint8_t* codes, const float* scales,
                  const uint16_t* q, const uint16_t* K, const uint16_t* V, int G, int P, int Hi,
                  int D, int Hq, int k, double tau, int64_t p, int32_t* sel, int32_t* nsel,
                  double* out, double* scores_out) {
  int64_t c = p / 8;
  double* sc = scores_out ? scores_out : (double*)malloc(sizeof(double) * (size_t)(G * (c > 0 ? c : 1)));
  or_scores(iq, z, codes, scales, G, P, Hi / G, c, sc);
  for (int g = 0; g < G; ++g) nsel[g] = or_select(sc + (int64_t)g * c, c, k, sel + (int64_t)g * k);
  or_attend(q, K, V, G, D, Hq, p, sel, nsel, k, tau, out);
  if (!scores_out) free(sc);
}
