/*
 * Device side of the synthetic input generator: writes the same values as
 * gen_host.c straight into GPU buffers, in the physical layouts the attention
 * library consumes, so full-size inputs never cross PCIe.  See gen_core.h.
 *
 * Physical layouts for a logical [B][T][G][C] tensor (token t of sequence b):
 *   GEN_L_GROUP_MAJOR : out[((b*G + g)*tcap + t % tmod)*C + c]
 *   GEN_L_REGION_T    : out[(((b*G + g)*(tcap/8) + s/8)*C + c)*8 + s%8], s = t % tmod
 *                       (8 consecutive tokens of one channel are contiguous)
 *   GEN_L_TOKEN_MAJOR : out[((b*nt + (t - t0))*G + g)*C + c]
 *   GEN_L_KTILED      : out[((b*G + g)*(tcap/8) + s/8)*1536 + koff(s%8, c)], C = 192, with
 *                       koff(p, c) = ((((p/4)*6 + (c%48)/8)*4 + c/48)*4 + p%4)*8 + c%8
 *                       (the attention library's key layout: MFMA A-operand order)
 * tmod is the ring size for ring buffers, or >= tcap for plain caches.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "gen_core.h"

#define GEN_L_GROUP_MAJOR 0
#define GEN_L_REGION_T 1
#define GEN_L_TOKEN_MAJOR 2
#define GEN_L_KTILED 3

struct GenTok {
  uint64_t key, kmask, kcoef;
  int64_t T, t0, nt, tcap, tmod;
  int32_t B, G, C, layout, planted;
  float scale;
};

__device__ static inline uint64_t gen_phys(const GenTok& a, int64_t b, int64_t t, int64_t g,
                                           int64_t c) {
  if (a.layout == GEN_L_TOKEN_MAJOR)
    return (((uint64_t)b * a.nt + (uint64_t)(t - a.t0)) * a.G + g) * a.C + c;
  int64_t s = t % a.tmod;
  if (a.layout == GEN_L_GROUP_MAJOR) return (((uint64_t)b * a.G + g) * a.tcap + s) * a.C + c;
  if (a.layout == GEN_L_KTILED) {
    const int64_t p = s % 8;
    return (((uint64_t)b * a.G + g) * (a.tcap / 8) + s / 8) * 1536 +
           (uint64_t)(((((p / 4) * 6 + (c % 48) / 8) * 4 + c / 48) * 4 + p % 4) * 8 + c % 8);
  }
  return ((((uint64_t)b * a.G + g) * (a.tcap / 8) + s / 8) * a.C + c) * 8 + (s % 8);
}

/* One block per token row (b, t) at a time; the block's threads cover its
 * G*C elements. */
__global__ void gen_tokens_kernel(GenTok a, uint16_t* __restrict__ out) {
  const uint64_t rows = (uint64_t)a.B * a.nt;
  const int32_t row_elems = a.G * a.C;
  for (uint64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    int64_t b = (int64_t)(row / (uint64_t)a.nt);
    int64_t t = a.t0 + (int64_t)(row % (uint64_t)a.nt);
    uint64_t lbase = ((uint64_t)b * a.T + t) * (uint64_t)row_elems;
    uint64_t breg = (uint64_t)b * (uint64_t)(a.T / 8) + (uint64_t)(t / 8);
    int planted = a.planted && gen_bernoulli(a.kmask, breg, GEN_P002_THRESH);
    for (int32_t e = threadIdx.x; e < row_elems; e += blockDim.x) {
      int32_t g = e / a.C, c = e - g * a.C;
      float x = gen_normal(a.key, lbase + (uint64_t)e) * a.scale;
      if (planted) x = x + gen_planted_beta(a.kcoef, breg, (uint32_t)g, (uint32_t)a.G, (uint32_t)c);
      out[gen_phys(a, b, t, g, c)] = gen_bf16_rne(x);
    }
  }
}

__global__ void gen_flat_kernel(uint64_t key, uint64_t start, uint64_t n, float scale, int kind,
                                void* __restrict__ out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (kind == 0)
      ((uint16_t*)out)[i] = gen_bf16_rne(gen_normal(key, start + i) * scale);
    else if (kind == 1)
      ((float*)out)[i] = gen_uniform(key, start + i);
    else
      ((float*)out)[i] = gen_normal(key, start + i) * scale;
  }
}

static int gen_grid(uint64_t total) {
  uint64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

extern "C" {

/* Returns 0 on success, else the hipError_t of the launch. */
int dsagen_dev_tokens(uint64_t seed, uint32_t tid, uint32_t tid_mask, uint32_t tid_coef,
                      int planted, int32_t B, int64_t T, int32_t G, int32_t C, int64_t t0,
                      int64_t nt, int64_t tcap, int64_t tmod, int32_t layout, float scale,
                      uint16_t* out, hipStream_t stream) {
  if (B <= 0 || nt <= 0) return 0;
  if (layout < 0 || layout > 3 || G <= 0 || C <= 0 || t0 < 0 || t0 + nt > T) return 1;
  if (layout == GEN_L_KTILED && C != 192) return 1;
  if (layout != GEN_L_TOKEN_MAJOR &&
      (tmod <= 0 || tcap <= 0 || ((layout == GEN_L_REGION_T || layout == GEN_L_KTILED) && (tcap % 8 || tmod % 8))))
    return 1;
  if (layout != GEN_L_TOKEN_MAJOR && tmod > tcap) return 1;
  GenTok a;
  a.key = gen_stream_key(seed, tid);
  a.kmask = gen_stream_key(seed, tid_mask);
  a.kcoef = gen_stream_key(seed, tid_coef);
  a.T = T; a.t0 = t0; a.nt = nt; a.tcap = tcap; a.tmod = tmod;
  a.B = B; a.G = G; a.C = C; a.layout = layout; a.planted = planted; a.scale = scale;
  uint64_t rows = (uint64_t)B * nt;
  int grid = rows > 262144 ? 262144 : (int)rows;
  hipLaunchKernelGGL(gen_tokens_kernel, dim3(grid), dim3(256), 0, stream, a, out);
  return (int)hipGetLastError();
}

/* kind 0: bf16 normal*scale, 1: f32 uniform, 2: f32 normal*scale. */
int dsagen_dev_flat(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float scale, int kind,
                    void* out, hipStream_t stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(gen_flat_kernel, dim3(gen_grid(n)), dim3(256), 0, stream,
                     gen_stream_key(seed, tid), start, n, scale, kind, out);
  return (int)hipGetLastError();
}
}
