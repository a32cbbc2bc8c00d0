// Region compression, device side (shared by the compression kernel and the
// decode step, which folds the compression of the region its query token
// completes into the scoring launch).
//
// Summary rule ([P1] kwkr.cn/news/601179, section DSA 稀疏注意力, steps ①②;
// [P2] yfxerp.com/news/376439, section 区域压缩（CSA）: every complete region of
// 8 tokens becomes one 256-d summary stored in FP8).  The pages give no maths
// for the summary; the stand-in rule is the mean of the 8 index_k rows of the
// group, quantised to OCP E4M3 with one fp32 scale amax/448 per (region,
// group).
#pragma once
#include "common.hpp"

namespace dsa {

// fp32 -> OCP E4M3 (e4m3fn): round to nearest even, saturate to +-448,
// keep the sign of zero.  Written from the format definition: normal values
// keep 3 mantissa bits (rounding on the fp32 bit pattern, the carry moves into
// the exponent), values below 2^-6 are multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  float af = __uint_as_float(a);
  if (af >= 448.0f) return sign | 0x7Eu;
  if (af < 0.015625f) return sign | (uint32_t)__builtin_rintf(af * 512.0f);
  uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

// One wave compresses region r of group g of sequence b: lane l owns
// channels 4l..4l+3.  index_k rows, summaries (tiled layout) and scales are
// found through the cache map (contiguous or paged).
__device__ __forceinline__ void compress_region_wave(const uint16_t* __restrict__ ik, const CacheMap& cm,
                                                     int64_t b, int64_t r, int g, uint8_t* __restrict__ summ,
                                                     float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t slot = region_slot(cm, b, g, r);
  const uint16_t* src = ik + slot * kRegion * kProxy + 4 * lane;
  uint2 row[kRegion];
#pragma unroll
  for (int t = 0; t < kRegion; ++t) row[t] = *(const uint2*)(src + (int64_t)t * kProxy);
  float m[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w0 = (e < 2) ? row[0].x : row[0].y;
    float s = __uint_as_float((e & 1) ? (w0 & 0xFFFF0000u) : (w0 << 16));
#pragma unroll
    for (int t = 1; t < kRegion; ++t) {
      const uint32_t w = (e < 2) ? row[t].x : row[t].y;
      s = s + __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    m[e] = s * 0.125f;
  }
  float amax = fmaxf(fmaxf(fabsf(m[0]), fabsf(m[1])), fmaxf(fabsf(m[2]), fabsf(m[3])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float sc = __fdiv_rn(amax, 448.0f);
  uint32_t packed = 0;
  if (sc != 0.0f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) packed |= e4m3_rne_sat(__fdiv_rn(m[e], sc)) << (8 * e);
  }
  // channels 4l..4l+3 of the region in its summary tile (slot/16)
  const int64_t off = summ_tile_base(slot) + (lane >> 4) * 1024 + ((lane & 15) >> 2) * 256 + (slot & 15) * 16 +
                      4 * (lane & 3);
  *(uint32_t*)(summ + off) = packed;
  if (lane == 0) scale[slot] = sc;
}

}  // namespace dsa
