// Sparse GQA (decode and chunked prefill) and sliding-window attention.
//
// [P1] kwkr.cn/news/601179, section DSA 稀疏注意力, step ④: attention runs over
// the real K/V of the selected regions only; [P3] kwkr.cn/news/593658, section
// 一: 64 query heads in 4 KV groups (GQA), kernels sparse_attention_prefill /
// _decode; [P2] yfxerp.com/news/376439, sections 512 Token 的环形缓冲区 and
// 给预填充做的小优化 for the sliding-window layers (512-slot ring written at
// position mod 512; banded prefill).
//
// One MFMA core serves every form.  A wave owns one (query, KV group): the 16
// query heads of the group are the N = 16 side of v_mfma_f32_16x16x32_bf16,
// so GQA maps onto the matrix cores without padding.  Regions are consumed
// four at a time (32 tokens):
//   S^T[token][head] = K(32x192) . Q^T  -> 2 tiles x 6 k-steps, A = K read
//     straight from the region-tiled K layout (one 16-byte load = 8 channels
//     of one token; a wave's load = four contiguous 256-byte pieces), B = Q^T
//     in registers.  Tile t row m holds token 8*(m/4) + 4t + m%4, which leaves
//     every lane with the 8 tokens of one region in order;
//   O^T[dv][head] += V^T(192x32) . P^T  -> 12 tiles, A = V^T read straight
//     from the region-transposed V layout (one 16-byte load = the 8 tokens of
//     a region for one channel), B = the lane's own 8 softmax weights.
// The core can keep O^T for a slice of the channels only (NT of the 12
// tiles): the sliding-window decode splits the output channels over blocks.
// Online softmax in fp32 (exp2 domain), weights rounded to bf16 for the PV
// product.  Masked positions get weight 0 and their V is zeroed, so stale or
// uninitialised cache rows can never leak in.
#include <math.h>
#include <type_traits>

#include "common.hpp"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;

// One region as the core sees it: its 1536 keys (region-tiled), its V pack
// [D][8], and the range [lo, hi] of valid positions inside the region
// (lo > hi: nothing valid).
struct Region {
  const uint16_t* k;
  const uint16_t* v;
  int lo, hi;
  // patched loads only (sliding-window decode): token tn of the region (-1:
  // none) is read from the new K/V row kn/vn (token-major [D]) instead; vn
  // must be readable whenever any lane of the wave patches
  const uint16_t* kn;
  const uint16_t* vn;
  int tn;
};

// A wave's running state: O^T tiles (NT tiles of 16 channels), the lane's
// reference max and partial denominator.
template <int NT>
struct CoreStateN {
  f32x4 o[NT];
  float m, l;
};
using CoreState = CoreStateN<12>;

template <int NT>
__device__ __forceinline__ void core_init(CoreStateN<NT>& st) {
#pragma unroll
  for (int i = 0; i < NT; ++i) st.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.0f;
}

// Q^T operand of head (16g + n) of query row `qrow`: channels 48kb + 8s + e.
__device__ __forceinline__ void load_q(const uint16_t* q, int64_t qrow, int g, bf16x8 qb[6]) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const uint16_t* p = q + (qrow * kQHeads + kHeadsPerGroup * g + n) * kHeadDim + 48 * kb;
#pragma unroll
  for (int s = 0; s < 6; ++s) qb[s] = as_bf16x8(ld16(p + 8 * s));
}

// The 4-region chunk as held in registers between its loads and its use:
// K rows of tile 0 and tile 1 (lane: one token, 48 channels) and the 12
// V^T operands (lane: one channel, the 8 tokens of region kb), plus the valid
// position range of the lane's softmax region.  NT < 12: the V^T operands of
// NT tiles only (16*NT channels from Region::v / Region::vn on).
template <int NT>
struct ChunkRegsN {
  u32x4 k0[6], k1[6], v[NT];
  int lo, hi;
  uint32_t vpatch[NT];  // patched loads only: the new token's V (channel 16nt + n) and its slot
  int tn;
};
using ChunkRegs = ChunkRegsN<12>;

// Issues the chunk's loads. ra = region of this lane's K rows (entry n/4),
// rb = region of this lane's softmax weights and V pack (entry kb).  PATCH:
// Region::tn / kn / vn are honoured.
template <bool PATCH = false, int NT = 12>
__device__ __forceinline__ void core_load(ChunkRegsN<NT>& c, const Region& ra, const Region& rb) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  // region-tiled K: unit ((t*6 + s)*4 + kb)*4 + (n&3) holds token 4t + n%4,
  // channels 48kb + 8s .. +7
  const uint16_t* kp = ra.k + (kb * 4 + (n & 3)) * 8;
  if constexpr (PATCH) {
    const bool p0 = ra.tn == (n & 3), p1 = ra.tn == 4 + (n & 3);
    const uint16_t* kn = ra.kn + 48 * kb;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      c.k0[s] = ld16(p0 ? kn + 8 * s : kp + (s * 16) * 8);
      c.k1[s] = ld16(p1 ? kn + 8 * s : kp + ((6 + s) * 16) * 8);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      c.k0[s] = ld16(kp + (s * 16) * 8);
      c.k1[s] = ld16(kp + ((6 + s) * 16) * 8);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) c.v[nt] = ld16(rb.v + (16 * nt + n) * 8);
  if constexpr (PATCH) {  // the new token's V, put into element tn when the chunk is used
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) c.vpatch[nt] = rb.vn[16 * nt + n];
    c.tn = rb.tn;
  }
  c.lo = rb.lo;
  c.hi = rb.hi;
}

// Puts the new token's V (patched loads) into element tn of the lane's V
// units; nothing when tn < 0.
template <int NT>
__device__ __forceinline__ void core_apply_patch(ChunkRegsN<NT>& c) {
  const int t = c.tn;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint32_t x = c.vpatch[nt];
    const uint32_t keep = (t & 1) ? 0x0000FFFFu : 0xFFFF0000u, put = (t & 1) ? x << 16 : x;
    c.v[nt].x = (t >> 1 == 0) ? (c.v[nt].x & keep) | put : c.v[nt].x;
    c.v[nt].y = (t >> 1 == 1) ? (c.v[nt].y & keep) | put : c.v[nt].y;
    c.v[nt].z = (t >> 1 == 2) ? (c.v[nt].z & keep) | put : c.v[nt].z;
    c.v[nt].w = (t >> 1 == 3) ? (c.v[nt].w & keep) | put : c.v[nt].w;
  }
}

// S^T tiles, online softmax update, O^T += V^T P^T for one loaded chunk.
template <int NT>
__device__ __forceinline__ void core_compute(CoreStateN<NT>& st, const bf16x8 qb[6], ChunkRegsN<NT>& c,
                                             float scale_log2) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    s0 = mfma16x16x32(as_bf16x8(c.k0[s]), qb[s], s0);
    s1 = mfma16x16x32(as_bf16x8(c.k1[s]), qb[s], s1);
  }
  float sv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (i >= c.lo && i <= c.hi) ? s0[i] * scale_log2 : -INFINITY;
    sv[4 + i] = (4 + i >= c.lo && 4 + i <= c.hi) ? s1[i] * scale_log2 : -INFINITY;
  }
  float cmax = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, sv[i]);
  cmax = max_across_rows(cmax);
  // Lazy rescaling: the reference max m only moves (and O, l are rescaled)
  // when some head's running max exceeds it by more than 8 (log2 units), so
  // every weight exp2(s - m) stays <= 256 and most chunks skip the rescale.
  // The first chunk with a valid score always moves m off -inf.
  const float m_new = fmaxf(st.m, cmax);
  if (__any(m_new > st.m + 8.0f)) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 when st.m = -inf
    st.l *= alpha;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) st.o[nt] *= alpha;
    st.m = m_new;
  }
  const float m_use = st.m == -INFINITY ? 0.0f : st.m;  // all masked so far: weights stay 0
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));

  // zero V of masked positions (only regions at the causal/window edge)
  const bool full = (c.lo <= 0 && c.hi >= 7);
  if (__any(!full)) {
    uint32_t mk[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bool a0 = (2 * w >= c.lo && 2 * w <= c.hi);
      const bool a1 = (2 * w + 1 >= c.lo && 2 * w + 1 <= c.hi);
      mk[w] = (a0 ? 0x0000FFFFu : 0u) | (a1 ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      c.v[nt].x &= mk[0];
      c.v[nt].y &= mk[1];
      c.v[nt].z &= mk[2];
      c.v[nt].w &= mk[3];
    }
  }
  u32x4 pp;
  pp.x = pack_bf16x2(p[0], p[1]);
  pp.y = pack_bf16x2(p[2], p[3]);
  pp.z = pack_bf16x2(p[4], p[5]);
  pp.w = pack_bf16x2(p[6], p[7]);
  const bf16x8 pb = as_bf16x8(pp);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) st.o[nt] = mfma16x16x32(as_bf16x8(c.v[nt]), pb, st.o[nt]);
}

// One chunk, loads then compute (no overlap).  The scheduling barrier keeps
// every K and V load issued before the first MFMA waits on any of them.
__device__ __forceinline__ void core_chunk(CoreState& st, const bf16x8 qb[6], const Region& ra,
                                           const Region& rb, float scale_log2) {
  ChunkRegs c;
  core_load(c, ra, rb);
  __builtin_amdgcn_sched_barrier(0);
  core_compute(st, qb, c, scale_log2);
}

// A run of chunks.  region_of(e, lane) gives the Region for list entry e as
// seen by this lane; entries >= n are invalid.  DEPTH 0: one chunk in
// registers (for kernels running several waves per SIMD, which overlap each
// other's loads); DEPTH 1 and 2: one and two chunks' loads in flight while a
// chunk computes (one wave per SIMD).
template <int DEPTH, bool PATCH = false, int NT = 12, class RegionOf>
__device__ __forceinline__ void core_run(CoreStateN<NT>& st, const bf16x8 qb[6], int64_t n, const RegionOf& region_of,
                                         float scale_log2) {
  const int lane = threadIdx.x & 63, nn = lane & 15, kb = lane >> 4;
  if (n <= 0) return;
  if constexpr (DEPTH == 0) {
    // one chunk in registers per wave; several waves per SIMD overlap the loads
    for (int64_t e0 = 0; e0 < n; e0 += 4) {
      ChunkRegsN<NT> c;
      core_load<PATCH>(c, region_of(e0 + (nn >> 2)), region_of(e0 + kb));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PATCH) core_apply_patch(c);
      core_compute(st, qb, c, scale_log2);
    }
    return;
  }
  // The prefetch is issued unconditionally (past the end it reads the dummy
  // region of an invalid entry), so the wait before each compute only covers
  // the chunk being used and not the ones in flight behind it.
  if constexpr (DEPTH >= 2) {
  // three chunks in registers: two in flight while one computes
  ChunkRegsN<NT> b0, b1, b2;
  core_load<PATCH>(b0, region_of(nn >> 2), region_of(kb));
  core_load<PATCH>(b1, region_of(4 + (nn >> 2)), region_of(4 + kb));
  for (int64_t e0 = 0; e0 < n; e0 += 12) {
    core_load<PATCH>(b2, region_of(e0 + 8 + (nn >> 2)), region_of(e0 + 8 + kb));
    if constexpr (PATCH) core_apply_patch(b0);
    core_compute(st, qb, b0, scale_log2);
    if (e0 + 4 >= n) break;
    core_load<PATCH>(b0, region_of(e0 + 12 + (nn >> 2)), region_of(e0 + 12 + kb));
    if constexpr (PATCH) core_apply_patch(b1);
    core_compute(st, qb, b1, scale_log2);
    if (e0 + 8 >= n) break;
    core_load<PATCH>(b1, region_of(e0 + 16 + (nn >> 2)), region_of(e0 + 16 + kb));
    if constexpr (PATCH) core_apply_patch(b2);
    core_compute(st, qb, b2, scale_log2);
  }
  } else {
  ChunkRegsN<NT> b0, b1;
  core_load<PATCH>(b0, region_of(nn >> 2), region_of(kb));
  for (int64_t e0 = 0; e0 < n; e0 += 8) {
    core_load<PATCH>(b1, region_of(e0 + 4 + (nn >> 2)), region_of(e0 + 4 + kb));
    if constexpr (PATCH) core_apply_patch(b0);
    core_compute(st, qb, b0, scale_log2);
    if (e0 + 4 >= n) break;
    core_load<PATCH>(b0, region_of(e0 + 8 + (nn >> 2)), region_of(e0 + 8 + kb));
    if constexpr (PATCH) core_apply_patch(b1);
    core_compute(st, qb, b1, scale_log2);
  }
  }
}

// Total softmax denominator of the lane's head (sum over the 4 kb lanes).
template <int NT>
__device__ __forceinline__ float core_total_l(const CoreStateN<NT>& st) {
  return sum_across_rows(st.l);
}

// Writes the normalised output of head (16g + n) of query row qrow.
__device__ __forceinline__ void core_store(const CoreState& st, uint16_t* out, int64_t qrow, int g) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const float l = core_total_l(st);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t* p = out + (qrow * kQHeads + kHeadsPerGroup * g + n) * kHeadDim + 4 * kb;
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) {
    uint2 w;
    w.x = pack_bf16x2(st.o[nt][0] * inv, st.o[nt][1] * inv);
    w.y = pack_bf16x2(st.o[nt][2] * inv, st.o[nt][3] * inv);
    *(uint2*)(p + 16 * nt) = w;
  }
}

// Region r of a DSA cache (sequence/group bases given), valid up to position p.
__device__ __forceinline__ Region dsa_region(const uint16_t* k, const uint16_t* v, int64_t slot, int32_t rid,
                                             int64_t p) {
  // region rid (its cache slot given) of a query at position p; ids outside
  // [0, p/8] give an empty region at the start of the cache
  Region rg;
  const int64_t c = p / kRegion;
  if (rid < 0 || rid > c) {
    rg.k = k;
    rg.v = v;
    rg.lo = 1;
    rg.hi = 0;
    return rg;
  }
  rg.k = k + slot * kRegionElems;
  rg.v = v + slot * kRegionElems;
  rg.lo = 0;
  const int64_t last = p - (int64_t)rid * kRegion;
  rg.hi = last >= 7 ? 7 : (int)last;
  return rg;
}

// ---------------------------------------------------------------------------
// FP8 K/V caches ([P3] section 一: an FP8 KV cache halves it).  Same core with
// E4M3 codes: the codes are turned into bf16 exactly (v_cvt_scalef32_pk_bf16_fp8,
// scale 1) right before their MFMA, the per-token K scale multiplies the
// token's scores, and the per-token V scale multiplies the token's softmax
// weight before P.V.  A 4-region chunk is 12 KB instead of 24 KB.
// ---------------------------------------------------------------------------
struct Region8 {
  const uint8_t* k;  // the region's K8 (1536 bytes, region-tiled)
  const uint8_t* v;  // its V8 ([D][8] bytes)
  const float* sc;   // its 16 scales: K of tokens 0..7, then V
  int lo, hi;
};

struct ChunkRegs8 {
  u32x4 k[2][3];  // tile t, channel block s2: 16 channels of the lane's K token
  uint2 v[12];    // the 8 tokens of region kb for channel 16nt + n
  f32x4 ks[2], vs[2];
  int lo, hi;
};

// 8 E4M3 codes (two dwords, channel order) -> bf16x8, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ Region8 dsa_region8(const uint8_t* k8, const uint8_t* v8, const float* kvs, int64_t slot,
                                               int32_t rid, int64_t p) {
  Region8 rg;
  const int64_t c = p / kRegion;
  if (rid < 0 || rid > c) {  // an empty region at the start of the cache
    rg.k = k8;
    rg.v = v8;
    rg.sc = kvs;
    rg.lo = 1;
    rg.hi = 0;
    return rg;
  }
  rg.k = k8 + slot * kRegionElems;
  rg.v = v8 + slot * kRegionElems;
  rg.sc = kvs + slot * kKvsPerRegion;
  rg.lo = 0;
  const int64_t last = p - (int64_t)rid * kRegion;
  rg.hi = last >= 7 ? 7 : (int)last;
  return rg;
}

// ra = region of this lane's K rows (entry n/4), rb = region of its softmax
// weights, V and scales (entry kb), as in core_load.
__device__ __forceinline__ void core_load8(ChunkRegs8& c, const Region8& ra, const Region8& rb) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const uint8_t* kp = ra.k + (kb * 4 + (n & 3)) * 16;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 3; ++s2) c.k[t][s2] = *(const u32x4*)(kp + (t * 3 + s2) * 256);
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) c.v[nt] = *(const uint2*)(rb.v + (16 * nt + n) * 8);
  c.ks[0] = *(const f32x4*)(rb.sc);
  c.ks[1] = *(const f32x4*)(rb.sc + 4);
  c.vs[0] = *(const f32x4*)(rb.sc + 8);
  c.vs[1] = *(const f32x4*)(rb.sc + 12);
  c.lo = rb.lo;
  c.hi = rb.hi;
}

__device__ __forceinline__ void core_compute8(CoreState& st, const bf16x8 qb[6], ChunkRegs8& c, float scale_log2) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const u32x4 a = c.k[0][s >> 1], b = c.k[1][s >> 1];
    const bf16x8 a0 = (s & 1) ? fp8x8_to_bf16(a.z, a.w) : fp8x8_to_bf16(a.x, a.y);
    const bf16x8 a1 = (s & 1) ? fp8x8_to_bf16(b.z, b.w) : fp8x8_to_bf16(b.x, b.y);
    s0 = mfma16x16x32(a0, qb[s], s0);
    s1 = mfma16x16x32(a1, qb[s], s1);
  }
  bool ok[8];
  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ok[i] = i >= c.lo && i <= c.hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = ok[i] ? s0[i] * c.ks[0][i] * scale_log2 : -INFINITY;
    sv[4 + i] = ok[4 + i] ? s1[i] * c.ks[1][i] * scale_log2 : -INFINITY;
  }
  float cmax = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, sv[i]);
  cmax = max_across_rows(cmax);
  const float m_new = fmaxf(st.m, cmax);
  if (__any(m_new > st.m + 8.0f)) {  // lazy rescaling, as in core_compute
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) st.o[nt] *= alpha;
    st.m = m_new;
  }
  const float m_use = st.m == -INFINITY ? 0.0f : st.m;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  // zero the V codes of masked positions (a stale code may be NaN) and take
  // each weight times its token's V scale (0 where masked)
  if (__any(!(c.lo <= 0 && c.hi >= 7))) {
    uint32_t mx = 0, my = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx |= ok[i] ? 0xFFu << (8 * i) : 0u;
      my |= ok[4 + i] ? 0xFFu << (8 * i) : 0u;
    }
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) {
      c.v[nt].x &= mx;
      c.v[nt].y &= my;
    }
  }
  float pw[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pw[i] = ok[i] ? p[i] * c.vs[0][i] : 0.0f;
    pw[4 + i] = ok[4 + i] ? p[4 + i] * c.vs[1][i] : 0.0f;
  }
  u32x4 pp;
  pp.x = pack_bf16x2(pw[0], pw[1]);
  pp.y = pack_bf16x2(pw[2], pw[3]);
  pp.z = pack_bf16x2(pw[4], pw[5]);
  pp.w = pack_bf16x2(pw[6], pw[7]);
  const bf16x8 pb = as_bf16x8(pp);
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) st.o[nt] = mfma16x16x32(fp8x8_to_bf16(c.v[nt].x, c.v[nt].y), pb, st.o[nt]);
}

// ---------------------------------------------------------------------------
// Decode: block = (sequence b, group g, split s of 16 selected regions); its
// 4 waves take one chunk of 4 regions each and are merged through LDS into
// one partial (max, sum, unnormalised O) per split; k_merge combines splits.
// ---------------------------------------------------------------------------
constexpr int kSplitRegions = 16;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_len;
  const int32_t* sel;
  const int32_t* nsel;
  float* part;  // [B][G][nsplit][16][kPartStride]
  CacheMap cm;  // where the K/V of each sequence live (capacity cm.R*8)
  const uint8_t* k8;  // FP8 caches (FP8 instances only)
  const uint8_t* v8;
  const float* kvs;
  int32_t topk, nsplit;
  float scale_log2;
};

constexpr int kPartStride = 4 + kHeadDim;  // per head: m, l, 2 unused, o[192] (16-byte aligned)

constexpr int kORow = kHeadDim + 4;  // padded LDS row of one head's partial O

template <bool FP8>
__global__ __launch_bounds__(256) void k_sgqa_decode(DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  __shared__ float sm_m[2][16], sm_l[2][16];
  __shared__ __attribute__((aligned(16))) float sm_o[2][16][kORow];

  // every load that does not depend on the list is issued at once: the
  // sequence length, the count, this lane's two list entries (clamped index)
  // and Q; the list decides the K/V addresses afterwards
  const int64_t sg = (int64_t)b * kGroups + g;
  const int32_t* lst = a.sel + sg * a.topk;
  const int e0 = split * kSplitRegions + wave * 4;
  const int ea = e0 + (n >> 2), eb = e0 + kb;
  int64_t L = a.seq_len[b];
  int32_t cnt = a.nsel[sg];
  const int32_t ida = lst[ea < a.topk ? ea : a.topk - 1];
  const int32_t idb = lst[eb < a.topk ? eb : a.topk - 1];
  bf16x8 qb[6];
  load_q(a.q, b, g, qb);
  const int64_t tcap = a.cm.R * kRegion;
  L = L < 1 ? 1 : (L > tcap ? tcap : L);
  const int64_t p = L - 1;
  cnt = cnt < 0 ? 0 : (cnt > a.topk ? a.topk : cnt);

  // (a chunk past the count reads the dummy region and contributes nothing)
  CoreState st;
  core_init(st);
  const int32_t ra_id = ea < cnt ? ida : -1, rb_id = eb < cnt ? idb : -1;
  const int64_t cr = p / kRegion;
  const int64_t slot_a = region_slot(a.cm, b, g, ra_id >= 0 && ra_id <= cr ? ra_id : 0);
  const int64_t slot_b = region_slot(a.cm, b, g, rb_id >= 0 && rb_id <= cr ? rb_id : 0);
  if constexpr (FP8) {
    ChunkRegs8 c;
    core_load8(c, dsa_region8(a.k8, a.v8, a.kvs, slot_a, ra_id, p), dsa_region8(a.k8, a.v8, a.kvs, slot_b, rb_id, p));
    __builtin_amdgcn_sched_barrier(0);
    core_compute8(st, qb, c, a.scale_log2);
  } else {
    core_chunk(st, qb, dsa_region(a.k, a.v, slot_a, ra_id, p), dsa_region(a.k, a.v, slot_b, rb_id, p), a.scale_log2);
  }
  // The 4 waves' partials combine in pairs through 25 KB of LDS (waves 2, 3
  // into 0, 1, then 1 into 0), so that 4 blocks fit per CU; wave 0 writes
  // the split's (max, sum, unnormalised O).  O^T lane layout: head n,
  // channels 16nt + 4kb + i.
  float l = core_total_l(st);
  auto put = [&](int slot) {
    if (kb == 0) {
      sm_m[slot][n] = st.m;
      sm_l[slot][n] = l;
    }
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) *(f32x4*)&sm_o[slot][n][16 * nt + 4 * kb] = st.o[nt];
  };
  auto take = [&](int slot) {
    const float mo = sm_m[slot][n], M = fmaxf(st.m, mo);
    const float fa = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.m - M);
    const float fb = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - M);
    l = fa * l + fb * sm_l[slot][n];
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) st.o[nt] = fa * st.o[nt] + fb * *(const f32x4*)&sm_o[slot][n][16 * nt + 4 * kb];
    st.m = M;
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) take(wave);
  __syncthreads();
  if (wave == 1) put(0);
  __syncthreads();
  if (wave == 0) {
    take(0);
    float* part = a.part + ((sg * a.nsplit) + split) * 16 * kPartStride + n * kPartStride;
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) *(f32x4*)(part + 4 + 16 * nt + 4 * kb) = st.o[nt];
    if (kb == 0) {
      part[0] = st.m;
      part[1] = l;
    }
  }
}

// One block per (head, group, query): block index h + 16 (g + G b); thread d
// owns output channel d.  Split weights exp2(m_s - M) are formed once in LDS
// by the first wave (nsplit <= 64).
template <int NS>
__global__ __launch_bounds__(kHeadDim) void k_sgqa_merge(const float* __restrict__ part,
                                                         uint16_t* __restrict__ out, int32_t nsplit) {
  static_assert(NS <= 64, "one wave forms the split weights");
  const int h = blockIdx.x % 16, g = (blockIdx.x / 16) % kGroups, d = threadIdx.x;
  const int64_t b = blockIdx.x / (16 * kGroups);
  const int64_t sg = (int64_t)b * kGroups + g;
  const float* pp = part + sg * nsplit * 16 * kPartStride + h * kPartStride;
  __shared__ float w[64];
  __shared__ float inv_l;
  // this thread's partial O of every split, loaded up front (clamped split)
  float o[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) o[s] = pp[(int64_t)(s < nsplit ? s : 0) * 16 * kPartStride + 4 + d];
  if (d < 64) {
    const int sd = d < nsplit ? d : 0;
    const float m0 = pp[(int64_t)sd * 16 * kPartStride], l0 = pp[(int64_t)sd * 16 * kPartStride + 1];
    const float m = d < nsplit ? m0 : -INFINITY;
    float M = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = (M == -INFINITY || d >= nsplit) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    w[d] = f;
    float l = d < nsplit ? f * l0 : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (d == 0) inv_l = l > 0.0f ? 1.0f / l : 0.0f;
  }
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s) acc += (s < nsplit ? w[s] : 0.0f) * o[s];
  out[(b * kQHeads + kHeadsPerGroup * g + h) * kHeadDim + d] = f32_to_bf16(acc * inv_l);
}

// ---------------------------------------------------------------------------
// Prefill: the candidate regions are cut into kPreSplits ranges, and one wave
// takes the entries of one (query, group)'s selection that fall in one range;
// k_sgqa_merge combines the ranges' partial results.  Blocks of one range
// are kPreSplits apart in launch order, and the GPU hands consecutive blocks
// to its 8 L2 slices (XCDs) in turn, so each slice only ever reads the K/V
// of one range: an eighth of a group's cache instead of all of it, which
// mostly stays in that slice's L2.
// ---------------------------------------------------------------------------
#ifndef DSA_PRE_SPLITS
#define DSA_PRE_SPLITS 8
#endif
constexpr int kPreSplits = DSA_PRE_SPLITS;

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* qseq;
  const int32_t* qpos;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* sel;
  const int32_t* nsel;
  uint16_t* part_o;  // [Nq][G][kPreSplits][16][D] bf16, unnormalised O
  float* part_ml;    // [Nq][G][kPreSplits][16][2] fp32, (max, sum)
  CacheMap cm;       // where the K/V of each sequence live (capacity cm.R*8)
  const uint8_t* k8;  // FP8 caches (FP8 instances only)
  const uint8_t* v8;
  const float* kvs;
  int32_t nq, n_seqs, topk, rsplit;  // rsplit: regions per range
  float scale_log2;
};

// Block = 4 waves = 4 consecutive queries of one KV group and one region
// range; block index = range + kPreSplits * (query block + nqb * group), so
// the GPU works through one group's K/V at a time.
template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_sgqa_prefill(PrefillArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nqb = (a.nq + 3) / 4;
  const int split = blockIdx.x % kPreSplits;
  const int rest = blockIdx.x / kPreSplits;
  const int g = rest / nqb;
  const int64_t qi = (int64_t)(rest % nqb) * 4 + wave;
  __shared__ int32_t ids[4][kMaxTopk];    // region ids of the wave's entries in this range
  __shared__ int32_t slots[4][kMaxTopk];  // their cache slots
  const bool live = qi < a.nq;
  int32_t s = live ? a.qseq[qi] : 0;
  s = s < 0 ? 0 : (s >= a.n_seqs ? a.n_seqs - 1 : s);
  const int64_t tcap = a.cm.R * kRegion;
  int64_t p = live ? a.qpos[qi] : 0;
  p = p < 0 ? 0 : (p >= tcap ? tcap - 1 : p);
  const int64_t pg = qi * kGroups + g;
  int32_t cnt = live ? a.nsel[pg] : 0;
  cnt = cnt < 0 ? 0 : (cnt > a.topk ? a.topk : cnt);
  // this range's entries of the list, in list order (repeats are dropped
  // below; ids outside every range are dropped here, as they are outside
  // [0, p/8] and would be ignored anyway)
  const int32_t* lst = a.sel + (live ? pg : 0) * a.topk;
  const int32_t r0 = split * a.rsplit, r1 = r0 + a.rsplit;
  int32_t mine[kMaxTopk / 64];
#pragma unroll
  for (int j = 0; j < kMaxTopk / 64; ++j) {
    const int i = 64 * j + lane;
    mine[j] = lst[i < cnt ? i : 0];
  }
  // paged caches: every entry's page, all lookups in flight at once
  int32_t pgs[kMaxTopk / 64];
#pragma unroll
  for (int j = 0; j < kMaxTopk / 64; ++j) {
    const int64_t r = mine[j] < 0 ? 0 : (mine[j] >= a.cm.R ? a.cm.R - 1 : mine[j]);
    pgs[j] = a.cm.bt ? page_of(a.cm, s, r) : 0;
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  int32_t n = 0;
#pragma unroll
  for (int j = 0; j < kMaxTopk / 64; ++j) {
    const bool in = 64 * j + lane < cnt && mine[j] >= r0 && mine[j] < r1 && mine[j] < a.cm.R;
    const uint64_t m = __ballot(in);
    if (in) {
      ids[wave][n + __popcll(m & lt)] = mine[j];
      slots[wave][n + __popcll(m & lt)] = (int32_t)slot_in(a.cm, pgs[j], s, g, mine[j]);
    }
    n += __popcll(m);
  }
  __syncthreads();
  if (!live) return;

  // A list is a set: a repeated id counts once.  A strictly ascending run of
  // entries (what dsa_score_topk writes) holds no repeats; otherwise every
  // entry whose id occurs earlier in the run is dropped (rare, caller-made
  // lists only).
  {
    bool unsorted = false;
    for (int e = lane; e + 1 < n; e += 64) unsorted |= ids[wave][e] >= ids[wave][e + 1];
    if (__any(unsorted)) {
      int32_t kid[kMaxTopk / 64], ksl[kMaxTopk / 64];
      bool keep[kMaxTopk / 64];
#pragma unroll
      for (int j = 0; j < kMaxTopk / 64; ++j) {
        const int e = 64 * j + lane;
        kid[j] = e < n ? ids[wave][e] : 0;
        ksl[j] = e < n ? slots[wave][e] : 0;
        bool first = e < n;
        for (int e2 = 0; first && e2 < e; ++e2) first = ids[wave][e2] != kid[j];
        keep[j] = first;
      }
      int32_t nk = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopk / 64; ++j) {
        const uint64_t m = __ballot(keep[j]);
        if (keep[j]) {
          ids[wave][nk + __popcll(m & lt)] = kid[j];
          slots[wave][nk + __popcll(m & lt)] = ksl[j];
        }
        nk += __popcll(m);
      }
      n = nk;
    }
  }

  bf16x8 qb[6];
  load_q(a.q, qi, g, qb);
  CoreState st;
  core_init(st);
  const int32_t* my = ids[wave];
  const int32_t* myslot = slots[wave];
  if constexpr (FP8) {
    const int nn = lane & 15, kb = lane >> 4;
    auto region8_of = [&](int64_t e) -> Region8 {
      return dsa_region8(a.k8, a.v8, a.kvs, e < n ? myslot[e] : 0, e < n ? my[e] : -1, p);
    };
    // one chunk in registers per wave (two waves per SIMD overlap the loads)
    for (int64_t e0 = 0; e0 < n; e0 += 4) {
      ChunkRegs8 c;
      core_load8(c, region8_of(e0 + (nn >> 2)), region8_of(e0 + kb));
      __builtin_amdgcn_sched_barrier(0);
      core_compute8(st, qb, c, a.scale_log2);
    }
  } else {
    auto region_of = [&](int64_t e) -> Region {
      return dsa_region(a.k, a.v, e < n ? myslot[e] : 0, e < n ? my[e] : -1, p);
    };
    core_run<0>(st, qb, n, region_of, a.scale_log2);
  }
  // partial (max, sum, unnormalised O^T in bf16) of this range; an empty
  // range leaves (-inf, 0, 0), which the merge weighs 0
  const int hn = lane & 15, kb = lane >> 4;
  const int64_t pr = ((pg * kPreSplits) + split) * 16 + hn;  // partial row of head hn
  const float l = core_total_l(st);
  // (streaming stores: the partials are read once, by the merge, and should
  // not displace this range's K/V from the L2)
  if (kb == 0) {
    __builtin_nontemporal_store(st.m, &a.part_ml[2 * pr]);
    __builtin_nontemporal_store(l, &a.part_ml[2 * pr + 1]);
  }
  uint32_t* po = (uint32_t*)(a.part_o + pr * kHeadDim + 4 * kb);
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) {
    __builtin_nontemporal_store(pack_bf16x2(st.o[nt][0], st.o[nt][1]), po + 8 * nt);
    __builtin_nontemporal_store(pack_bf16x2(st.o[nt][2], st.o[nt][3]), po + 8 * nt + 1);
  }
}

// Prefill merge: block = (query, group), thread t = head t/16, channels
// 12(t%16) .. +11 of that head, over the kPreSplits partials.
__global__ __launch_bounds__(256) void k_sgqa_merge_pre(const uint16_t* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        uint16_t* __restrict__ out) {
  const int64_t pg = blockIdx.x;  // query * G + group
  const int h = threadIdx.x >> 4, c0 = 12 * (threadIdx.x & 15);
  float2 ml[kPreSplits];
  uint2 o[kPreSplits][3];
#pragma unroll
  for (int sp = 0; sp < kPreSplits; ++sp) {
    const int64_t pr = (pg * kPreSplits + sp) * 16 + h;
    ml[sp] = *(const float2*)&part_ml[2 * pr];
    const uint16_t* po = part_o + pr * kHeadDim + c0;
#pragma unroll
    for (int j = 0; j < 3; ++j) o[sp][j] = *(const uint2*)(po + 4 * j);
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kPreSplits; ++sp) M = fmaxf(M, ml[sp].x);
  float acc[12], L = 0.0f;
#pragma unroll
  for (int i = 0; i < 12; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int sp = 0; sp < kPreSplits; ++sp) {
    const float f = (ml[sp].x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml[sp].x - M);
    L += f * ml[sp].y;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      acc[4 * j + 0] += f * bf16_lo(o[sp][j].x);
      acc[4 * j + 1] += f * bf16_hi(o[sp][j].x);
      acc[4 * j + 2] += f * bf16_lo(o[sp][j].y);
      acc[4 * j + 3] += f * bf16_hi(o[sp][j].y);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t q = pg / kGroups, g = pg % kGroups;
  uint16_t* op = out + (q * kQHeads + kHeadsPerGroup * g + h) * kHeadDim + c0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    uint2 w;
    w.x = pack_bf16x2(acc[4 * j] * inv, acc[4 * j + 1] * inv);
    w.y = pack_bf16x2(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv);
    *(uint2*)(op + 4 * j) = w;
  }
}

// ---------------------------------------------------------------------------
// Sliding window.  The ring holds positions < P0 (first new position of the
// sequence); the new tokens and the old positions sharing P0's region are
// staged into a region-aligned buffer so that every region the core reads
// comes from exactly one source.
// ---------------------------------------------------------------------------
struct SwaArgs {
  const int32_t* pos0;  // [S]
  const int32_t* row0;  // [S+1]
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* k_ring;
  const uint16_t* v_ring;
  uint16_t* out;
  uint16_t* st_k;  // [S][G][nst][1536] region-tiled
  uint16_t* st_v;  // [S][G][nst][D][8]
  int32_t n_seqs, max_new, nst, window;
  int64_t rows;
  float scale_log2;
};

__device__ __forceinline__ void seq_rows(const SwaArgs& a, int s, int64_t& p0, int64_t& r0, int64_t& nnew) {
  p0 = a.pos0[s];
  p0 = p0 < 0 ? 0 : p0;
  if (!a.row0) {  // one new token per sequence, in row s
    r0 = s;
    nnew = 1;
    return;
  }
  r0 = a.row0[s];
  int64_t r1 = a.row0[s + 1];
  r0 = r0 < 0 ? 0 : (r0 > a.rows ? a.rows : r0);
  r1 = r1 < r0 ? r0 : (r1 > a.rows ? a.rows : r1);
  nnew = r1 - r0;
  if (nnew > a.max_new) nnew = a.max_new;
}

// block = (staged region j, sequence s).  A staged region has the ring's
// layouts, so K is 192 units of 8 channels of one token and V 192 units of
// one channel's 8 tokens, per group; thread t owns units t, t+256, ... of the
// 4 groups' 384 units each, and every load is issued before the first store.
__global__ __launch_bounds__(256) void k_swa_stage(SwaArgs a) {
  constexpr int kUnits = kGroups * 2 * kHeadDim, kPer = kUnits / 256;
  const int j = blockIdx.x, s = blockIdx.y;
  int64_t p0, r0, nnew;
  seq_rows(a, s, p0, r0, nnew);
  const int64_t base_pos = (p0 / kRegion) * kRegion + (int64_t)j * kRegion;
  if (nnew <= 0 || base_pos >= p0 + nnew) return;
  const int W = a.window;
  const int64_t rslot = (base_pos % W) / kRegion;  // ring region of the old positions of this region
  u32x4 val[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int u = threadIdx.x + 256 * k;
    const int g = u / (2 * kHeadDim), rest = u - g * 2 * kHeadDim;
    const int64_t sg = (int64_t)s * kGroups + g;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (rest < kHeadDim) {  // K unit: token t, channels d0 .. d0+7
      const int q = rest;
      const int t = (q / 96) * 4 + (q & 3), d0 = 48 * ((q >> 2) & 3) + 8 * ((q >> 4) % 6);
      const int64_t pos = base_pos + t;
      if (pos < p0) v = ld16(a.k_ring + (sg * (W / kRegion) + rslot) * kRegionElems + 8 * q);
      else if (pos < p0 + nnew) v = ld16(a.k_new + ((r0 + pos - p0) * kGroups + g) * kHeadDim + d0);
    } else {  // V unit: channel d, tokens 0..7
      const int d = rest - kHeadDim;
      if (base_pos < p0) v = ld16(a.v_ring + ((sg * (W / kRegion) + rslot) * kHeadDim + d) * kRegion);
      uint16_t e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int64_t pos = base_pos + t;
        const int64_t off = pos - p0;
        const int64_t row = r0 + (off >= 0 && off < nnew ? off : 0);  // a new row (clamped otherwise)
        const uint16_t nv = a.v_new[(row * kGroups + g) * kHeadDim + d];
        const uint32_t w = t < 2 ? v.x : t < 4 ? v.y : t < 6 ? v.z : v.w;
        const uint16_t ov = (uint16_t)(t & 1 ? w >> 16 : w & 0xFFFFu);
        e[t] = pos < p0 ? ov : (pos < p0 + nnew ? nv : (uint16_t)0);
      }
      v.x = e[0] | ((uint32_t)e[1] << 16);
      v.y = e[2] | ((uint32_t)e[3] << 16);
      v.z = e[4] | ((uint32_t)e[5] << 16);
      v.w = e[6] | ((uint32_t)e[7] << 16);
    }
    val[k] = v;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int u = threadIdx.x + 256 * k;
    const int g = u / (2 * kHeadDim), rest = u - g * 2 * kHeadDim;
    const int64_t sg = (int64_t)s * kGroups + g;
    uint16_t* dst = rest < kHeadDim ? a.st_k + (sg * a.nst + j) * kRegionElems + 8 * rest
                                    : a.st_v + ((sg * a.nst + j) * kHeadDim + (rest - kHeadDim)) * kRegion;
    *(u32x4*)dst = val[k];
  }
}

// Short chunks (fewer than two band tiles per sequence): block = (new token
// i of sequence s, group g); the window's regions go to the 4 waves in chunks
// of 4 (wave w: chunks w, w+4, ...), whose partial (max, sum, O) merge through
// LDS.  The chunk's own positions come from the staged regions.  DEPTH as for
// core_run: 2 for few blocks (latency), 0 with two blocks per CU for many.
template <int DEPTH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DEPTH == 0 ? 2 : 1, DEPTH == 0 ? 2 : 1)))
void k_swa_attend(SwaArgs a) {
  const int64_t i = blockIdx.x;
  const int s = blockIdx.y, g = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  __shared__ float sm_m[4][16], sm_l[4][16];
  __shared__ __attribute__((aligned(16))) float sm_o[4][16][kORow];
  int64_t p0, r0, nnew;
  seq_rows(a, s, p0, r0, nnew);
  if (i >= nnew) return;
  const int64_t p = p0 + i, row = r0 + i;
  const int W = a.window;
  const int64_t lo = p - W + 1 < 0 ? 0 : p - W + 1;
  const int64_t rlo = lo / kRegion, rhi = p / kRegion, rst = p0 / kRegion;
  const int64_t sg = (int64_t)s * kGroups + g;
  const uint16_t* rk = a.k_ring + sg * W * kHeadDim;
  const uint16_t* rv = a.v_ring + sg * (W / kRegion) * kHeadDim * kRegion;
  const uint16_t* sk = a.st_k + sg * a.nst * kRegion * kHeadDim;
  const uint16_t* sv = a.st_v + sg * a.nst * kHeadDim * kRegion;

  bf16x8 qb[6];
  load_q(a.q, row, g, qb);
  CoreState st;
  core_init(st);
  const int64_t nreg = rhi - rlo + 1;
  const int64_t nch = (nreg + 3) / 4;
  const int64_t mine = wave < nch ? 4 * ((nch - wave + 3) / 4) : 0;  // this wave's list entries
  auto region_of = [&](int64_t e) -> Region {
    const int64_t er = 4 * (wave + 4 * (e >> 2)) + (e & 3);  // window region index of entry e
    Region rg;
    if (e >= mine || er >= nreg) {
      rg.k = rk; rg.v = rv; rg.lo = 1; rg.hi = 0;
      return rg;
    }
    const int64_t r = rlo + er;
    if (r < rst) {
      const int64_t pk = r % (W / kRegion);
      rg.k = rk + pk * kRegion * kHeadDim;
      rg.v = rv + pk * kHeadDim * kRegion;
    } else {
      rg.k = sk + (r - rst) * kRegion * kHeadDim;
      rg.v = sv + (r - rst) * kHeadDim * kRegion;
    }
    rg.tn = -1;
    const int64_t first = r * kRegion;
    rg.lo = (int)((lo > first ? lo : first) - first);
    rg.hi = (int)((p < first + 7 ? p : first + 7) - first);
    return rg;
  };
  core_run<DEPTH>(st, qb, mine, region_of, a.scale_log2);
  // wave partials -> LDS (O^T lane layout: head n, channels 16nt + 4kb + i), then the merged,
  // normalised output
  const float lt = core_total_l(st);
  if (kb == 0) {
    sm_m[wave][n] = st.m;
    sm_l[wave][n] = lt;
  }
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) *(f32x4*)&sm_o[wave][n][16 * nt + 4 * kb] = st.o[nt];
  __syncthreads();
  uint16_t* op = a.out + (row * kQHeads + kHeadsPerGroup * g) * kHeadDim;
  for (int e = threadIdx.x; e < 16 * kHeadDim; e += 256) {
    const int h = e / kHeadDim, d = e - h * kHeadDim;
    const float M = fmaxf(fmaxf(sm_m[0][h], sm_m[1][h]), fmaxf(sm_m[2][h], sm_m[3][h]));
    float acc = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
        acc += f * sm_o[w][h][d];
        lsum += f * sm_l[w][h];
      }
    }
    op[h * kHeadDim + d] = f32_to_bf16(lsum > 0.0f ? acc / lsum : 0.0f);
  }
}

// Sliding-window decode, one new token per sequence, in one launch.  The
// window of position p (a = p/8, b = p mod 8) is exactly the ring's W/8
// region slots: slot a mod (W/8) holds the current region's tokens at
// offsets 0..b (the new token patched in at b when loaded) and, above b,
// the window's first region's; every other slot holds a whole region of the
// window.  Before the ring has filled (p < W - 1), slots 0..a hold the
// window, slot a up to offset b.  The 16 chunks of 4 slots go to the block's
// WV waves (8 waves of two chunks by default, both chunks' loads in flight
// at once).  A block owns one (sequence, group) and the 16*NT output channels
// of slice `slice`: every wave scores all 16 heads over the full 192 channels
// (the same scores in every slice block) and accumulates P.V on its slice
// only, and the waves' partials combine in LDS.  Blocks go to the 8 XCDs round
// robin by index, so the 12/NT slice blocks of one (sequence, group) are
// placed on one XCD and share its L2 for K.
// APPEND: slice 0 then writes the new token's K/V into the ring at slot p mod
// W, offset b of region slot a mod (W/8), while other blocks may still read
// that slot: their K rows of offset b come from the new token instead, and
// the bytes of offset b in their V loads are replaced by the new token's, so
// no value read from those bytes is used.
constexpr int kSwdSlots = kWindow / kRegion;  // ring region slots = window regions
static_assert(kSwdSlots % 4 == 0, "whole 4-slot chunks");

// A chunk of 4 ring slots as a sliding-window decode wave holds it: every
// load is issued before the position is known (the slots do not depend on
// it), the new token's K and V included; which token is patched and which
// are masked is settled once the position arrives.
template <int NT>
struct SwdChunk {
  ChunkRegsN<NT> c;
  u32x4 kq[6];  // the new token's K, channels 48kb + 8s .. +7
};

template <int NT>
__device__ __forceinline__ void swd_load(SwdChunk<NT>& x, const uint16_t* rk, const uint16_t* rv,
                                         const uint16_t* knew, const uint16_t* vnew, int slot0) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const uint16_t* kp = rk + (int64_t)(slot0 + (n >> 2)) * kRegion * kHeadDim + (kb * 4 + (n & 3)) * 8;
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    x.c.k0[s] = ld16(kp + (s * 16) * 8);
    x.c.k1[s] = ld16(kp + ((6 + s) * 16) * 8);
  }
  const uint16_t* vp = rv + (int64_t)(slot0 + kb) * kHeadDim * kRegion;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) x.c.v[nt] = ld16(vp + (16 * nt + n) * 8);
#pragma unroll
  for (int s = 0; s < 6; ++s) x.kq[s] = ld16(knew + 48 * kb + 8 * s);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) x.c.vpatch[nt] = vnew[16 * nt + n];
}

// Settles the chunk for position p (current slot cur, offset cb, region ca;
// full: the ring holds the whole window): the new token replaces offset cb
// of slot cur in K and V, slots past ca are empty until the ring has filled.
template <int NT>
__device__ __forceinline__ void swd_settle(SwdChunk<NT>& x, int slot0, int cur, int cb, int64_t ca, bool full) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const int jk = slot0 + (n >> 2), jv = slot0 + kb;
  const bool p0 = jk == cur && cb == (n & 3), p1 = jk == cur && cb == 4 + (n & 3);
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    x.c.k0[s] = p0 ? x.kq[s] : x.c.k0[s];
    x.c.k1[s] = p1 ? x.kq[s] : x.c.k1[s];
  }
  x.c.tn = jv == cur ? cb : -1;
  x.c.lo = (full || jv <= ca) ? 0 : 1;
  x.c.hi = (full || jv < ca) ? 7 : (jv == ca ? cb : 0);
  core_apply_patch(x.c);
}

template <int NT, int WV, bool APPEND>
__global__ __launch_bounds__(64 * WV) void k_swa_decode(SwaArgs a, uint16_t* k_ring_w, uint16_t* v_ring_w) {
  constexpr int kCpw = kSwdSlots / 4 / WV;  // chunks per wave
  static_assert(kCpw * WV * 4 == kSwdSlots, "the waves cover the ring");
  constexpr int kSlices = 12 / NT;
  static_assert(kSlices * NT == 12, "slices of whole 16-channel tiles");
  constexpr int kCh = 16 * NT;  // output channels per block
  const int L = blockIdx.x, xcd = L & 7, k = L >> 3;
  const int slice = k % kSlices;
  const int64_t sg = (int64_t)(k / kSlices) * 8 + xcd;
  if (sg >= (int64_t)a.n_seqs * kGroups) return;
  const int s = (int)(sg / kGroups), g = (int)(sg % kGroups);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  __shared__ float sm_m[WV][16], sm_l[WV][16];
  __shared__ __attribute__((aligned(16))) float sm_o[WV][16][kCh + 4];
  // the position first, then every load that does not depend on it
  const int32_t praw = a.pos0[s];
  int64_t row = s;
  if (a.row0) {  // (swa_attention with one new row per sequence at most)
    int64_t r0 = a.row0[s], r1 = a.row0[s + 1];
    r0 = r0 < 0 ? 0 : (r0 > a.rows ? a.rows : r0);
    r1 = r1 < r0 ? r0 : (r1 > a.rows ? a.rows : r1);
    if (r1 <= r0) return;
    row = r0;
  }
  const int W = a.window;
  const int nslot = W / kRegion;
  const uint16_t* rk = a.k_ring + sg * W * kHeadDim;
  const uint16_t* rv = a.v_ring + sg * nslot * kHeadDim * kRegion + kCh * slice * kRegion;
  const uint16_t* knew = a.k_new + (row * kGroups + g) * kHeadDim;
  const uint16_t* vnew = a.v_new + (row * kGroups + g) * kHeadDim + kCh * slice;
  bf16x8 qb[6];
  load_q(a.q, row, g, qb);
  SwdChunk<NT> x[kCpw];
#pragma unroll
  for (int j = 0; j < kCpw; ++j) swd_load(x[j], rk, rv, knew, vnew, 4 * (wave + WV * j));
  // the append's copy of the new token (slice 0, whose vnew is the whole
  // row): K units for threads 0..23, V channels for threads 64..255
  static_assert(64 * WV >= 64 + kHeadDim, "a thread per V channel of the append");
  const int t = threadIdx.x;
  u32x4 akv = {0u, 0u, 0u, 0u};
  uint16_t avv = 0;
  if (APPEND && slice == 0) {
    if (t < kHeadDim / 8) akv = ld16(knew + 8 * t);
    else if (t >= 64 && t < 64 + kHeadDim) avv = vnew[t - 64];
  }
  __builtin_amdgcn_sched_barrier(0);  // (every load issued before any is waited for)
  const int64_t p = praw < 0 ? 0 : praw;
  const int64_t ca = p / kRegion;
  const int cb = (int)(p % kRegion), cur = (int)(ca % nslot);
  CoreStateN<NT> st;
  core_init(st);
#pragma unroll
  for (int j = 0; j < kCpw; ++j) {
    swd_settle(x[j], 4 * (wave + WV * j), cur, cb, ca, p >= W - 1);
    core_compute(st, qb, x[j].c, a.scale_log2);
  }
  const float lt = core_total_l(st);
  if (kb == 0) {
    sm_m[wave][n] = st.m;
    sm_l[wave][n] = lt;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) *(f32x4*)&sm_o[wave][n][16 * nt + 4 * kb] = st.o[nt];
  __syncthreads();
  // item e: head e / (kCh/4), channels 4q..4q+3 of the slice
  for (int e = t; e < 16 * kCh / 4; e += 64 * WV) {
    const int h = e / (kCh / 4), q4 = 4 * (e - h * (kCh / 4));
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < WV; ++w) M = fmaxf(M, sm_m[w][h]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float Lsum = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < WV; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
        acc += f * *(const f32x4*)&sm_o[w][h][q4];
        Lsum += f * sm_l[w][h];
      }
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    uint2 o2;
    o2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    o2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *(uint2*)(a.out + (row * kQHeads + kHeadsPerGroup * g + h) * kHeadDim + kCh * slice + q4) = o2;
  }
  if constexpr (APPEND) {
    if (slice == 0) {
      const int64_t slot = p % W;
      if (t < kHeadDim / 8)  // K: 24 units of 8 channels
        *(u32x4*)(k_ring_w + (sg * nslot + slot / kRegion) * kRegionElems + k_tile_offset(slot % kRegion, 8 * t)) =
            akv;
      else if (t >= 64 && t < 64 + kHeadDim)  // V: 192 channels
        v_ring_w[((sg * nslot + slot / kRegion) * kHeadDim + (t - 64)) * kRegion + slot % kRegion] = avv;
    }
  }
}

#ifndef DSA_SWD_NT
#define DSA_SWD_NT 2
#endif
#ifndef DSA_SWD_WV
#define DSA_SWD_WV 8
#endif

// One launch: (sequence, group) x channel slice blocks, the slices of one
// (sequence, group) on one XCD (see k_swa_decode).
static void swa_decode_launch(const SwaArgs& a, uint16_t* k_ring_w, uint16_t* v_ring_w, hipStream_t s) {
  ProfScope prof_("k_swa_decode", s);
  constexpr int NT = DSA_SWD_NT, WV = DSA_SWD_WV;
  const int64_t nsg = (int64_t)a.n_seqs * kGroups;
  const dim3 grid((unsigned)((nsg + 7) / 8 * 8 * (12 / NT)));
  if (k_ring_w)
    hipLaunchKernelGGL((k_swa_decode<NT, WV, true>), grid, dim3(64 * WV), 0, s, a, k_ring_w, v_ring_w);
  else
    hipLaunchKernelGGL((k_swa_decode<NT, WV, false>), grid, dim3(64 * WV), 0, s, a, (uint16_t*)nullptr,
                       (uint16_t*)nullptr);
}


// S^T tiles, online softmax and O^T += V^T P^T of one chunk for NQ queries
// that share its K/V registers (the neighbour-merged prefill: consecutive
// queries of one group walk the union of their selections).  lo[j]/hi[j]: query j's valid positions
// in the lane's softmax region.  Positions no query of the wave uses get
// their V zeroed; a position one query uses and another masks holds real
// data and gets weight 0 from the latter.
// after_s() runs once the S tiles are issued (a caller may load c.v there);
// c.v is first used after the softmax.
struct NoOp {
  __device__ __forceinline__ void operator()() const {}
};
template <int NQ, class QOf, class AfterS = NoOp>
__device__ __forceinline__ void core_compute_band(CoreState (&st)[NQ], const QOf& q_of, ChunkRegs& c,
                                                  const int (&lo)[NQ], const int (&hi)[NQ], float scale_log2,
                                                  const AfterS& after_s = AfterS()) {
  constexpr bool kLateV = !__is_same(AfterS, NoOp);  // V arrives in after_s: mask it after the softmax
  int ulo = lo[0], uhi = hi[0];
#pragma unroll
  for (int j = 1; j < NQ; ++j) {
    ulo = lo[j] < ulo ? lo[j] : ulo;
    uhi = hi[j] > uhi ? hi[j] : uhi;
  }
  const bool full = (ulo <= 0 && uhi >= 7);
  auto mask_v = [&]() {
    if (__any(!full)) {
      uint32_t mk[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bool a0 = (2 * w >= ulo && 2 * w <= uhi);
        const bool a1 = (2 * w + 1 >= ulo && 2 * w + 1 <= uhi);
        mk[w] = (a0 ? 0x0000FFFFu : 0u) | (a1 ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int nt = 0; nt < 12; ++nt) {
        c.v[nt].x &= mk[0];
        c.v[nt].y &= mk[1];
        c.v[nt].z &= mk[2];
        c.v[nt].w &= mk[3];
      }
    }
  };
  if constexpr (!kLateV) mask_v();
  // three phases over the NQ queries (S tiles, softmax, P.V) so that one
  // query's MFMAs overlap another's VALU work
  f32x4 s0[NQ], s1[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    s0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    s1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int q = 0; q < 6; ++q)
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const bf16x8 qv = q_of(j, q);
      s0[j] = mfma16x16x32(as_bf16x8(c.k0[q]), qv, s0[j]);
      s1[j] = mfma16x16x32(as_bf16x8(c.k1[q]), qv, s1[j]);
    }
  after_s();
  float sv[NQ][8], m_new[NQ];
  bool grow = false;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[j][i] = (i >= lo[j] && i <= hi[j]) ? s0[j][i] * scale_log2 : -INFINITY;
      sv[j][4 + i] = (4 + i >= lo[j] && 4 + i <= hi[j]) ? s1[j][i] * scale_log2 : -INFINITY;
    }
    float cmax = sv[j][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, sv[j][i]);
    m_new[j] = fmaxf(st[j].m, max_across_rows(cmax));
    grow |= m_new[j] > st[j].m + 8.0f;
  }
  // lazy rescaling as in core_compute, one branch for the wave's queries
  if (__any(grow)) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (__any(m_new[j] > st[j].m + 8.0f)) {
        const float alpha = __builtin_amdgcn_exp2f(st[j].m - m_new[j]);
        st[j].l *= alpha;
#pragma unroll
        for (int nt = 0; nt < 12; ++nt) st[j].o[nt] *= alpha;
        st[j].m = m_new[j];
      }
    }
  }
  if constexpr (kLateV) mask_v();
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const float m_use = st[j].m == -INFINITY ? 0.0f : st[j].m;
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(sv[j][i] - m_use);
    st[j].l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    u32x4 pp;
    pp.x = pack_bf16x2(pr[0], pr[1]);
    pp.y = pack_bf16x2(pr[2], pr[3]);
    pp.z = pack_bf16x2(pr[4], pr[5]);
    pp.w = pack_bf16x2(pr[6], pr[7]);
    const bf16x8 pb = as_bf16x8(pp);
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) st[j].o[nt] = mfma16x16x32(as_bf16x8(c.v[nt]), pb, st[j].o[nt]);
  }
}

constexpr int kRegionBytes = kRegionElems * 2;    // K (or V) of one region
constexpr int kBandRegion = 2 * kRegionBytes + 64;  // a region's K then V in LDS; the 64-byte pad puts
                                                     // the 4 regions' K rows a wave reads together in
                                                     // different banks
constexpr int kChunkBytes = 4 * kBandRegion;

// Chunked prefill: block = (8 consecutive new tokens of sequence s, group
// g), 4 waves of 2 tokens.  The tokens' windows nearly coincide, so the
// block streams the union of the windows (about 66 regions) once through an
// LDS ring of 4-region chunks (direct-to-LDS copies, 24 of 1 KB per chunk:
// wave w copies region w, two chunks ahead); each wave applies a chunk to
// its 2 tokens under their band masks, so a K/V byte read from L2 feeds 8
// queries.  A wave's count of outstanding memory operations (the loop
// issues nothing else) tells when its copies landed, and a barrier makes
// the whole chunk visible and frees the slot refilled next.  The ring holds
// 3 chunks (74.5 KB), so two blocks share a CU and each SIMD runs two waves:
// one wave's softmax VALU work runs under the other's MFMAs (with one wave
// per SIMD they run one after another).  The operands are read from LDS as
// they are used (the K rows of one k-step, the V^T operand of one channel
// tile), which keeps a wave within the 256 registers two waves per SIMD
// allow.  V of positions outside the union of the block's windows (in the
// union's first and last regions only) is zeroed in LDS by the wave that
// copied the region, so P.V needs no mask: every other position holds a
// token of some window, and its weight is exactly 0 for the tokens whose
// band leaves it out.  Chunks inside every window of the block (all but the
// first and last few) take a form without the band masks.
constexpr int kBandNQ = 2;               // tokens per wave
constexpr int kBandQ = 4 * kBandNQ;       // tokens per block
constexpr int kBandDepth = 3;             // chunks in the LDS ring

// One chunk for NQ tokens (see above).  MASKED: lo/hi give each token's
// valid offsets in the lane's softmax region kb (lo > hi: none); otherwise
// every position of the chunk is inside every token's band.
template <int NQ, bool MASKED>
__device__ __forceinline__ void band_chunk(CoreState (&st)[NQ], const bf16x8 (&qb)[NQ][6], const uint8_t* ch,
                                            const int (&lo)[NQ], const int (&hi)[NQ], float scale_log2) {
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  // K rows of region n/4 (tile layout as in memory), V^T of region kb
  const uint8_t* kp = ch + (n >> 2) * kBandRegion + ((kb * 4 + (n & 3)) * 8) * 2;
  const uint8_t* vp = ch + kb * kBandRegion + kRegionBytes;
  f32x4 s0[NQ], s1[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    s0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    s1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    const bf16x8 k0 = as_bf16x8(*(const u32x4*)(kp + (q * 16) * 16));
    const bf16x8 k1 = as_bf16x8(*(const u32x4*)(kp + ((6 + q) * 16) * 16));
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      s0[j] = mfma16x16x32(k0, qb[j][q], s0[j]);
      s1[j] = mfma16x16x32(k1, qb[j][q], s1[j]);
    }
  }
  // raw scores (masked ones -inf); the scale (> 0) is applied to the row
  // maximum and folded into the exponent below
  float sv[NQ][8];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (MASKED) {
        sv[j][i] = (i >= lo[j] && i <= hi[j]) ? s0[j][i] : -INFINITY;
        sv[j][4 + i] = (4 + i >= lo[j] && 4 + i <= hi[j]) ? s1[j][i] : -INFINITY;
      } else {
        sv[j][i] = s0[j][i];
        sv[j][4 + i] = s1[j][i];
      }
    }
  float m_new[NQ];
  bool grow = false;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    float cmax = sv[j][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, sv[j][i]);
    m_new[j] = fmaxf(st[j].m, max_across_rows(cmax) * scale_log2);
    grow |= m_new[j] > st[j].m + 8.0f;
  }
  // lazy rescaling as in core_compute
  if (__any(grow)) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (__any(m_new[j] > st[j].m + 8.0f)) {
        const float alpha = __builtin_amdgcn_exp2f(st[j].m - m_new[j]);
        st[j].l *= alpha;
#pragma unroll
        for (int nt = 0; nt < 12; ++nt) st[j].o[nt] *= alpha;
        st[j].m = m_new[j];
      }
    }
  }
  bf16x8 pb[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const float m_use = st[j].m == -INFINITY ? 0.0f : st[j].m;
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(sv[j][i], scale_log2, -m_use));
    st[j].l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    u32x4 pp;
    pp.x = pack_bf16x2(pr[0], pr[1]);
    pp.y = pack_bf16x2(pr[2], pr[3]);
    pp.z = pack_bf16x2(pr[4], pr[5]);
    pp.w = pack_bf16x2(pr[6], pr[7]);
    pb[j] = as_bf16x8(pp);
  }
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) {
    const bf16x8 v = as_bf16x8(*(const u32x4*)(vp + (16 * nt + n) * 16));
#pragma unroll
    for (int j = 0; j < NQ; ++j) st[j].o[nt] = mfma16x16x32(v, pb[j], st[j].o[nt]);
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_swa_band(SwaArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, kb = lane >> 4;
  const int s = blockIdx.y, g = blockIdx.z;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kBandDepth][kChunkBytes];
  int64_t p0, r0, nnew;
  seq_rows(a, s, p0, r0, nnew);
  // gridDim.x is a multiple of 8 and consecutive blocks go to the 8 XCDs in
  // turn, so XCD x gets blocks x, x+8, ...: give it a contiguous run of
  // query tiles, whose windows overlap and stay in its L2
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int64_t i0 = tile * kBandQ;
  if (i0 >= nnew) return;  // the same for the whole block
  constexpr int W = kWindow, kSlots = kWindow / kRegion;
  const int64_t i1 = (i0 + kBandQ < nnew ? i0 + kBandQ : nnew) - 1;
  const int64_t ulo = p0 + i0 - W + 1 < 0 ? 0 : p0 + i0 - W + 1;  // union of the block's windows
  const int64_t uhi = p0 + i1;
  const int64_t rlo = ulo / kRegion, rhi = uhi / kRegion, rst = p0 / kRegion;
  const int nch = (int)((rhi - rlo + 1 + 3) / 4);
  const int64_t sg = (int64_t)s * kGroups + g;
  const uint8_t* rk = (const uint8_t*)(a.k_ring + sg * W * kHeadDim);
  const uint8_t* rv = (const uint8_t*)(a.v_ring + sg * kSlots * kHeadDim * kRegion);
  const uint8_t* sk = (const uint8_t*)(a.st_k + sg * a.nst * kRegionElems);
  const uint8_t* sv = (const uint8_t*)(a.st_v + sg * a.nst * kRegionElems);
  // wave w copies region w of each chunk, K then V (past rhi: a re-read of
  // region rhi, which no token weighs)
#define DSA_BAND_ISSUE(c_)                                                                                  \
  do {                                                                                                       \
    int64_t r_ = rlo + 4 * (int64_t)(c_) + wave;                                                             \
    r_ = r_ > rhi ? rhi : r_;                                                                                \
    const int64_t o_ = r_ < rst ? (r_ & (kSlots - 1)) * kRegionBytes : (r_ - rst) * kRegionBytes;           \
    const uint8_t* bk_ = (r_ < rst ? rk : sk) + o_;                                                          \
    const uint8_t* bv_ = (r_ < rst ? rv : sv) + o_;                                                          \
    LdsPtr d_ = (LdsPtr)(&ring[(c_) % kBandDepth][0] + wave * kBandRegion);                                 \
    _Pragma("unroll") for (int k_ = 0; k_ < 3; ++k_) {                                                       \
      __builtin_amdgcn_global_load_lds((const void*)(bk_ + 1024 * k_ + 16 * lane), d_ + 1024 * k_, 16, 0, 0);  \
      __builtin_amdgcn_global_load_lds((const void*)(bv_ + 1024 * k_ + 16 * lane), d_ + kRegionBytes + 1024 * k_, \
                                       16, 0, 0);                                                            \
    }                                                                                                        \
  } while (0)
  // this wave's tokens (idle ones shadow the last token and store nothing);
  // Q first, so that waiting for it does not wait for the copies
  bf16x8 qb[kBandNQ][6];
  CoreState st[kBandNQ];
  int64_t pj[kBandNQ];
#pragma unroll
  for (int j = 0; j < kBandNQ; ++j) {
    const int64_t i = i0 + kBandNQ * wave + j;
    const int64_t ic = i < nnew ? i : nnew - 1;
    pj[j] = p0 + ic;
    load_q(a.q, r0 + ic, g, qb[j]);
    core_init(st[j]);
  }
  if (nch > 0)
#pragma unroll
    for (int c = 0; c < kBandDepth - 1; ++c) DSA_BAND_ISSUE(c);
  // chunk c: wait for its copies, clear V outside the union, then apply it
  // (MASKED: with each token's band; the chunks inside every window of the
  // block, from the last token's window start to the first token's
  // position, need none)
  auto body = [&](int c, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    // the chunk's 6 copies are older than the 6 issued since
    static_assert(kBandDepth == 3, "wait count below");
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    {  // zero V outside [ulo, uhi] in the region this wave copied
      int64_t r_ = rlo + 4 * (int64_t)c + wave;
      r_ = r_ > rhi ? rhi : r_;
      const int64_t f_ = r_ * kRegion;
      const int zlo = ulo > f_ ? (int)(ulo - f_) : 0;
      const int zhi = uhi < f_ + 7 ? (int)(uhi - f_) : 7;
      if (zlo > 0 || zhi < 7) {  // uniform: the union's first or last region
        uint32_t mk[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          mk[w] = ((2 * w >= zlo && 2 * w <= zhi) ? 0x0000FFFFu : 0u) |
                  ((2 * w + 1 >= zlo && 2 * w + 1 <= zhi) ? 0xFFFF0000u : 0u);
        uint8_t* vrow = &ring[c % kBandDepth][0] + wave * kBandRegion + kRegionBytes;
#pragma unroll
        for (int d = 0; d < kHeadDim; d += 64) {
          u32x4 x = *(u32x4*)(vrow + (d + lane) * 16);
          x.x &= mk[0];
          x.y &= mk[1];
          x.z &= mk[2];
          x.w &= mk[3];
          *(u32x4*)(vrow + (d + lane) * 16) = x;
        }
      }
    }
    __syncthreads();
    DSA_BAND_ISSUE(c + kBandDepth - 1);
    const uint8_t* ch = &ring[c % kBandDepth][0];
    int lo[kBandNQ], hi[kBandNQ];
    if constexpr (kMasked) {
      const int64_t r = rlo + 4 * c + kb, first = r * kRegion;
#pragma unroll
      for (int j = 0; j < kBandNQ; ++j) {
        const int64_t qlo = pj[j] - W + 1;
        const bool in = r <= pj[j] / kRegion && first + 7 >= qlo;
        lo[j] = in ? (int)((qlo > first ? qlo : first) - first) : 1;
        hi[j] = in ? (int)((pj[j] < first + 7 ? pj[j] : first + 7) - first) : 0;
      }
    }
    band_chunk<kBandNQ, kMasked>(st, qb, ch, lo, hi, a.scale_log2);
  };
  auto interior = [&](int c) {
    const int64_t cf = (rlo + 4 * (int64_t)c) * kRegion;
    return cf >= uhi - W + 1 && cf + 4 * kRegion - 1 <= p0 + i0;
  };
  // the interior chunks form one run
  int c = 0;
  for (; c < nch && !interior(c); ++c) body(c, std::true_type());
  for (; c < nch && interior(c); ++c) body(c, std::false_type());
  for (; c < nch; ++c) body(c, std::true_type());
  // copies issued past the last chunk must land before the block's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < kBandNQ; ++j) {
    const int64_t i = i0 + kBandNQ * wave + j;
    if (i < nnew) core_store(st[j], a.out, r0 + i, g);
  }
#undef DSA_BAND_ISSUE
}

// ---------------------------------------------------------------------------
// Neighbour-merged prefill ([P5], Sparse GQA paragraph: the selections of
// neighbouring tokens are merged so that the GPU is used better).  Exact
// form: a wave takes 2 consecutive queries of one KV group and walks the
// union of their selections inside one region range, ascending; each union
// region's K/V is read once and applied to both queries under their
// membership bits (a query that did not select the region gives it weight
// 0), so every query gets the attention over its own selection.  A query's
// list is taken as a set (a repeated id counts once).  When the 2 queries
// belong to different sequences, the wave makes one pass per sequence.
//
// The union of the range is built in windows of kMrgWin regions: a byte per
// region collects the membership bits (LDS atomics), a wave-wide scan of the
// nonzero bytes lists the union in ascending order, then the entries' cache
// slots are looked up.  The queries' Q^T operands sit in LDS, which leaves
// room for two waves per SIMD (242 VGPRs): chunks load straight into
// registers, K first and V once the S tiles are issued, and the other wave
// of the SIMD covers the waits.  No barrier is shared between waves.
// Partials go to the layout of k_sgqa_prefill and k_sgqa_merge_pre merges.
// (Four queries per wave, one wave per SIMD, with the next chunk copied into
// LDS ahead, measured slower: 1.19 ms against 0.93 ms on the correlated 64K
// chunk.)
// ---------------------------------------------------------------------------
constexpr int kMrgQ = 2;       // queries per wave
constexpr int kMrgWin = 512;   // regions per union window (64 lanes x 8 bytes)

struct MergeWave {
  u32x4 q[kMrgQ][6][64];        // Q^T operand of query j, k-step s, lane
  uint32_t bits[kMrgWin / 4];   // membership byte of each region of the window
  int32_t rid[kMrgWin];         // the window's union, ascending
  int32_t slot[kMrgWin];        // its cache slots
  uint8_t msk[kMrgWin];         // its membership bytes
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_sgqa_prefill_merged(
    PrefillArgs a) {
  constexpr int NQ = kMrgQ;
  constexpr int kWin = kMrgWin;
  constexpr int kBytesPerLane = kWin / 64;  // membership bytes a lane scans
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, nn = lane & 15, kb = lane >> 4;
  const int nqb = (a.nq + 4 * NQ - 1) / (4 * NQ);
  const int split = blockIdx.x % kPreSplits;
  const int rest = blockIdx.x / kPreSplits;
  const int g = rest / nqb;
  const int64_t q0 = ((int64_t)(rest % nqb) * 4 + wave) * NQ;
  __shared__ __attribute__((aligned(16))) MergeWave lds_all[4];
  MergeWave& L = lds_all[wave];
  if (q0 >= a.nq) return;  // the whole wave; no barrier is shared with the others
  const int64_t tcap = a.cm.R * kRegion;
  int32_t sq[NQ], cq[NQ];
  int64_t pq[NQ];
  uint32_t todo = 0;
  CoreState st[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int64_t qi = q0 + j;
    const bool live = qi < a.nq;
    const int64_t qc = live ? qi : q0;
    int32_t s = a.qseq[qc];
    sq[j] = s < 0 ? 0 : (s >= a.n_seqs ? a.n_seqs - 1 : s);
    int64_t p = a.qpos[qc];
    pq[j] = p < 0 ? 0 : (p >= tcap ? tcap - 1 : p);
    int32_t c = live ? a.nsel[qc * kGroups + g] : 0;
    cq[j] = c < 0 ? 0 : (c > a.topk ? a.topk : c);
    todo |= live ? 1u << j : 0u;
    bf16x8 t[6];
    load_q(a.q, qc, g, t);
#pragma unroll
    for (int q = 0; q < 6; ++q) L.q[j][q][lane] = *(const u32x4*)&t[q];
    core_init(st[j]);
  }
  const int64_t r0 = (int64_t)split * a.rsplit;
  const int64_t r1 = r0 + a.rsplit < a.cm.R ? r0 + a.rsplit : a.cm.R;
  while (todo) {
    // one pass per sequence among the wave's queries
    const int lead = __builtin_ctz(todo);
    int32_t sp = sq[0];
#pragma unroll
    for (int j = 1; j < NQ; ++j) sp = lead == j ? sq[j] : sp;
    uint32_t mem = 0;
#pragma unroll
    for (int j = 0; j < NQ; ++j) mem |= ((todo >> j) & 1u) && sq[j] == sp ? 1u << j : 0u;
    todo &= ~mem;
    for (int64_t w0 = r0; w0 < r1; w0 += kWin) {
      const int64_t w1 = w0 + kWin < r1 ? w0 + kWin : r1;
      // membership bytes (a wave's LDS operations complete in issue order)
#pragma unroll
      for (int i = 0; i < kWin / 4 / 64; ++i) L.bits[64 * i + lane] = 0u;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        if (!((mem >> j) & 1u)) continue;
        const int32_t* lst = a.sel + ((q0 + j) * kGroups + g) * a.topk;
        const int64_t cur = pq[j] / kRegion;
        for (int e = lane; e < cq[j]; e += 64) {
          const int64_t r = lst[e];
          if (r >= w0 && r < w1 && r <= cur) {
            const int o = (int)(r - w0);
            atomicOr(&L.bits[o >> 2], (1u << j) << (8 * (o & 3)));
          }
        }
      }
      // the union in ascending order: lane l owns regions w0 + l*kBytesPerLane ...
      uint32_t words[kBytesPerLane / 4];
#pragma unroll
      for (int w = 0; w < kBytesPerLane / 4; ++w) words[w] = L.bits[(kBytesPerLane / 4) * lane + w];
      uint32_t cnt = 0;
#pragma unroll
      for (int w = 0; w < kBytesPerLane / 4; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) cnt += ((words[w] >> (8 * b)) & 0xffu) ? 1u : 0u;
      const uint32_t incl = wave_incl_scan(cnt);
      const int nu = __builtin_amdgcn_readlane((int)incl, 63);
      uint32_t at = incl - cnt;
#pragma unroll
      for (int w = 0; w < kBytesPerLane / 4; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t m = (words[w] >> (8 * b)) & 0xffu;
          if (m) {
            L.rid[at] = (int32_t)(w0 + kBytesPerLane * lane + 4 * w + b);
            L.msk[at] = (uint8_t)m;
            ++at;
          }
        }
      if (nu == 0) continue;
      for (int e = lane; e < nu; e += 64) {
        const int32_t r = L.rid[e];
        L.slot[e] = (int32_t)slot_in(a.cm, a.cm.bt ? page_of(a.cm, sp, r) : 0, sp, g, r);
      }
      auto masks = [&](int e0, int (&lo)[NQ], int (&hi)[NQ]) {
        const int e = e0 + kb;
        const int m = e < nu ? L.msk[e] : 0;
        const int64_t first = (int64_t)(e < nu ? L.rid[e] : 0) * kRegion;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          const bool in = (m >> j) & 1;
          const int64_t last = pq[j] - first;
          lo[j] = in ? 0 : 1;
          hi[j] = in ? (last >= 7 ? 7 : (int)last) : 0;
        }
      };
      // walk the union 4 regions at a time
      {
        auto region_of = [&](int e) -> Region {
          Region rg;
          const int64_t sl = e < nu ? L.slot[e] : L.slot[nu - 1];  // past the end: a re-read, masked
          rg.k = a.k + sl * kRegionElems;
          rg.v = a.v + sl * kRegionElems;
          rg.lo = 0;
          rg.hi = 7;
          return rg;
        };
        // K rows of region (e0 + nn/4) first; the V pack of region (e0 + kb)
        // once the S tiles are issued (K and V are then not live together,
        // which keeps two waves per SIMD; the other wave covers the waits)
        for (int e0 = 0; e0 < nu; e0 += 4) {
          ChunkRegs cr;
          const uint16_t* kp = region_of(e0 + (nn >> 2)).k + (kb * 4 + (nn & 3)) * 8;
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            cr.k0[q] = ld16(kp + (q * 16) * 8);
            cr.k1[q] = ld16(kp + ((6 + q) * 16) * 8);
          }
          const uint16_t* vb = region_of(e0 + kb).v;
          int lo[NQ], hi[NQ];
          masks(e0, lo, hi);
          core_compute_band<NQ>(
              st, [&](int j, int q) { const u32x4 v = L.q[j][q][lane]; return as_bf16x8(v); }, cr, lo, hi,
              a.scale_log2, [&]() {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < 12; ++nt) cr.v[nt] = ld16(vb + (16 * nt + nn) * 8);
                __builtin_amdgcn_sched_barrier(0);
              });
        }
      }
    }
  }
  // partials of this range for the live queries (layout of k_sgqa_prefill)
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    if (q0 + j >= a.nq) continue;
    const int64_t pr = (((q0 + j) * kGroups + g) * kPreSplits + split) * 16 + nn;
    const float l = core_total_l(st[j]);
    if (kb == 0) {
      __builtin_nontemporal_store(st[j].m, &a.part_ml[2 * pr]);
      __builtin_nontemporal_store(l, &a.part_ml[2 * pr + 1]);
    }
    uint32_t* po = (uint32_t*)(a.part_o + pr * kHeadDim + 4 * kb);
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) {
      __builtin_nontemporal_store(pack_bf16x2(st[j].o[nt][0], st[j].o[nt][1]), po + 8 * nt);
      __builtin_nontemporal_store(pack_bf16x2(st[j].o[nt][2], st[j].o[nt][3]), po + 8 * nt + 1);
    }
  }
}

// block = (new token i of sequence s): writes it to the ring if it is among
// the last `window` new tokens of its sequence (K as 96 units of 8 channels,
// V element-wise; all loads issued before the stores).
__global__ __launch_bounds__(256) void k_ring_append(SwaArgs a, uint16_t* k_ring, uint16_t* v_ring) {
  const int64_t i = blockIdx.x;
  const int s = blockIdx.y;
  int64_t p0, r0, nnew;
  seq_rows(a, s, p0, r0, nnew);
  if (i >= nnew || i < nnew - a.window) return;
  const int W = a.window;
  const int64_t pos = p0 + i, row = r0 + i, slot = pos % W;
  const int t = threadIdx.x;
  // K: 4 groups x 24 units of 8 channels (threads 0..95)
  if (t < kGroups * kHeadDim / 8) {
    const int g = t / (kHeadDim / 8), d0 = 8 * (t % (kHeadDim / 8));
    const int64_t sg = (int64_t)s * kGroups + g;
    const u32x4 v = ld16(a.k_new + (row * kGroups + g) * kHeadDim + d0);
    *(u32x4*)(k_ring + (sg * (W / kRegion) + slot / kRegion) * kRegionElems + k_tile_offset(slot % kRegion, d0)) = v;
  }
  // V: 768 elements, 3 per thread
  uint16_t vv[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int e = t + 256 * k, g = e / kHeadDim, d = e - g * kHeadDim;
    vv[k] = a.v_new[(row * kGroups + g) * kHeadDim + d];
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int e = t + 256 * k, g = e / kHeadDim, d = e - g * kHeadDim;
    const int64_t sg = (int64_t)s * kGroups + g;
    v_ring[((sg * (W / kRegion) + slot / kRegion) * kHeadDim + d) * kRegion + slot % kRegion] = vv[k];
  }
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static int32_t nsplit_of(int32_t topk) { return (topk + kSplitRegions - 1) / kSplitRegions; }
static int32_t nstage_of(int32_t max_new) { return (max_new + kRegion - 1) / kRegion + 1; }

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_sparse_gqa_workspace_size(const dsa_geometry* geom, int32_t batch) {
  const int32_t topk = (geom && geom->topk > 0 && geom->topk <= kMaxTopk) ? geom->topk : kMaxTopk;
  if (batch <= 0) return 256;
  return (size_t)batch * kGroups * nsplit_of(topk) * 16 * kPartStride * sizeof(float) + 256;
}

namespace dsa {
dsa_status sparse_gqa_decode(const char* who, const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                             const uint16_t* k_cache, const uint16_t* v_cache, const CacheMap& cm,
                             const int32_t* seq_len, const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                             void* workspace, size_t workspace_bytes, void* stream, const Fp8Kv* f8) {
  const std::string w(who);
  if (batch < 0) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": batch must be >= 0");
  if (batch == 0) return DSA_OK;
  const bool kv_ok = f8 ? (f8->k8 && f8->v8 && f8->kvs) : (k_cache && v_cache);
  if (!q || !kv_ok || !seq_len || !sel || !n_sel || !out || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, w + ": NULL pointer");
  if ((size_t)workspace & 255) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": workspace must be 256-byte aligned");
  if (workspace_bytes < dsa_sparse_gqa_workspace_size(geom, batch))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, w + ": workspace too small");
  if (batch > 65535) return fail(DSA_ERR_UNSUPPORTED, w + ": batch > 65535");
  DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.seq_len = seq_len; a.sel = sel; a.nsel = n_sel;
  a.part = (float*)workspace; a.cm = cm; a.topk = geom->topk; a.nsplit = nsplit_of(geom->topk);
  a.k8 = f8 ? f8->k8 : nullptr; a.v8 = f8 ? f8->v8 : nullptr; a.kvs = f8 ? f8->kvs : nullptr;
  a.scale_log2 = geom->softmax_scale * kLog2e;
  hipStream_t s = as_stream(stream);
  {
    ProfScope prof_("k_sgqa_decode", s);
    if (f8) hipLaunchKernelGGL(k_sgqa_decode<true>, dim3(a.nsplit, kGroups, batch), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_sgqa_decode<false>, dim3(a.nsplit, kGroups, batch), dim3(256), 0, s, a);
  }
  dsa_status st = check_launch(who);
  if (st != DSA_OK) return st;
  {
    ProfScope prof_("k_sgqa_merge", s);
    hipLaunchKernelGGL(k_sgqa_merge<kMaxTopk / kSplitRegions>, dim3((unsigned)(16 * kGroups * batch)),
                       dim3(kHeadDim), 0, s, (const float*)workspace, out, a.nsplit);
  }
  return check_launch(who);
}
}  // namespace dsa

extern "C" dsa_status dsa_sparse_gqa_decode(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                            const uint16_t* k_cache, const uint16_t* v_cache,
                                            int64_t tcap, const int32_t* seq_len,
                                            const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_sparse_gqa_decode: tcap must be a positive multiple of 128");
  return sparse_gqa_decode("dsa_sparse_gqa_decode", geom, batch, q, k_cache, v_cache, contiguous_map(tcap), seq_len,
                           sel, n_sel, out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_sparse_gqa_decode_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                                  const dsa_page_table* pages, const uint16_t* k_pool,
                                                  const uint16_t* v_pool, const int32_t* seq_len,
                                                  const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                                  void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_sparse_gqa_decode_paged", pages, &cm);
  if (st != DSA_OK) return st;
  return sparse_gqa_decode("dsa_sparse_gqa_decode_paged", geom, batch, q, k_pool, v_pool, cm, seq_len, sel, n_sel,
                           out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_sparse_gqa_decode_fp8(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                                const uint8_t* k8_cache, const uint8_t* v8_cache, const float* kv_scale,
                                                int64_t tcap, const int32_t* seq_len, const int32_t* sel,
                                                const int32_t* n_sel, uint16_t* out, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_sparse_gqa_decode_fp8: tcap must be a positive multiple of 128");
  const Fp8Kv f8{k8_cache, v8_cache, kv_scale};
  return sparse_gqa_decode("dsa_sparse_gqa_decode_fp8", geom, batch, q, nullptr, nullptr, contiguous_map(tcap),
                           seq_len, sel, n_sel, out, workspace, workspace_bytes, stream, &f8);
}

extern "C" dsa_status dsa_sparse_gqa_decode_fp8_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                                      const dsa_page_table* pages, const uint8_t* k8_pool,
                                                      const uint8_t* v8_pool, const float* kvs_pool,
                                                      const int32_t* seq_len, const int32_t* sel, const int32_t* n_sel,
                                                      uint16_t* out, void* workspace, size_t workspace_bytes,
                                                      void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_sparse_gqa_decode_fp8_paged", pages, &cm);
  if (st != DSA_OK) return st;
  const Fp8Kv f8{k8_pool, v8_pool, kvs_pool};
  return sparse_gqa_decode("dsa_sparse_gqa_decode_fp8_paged", geom, batch, q, nullptr, nullptr, cm, seq_len, sel,
                           n_sel, out, workspace, workspace_bytes, stream, &f8);
}

extern "C" size_t dsa_sparse_gqa_prefill_workspace_size(const dsa_geometry* geom, int32_t n_queries) {
  (void)geom;
  if (n_queries <= 0) return 256;
  const size_t rows = (size_t)n_queries * kGroups * kPreSplits * 16;
  return align256(rows * kHeadDim * sizeof(uint16_t)) + rows * 2 * sizeof(float) + 256;
}

static dsa_status sparse_gqa_prefill(const char* who, const dsa_geometry* geom, int32_t n_queries,
                                     const uint16_t* q, const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                     const uint16_t* k_cache, const uint16_t* v_cache, const CacheMap& cm,
                                     const int32_t* sel, const int32_t* n_sel, uint16_t* out, void* workspace,
                                     size_t workspace_bytes, void* stream, const Fp8Kv* f8 = nullptr,
                                     bool merged = false) {
  const std::string w(who);
  if (n_queries < 0 || n_seqs < 0) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": bad sizes");
  if (n_queries == 0) return DSA_OK;
  if (n_seqs == 0) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": n_seqs must be positive");
  const bool kv_ok = f8 ? (f8->k8 && f8->v8 && f8->kvs) : (k_cache && v_cache);
  if (!q || !q_seq || !q_pos || !kv_ok || !sel || !n_sel || !out || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, w + ": NULL pointer");
  if ((size_t)workspace & 255) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": workspace must be 256-byte aligned");
  if (workspace_bytes < dsa_sparse_gqa_prefill_workspace_size(geom, n_queries))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, w + ": workspace too small");
  if (n_queries > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, w + ": more than 2^24 queries");
  // region slots are kept as 32-bit values
  if (!cm.bt && (int64_t)n_seqs * kGroups * cm.R > ((int64_t)1 << 31))
    return fail(DSA_ERR_UNSUPPORTED, w + ": n_seqs * 4 * tcap/8 must stay below 2^31");
  PrefillArgs a;
  a.q = q; a.qseq = q_seq; a.qpos = q_pos; a.k = k_cache; a.v = v_cache; a.sel = sel; a.nsel = n_sel;
  const size_t rows = (size_t)n_queries * kGroups * kPreSplits * 16;
  a.part_o = (uint16_t*)workspace;
  a.part_ml = (float*)((char*)workspace + align256(rows * kHeadDim * sizeof(uint16_t)));
  a.cm = cm; a.nq = n_queries; a.n_seqs = n_seqs; a.topk = geom->topk;
  a.k8 = f8 ? f8->k8 : nullptr; a.v8 = f8 ? f8->v8 : nullptr; a.kvs = f8 ? f8->kvs : nullptr;
  a.rsplit = (int32_t)((cm.R + kPreSplits - 1) / kPreSplits);
  a.scale_log2 = geom->softmax_scale * kLog2e;
  hipStream_t s = as_stream(stream);
  if (merged) {
    ProfScope prof_("k_sgqa_prefill_merged", s);
    const dim3 grid((unsigned)(kPreSplits * kGroups * ((n_queries + 4 * kMrgQ - 1) / (4 * kMrgQ))));
    hipLaunchKernelGGL(k_sgqa_prefill_merged, grid, dim3(256), 0, s, a);
  } else {
    ProfScope prof_("k_sgqa_prefill", s);
    const dim3 grid((unsigned)(kPreSplits * kGroups * ((n_queries + 3) / 4)));
    if (f8) hipLaunchKernelGGL(k_sgqa_prefill<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_sgqa_prefill<false>, grid, dim3(256), 0, s, a);
  }
  dsa_status st = check_launch(who);
  if (st != DSA_OK) return st;
  {
    ProfScope prof_("k_sgqa_merge", s);
    hipLaunchKernelGGL(k_sgqa_merge_pre, dim3((unsigned)(kGroups * (int64_t)n_queries)), dim3(256), 0, s,
                       (const uint16_t*)a.part_o, (const float*)a.part_ml, out);
  }
  return check_launch(who);
}

extern "C" dsa_status dsa_sparse_gqa_prefill(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                             const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                             const uint16_t* k_cache, const uint16_t* v_cache,
                                             int64_t tcap, const int32_t* sel, const int32_t* n_sel,
                                             uint16_t* out, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_sparse_gqa_prefill: tcap must be a positive multiple of 128");
  return sparse_gqa_prefill("dsa_sparse_gqa_prefill", geom, n_queries, q, q_seq, q_pos, n_seqs, k_cache, v_cache,
                            contiguous_map(tcap), sel, n_sel, out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_sparse_gqa_prefill_merged(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                                    const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                                    const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                                    const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                                    void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_sparse_gqa_prefill_merged: tcap must be a positive multiple of 128");
  return sparse_gqa_prefill("dsa_sparse_gqa_prefill_merged", geom, n_queries, q, q_seq, q_pos, n_seqs, k_cache,
                            v_cache, contiguous_map(tcap), sel, n_sel, out, workspace, workspace_bytes, stream,
                            nullptr, true);
}

extern "C" dsa_status dsa_sparse_gqa_prefill_merged_paged(const dsa_geometry* geom, int32_t n_queries,
                                                          const uint16_t* q, const int32_t* q_seq,
                                                          const int32_t* q_pos, int32_t n_seqs,
                                                          const dsa_page_table* pages, const uint16_t* k_pool,
                                                          const uint16_t* v_pool, const int32_t* sel,
                                                          const int32_t* n_sel, uint16_t* out, void* workspace,
                                                          size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_sparse_gqa_prefill_merged_paged", pages, &cm);
  if (st != DSA_OK) return st;
  return sparse_gqa_prefill("dsa_sparse_gqa_prefill_merged_paged", geom, n_queries, q, q_seq, q_pos, n_seqs, k_pool,
                            v_pool, cm, sel, n_sel, out, workspace, workspace_bytes, stream, nullptr, true);
}

extern "C" dsa_status dsa_sparse_gqa_prefill_paged(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                                   const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                                   const dsa_page_table* pages, const uint16_t* k_pool,
                                                   const uint16_t* v_pool, const int32_t* sel, const int32_t* n_sel,
                                                   uint16_t* out, void* workspace, size_t workspace_bytes,
                                                   void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_sparse_gqa_prefill_paged", pages, &cm);
  if (st != DSA_OK) return st;
  return sparse_gqa_prefill("dsa_sparse_gqa_prefill_paged", geom, n_queries, q, q_seq, q_pos, n_seqs, k_pool,
                            v_pool, cm, sel, n_sel, out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_sparse_gqa_prefill_fp8(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                                 const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                                 const uint8_t* k8_cache, const uint8_t* v8_cache,
                                                 const float* kv_scale, int64_t tcap, const int32_t* sel,
                                                 const int32_t* n_sel, uint16_t* out, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_sparse_gqa_prefill_fp8: tcap must be a positive multiple of 128");
  const Fp8Kv f8{k8_cache, v8_cache, kv_scale};
  return sparse_gqa_prefill("dsa_sparse_gqa_prefill_fp8", geom, n_queries, q, q_seq, q_pos, n_seqs, nullptr, nullptr,
                            contiguous_map(tcap), sel, n_sel, out, workspace, workspace_bytes, stream, &f8);
}

extern "C" dsa_status dsa_sparse_gqa_prefill_fp8_paged(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                                       const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                                       const dsa_page_table* pages, const uint8_t* k8_pool,
                                                       const uint8_t* v8_pool, const float* kvs_pool,
                                                       const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                                       void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_sparse_gqa_prefill_fp8_paged", pages, &cm);
  if (st != DSA_OK) return st;
  const Fp8Kv f8{k8_pool, v8_pool, kvs_pool};
  return sparse_gqa_prefill("dsa_sparse_gqa_prefill_fp8_paged", geom, n_queries, q, q_seq, q_pos, n_seqs, nullptr,
                            nullptr, cm, sel, n_sel, out, workspace, workspace_bytes, stream, &f8);
}

extern "C" size_t swa_attention_workspace_size(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                                               int32_t max_new_per_seq) {
  (void)geom;
  (void)window;
  if (n_seqs <= 0 || max_new_per_seq <= 0) return 256;
  if (max_new_per_seq == 1) return 256;  // decode: one launch, no workspace
  const size_t one = (size_t)n_seqs * kGroups * nstage_of(max_new_per_seq) * kRegion * kHeadDim * sizeof(uint16_t);
  return 2 * ((one + 255) / 256 * 256) + 256;
}

static dsa_status swa_check(const dsa_geometry* geom, int32_t window, int32_t n_seqs, int32_t max_new,
                            const char* who) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (window != kWindow) return fail(DSA_ERR_UNSUPPORTED, std::string(who) + ": window must be 512");
  if (n_seqs < 0 || max_new < 0) return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": negative size");
  if (n_seqs > 65535) return fail(DSA_ERR_UNSUPPORTED, std::string(who) + ": n_seqs > 65535");
  return DSA_OK;
}

extern "C" dsa_status swa_attention(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                                    int32_t max_new_per_seq, const int32_t* seq_pos0, const int32_t* seq_row0,
                                    const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                    const uint16_t* k_ring, const uint16_t* v_ring, uint16_t* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = swa_check(geom, window, n_seqs, max_new_per_seq, "swa_attention");
  if (st != DSA_OK) return st;
  if (n_seqs == 0 || max_new_per_seq == 0) return DSA_OK;
  if (!seq_pos0 || !seq_row0 || !q || !k_new || !v_new || !k_ring || !v_ring || !out || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, "swa_attention: NULL pointer");
  if ((size_t)workspace & 255)
    return fail(DSA_ERR_INVALID_ARGUMENT, "swa_attention: workspace must be 256-byte aligned");
  if (workspace_bytes < swa_attention_workspace_size(geom, window, n_seqs, max_new_per_seq))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "swa_attention: workspace too small");
  SwaArgs a;
  a.pos0 = seq_pos0; a.row0 = seq_row0; a.q = q; a.k_new = k_new; a.v_new = v_new;
  a.k_ring = k_ring; a.v_ring = v_ring; a.out = out;
  a.n_seqs = n_seqs; a.max_new = max_new_per_seq; a.nst = nstage_of(max_new_per_seq); a.window = window;
  a.rows = (int64_t)n_seqs * max_new_per_seq;
  a.scale_log2 = geom->softmax_scale * kLog2e;
  const size_t one = (size_t)n_seqs * kGroups * a.nst * kRegion * kHeadDim * sizeof(uint16_t);
  a.st_k = (uint16_t*)workspace;
  a.st_v = (uint16_t*)((char*)workspace + (one + 255) / 256 * 256);
  hipStream_t s = as_stream(stream);
  if (max_new_per_seq == 1) {  // decode: the attention kernels patch the new token in themselves
    swa_decode_launch(a, nullptr, nullptr, s);
    return check_launch("swa_attention");
  }
  {
    ProfScope prof_("k_swa_stage", s);
    hipLaunchKernelGGL(k_swa_stage, dim3(a.nst, n_seqs), dim3(256), 0, s, a);
  }
  st = check_launch("swa_attention: stage");
  if (st != DSA_OK) return st;
  if (max_new_per_seq >= 2 * kBandQ) {  // chunks: the band kernel shares each window across 8 tokens
    ProfScope prof_("k_swa_band", s);
    const unsigned tiles = (unsigned)((max_new_per_seq + kBandQ - 1) / kBandQ);
    hipLaunchKernelGGL(k_swa_band, dim3((tiles + 7) / 8 * 8, n_seqs, kGroups), dim3(256), 0, s, a);
  } else {
    // few blocks: keep two chunks in flight per wave; many: two blocks per CU instead
    ProfScope prof_("k_swa_attend", s);
    {
      const dim3 grid(max_new_per_seq, n_seqs, kGroups);
      if ((int64_t)max_new_per_seq * n_seqs * kGroups < 1024)
        hipLaunchKernelGGL((k_swa_attend<2>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((k_swa_attend<0>), grid, dim3(256), 0, s, a);
    }
  }
  return check_launch("swa_attention");
}

extern "C" dsa_status swa_decode_step(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                                      const int32_t* seq_pos, const uint16_t* q, const uint16_t* k_new,
                                      const uint16_t* v_new, uint16_t* k_ring, uint16_t* v_ring, uint16_t* out,
                                      void* stream) {
  dsa_status st = swa_check(geom, window, n_seqs, 1, "swa_decode_step");
  if (st != DSA_OK) return st;
  if (n_seqs == 0) return DSA_OK;
  if (!seq_pos || !q || !k_new || !v_new || !k_ring || !v_ring || !out)
    return fail(DSA_ERR_INVALID_ARGUMENT, "swa_decode_step: NULL pointer");
  SwaArgs a = {};
  a.pos0 = seq_pos; a.row0 = nullptr; a.q = q; a.k_new = k_new; a.v_new = v_new;
  a.k_ring = k_ring; a.v_ring = v_ring; a.out = out;
  a.n_seqs = n_seqs; a.max_new = 1; a.window = window; a.rows = n_seqs;
  a.scale_log2 = geom->softmax_scale * kLog2e;
  swa_decode_launch(a, k_ring, v_ring, as_stream(stream));
  return check_launch("swa_decode_step");
}

extern "C" dsa_status swa_ring_append(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                                      int32_t max_new_per_seq, const int32_t* seq_pos0, const int32_t* seq_row0,
                                      const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_ring,
                                      uint16_t* v_ring, void* stream) {
  dsa_status st = swa_check(geom, window, n_seqs, max_new_per_seq, "swa_ring_append");
  if (st != DSA_OK) return st;
  if (n_seqs == 0 || max_new_per_seq == 0) return DSA_OK;
  if (!seq_pos0 || !seq_row0 || !k_new || !v_new || !k_ring || !v_ring)
    return fail(DSA_ERR_INVALID_ARGUMENT, "swa_ring_append: NULL pointer");
  SwaArgs a = {};
  a.pos0 = seq_pos0; a.row0 = seq_row0; a.k_new = k_new; a.v_new = v_new;
  a.n_seqs = n_seqs; a.max_new = max_new_per_seq; a.window = window;
  a.rows = (int64_t)n_seqs * max_new_per_seq;
  {
    ProfScope prof_("k_ring_append", as_stream(stream));
    hipLaunchKernelGGL(k_ring_append, dim3(max_new_per_seq, n_seqs), dim3(256), 0, as_stream(stream), a,
                       k_ring, v_ring);
  }
  return check_launch("swa_ring_append");
}
