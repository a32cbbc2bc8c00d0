// Region compression (CSA summaries) and cache writes.
#include "compress_dev.hpp"

namespace dsa {

// One wave per (region, group): lane l owns channels 4l..4l+3.  The block's
// four waves are the four groups of one region.
__global__ __launch_bounds__(256) void k_compress(const uint16_t* __restrict__ ik, CacheMap cm,
                                                  const int32_t* __restrict__ rbeg,
                                                  const int32_t* __restrict__ rend,
                                                  int32_t max_span, uint8_t* __restrict__ summ,
                                                  float* __restrict__ scale) {
  const int b = blockIdx.y;
  const int g = threadIdx.x >> 6;
  const int64_t R = cm.R;
  int64_t r0 = rbeg[b], r1 = rend[b];
  r0 = r0 < 0 ? 0 : (r0 > R ? R : r0);
  r1 = r1 < r0 ? r0 : (r1 > R ? R : r1);
  if (r1 - r0 > max_span) r1 = r0 + max_span;
  const int64_t r = r0 + blockIdx.x;
  if (r >= r1) return;
  compress_region_wave(ik, cm, b, r, g, summ, scale);
}

// One block per new token row: copies K/V (and index_k) into the cache
// layouts (K region-tiled, V region-transposed).
__global__ __launch_bounds__(256) void k_cache_write(
    const int32_t* __restrict__ tok_seq, const int32_t* __restrict__ tok_pos,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ ik_new, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, uint16_t* __restrict__ ik_cache, int32_t n_seqs,
    CacheMap cm) {
  const int64_t i = blockIdx.x;
  const int s = tok_seq[i];
  const int64_t t = tok_pos[i];
  if (s < 0 || s >= n_seqs || t < 0 || t >= cm.R * kRegion) return;
  const int64_t r = t / kRegion;
  const int32_t pg = cm.bt ? page_of(cm, s, r) : 0;
  for (int e = threadIdx.x; e < kGroups * kHeadDim; e += blockDim.x) {
    const int g = e / kHeadDim, d = e - g * kHeadDim;
    const int64_t slot = slot_in(cm, pg, s, g, r);
    k_cache[slot * kRegionElems + k_tile_offset((int)(t % kRegion), d)] = k_new[i * kGroups * kHeadDim + e];
    v_cache[(slot * kHeadDim + d) * kRegion + (t % kRegion)] = v_new[i * kGroups * kHeadDim + e];
  }
  if (ik_new) {
    for (int e = threadIdx.x; e < kGroups * kProxy; e += blockDim.x) {
      const int g = e / kProxy, d = e - g * kProxy;
      const int64_t slot = slot_in(cm, pg, s, g, r);
      ik_cache[(slot * kRegion + t % kRegion) * kProxy + d] = ik_new[i * kGroups * kProxy + e];
    }
  }
}

// FP8 cache write: block = one token row, wave g = group g; lane l owns
// channels 3l..3l+2.  Each (token, group) row of K and of V gets one fp32
// scale amax/448 and its values x/scale (fp32) rounded once to E4M3 (the
// summary rule applied per cached row; the pages only say an FP8 KV cache
// halves it).
__global__ __launch_bounds__(256) void k_cache_write_fp8(const int32_t* __restrict__ tok_seq,
                                                         const int32_t* __restrict__ tok_pos,
                                                         const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new, uint8_t* __restrict__ k8,
                                                         uint8_t* __restrict__ v8, float* __restrict__ kvs,
                                                         int32_t n_seqs, CacheMap cm) {
  const int64_t i = blockIdx.x;
  const int s = tok_seq[i];
  const int64_t t = tok_pos[i];
  if (s < 0 || s >= n_seqs || t < 0 || t >= cm.R * kRegion) return;
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pos = (int)(t % kRegion);
  const int64_t slot = region_slot(cm, s, g, t / kRegion);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = (which ? v_new : k_new) + (i * kGroups + g) * kHeadDim + 3 * lane;
    float x[3];
#pragma unroll
    for (int e = 0; e < 3; ++e) x[e] = bf16_to_f32(src[e]);
    float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fabsf(x[2]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sc = __fdiv_rn(amax, 448.0f);
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const int d = 3 * lane + e;
      const uint8_t code = sc == 0.0f ? 0 : (uint8_t)e4m3_rne_sat(__fdiv_rn(x[e], sc));
      if (which == 0) k8[slot * kRegionElems + k8_tile_offset(pos, d)] = code;
      else v8[slot * kRegionElems + d * kRegion + pos] = code;
    }
    if (lane == 0) kvs[slot * kKvsPerRegion + which * kRegion + pos] = sc;
  }
}

}  // namespace dsa

using namespace dsa;

static dsa_status cache_write_fp8(const char* who, int32_t n_tokens, const int32_t* tok_seq, const int32_t* tok_pos,
                                  const uint16_t* k_new, const uint16_t* v_new, uint8_t* k8, uint8_t* v8, float* kvs,
                                  int32_t n_seqs, const CacheMap& cm, void* stream) {
  if (n_tokens < 0 || n_seqs < 0) return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": bad sizes");
  if (n_tokens == 0 || n_seqs == 0) return DSA_OK;
  if (!tok_seq || !tok_pos || !k_new || !v_new || !k8 || !v8 || !kvs)
    return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": NULL pointer");
  {
    ProfScope prof_("k_cache_write", as_stream(stream));
    hipLaunchKernelGGL(k_cache_write_fp8, dim3(n_tokens), dim3(256), 0, as_stream(stream), tok_seq, tok_pos, k_new,
                       v_new, k8, v8, kvs, n_seqs, cm);
  }
  return check_launch(who);
}

extern "C" dsa_status dsa_cache_write_fp8(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                                          const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                                          uint8_t* k8_cache, uint8_t* v8_cache, float* kv_scale, int32_t n_seqs,
                                          int64_t tcap, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_cache_write_fp8: tcap must be a positive multiple of 128");
  return cache_write_fp8("dsa_cache_write_fp8", n_tokens, tok_seq, tok_pos, k_new, v_new, k8_cache, v8_cache, kv_scale,
                         n_seqs, contiguous_map(tcap), stream);
}

extern "C" dsa_status dsa_cache_write_fp8_paged(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                                                const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                                                const dsa_page_table* pages, int32_t n_seqs, uint8_t* k8_pool,
                                                uint8_t* v8_pool, float* kvs_pool, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_cache_write_fp8_paged", pages, &cm);
  if (st != DSA_OK) return st;
  return cache_write_fp8("dsa_cache_write_fp8_paged", n_tokens, tok_seq, tok_pos, k_new, v_new, k8_pool, v8_pool,
                         kvs_pool, n_seqs, cm, stream);
}

// Host: shared bodies of the contiguous and paged entry points.
static dsa_status compress_regions(const char* who, const dsa_geometry* geom, int32_t batch,
                                   const uint16_t* index_k, const CacheMap& cm, const int32_t* region_begin,
                                   const int32_t* region_end, int32_t max_span, uint8_t* summ, float* scale,
                                   void* stream) {
  if (batch == 0 || max_span == 0) return DSA_OK;
  if (!index_k || !region_begin || !region_end || !summ || !scale)
    return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": NULL pointer");
  if (max_span > cm.R) max_span = (int32_t)cm.R;
  if (batch > 65535) return fail(DSA_ERR_UNSUPPORTED, std::string(who) + ": batch > 65535");
  {
    ProfScope prof_("k_compress", as_stream(stream));
    hipLaunchKernelGGL(k_compress, dim3(max_span, batch), dim3(256), 0, as_stream(stream), index_k, cm,
                       region_begin, region_end, max_span, summ, scale);
  }
  return check_launch(who);
}

static dsa_status cache_write(const char* who, int32_t n_tokens, const int32_t* tok_seq, const int32_t* tok_pos,
                              const uint16_t* k_new, const uint16_t* v_new, const uint16_t* ik_new,
                              uint16_t* k_cache, uint16_t* v_cache, uint16_t* ik_cache, int32_t n_seqs,
                              const CacheMap& cm, void* stream) {
  if (n_tokens == 0 || n_seqs == 0) return DSA_OK;
  if (!tok_seq || !tok_pos || !k_new || !v_new || !k_cache || !v_cache)
    return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": NULL pointer");
  if ((ik_new == nullptr) != (ik_cache == nullptr))
    return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": ik_new and the index_k cache must both be set or both NULL");
  {
    ProfScope prof_("k_cache_write", as_stream(stream));
    hipLaunchKernelGGL(k_cache_write, dim3(n_tokens), dim3(256), 0, as_stream(stream), tok_seq, tok_pos, k_new,
                       v_new, ik_new, k_cache, v_cache, ik_cache, n_seqs, cm);
  }
  return check_launch(who);
}

extern "C" dsa_status dsa_compress_regions(const dsa_geometry* geom, int32_t batch,
                                           const uint16_t* index_k, int64_t tcap,
                                           const int32_t* region_begin, const int32_t* region_end,
                                           int32_t max_span, uint8_t* summ, float* scale,
                                           void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (batch < 0 || max_span < 0 || tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_compress_regions: batch/max_span must be >= 0 and tcap a positive multiple of 128");
  return compress_regions("dsa_compress_regions", geom, batch, index_k, contiguous_map(tcap), region_begin,
                          region_end, max_span, summ, scale, stream);
}

extern "C" dsa_status dsa_compress_regions_paged(const dsa_geometry* geom, int32_t batch,
                                                 const dsa_page_table* pages, const uint16_t* ik_pool,
                                                 const int32_t* region_begin, const int32_t* region_end,
                                                 int32_t max_span, uint8_t* summ_pool, float* scale_pool,
                                                 void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_compress_regions_paged", pages, &cm);
  if (st != DSA_OK) return st;
  if (batch < 0 || max_span < 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_compress_regions_paged: batch/max_span must be >= 0");
  return compress_regions("dsa_compress_regions_paged", geom, batch, ik_pool, cm, region_begin, region_end,
                          max_span, summ_pool, scale_pool, stream);
}

extern "C" dsa_status dsa_cache_write(const dsa_geometry* geom, int32_t n_tokens,
                                      const int32_t* tok_seq, const int32_t* tok_pos,
                                      const uint16_t* k_new, const uint16_t* v_new,
                                      const uint16_t* ik_new, uint16_t* k_cache,
                                      uint16_t* v_cache, uint16_t* ik_cache, int32_t n_seqs,
                                      int64_t tcap, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (n_tokens < 0 || n_seqs < 0 || tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_cache_write: bad sizes (tcap must be a positive multiple of 128)");
  return cache_write("dsa_cache_write", n_tokens, tok_seq, tok_pos, k_new, v_new, ik_new, k_cache, v_cache, ik_cache,
                     n_seqs, contiguous_map(tcap), stream);
}

extern "C" dsa_status dsa_cache_write_paged(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                                            const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                                            const uint16_t* ik_new, const dsa_page_table* pages, int32_t n_seqs,
                                            uint16_t* k_pool, uint16_t* v_pool, uint16_t* ik_pool, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_cache_write_paged", pages, &cm);
  if (st != DSA_OK) return st;
  if (n_tokens < 0 || n_seqs < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_cache_write_paged: bad sizes");
  return cache_write("dsa_cache_write_paged", n_tokens, tok_seq, tok_pos, k_new, v_new, ik_new, k_pool, v_pool,
                     ik_pool, n_seqs, cm, stream);
}
