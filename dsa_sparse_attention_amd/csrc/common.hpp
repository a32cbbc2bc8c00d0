// Shared device/host helpers of the gfx950 DSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/dsa.h"

namespace dsa {

// Compiled geometry ([P2] sparse_config table; [P3] section 一 config table).
constexpr int kRegion = 8;
constexpr int kProxy = 256;
constexpr int kGroups = 4;
constexpr int kIdxHeads = 16;
constexpr int kIdxHeadsPerGroup = kIdxHeads / kGroups;  // 4
constexpr int kQHeads = 64;
constexpr int kHeadsPerGroup = kQHeads / kGroups;  // 16 = one MFMA tile edge
constexpr int kHeadDim = 192;
constexpr int kMaxTopk = 512;
constexpr int kWindow = 512;
constexpr int kTcapAlign = 128;  // cache capacity granule: 16 regions = one summary tile

// Summaries of one (sequence, group) are stored in tiles of 16 regions
// (4096 bytes).  Byte j of region r lives at
//   (r/16)*4096 + (j/64)*1024 + ((j%64)/16)*256 + (r%16)*16 + j%16,
// i.e. each 1 KB quarter of a tile holds, for every region of the tile, the
// 16-byte pieces that one 64-lane load instruction hands to the MFMA
// B operand (lane 16*kb + n <- region n, channels 64q + 16kb .. +15).
__device__ __forceinline__ int64_t summ_tile_base(int64_t r) { return (r >> 4) * 4096; }

// Where the caches of a sequence live.  Every cached tensor of the layer is
// stored per region slot: one region of one group (1536 bf16 of K, 1536 of
// V, 8 index_k rows, 256 summary bytes, one scale).
//   contiguous caches (capacity tcap, R = tcap/8 regions per sequence):
//     slot(s, g, r) = (s*G + g)*R + r
//   paged caches (pages of 128 positions = 16 regions, one page id for every
//   tensor of the cache, block table bt[n_seqs][max_pages]):
//     slot(s, g, r) = (bt[s][r/16]*G + g)*16 + r%16
// In both, summary tile slot(s, g, r)/16 holds region r's summary at
// position slot%16 == r%16, and index_k row t of region r is row 8*slot + t.
constexpr int kPageRegions = 16;  // regions per page (128 positions, one summary tile)
struct CacheMap {
  const int32_t* bt;  // block table, or nullptr for contiguous caches
  int64_t R;          // regions per sequence: tcap/8, or max_pages*16
  int32_t bt_stride;  // max_pages (row length of the block table)
  int32_t n_pages;    // pages in every pool; page ids are clamped into [0, n_pages)
};
__device__ __forceinline__ int32_t clamp_page(const CacheMap& m, int32_t pg) {
  return pg < 0 ? 0 : (pg >= m.n_pages ? m.n_pages - 1 : pg);
}
// Block-table entry of region r of sequence s (paged caches; r in [0, R)),
// unclamped, so that a caller can issue the load early and clamp at use.
__device__ __forceinline__ int32_t page_entry(const CacheMap& m, int64_t s, int64_t r) {
  return m.bt[s * m.bt_stride + (r >> 4)];
}
// Page id of region r of sequence s (paged caches; r in [0, R)).
__device__ __forceinline__ int32_t page_of(const CacheMap& m, int64_t s, int64_t r) {
  return clamp_page(m, page_entry(m, s, r));
}
// Slot of region r given its page id (ignored for contiguous caches).
__device__ __forceinline__ int64_t slot_in(const CacheMap& m, int32_t pg, int64_t s, int g, int64_t r) {
  return m.bt ? ((int64_t)pg * kGroups + g) * kPageRegions + (r & (kPageRegions - 1))
              : (s * kGroups + g) * m.R + r;
}
__device__ __forceinline__ int64_t region_slot(const CacheMap& m, int64_t s, int g, int64_t r) {
  return slot_in(m, m.bt ? page_of(m, s, r) : 0, s, g, r);
}

// Keys are stored per region of 8 tokens (1536 bf16) in MFMA A-operand
// order: element (token pos of the region, channel d) lives at
//   ((((pos/4)*6 + (d%48)/8)*4 + d/48)*4 + pos%4)*8 + d%8,
// i.e. 16-byte units ordered (tile pos/4, k-step (d%48)/8, lane slot d/48,
// token pos%4): one 64-lane load of a 4-region chunk reads four contiguous
// 256-byte pieces.
constexpr int kRegionElems = kRegion * kHeadDim;  // 1536
__device__ __forceinline__ int k_tile_offset(int pos, int d) {
  return ((((pos >> 2) * 6 + (d % 48) / 8) * 4 + d / 48) * 4 + (pos & 3)) * 8 + (d & 7);
}

// FP8 K/V caches (per region slot): K8 [1536] bytes, region-tiled: the
// 16-byte unit ((t*3 + s2)*4 + kb)*4 + pos%4 holds token pos (t = pos/4),
// channels 48kb + 16s2 .. +15; V8 [D][8] bytes, region-transposed; KVS [16]
// fp32: the K scales of the 8 tokens, then their V scales.
__device__ __forceinline__ int k8_tile_offset(int pos, int d) {
  return ((((pos >> 2) * 3 + (d % 48) / 16) * 4 + d / 48) * 4 + (pos & 3)) * 16 + (d & 15);
}
constexpr int kKvsPerRegion = 16;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(3))) uint8_t* LdsPtr;  // LDS destination of direct-to-LDS loads

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts inside
// each row of 16 lanes, then row broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// the low and high bf16 of a packed pair, as fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup barrier for hand-offs through LDS only: waits for this wave's LDS
// operations, but not for its global loads still in flight, which
// __syncthreads() (a workgroup fence) would drain first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Max / sum of x over lanes l, l^16, l^32 and l^48 of the wave with gfx950's
// row swaps (each leaves lane l holding x_l and x_{l^16}, or x_l and
// x_{l^32}, in its two results): VALU only, no LDS round trip.
__device__ __forceinline__ float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// D = A(16x32) * B(32x16) + C on the matrix cores; lane l holds A row l%16,
// B column l%16 (8 contraction elements each, slot l/16) and D rows
// 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

#ifndef DSA_NT_LOADS
#define DSA_NT_LOADS 1
#endif
// 16-byte load of data streamed once (non-temporal hint).
__device__ __forceinline__ u32x4 ldg16(const void* p) {
#if DSA_NT_LOADS
  return __builtin_nontemporal_load((const u32x4*)p);
#else
  return *(const u32x4*)p;
#endif
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

}  // namespace dsa

// ---- host-side helpers (api.hip) ----
namespace dsa {
dsa_status fail(dsa_status s, const std::string& msg);
dsa_status check_geometry(const dsa_geometry* g);
dsa_status check_launch(const char* what);
inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Cache maps of the two cache arrangements (host side).
inline CacheMap contiguous_map(int64_t tcap) {
  CacheMap m;
  m.bt = nullptr;
  m.R = tcap / kRegion;
  m.bt_stride = 0;
  m.n_pages = 0;
  return m;
}
// Checks a page table (non-NULL block table, max_pages and n_pages > 0,
// n_pages <= kMaxPages so that region slots fit 31 bits) and builds its map.
constexpr int32_t kMaxPages = 1 << 25;
dsa_status paged_map(const char* who, const dsa_page_table* pt, CacheMap* m);
// FP8 K/V caches (K8, V8, scales; layouts above).
struct Fp8Kv {
  const uint8_t* k8;
  const uint8_t* v8;
  const float* kvs;
};
// Sparse GQA decode over either cache arrangement, bf16 K/V (k_cache, v_cache)
// or, when f8 is given, FP8 K/V (the decode steps call it).
dsa_status sparse_gqa_decode(const char* who, const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                             const uint16_t* k_cache, const uint16_t* v_cache, const CacheMap& cm,
                             const int32_t* seq_len, const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                             void* workspace, size_t workspace_bytes, void* stream, const Fp8Kv* f8 = nullptr);

// Instrumentation: while enabled (dsa_profile_enable), a ProfScope brackets
// the kernel launched inside its lifetime with two hipEvents on the launch
// stream; dsa_profile_kernel_stats sums the intervals per kernel name.
struct ProfScope {
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  int rec;
  hipStream_t stream;
};
}  // namespace dsa
