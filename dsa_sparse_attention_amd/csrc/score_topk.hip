// Indexer scoring and top-k region selection.
//
// [P2] yfxerp.com/news/376439, section 索引器打分 + Top-K 选择: score_regions
// rates every region summary of the request against the query, a radix-style
// top-k keeps the best 512 and the region holding the query is always kept;
// [P3] kwkr.cn/news/593658, section 一, kernel list (indexer logits + radix
// top-k threshold).  The score maths is not on the pages; the stand-in is
//   s_g(r) = sum_{h in 4g..4g+3} z_h * ReLU(q_h . S_g[r]),
// S_g[r] = E4M3 summary * scale, heads 4g..4g+3 feeding KV group g ([P2]
// same section: regions are tied one-to-one to the 4 GQA groups).
//
// Design (gfx950):
//  * k_score streams the summaries once, coalesced, with the dot products on
//    the matrix cores: A = the query's 4 group heads (rows; up to 4 queries
//    per 16-row MFMA tile), B = 16 regions x 32 channels of E4M3 codes turned
//    into bf16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1).  The channel
//    order inside one 256-d dot is permuted so that each lane reads 64
//    contiguous bytes of one region; A uses the same permutation.  For decode
//    it also builds a 4096-bin histogram of the top 12 bits of each score's
//    order-preserving key (LDS atomics, flushed with integer atomics).
//  * k_select (one block per (query, group)) finds the exact k-th largest
//    64-bit key (score key << 32 | ~region) by radix narrowing: 12-bit digits
//    over global memory until the candidates fit in LDS, then 8-bit digits in
//    LDS.  Keys are unique, so ties go to the lower region exactly.  The
//    selected regions are bitonic-sorted ascending.
#include "common.hpp"

namespace dsa {

constexpr int kScoreRange = 1024;  // regions per k_score block
constexpr int kTile = 16;          // regions per MFMA tile
constexpr int kHistBins = 4096;    // level-0 digit: key bits 31..20
constexpr int kSelThreads = 512;
constexpr int kSelCap = 4096;      // LDS candidate capacity of k_select

struct ScoreArgs {
  const uint16_t* iq;   // [Nq][16][P]
  const float* z;       // [Nq][16]
  const int32_t* qseq;  // [Nq]
  const int32_t* qpos;  // [Nq]
  const uint8_t* summ;  // [S][G][R][P]
  const float* scale;   // [S][G][R]
  float* scores;        // workspace [Nq][G][ws_stride]
  float* scores_out;    // nullable [Nq][G][max_regions]
  uint32_t* hist;       // [Nq][G][4096] (decode only)
  int64_t R;            // tcap / 8
  int32_t nq, n_seqs, max_regions, ws_stride;
};

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Current region c of a query (clamped so every index stays in bounds).
__device__ __forceinline__ int64_t current_region(int32_t pos, int64_t R, int32_t max_regions) {
  int64_t c = pos < 0 ? 0 : (int64_t)pos / kRegion;
  if (c > R - 1) c = R - 1;
  if (c > max_regions - 1) c = max_regions - 1;
  return c;
}

// 16 E4M3 codes -> two bf16x8 operands (exact conversion).
__device__ __forceinline__ void codes_to_bf16(u32x4 c, bf16x8& lo, bf16x8& hi) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, true);
  bf16x2 p4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.z, 1.0f, false);
  bf16x2 p5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.z, 1.0f, true);
  bf16x2 p6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.w, 1.0f, false);
  bf16x2 p7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.w, 1.0f, true);
  lo = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  hi = bf16x8{p4[0], p4[1], p5[0], p5[1], p6[0], p6[1], p7[0], p7[1]};
}

// QW queries per wave (1: decode, rows 0..3 of the tile used; 16: prefill,
// four row-sets of 4 queries x 4 heads).  Block = 4 waves sharing
// (region range, group, query block); wave w takes tiles w, w+4, ...
template <int QW>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a) {
  constexpr int NRS = (QW + 3) / 4;
  const int g = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kb = lane >> 4;
  const int q0 = blockIdx.z * QW;
  const int64_t range0 = (int64_t)blockIdx.x * kScoreRange;

  __shared__ uint32_t hist_lds[QW == 1 ? kHistBins : 1];
  if (QW == 1) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) hist_lds[i] = 0;
    __syncthreads();
  }

  // Per-query info of the queries this lane's output rows belong to.
  uint32_t remaining = 0;  // bit j: query q0+j still to process
  for (int j = 0; j < QW; ++j)
    if (q0 + j < a.nq) remaining |= 1u << j;

  while (remaining) {
    const int lead = __builtin_ctz(remaining);
    int32_t seq = a.qseq[q0 + lead];
    seq = seq < 0 ? 0 : (seq >= a.n_seqs ? a.n_seqs - 1 : seq);
    uint32_t active = 0;
    int64_t cmax = 0;
    for (int j = 0; j < QW; ++j) {
      if (!(remaining >> j & 1u)) continue;
      int32_t sj = a.qseq[q0 + j];
      sj = sj < 0 ? 0 : (sj >= a.n_seqs ? a.n_seqs - 1 : sj);
      if (sj == seq) {
        active |= 1u << j;
        int64_t cj = current_region(a.qpos[q0 + j], a.R, a.max_regions);
        cmax = cj > cmax ? cj : cmax;
      }
    }
    remaining &= ~active;

    // A operand: rows = (query, head) pairs of group g; channel permutation
    // pi(s, kb, e) = 64*(s/2) + 16*kb + 8*(s%2) + e.
    bf16x8 A[NRS][8];
    float zq[NRS][4];
    int64_t cq[NRS];
    int32_t qidx[NRS];
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      const int jrow = (QW == 1) ? 0 : 4 * rs + (n >> 2);     // query of A row n
      const bool rvalid = (QW == 1 ? n < 4 : true) && (active >> jrow & 1u);
      const int hh = 4 * g + (n & 3);
      const uint16_t* qp = a.iq + ((int64_t)(q0 + jrow) * kIdxHeads + hh) * kProxy + 16 * kb;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 v = {0, 0, 0, 0};
        if (rvalid) v = ld16(qp + 64 * (s >> 1) + 8 * (s & 1));
        A[rs][s] = as_bf16x8(v);
      }
      // output rows 4kb..4kb+3 of row-set rs belong to query jout
      const int jout = (QW == 1) ? 0 : 4 * rs + kb;
      const bool ovalid = (QW == 1 ? kb == 0 : true) && (active >> jout & 1u);
      qidx[rs] = ovalid ? q0 + jout : -1;
      if (ovalid) {
        f32x4 zz = *(const f32x4*)(a.z + (int64_t)(q0 + jout) * kIdxHeads + 4 * g);
        zq[rs][0] = zz[0]; zq[rs][1] = zz[1]; zq[rs][2] = zz[2]; zq[rs][3] = zz[3];
        cq[rs] = current_region(a.qpos[q0 + jout], a.R, a.max_regions);
      } else {
        zq[rs][0] = zq[rs][1] = zq[rs][2] = zq[rs][3] = 0.0f;
        cq[rs] = 0;
      }
    }

    const int64_t rend = (range0 + kScoreRange < cmax) ? range0 + kScoreRange : cmax;
    const uint8_t* sbase = a.summ + ((int64_t)seq * kGroups + g) * a.R * kProxy;
    const float* scbase = a.scale + ((int64_t)seq * kGroups + g) * a.R;
#pragma unroll 2
    for (int64_t t0 = range0 + (int64_t)wave * kTile; t0 < rend; t0 += 4 * kTile) {
      int64_t r = t0 + n;
      const int64_t rl = r < a.R ? r : a.R - 1;
      const uint8_t* rp = sbase + rl * kProxy + 16 * kb;
      u32x4 c0 = ldg16(rp), c1 = ldg16(rp + 64), c2 = ldg16(rp + 128), c3 = ldg16(rp + 192);
      const float sc = scbase[rl];
      bf16x8 B[8];
      codes_to_bf16(c0, B[0], B[1]);
      codes_to_bf16(c1, B[2], B[3]);
      codes_to_bf16(c2, B[4], B[5]);
      codes_to_bf16(c3, B[6], B[7]);
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma16x16x32(A[rs][s], B[s], acc);
        if (qidx[rs] >= 0 && r < cq[rs]) {
          float s = zq[rs][0] * fmaxf(acc[0], 0.0f);
          s = fmaf(zq[rs][1], fmaxf(acc[1], 0.0f), s);
          s = fmaf(zq[rs][2], fmaxf(acc[2], 0.0f), s);
          s = fmaf(zq[rs][3], fmaxf(acc[3], 0.0f), s);
          s *= sc;
          const int64_t pq = (int64_t)qidx[rs] * kGroups + g;
          a.scores[pq * a.ws_stride + r] = s;
          if (a.scores_out) a.scores_out[pq * a.max_regions + r] = s;
          if (QW == 1) atomicAdd(&hist_lds[score_key(s) >> 20], 1u);
        }
      }
    }
  }

  if (QW == 1) {
    __syncthreads();
    if (q0 < a.nq) {
      uint32_t* gh = a.hist + ((int64_t)q0 * kGroups + g) * kHistBins;
      for (int i = threadIdx.x; i < kHistBins; i += 256) {
        uint32_t v = hist_lds[i];
        if (v) atomicAdd(gh + i, v);
      }
    }
  }
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------
// k_select
// ---------------------------------------------------------------------------

// Exclusive prefix sum over the block (kSelThreads threads).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < kSelThreads / 64; ++i) {
    if (i < w) base += wsum[i];
    tot += wsum[i];
  }
  if (total) *total = tot;
  __syncthreads();
  return base + x - v;
}

// Given hist[0..nb) of the elements still in play, find digit d (scanning
// from the top) with above(d) < need <= above(d) + hist[d].  Returns d and
// writes above(d) to *above_out.  All threads get the result.
__device__ __forceinline__ int find_digit(const uint32_t* hist, int nb, uint32_t need,
                                          uint32_t* above_out, uint32_t* wsum, int* sh_d,
                                          uint32_t* sh_above) {
  // thread t owns bins [per*t', per*t'+per) with t' counted from the top.
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  const int tr = threadIdx.x;  // rank from the top
  const int hi_bin = nb - 1 - per * tr;  // highest bin of this thread
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) {
    int bin = hi_bin - i;
    if (bin >= 0) local += hist[bin];
  }
  uint32_t run = block_excl_scan(local, wsum, nullptr);
  for (int i = 0; i < per; ++i) {
    int bin = hi_bin - i;
    if (bin < 0) break;
    uint32_t h = hist[bin];
    if (run < need && run + h >= need) {
      *sh_d = bin;
      *sh_above = run;
    }
    run += h;
  }
  __syncthreads();
  *above_out = *sh_above;
  int d = *sh_d;
  __syncthreads();
  return d;
}

struct SelectArgs {
  const float* scores;   // [Nq][G][ws_stride]
  uint32_t* hist;        // [Nq][G][4096] or nullptr (computed here)
  const int32_t* qpos;
  int32_t* sel;          // [Nq][G][topk]
  int32_t* nsel;         // [Nq][G]
  int64_t R;
  int32_t nq, max_regions, ws_stride, topk;
};

__device__ __forceinline__ uint64_t cand_key(const float* sc, int64_t r) {
  return ((uint64_t)score_key(sc[r]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)r);
}

__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs a) {
  const int64_t pq = blockIdx.x;  // (query, group)
  const int qi = (int)(pq / kGroups);
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint64_t list[kSelCap];
  __shared__ int32_t outl[kMaxTopk];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ int sh_d;
  __shared__ uint32_t sh_above, sh_count;

  if (tid == 0) {
    sh_d = 0;
    sh_above = 0;
  }
  __syncthreads();
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const int64_t need64 = (c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1);
  const uint32_t need = (uint32_t)need64;
  int32_t* sel = a.sel + pq * a.topk;
  const float* sc = a.scores + pq * a.ws_stride;

  if (need64 == c) {  // every candidate fits: regions 0..c
    for (int i = tid; i < a.topk; i += kSelThreads) sel[i] = (i <= c) ? i : -1;
    if (tid == 0) a.nsel[pq] = (int32_t)(c + 1);
    return;
  }
  if (need == 0) {  // topk == 1: only the current region
    for (int i = tid; i < a.topk; i += kSelThreads) sel[i] = (i == 0) ? (int32_t)c : -1;
    if (tid == 0) a.nsel[pq] = 1;
    return;
  }

  // ---- level 0: 12-bit digit of the score key (bits 63..52 of the 64-bit key)
  if (a.hist) {
    const uint32_t* gh = a.hist + pq * kHistBins;
    for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = gh[i];
  } else {
    for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t r = tid; r < c; r += kSelThreads) atomicAdd(&hist[score_key(sc[r]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t above;
  int d = find_digit(hist, kHistBins, need, &above, wsum, &sh_d, &sh_above);
  uint64_t prefix = (uint64_t)d;
  int shift = 52;
  uint32_t inbin = hist[d];
  __syncthreads();

  // ---- narrow over global memory until the candidates fit in LDS
  while (above + inbin > (uint32_t)kSelCap && shift > 0) {
    const int width = shift >= 12 ? 12 : shift;
    const int nshift = shift - width;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t r = tid; r < c; r += kSelThreads) {
      uint64_t k = cand_key(sc, r);
      if ((k >> shift) == prefix) atomicAdd(&hist[(uint32_t)(k >> nshift) & (nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t ab;
    d = find_digit(hist, nb, need - above, &ab, wsum, &sh_d, &sh_above);
    above += ab;
    inbin = hist[d];
    prefix = (prefix << width) | (uint64_t)d;
    shift = nshift;
    __syncthreads();
  }

  // ---- collect everything at or above the current bin into LDS
  if (tid == 0) sh_count = 0;
  __syncthreads();
  for (int64_t r = tid; r < c; r += kSelThreads) {
    uint64_t k = cand_key(sc, r);
    if ((k >> shift) >= prefix) {
      uint32_t pos = atomicAdd(&sh_count, 1u);
      if (pos < (uint32_t)kSelCap) list[pos] = k;
    }
  }
  __syncthreads();
  const uint32_t M = sh_count < (uint32_t)kSelCap ? sh_count : (uint32_t)kSelCap;
  uint32_t need_in = need - above;

  // ---- finish in LDS with 8-bit digits
  while (shift > 0 && inbin != need_in) {
    const int width = shift >= 8 ? 8 : shift;
    const int nshift = shift - width;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < M; i += kSelThreads) {
      uint64_t k = list[i];
      if ((k >> shift) == prefix) atomicAdd(&hist[(uint32_t)(k >> nshift) & (nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t ab;
    d = find_digit(hist, nb, need_in, &ab, wsum, &sh_d, &sh_above);
    need_in -= ab;
    inbin = hist[d];
    prefix = (prefix << width) | (uint64_t)d;
    shift = nshift;
    __syncthreads();
  }

  // ---- selected = list entries with (key >> shift) >= prefix (exactly need)
  if (tid == 0) sh_count = 0;
  __syncthreads();
  for (uint32_t i = tid; i < M; i += kSelThreads) {
    uint64_t k = list[i];
    if ((k >> shift) >= prefix) {
      uint32_t pos = atomicAdd(&sh_count, 1u);
      if (pos < (uint32_t)kMaxTopk - 1) outl[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
    }
  }
  __syncthreads();
  const uint32_t nsel = need + 1;
  for (int i = tid; i < kMaxTopk; i += kSelThreads) {
    if ((uint32_t)i == need) outl[i] = (int32_t)c;
    else if ((uint32_t)i > need) outl[i] = 0x7FFFFFFF;
  }
  __syncthreads();
  // bitonic sort of 512 ascending
  for (int size = 2; size <= kMaxTopk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < kMaxTopk; i += kSelThreads) {
        int j = i ^ stride;
        if (j > i) {
          bool up = ((i & size) == 0);
          int32_t x = outl[i], y = outl[j];
          if ((x > y) == up) {
            outl[i] = y;
            outl[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < a.topk; i += kSelThreads) sel[i] = ((uint32_t)i < nsel) ? outl[i] : -1;
  if (tid == 0) a.nsel[pq] = (int32_t)nsel;
}

static int64_t ws_stride_of(int32_t max_regions) { return ((int64_t)max_regions + 63) / 64 * 64; }

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_score_topk_workspace_size(const dsa_geometry* geom, int32_t n_queries,
                                                int32_t max_regions) {
  (void)geom;
  if (n_queries <= 0 || max_regions <= 0) return 256;
  size_t hist = (size_t)n_queries * kGroups * kHistBins * sizeof(uint32_t);
  size_t sc = (size_t)n_queries * kGroups * (size_t)ws_stride_of(max_regions) * sizeof(float);
  return hist + sc + 256;
}

extern "C" dsa_status dsa_score_topk(const dsa_geometry* geom, int32_t n_queries,
                                     const uint16_t* index_q, const float* z,
                                     const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                     const uint8_t* summ, const float* scale, int64_t tcap,
                                     int32_t max_regions, int32_t* sel, int32_t* n_sel,
                                     float* scores_out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (n_queries < 0 || n_seqs < 0 || max_regions < 0 || tcap <= 0 || tcap % kRegion)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: bad sizes (tcap must be a positive multiple of 8)");
  if (n_queries == 0) return DSA_OK;
  if (n_seqs == 0 || max_regions == 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: n_seqs and max_regions must be positive");
  if (!index_q || !z || !q_seq || !q_pos || !summ || !scale || !sel || !n_sel || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: NULL pointer");
  if ((size_t)workspace & 255)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: workspace must be 256-byte aligned");
  if (workspace_bytes < dsa_score_topk_workspace_size(geom, n_queries, max_regions))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_score_topk: workspace too small");
  hipStream_t s = as_stream(stream);

  uint32_t* hist = (uint32_t*)workspace;
  const int64_t hist_n = (int64_t)n_queries * kGroups * kHistBins;
  float* scores = (float*)(hist + hist_n);
  const int32_t stride = (int32_t)ws_stride_of(max_regions);

  ScoreArgs sa;
  sa.iq = index_q; sa.z = z; sa.qseq = q_seq; sa.qpos = q_pos; sa.summ = summ; sa.scale = scale;
  sa.scores = scores; sa.scores_out = scores_out; sa.hist = hist; sa.R = tcap / kRegion;
  sa.nq = n_queries; sa.n_seqs = n_seqs; sa.max_regions = max_regions; sa.ws_stride = stride;
  const int ranges = (max_regions + kScoreRange - 1) / kScoreRange;
  // Decode-shaped calls (few queries, many regions) score one query per wave
  // and build the level-0 histogram on the fly; prefill-shaped calls score
  // 16 queries per wave so each summary tile feeds 4 MFMA row-sets.
  const bool decode_shape = n_queries < 64;
  if (decode_shape) {
    int64_t fill_blocks = (hist_n + 255) / 256;
    if (fill_blocks > 4096) fill_blocks = 4096;
    {
      ProfScope prof_("k_fill_u32", s);
      hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)fill_blocks), dim3(256), 0, s, hist, hist_n, 0u);
    }
    {
      ProfScope prof_("k_score_decode", s);
      hipLaunchKernelGGL(k_score<1>, dim3(ranges, kGroups, n_queries), dim3(256), 0, s, sa);
    }
  } else {
    {
      ProfScope prof_("k_score_prefill", s);
      hipLaunchKernelGGL(k_score<16>, dim3(ranges, kGroups, (n_queries + 15) / 16), dim3(256), 0, s, sa);
    }
  }
  st = check_launch("dsa_score_topk: score");
  if (st != DSA_OK) return st;

  SelectArgs se;
  se.scores = scores; se.hist = decode_shape ? hist : nullptr; se.qpos = q_pos; se.sel = sel;
  se.nsel = n_sel; se.R = tcap / kRegion; se.nq = n_queries; se.max_regions = max_regions;
  se.ws_stride = stride; se.topk = geom->topk;
  {
    ProfScope prof_("k_select", s);
    hipLaunchKernelGGL(k_select, dim3((unsigned)((int64_t)n_queries * kGroups)), dim3(kSelThreads), 0, s, se);
  }
  return check_launch("dsa_score_topk: select");
}
