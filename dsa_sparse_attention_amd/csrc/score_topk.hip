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
constexpr int kHistCopies = 8;     // decode histogram stripes (one per XCD by block index)
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
  uint32_t* hist;       // [Nq][G][8][4096] striped level-0 histogram (decode only)
  int64_t R;            // tcap / 8
  int32_t nq, n_seqs, max_regions, ws_stride, topk;
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

// Exclusive prefix sum over a block of NT threads.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i)
    if (i < w) base += wsum[i];
  __syncthreads();
  return base + x - v;
}

// Given hist[0..nb) of the elements still in play, finds digit d (scanning
// from the top) with above(d) < need <= above(d) + hist[d]; returns d and
// sets *above_out.  Every thread of the block gets the result.
template <int NT>
__device__ __forceinline__ int find_digit(const uint32_t* hist, int nb, uint32_t need, uint32_t* above_out,
                                          uint32_t* wsum, int* sh_d, uint32_t* sh_above) {
  const int per = (nb + NT - 1) / NT;
  const int hi_bin = nb - 1 - per * (int)threadIdx.x;  // this thread's bins, counted from the top
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) {
    const int bin = hi_bin - i;
    if (bin >= 0) local += hist[bin];
  }
  uint32_t run = block_excl_scan<NT>(local, wsum);
  for (int i = 0; i < per; ++i) {
    const int bin = hi_bin - i;
    if (bin < 0) break;
    const uint32_t h = hist[bin];
    if (run < need && run + h >= need) {
      *sh_d = bin;
      *sh_above = run;
    }
    run += h;
  }
  __syncthreads();
  *above_out = *sh_above;
  const int d = *sh_d;
  __syncthreads();
  return d;
}

// Wave-aggregated append: one atomic per wave; returns this lane's slot when
// pred holds.  Must be reached by every active lane of the wave.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __ballot(pred);
  const int lane = threadIdx.x & 63;
  uint32_t base = 0;
  if (mask) {
    const int leader = __ffsll((long long)mask) - 1;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = __shfl(base, leader);
  }
  return base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

#ifndef DSA_SCORE_DEC_RANGE
#define DSA_SCORE_DEC_RANGE 512
#endif
#ifndef DSA_SCORE_DEC_DEPTH
#define DSA_SCORE_DEC_DEPTH 4
#endif
constexpr int kDecRange = DSA_SCORE_DEC_RANGE;  // regions per decode-score block
constexpr int kDecDepth = DSA_SCORE_DEC_DEPTH;  // tiles in flight per wave

// Decode scoring: one query per block, one (query, group) region range.
// Each wave streams a contiguous run of 16-region tiles with kDecDepth tiles
// of summary loads in flight; A holds the query's 4 heads of group g in rows
// 0..3.  Lanes 0..15 turn MFMA rows 0..3 into the region's score, store it
// and count its level-0 key digit in the block's LDS histogram, which is
// flushed to the (query, group) histogram with integer atomics.
__global__ __launch_bounds__(256) void k_score_dec(ScoreArgs a) {
  const int g = blockIdx.y;
  const int qi = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kb = lane >> 4;
  __shared__ uint32_t hist_lds[kHistBins];
  for (int i = threadIdx.x; i < kHistBins; i += 256) hist_lds[i] = 0;

  int32_t seq = a.qseq[qi];
  seq = seq < 0 ? 0 : (seq >= a.n_seqs ? a.n_seqs - 1 : seq);
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  bf16x8 A[8];
  {
    const uint16_t* qp = a.iq + ((int64_t)qi * kIdxHeads + 4 * g + (n & 3)) * kProxy + 16 * kb;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = {0, 0, 0, 0};
      if (n < 4) v = ld16(qp + 64 * (s >> 1) + 8 * (s & 1));
      A[s] = as_bf16x8(v);
    }
  }
  const f32x4 zz = *(const f32x4*)(a.z + (int64_t)qi * kIdxHeads + 4 * g);
  __syncthreads();

  // this wave's tiles: contiguous quarter of the block's range
  constexpr int kWaveRegions = kDecRange / 4;
  const int64_t w0 = (int64_t)blockIdx.x * kDecRange + (int64_t)wave * kWaveRegions;
  int64_t w1 = w0 + kWaveRegions;
  if (w1 > c) w1 = c;
  const int ntile = w0 < w1 ? (int)((w1 - w0 + kTile - 1) / kTile) : 0;
  const uint8_t* sbase = a.summ + ((int64_t)seq * kGroups + g) * a.R * kProxy;
  const float* scbase = a.scale + ((int64_t)seq * kGroups + g) * a.R;
  const int64_t pq = (int64_t)qi * kGroups + g;
  float* scores = a.scores + pq * a.ws_stride;
  float* scores_out = a.scores_out ? a.scores_out + pq * a.max_regions : nullptr;

  u32x4 buf[kDecDepth][4];
  float bsc[kDecDepth];
  auto issue = [&](int t, int slot) {
    const int64_t r = w0 + (int64_t)t * kTile + n;
    const int64_t rl = r < a.R ? r : a.R - 1;
    const uint8_t* rp = sbase + summ_tile_base(rl) + 16 * lane;
    buf[slot][0] = ldg16(rp);
    buf[slot][1] = ldg16(rp + 1024);
    buf[slot][2] = ldg16(rp + 2048);
    buf[slot][3] = ldg16(rp + 3072);
    bsc[slot] = scbase[rl];
  };
#pragma unroll
  for (int t = 0; t < kDecDepth - 1; ++t)
    if (t < ntile) issue(t, t);
  for (int t0 = 0; t0 < ntile; t0 += kDecDepth) {
#pragma unroll
    for (int u = 0; u < kDecDepth; ++u) {
      const int t = t0 + u;
      if (t >= ntile) break;
      const int nxt = t + kDecDepth - 1;
      if (nxt < ntile) issue(nxt, (u + kDecDepth - 1) % kDecDepth);
      bf16x8 B[8];
      codes_to_bf16(buf[u][0], B[0], B[1]);
      codes_to_bf16(buf[u][1], B[2], B[3]);
      codes_to_bf16(buf[u][2], B[4], B[5]);
      codes_to_bf16(buf[u][3], B[6], B[7]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc = mfma16x16x32(A[s], B[s], acc);
      const int64_t r = w0 + (int64_t)t * kTile + n;
      if (kb == 0 && r < w1) {
        float sv = zz[0] * fmaxf(acc[0], 0.0f);
        sv = fmaf(zz[1], fmaxf(acc[1], 0.0f), sv);
        sv = fmaf(zz[2], fmaxf(acc[2], 0.0f), sv);
        sv = fmaf(zz[3], fmaxf(acc[3], 0.0f), sv);
        sv *= bsc[u];
        scores[r] = sv;
        if (scores_out) scores_out[r] = sv;
        atomicAdd(&hist_lds[score_key(sv) >> 20], 1u);
      }
    }
  }
  __syncthreads();
  // blocks are dealt round-robin to the XCDs; striping the flush by block
  // index keeps same-address atomics from all blocks off one counter
  uint32_t* gh = a.hist + (pq * kHistCopies + (blockIdx.x % kHistCopies)) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t v = hist_lds[i];
    if (v) atomicAdd(gh + i, v);
  }
}

// Prefill scoring: 16 queries per wave as four MFMA row-sets (4 queries x
// 4 heads each), so every summary tile loaded feeds 4 MFMAs per k-step.
// Block = 4 waves sharing (region range of kScoreRange, group, 16-query
// block); wave w takes tiles w, w+4, ...  Queries of one block that belong
// to different sequences are handled one sequence at a time.
__global__ __launch_bounds__(256) void k_score_pre(ScoreArgs a) {
  constexpr int QW = 16, NRS = 4;
  const int g = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kb = lane >> 4;
  const int q0 = blockIdx.z * QW;
  const int64_t range0 = (int64_t)blockIdx.x * kScoreRange;

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
        const int64_t cj = current_region(a.qpos[q0 + j], a.R, a.max_regions);
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
      const int jrow = 4 * rs + (n >> 2);  // query of A row n
      const bool rvalid = (active >> jrow & 1u);
      const int hh = 4 * g + (n & 3);
      const uint16_t* qp = a.iq + ((int64_t)(q0 + jrow) * kIdxHeads + hh) * kProxy + 16 * kb;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 v = {0, 0, 0, 0};
        if (rvalid) v = ld16(qp + 64 * (s >> 1) + 8 * (s & 1));
        A[rs][s] = as_bf16x8(v);
      }
      // output rows 4kb..4kb+3 of row-set rs belong to query jout
      const int jout = 4 * rs + kb;
      const bool ovalid = (active >> jout & 1u);
      qidx[rs] = ovalid ? q0 + jout : -1;
      if (ovalid) {
        const f32x4 zz = *(const f32x4*)(a.z + (int64_t)(q0 + jout) * kIdxHeads + 4 * g);
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
    for (int64_t t0 = range0 + (int64_t)wave * kTile; t0 < rend; t0 += 4 * kTile) {
      const int64_t r = t0 + n;
      const int64_t rl = r < a.R ? r : a.R - 1;
      const uint8_t* rp = sbase + summ_tile_base(rl) + 16 * lane;
      u32x4 c0 = ldg16(rp), c1 = ldg16(rp + 1024), c2 = ldg16(rp + 2048), c3 = ldg16(rp + 3072);
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
          float sv = zq[rs][0] * fmaxf(acc[0], 0.0f);
          sv = fmaf(zq[rs][1], fmaxf(acc[1], 0.0f), sv);
          sv = fmaf(zq[rs][2], fmaxf(acc[2], 0.0f), sv);
          sv = fmaf(zq[rs][3], fmaxf(acc[3], 0.0f), sv);
          sv *= sc;
          const int64_t pq = (int64_t)qidx[rs] * kGroups + g;
          a.scores[pq * a.ws_stride + r] = sv;
          if (a.scores_out) a.scores_out[pq * a.max_regions + r] = sv;
        }
      }
    }
  }
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------

struct SelectArgs {
  const float* scores;  // [Nq][G][ws_stride]
  const uint32_t* hist; // [Nq][G][8][4096] level-0 histogram stripes, or nullptr (computed in k_select)
  uint32_t* bcnt;       // [Nq][G][nblk] candidates found by each collect block (decode)
  uint64_t* cand;       // [Nq][G][nblk][kCollectChunk] candidate keys (decode), or nullptr
  uint32_t* thr;        // [Nq][G][4] level-0 threshold: digit, count above, count in digit (decode)
  int32_t nblk;         // collect blocks per (query, group)
  const int32_t* qpos;
  int32_t* sel;         // [Nq][G][topk]
  int32_t* nsel;        // [Nq][G]
  int64_t R;
  int32_t nq, max_regions, ws_stride, topk;
};

__device__ __forceinline__ uint64_t cand_key(const float* sc, int64_t r) {
  return ((uint64_t)score_key(sc[r]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)r);
}

constexpr int kCollectThreads = 256;
constexpr int kCollectPer = 8;  // consecutive scores per thread
constexpr int kCollectChunk = kCollectThreads * kCollectPer;

// Decode, step 1: one block per (query, group) sums the histogram stripes
// built by k_score_dec and finds the threshold digit (the digit holding the
// k-th key), publishing (digit, keys above it, keys in it).
constexpr int kThreshThreads = 1024;
__global__ __launch_bounds__(kThreshThreads) void k_select_thresh(SelectArgs a) {
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[kThreshThreads / 64];
  __shared__ int sh_d;
  __shared__ uint32_t sh_above;
  if (threadIdx.x == 0) {
    sh_d = 0;
    sh_above = 0;
  }
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const int64_t need = (c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1);
  if (need == c || need == 0) return;
  const uint32_t* gh = a.hist + pq * kHistCopies * kHistBins;
  constexpr int kPer = kHistBins / kThreshThreads;
  uint32_t v[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) v[e] = 0;
#pragma unroll
  for (int k = 0; k < kHistCopies; ++k)
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] += gh[k * kHistBins + e * kThreshThreads + threadIdx.x];
#pragma unroll
  for (int e = 0; e < kPer; ++e) hist[e * kThreshThreads + threadIdx.x] = v[e];
  __syncthreads();
  uint32_t above;
  const int d = find_digit<kThreshThreads>(hist, kHistBins, (uint32_t)need, &above, wsum, &sh_d, &sh_above);
  if (threadIdx.x == 0) {
    a.thr[pq * 4 + 0] = (uint32_t)d;
    a.thr[pq * 4 + 1] = above;
    a.thr[pq * 4 + 2] = hist[d];
  }
}

// Decode, step 2: block j of (query, group) scans scores [2048j, 2048j+2048)
// and keeps every key whose level-0 digit is at or above the threshold digit.
// The kept keys are compacted in index order (block-wide scan, no atomics)
// into the block's slice of the candidate buffer, with their count, so the
// concatenation over blocks is in ascending region order.  Blocks write
// count 0 when the problem needs no list or the list would not fit.
__global__ __launch_bounds__(kCollectThreads) void k_select_collect(SelectArgs a) {
  const int64_t pq = (int64_t)blockIdx.z * kGroups + blockIdx.y;
  const int qi = blockIdx.z;
  const int blk = blockIdx.x;
  __shared__ uint32_t wsum[kCollectThreads / 64];
  __shared__ uint32_t total;
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const int64_t need = (c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1);
  uint32_t* bc = a.bcnt + pq * a.nblk + blk;
  const int64_t rb = (int64_t)blk * kCollectChunk;
  if (need == c || need == 0 || rb >= c || a.thr[pq * 4 + 1] + a.thr[pq * 4 + 2] > (uint32_t)kSelCap) {
    if (threadIdx.x == 0) *bc = 0;
    return;
  }
  const int d = (int)a.thr[pq * 4 + 0];
  const float* sc = a.scores + pq * a.ws_stride;
  const int64_t r0 = rb + (int64_t)threadIdx.x * kCollectPer;
  float v[kCollectPer];
  if (r0 + kCollectPer <= c) {
    const f32x4 x0 = *(const f32x4*)(sc + r0), x1 = *(const f32x4*)(sc + r0 + 4);
    v[0] = x0[0]; v[1] = x0[1]; v[2] = x0[2]; v[3] = x0[3];
    v[4] = x1[0]; v[5] = x1[1]; v[6] = x1[2]; v[7] = x1[3];
  } else {
#pragma unroll
    for (int e = 0; e < kCollectPer; ++e) v[e] = (r0 + e < c) ? sc[r0 + e] : 0.0f;
  }
  uint32_t key[kCollectPer];
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kCollectPer; ++e) {
    key[e] = score_key(v[e]);
    if (r0 + e < c && (int)(key[e] >> 20) >= d) ++mine;
  }
  const uint32_t off = block_excl_scan<kCollectThreads>(mine, wsum);
  if (threadIdx.x == kCollectThreads - 1) total = off + mine;
  uint64_t* out = a.cand + (pq * a.nblk + blk) * kCollectChunk + off;
  uint32_t j = 0;
#pragma unroll
  for (int e = 0; e < kCollectPer; ++e) {
    const int64_t r = r0 + e;
    if (r < c && (int)(key[e] >> 20) >= d)
      out[j++] = ((uint64_t)key[e] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)r);
  }
  __syncthreads();
  if (threadIdx.x == 0) *bc = total;
}

// ---------------------------------------------------------------------------
// Ordered selection on keys held in registers.  Entry e of thread t is the
// (e*NT + t)-th entry of an index-ordered candidate sequence (coalesced
// loads); absent entries carry key 0.  The need-th largest key T is found by
// bisection on its bits, with block-wide counts of keys >= a trial value
// (ballot + scalar popcount per wave).  Keys above T are all taken; keys
// equal to T are taken lowest index first; the selection is written in
// ascending index order (ranks from a per-(entry slot, wave) table and one
// block scan), followed by the forced current region c.
// ---------------------------------------------------------------------------

// Sum over the block of per-wave totals (each wave passes the same value in
// every lane); `slot` alternates so one barrier per call suffices.
template <int NT>
__device__ __forceinline__ uint32_t block_sum_waves(uint32_t wave_total, uint32_t* red, int slot) {
  if ((threadIdx.x & 63) == 0) red[slot * (NT / 64) + (threadIdx.x >> 6)] = wave_total;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[slot * (NT / 64) + i];
  return t;
}

// Number of keys >= trial held by this wave (trial is never 0).
template <int KPT>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&key)[KPT], uint32_t trial) {
  uint32_t n = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) n += (uint32_t)__popcll(__ballot(key[e] >= trial));
  return n;
}

// Exclusive scan, in place, of tab[0..n) laid out slot-major (slot, wave);
// n <= NT.
template <int NT>
__device__ __forceinline__ void scan_table(uint32_t* tab, int n, uint32_t* wsum) {
  __syncthreads();
  const uint32_t v = threadIdx.x < n ? tab[threadIdx.x] : 0u;
  const uint32_t ex = block_excl_scan<NT>(v, wsum);
  if (threadIdx.x < n) tab[threadIdx.x] = ex;
  __syncthreads();
}

// The need-th largest key by bisection over all register-held keys.
template <int NT, int KPT>
__device__ uint32_t kth_key_bisect(const uint32_t (&key)[KPT], uint32_t need, uint32_t* red) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = T | (1u << bit);
    if (block_sum_waves<NT>(wave_count_ge<KPT>(key, trial), red, bit & 1) >= need) T = trial;
  }
  return T;
}

// Writes the selection given T = the need-th largest key: keys above T, then
// keys equal to T lowest index first, in ascending index order, then c.
template <int NT, int KPT>
__device__ void emit_selection(const uint32_t (&key)[KPT], const int32_t (&idx)[KPT], uint32_t T, uint32_t need,
                               int64_t c, int32_t* sel, int32_t* nsel_out, int topk, uint32_t* red, uint32_t* tab,
                               uint32_t* wsum) {
  constexpr int NW = NT / 64;
  static_assert(KPT * NW <= NT, "rank table larger than the block");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  __syncthreads();
  const uint32_t above = (T == 0xFFFFFFFFu) ? 0u : block_sum_waves<NT>(wave_count_ge<KPT>(key, T + 1), red, 1);
  const uint32_t need_eq = need - above;  // >= 1 by the choice of T
  // ranks of keys equal to T, in index order
  uint64_t meq[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    meq[e] = __ballot(key[e] == T);
    if (lane == 0) tab[e * NW + w] = (uint32_t)__popcll(meq[e]);
  }
  scan_table<NT>(tab, KPT * NW, wsum);
  uint64_t msel[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    // absent entries (key 0) have the highest indices, so they can only rank
    // after every present key equal to T and are never taken
    const bool s = key[e] > T || (key[e] == T && tab[e * NW + w] + (uint32_t)__popcll(meq[e] & lt) < need_eq);
    msel[e] = __ballot(s);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if (lane == 0) tab[e * NW + w] = (uint32_t)__popcll(msel[e]);
  scan_table<NT>(tab, KPT * NW, wsum);
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if ((msel[e] >> lane) & 1ull) sel[tab[e * NW + w] + (uint32_t)__popcll(msel[e] & lt)] = idx[e];
  for (int i = (int)need + 1 + threadIdx.x; i < topk; i += NT) sel[i] = -1;
  if (threadIdx.x == 0) {
    sel[need] = (int32_t)c;
    *nsel_out = (int32_t)need + 1;
  }
}

template <int NT, int KPT>
__device__ void select_strided(const uint32_t (&key)[KPT], const int32_t (&idx)[KPT], uint32_t need, int64_t c,
                               int32_t* sel, int32_t* nsel_out, int topk, uint32_t* red, uint32_t* tab,
                               uint32_t* wsum) {
  const uint32_t T = kth_key_bisect<NT, KPT>(key, need, red);
  emit_selection<NT, KPT>(key, idx, T, need, c, sel, nsel_out, topk, red, tab, wsum);
}

// Trivial cases shared by the selection kernels.  Returns true when handled.
__device__ __forceinline__ bool select_trivial(int64_t c, uint32_t need, int32_t* sel, int32_t* nsel, int topk,
                                               int nt) {
  if ((int64_t)need == c) {  // every candidate fits: regions 0..c
    for (int i = threadIdx.x; i < topk; i += nt) sel[i] = (i <= c) ? i : -1;
    if (threadIdx.x == 0) *nsel = (int32_t)(c + 1);
    return true;
  }
  if (need == 0) {  // topk == 1: only the current region
    for (int i = threadIdx.x; i < topk; i += nt) sel[i] = (i == 0) ? (int32_t)c : -1;
    if (threadIdx.x == 0) *nsel = 1;
    return true;
  }
  return false;
}

#ifndef DSA_PRE_SELECT_NT
#define DSA_PRE_SELECT_NT 256
#endif
constexpr int kPreNT = DSA_PRE_SELECT_NT;  // threads of the prefill selection block (<= 8192 regions)

// Prefill: one block per (query, group); the problem's scores (c <= NT*KPT)
// are loaded straight into registers in index order.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void k_select_pre(SelectArgs a) {
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  __shared__ uint32_t red[2 * (NT / 64)];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t tab[KPT * (NT / 64)];
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const uint32_t need = (uint32_t)((c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1));
  int32_t* sel = a.sel + pq * a.topk;
  if (select_trivial(c, need, sel, a.nsel + pq, a.topk, NT)) return;
  const float* sc = a.scores + pq * a.ws_stride;
  uint32_t key[KPT];
  int32_t idx[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int64_t r = (int64_t)e * NT + threadIdx.x;
    key[e] = r < c ? score_key(sc[r]) : 0u;
    idx[e] = (int32_t)r;
  }
  select_strided<NT, KPT>(key, idx, need, c, sel, a.nsel + pq, a.topk, red, tab, wsum);
}

// Decode fallback and very long prefill contexts: exact selection by radix
// narrowing over the scores in global memory (12-bit digits) until the
// candidates fit in LDS, 8-bit digits in LDS, bitonic sort of the result.
template <int NT>
__device__ void select_fallback(const SelectArgs& a, int64_t pq) {
  const int qi = (int)(pq / kGroups);
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint64_t list[kSelCap];
  __shared__ int32_t outl[kMaxTopk];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ int sh_d;
  __shared__ uint32_t sh_above, sh_count;

  if (tid == 0) {
    sh_d = 0;
    sh_above = 0;
    sh_count = 0;
  }
  __syncthreads();
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const int64_t need64 = (c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1);
  const uint32_t need = (uint32_t)need64;
  int32_t* sel = a.sel + pq * a.topk;
  const float* sc = a.scores + pq * a.ws_stride;

  if (need64 == c) {  // every candidate fits: regions 0..c
    for (int i = tid; i < a.topk; i += NT) sel[i] = (i <= c) ? i : -1;
    if (tid == 0) a.nsel[pq] = (int32_t)(c + 1);
    return;
  }
  if (need == 0) {  // topk == 1: only the current region
    for (int i = tid; i < a.topk; i += NT) sel[i] = (i == 0) ? (int32_t)c : -1;
    if (tid == 0) a.nsel[pq] = 1;
    return;
  }

  // ---- level 0: 12-bit digit of the score key (bits 63..52 of the 64-bit key),
  // published by k_select_thresh for decode, found here for prefill
  uint32_t above, inbin;
  int d;
  if (a.thr) {
    d = (int)a.thr[pq * 4 + 0];
    above = a.thr[pq * 4 + 1];
    inbin = a.thr[pq * 4 + 2];
  } else {
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0;
    __syncthreads();
    for (int64_t r = tid; r < c; r += NT) atomicAdd(&hist[score_key(sc[r]) >> 20], 1u);
    __syncthreads();
    d = find_digit<NT>(hist, kHistBins, need, &above, wsum, &sh_d, &sh_above);
    inbin = hist[d];
  }
  uint64_t prefix = (uint64_t)d;
  int shift = 52;
  __syncthreads();
  // ---- narrow over global memory until the candidates fit in LDS
  while (above + inbin > (uint32_t)kSelCap && shift > 0) {
    const int width = shift >= 12 ? 12 : shift;
    const int nshift = shift - width;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += NT) hist[i] = 0;
    __syncthreads();
    for (int64_t r = tid; r < c; r += NT) {
      const uint64_t k = cand_key(sc, r);
      if ((k >> shift) == prefix) atomicAdd(&hist[(uint32_t)(k >> nshift) & (nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t ab;
    d = find_digit<NT>(hist, nb, need - above, &ab, wsum, &sh_d, &sh_above);
    above += ab;
    inbin = hist[d];
    prefix = (prefix << width) | (uint64_t)d;
    shift = nshift;
    __syncthreads();
  }
  // ---- collect everything at or above the current bin into LDS
  for (int64_t base = 0; base < c; base += NT) {
    const int64_t r = base + tid;
    uint64_t k = 0;
    bool take = false;
    if (r < c) {
      k = cand_key(sc, r);
      take = (k >> shift) >= prefix;
    }
    const uint32_t pos = wave_append(take, &sh_count);
    if (take && pos < (uint32_t)kSelCap) list[pos] = k;
  }
  __syncthreads();
  const uint32_t M = sh_count < (uint32_t)kSelCap ? sh_count : (uint32_t)kSelCap;
  uint32_t need_in = need - above;

  // ---- finish in LDS with 8-bit digits
  while (shift > 0 && inbin != need_in) {
    const int width = shift >= 8 ? 8 : shift;
    const int nshift = shift - width;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += NT) hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < M; i += NT) {
      const uint64_t k = list[i];
      if ((k >> shift) == prefix) atomicAdd(&hist[(uint32_t)(k >> nshift) & (nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t ab;
    d = find_digit<NT>(hist, nb, need_in, &ab, wsum, &sh_d, &sh_above);
    need_in -= ab;
    inbin = hist[d];
    prefix = (prefix << width) | (uint64_t)d;
    shift = nshift;
    __syncthreads();
  }

  // ---- selected = list entries with (key >> shift) >= prefix (exactly need)
  if (tid == 0) sh_count = 0;
  __syncthreads();
  for (uint32_t base = 0; base < M; base += NT) {
    const uint32_t i = base + tid;
    uint64_t k = 0;
    bool take = false;
    if (i < M) {
      k = list[i];
      take = (k >> shift) >= prefix;
    }
    const uint32_t pos = wave_append(take, &sh_count);
    if (take && pos < (uint32_t)kMaxTopk - 1) outl[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
  }
  __syncthreads();
  const uint32_t nsel = need + 1;
  for (int i = tid; i < kMaxTopk; i += NT) {
    if ((uint32_t)i == need) outl[i] = (int32_t)c;
    else if ((uint32_t)i > need) outl[i] = 0x7FFFFFFF;
  }
  __syncthreads();
  // bitonic sort of 512 ascending; sorted prefix [0, nsel) is the selection
  for (int size = 2; size <= kMaxTopk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < kMaxTopk / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const int32_t x = outl[lo], y = outl[hi];
        if ((x > y) == up) {
          outl[lo] = y;
          outl[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < a.topk; i += NT) sel[i] = ((uint32_t)i < nsel) ? outl[i] : -1;
  if (tid == 0) a.nsel[pq] = (int32_t)nsel;
}


// Prefill with more than 32768 candidate regions per query.
__global__ __launch_bounds__(512) void k_select_long(SelectArgs a) {
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const uint32_t need = (uint32_t)((c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1));
  if (select_trivial(c, need, a.sel + pq * a.topk, a.nsel + pq, a.topk, 512)) return;
  select_fallback<512>(a, pq);
}

// Decode, step 3: one block per (query, group).  The collected list (index
// order, at most kSelCap keys) is loaded into registers and finished with the
// ordered selection; problems whose list would not fit use the fallback.
constexpr int kFinalThreads = 512;
constexpr int kFinalKpt = kSelCap / kFinalThreads;  // 8
__global__ __launch_bounds__(kFinalThreads) void k_select_dec(SelectArgs a) {
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  __shared__ uint32_t red[2 * (kFinalThreads / 64)];
  __shared__ uint32_t wsum[kFinalThreads / 64];
  __shared__ uint32_t offs[kMaxTopk + 1];
  __shared__ uint32_t tab[kFinalKpt * (kFinalThreads / 64)];
  __shared__ uint32_t sh_total;
  const int64_t c = current_region(a.qpos[qi], a.R, a.max_regions);
  const uint32_t need = (uint32_t)((c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1));
  int32_t* sel = a.sel + pq * a.topk;
  if (select_trivial(c, need, sel, a.nsel + pq, a.topk, kFinalThreads)) return;
  const bool fits = a.nblk <= kMaxTopk && a.thr[pq * 4 + 1] + a.thr[pq * 4 + 2] <= (uint32_t)kSelCap;
  if (!fits) {
    select_fallback<kFinalThreads>(a, pq);
    return;
  }
  // offsets of the blocks' lists (rounds of kFinalThreads blocks)
  uint32_t base = 0;
  for (int j0 = 0; j0 < a.nblk; j0 += kFinalThreads) {
    const int j = j0 + threadIdx.x;
    const uint32_t cj = j < a.nblk ? a.bcnt[pq * a.nblk + j] : 0u;
    const uint32_t ex = block_excl_scan<kFinalThreads>(cj, wsum);
    if (j < a.nblk) offs[j] = base + ex;
    if (threadIdx.x == kFinalThreads - 1) sh_total = base + ex + cj;
    __syncthreads();
    base = sh_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) offs[a.nblk] = base;
  __syncthreads();
  const uint32_t m = base < (uint32_t)kSelCap ? base : (uint32_t)kSelCap;
  uint32_t key[kFinalKpt];
  int32_t idx[kFinalKpt];
#pragma unroll
  for (int e = 0; e < kFinalKpt; ++e) {
    const uint32_t i = (uint32_t)e * kFinalThreads + threadIdx.x;
    key[e] = 0;
    idx[e] = 0;
    if (i < m) {
      int lo = 0, hi = a.nblk - 1;  // collect block holding entry i: last j with offs[j] <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const uint64_t k = a.cand[(pq * a.nblk + lo) * kCollectChunk + (i - offs[lo])];
      key[e] = (uint32_t)(k >> 32);
      idx[e] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
    }
  }
  select_strided<kFinalThreads, kFinalKpt>(key, idx, need, c, sel, a.nsel + pq, a.topk, red, tab, wsum);
}

static int64_t ws_stride_of(int32_t max_regions) { return ((int64_t)max_regions + 63) / 64 * 64; }
static bool decode_shaped(int32_t n_queries) { return n_queries < 64; }

struct ScoreWs {
  uint32_t* hist;
  uint32_t* thr;
  uint32_t* bcnt;
  uint64_t* cand;
  float* scores;
  size_t bytes;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int32_t collect_blocks(int32_t max_regions) { return (max_regions + kCollectChunk - 1) / kCollectChunk; }

static ScoreWs score_ws_layout(void* base, int32_t nq, int32_t max_regions) {
  ScoreWs w;
  char* p = (char*)base;
  const size_t np = (size_t)nq * kGroups;
  const bool dec = decode_shaped(nq);
  const size_t nblk = (size_t)collect_blocks(max_regions);
  size_t off = 0;
  w.hist = (uint32_t*)(p + off);
  off += align256(np * (dec ? kHistCopies : 1) * kHistBins * 4);
  w.thr = (uint32_t*)(p + off);
  off += align256(np * 4 * 4);
  w.bcnt = (uint32_t*)(p + off);
  off += align256(np * nblk * 4);
  w.cand = dec ? (uint64_t*)(p + off) : nullptr;
  if (dec) off += align256(np * nblk * kCollectChunk * 8);
  w.scores = (float*)(p + off);
  off += align256(np * (size_t)ws_stride_of(max_regions) * 4);
  w.bytes = off;
  return w;
}

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_score_topk_workspace_size(const dsa_geometry* geom, int32_t n_queries,
                                                int32_t max_regions) {
  (void)geom;
  if (n_queries <= 0 || max_regions <= 0) return 256;
  return score_ws_layout(nullptr, n_queries, max_regions).bytes;
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
  if (n_queries < 0 || n_seqs < 0 || max_regions < 0 || tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: bad sizes (tcap must be a positive multiple of 128)");
  if (n_queries == 0) return DSA_OK;
  if (n_seqs == 0 || max_regions == 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: n_seqs and max_regions must be positive");
  if (!index_q || !z || !q_seq || !q_pos || !summ || !scale || !sel || !n_sel || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: NULL pointer");
  if ((size_t)workspace & 255)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: workspace must be 256-byte aligned");
  if (workspace_bytes < dsa_score_topk_workspace_size(geom, n_queries, max_regions))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_score_topk: workspace too small");
  if (n_queries > 65535 * 16) return fail(DSA_ERR_UNSUPPORTED, "dsa_score_topk: too many queries");
  hipStream_t s = as_stream(stream);
  const ScoreWs w = score_ws_layout(workspace, n_queries, max_regions);
  const int32_t stride = (int32_t)ws_stride_of(max_regions);

  ScoreArgs sa;
  sa.iq = index_q; sa.z = z; sa.qseq = q_seq; sa.qpos = q_pos; sa.summ = summ; sa.scale = scale;
  sa.scores = w.scores; sa.scores_out = scores_out; sa.hist = w.hist;
  sa.R = tcap / kRegion; sa.nq = n_queries; sa.n_seqs = n_seqs; sa.max_regions = max_regions;
  sa.ws_stride = stride; sa.topk = geom->topk;
  const int ranges = (max_regions + kScoreRange - 1) / kScoreRange;
  // Decode-shaped calls (few queries, many regions) score one query per wave,
  // build the level-0 histogram on the fly and collect candidates with many
  // blocks; prefill-shaped calls score 16 queries per wave so each summary
  // tile feeds 4 MFMA row-sets, and select with one block per problem.
  const bool dec = decode_shaped(n_queries);
  SelectArgs se;
  se.scores = w.scores; se.hist = dec ? w.hist : nullptr; se.bcnt = w.bcnt; se.cand = w.cand;
  se.thr = dec ? w.thr : nullptr;
  se.nblk = collect_blocks(max_regions); se.qpos = q_pos;
  se.sel = sel; se.nsel = n_sel; se.R = tcap / kRegion; se.nq = n_queries; se.max_regions = max_regions;
  se.ws_stride = stride; se.topk = geom->topk;
  if (dec) {
    const int64_t fill_n = (int64_t)n_queries * kGroups * kHistCopies * kHistBins;
    int64_t fill_blocks = (fill_n + 255) / 256;
    if (fill_blocks > 4096) fill_blocks = 4096;
    {
      ProfScope prof_("k_fill_u32", s);
      hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)fill_blocks), dim3(256), 0, s, w.hist, fill_n, 0u);
    }
    {
      ProfScope prof_("k_score_decode", s);
      hipLaunchKernelGGL(k_score_dec, dim3((max_regions + kDecRange - 1) / kDecRange, kGroups, n_queries),
                         dim3(256), 0, s, sa);
    }
    st = check_launch("dsa_score_topk: score");
    if (st != DSA_OK) return st;
    {
      ProfScope prof_("k_select_thresh", s);
      hipLaunchKernelGGL(k_select_thresh, dim3((unsigned)((int64_t)n_queries * kGroups)), dim3(kThreshThreads), 0,
                         s, se);
    }
    {
      ProfScope prof_("k_select_collect", s);
      hipLaunchKernelGGL(k_select_collect, dim3(se.nblk, kGroups, n_queries), dim3(kCollectThreads), 0, s, se);
    }
    st = check_launch("dsa_score_topk: collect");
    if (st != DSA_OK) return st;
    {
      ProfScope prof_("k_select", s);
      hipLaunchKernelGGL(k_select_dec, dim3((unsigned)((int64_t)n_queries * kGroups)), dim3(kFinalThreads), 0,
                         s, se);
    }
  } else {
    {
      ProfScope prof_("k_score_prefill", s);
      hipLaunchKernelGGL(k_score_pre, dim3(ranges, kGroups, (n_queries + 15) / 16), dim3(256), 0, s, sa);
    }
    st = check_launch("dsa_score_topk: score");
    if (st != DSA_OK) return st;
    {
      ProfScope prof_("k_select", s);
      const dim3 grid((unsigned)((int64_t)n_queries * kGroups));
      if (max_regions <= kPreNT * (8192 / kPreNT))
        hipLaunchKernelGGL((k_select_pre<kPreNT, 8192 / kPreNT>), grid, dim3(kPreNT), 0, s, se);
      else if (max_regions <= 1024 * 32)
        hipLaunchKernelGGL((k_select_pre<1024, 32>), grid, dim3(1024), 0, s, se);
      else
        hipLaunchKernelGGL(k_select_long, grid, dim3(512), 0, s, se);
    }
  }
  return check_launch("dsa_score_topk: select");
}
