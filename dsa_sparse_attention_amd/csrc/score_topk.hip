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
//  * Scoring streams the summaries once, coalesced, with the dot products on
//    the matrix cores: B = 16 regions x 32 channels of E4M3 codes turned into
//    bf16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1), A = query heads of
//    the group.  The channel order inside one 256-d dot is permuted so that
//    each lane reads 64 contiguous bytes of one region; A uses the same
//    permutation.  k_score_dec (few queries, long contexts) gives each block
//    one (query, group) and a run of regions, the 4 heads in MFMA rows 0..3;
//    k_score_pre (prefill chunks) gives each wave 16 queries as four row-sets
//    that share every summary tile, which the block streams through an LDS
//    ring.  Both can store, per 16-region tile, the largest order-preserving
//    score key of the tile.
//  * Selection ranks regions by (score desc, region asc) with 32-bit keys.
//    Problems of up to 8192 candidates keep their keys in registers
//    (k_select_pre): a histogram on a linear score scale finds the bin of
//    the need-th key, whose few keys are ranked exactly.  Longer problems go
//    through the tile maxima: the need-th largest tile maximum bounds the
//    need-th score from below, so only tiles reaching that bound can hold a
//    selected region.  Decode-shaped problems (k_select_dec) take a digit of
//    the tile maxima as the bound and finish with a wave-level radix on the
//    candidates' keys; prefill-shaped ones (k_select_tiles) take the need
//    best tiles and rank their regions.  A radix fallback in global memory
//    covers problems beyond the register capacity.
#include <mutex>

#include "compress_dev.hpp"

namespace dsa {

constexpr int kScoreRange = 1024;  // regions per k_score block
constexpr int kPreQ = 64;          // queries per prefill scoring block (16 per wave)
constexpr int kPreSlot = 4096 + 4 * 256;  // one summary tile in the block's LDS ring: 4 KB of codes,
                                          // then one scale copy per wave (lanes 0..15 hold the scales)
#ifndef DSA_PRE_WAVES
#define DSA_PRE_WAVES 2
#endif
constexpr int kTile = 16;          // regions per MFMA tile
constexpr int kHistBins = 4096;    // level-0 digit: key bits 31..20
constexpr int kSelCap = 4096;      // LDS candidate capacity of the radix fallback
constexpr int kCandCap = 2048;     // decode candidates at or above the level-0 digit
constexpr int kDirectMax = 8192;   // longest problem selected straight from its scores

struct ScoreArgs {
  const uint16_t* iq;   // [Nq][16][P]
  const float* z;       // [Nq][16]
  const int32_t* qseq;  // [Nq], or nullptr: query i belongs to sequence i
  const int32_t* qpos;  // [Nq], or nullptr: position slen[i] - 1
  const int32_t* slen;  // [Nq] sequence lengths when qpos is nullptr
  const uint8_t* summ;  // summary tiles, found through cm
  const float* scale;   // scales, found through cm
  float* scores;        // workspace [Nq][G][ws_stride]
  float* scores_out;    // nullable [Nq][G][max_regions]
  uint32_t* tilemax;    // nullable workspace [Nq][G][tm_stride]: largest key of each 16-region tile
  CacheMap cm;          // where the sequences' summaries live (cm.R regions each)
  int32_t nq, n_seqs, max_regions, ws_stride, tm_stride, topk;
};

// Order-preserving key of a score; NaN maps to 0 and ranks below every number.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Current region c of a query (clamped so every index stays in bounds).  Its
// candidates are regions 0..c-1, so c = max_regions still fits every array
// sized by max_regions (scores, tile maxima, the scoring grid); a decode query
// in a partial region c = seq_len/8 is thus covered by max_regions = seq_len/8.
__device__ __forceinline__ int64_t current_region(int32_t pos, int64_t R, int32_t max_regions) {
  int64_t c = pos < 0 ? 0 : (int64_t)pos / kRegion;
  if (c > R - 1) c = R - 1;
  if (c > max_regions) c = max_regions;
  return c;
}

// Position and sequence of query i: explicit arrays, or (decode step) query
// i is the last token of sequence i.
__device__ __forceinline__ int32_t query_pos(const int32_t* qpos, const int32_t* slen, int64_t i) {
  return qpos ? qpos[i] : slen[i] - 1;
}
__device__ __forceinline__ int32_t query_seq(const int32_t* qseq, int64_t i) {
  return qseq ? qseq[i] : (int32_t)i;
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

// max(x, 0) in one instruction: the median of (x, 0, FLT_MAX), equal to it
// for every x but +inf.  fmaxf(x, 0) costs two (the compiler first quiets a
// possible signalling NaN), and so does a median with +inf, which it turns
// back into fmaxf.  (Not inline asm: the compiler inserts no wait states
// before an asm block that reads an MFMA result, which can then read the
// register before the MFMA has written it.)
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e38f); }

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
#define DSA_SCORE_DEC_RANGE 384
#endif
#ifndef DSA_SCORE_DEC_DEPTH
#define DSA_SCORE_DEC_DEPTH 4
#endif
constexpr int kDecRange = DSA_SCORE_DEC_RANGE;  // regions per decode-score block
constexpr int kDecRangeShort = 128;               // the same for problems of <= 8192 regions
constexpr int kDecDepth = DSA_SCORE_DEC_DEPTH;  // tiles in flight per wave

// Decode scoring: one query per block, one (query, group) region range.
// Each wave streams a contiguous run of 16-region tiles with kDecDepth tiles
// of summary loads in flight; A holds the query's 4 heads of group g in rows
// 0..3.  Lanes 0..15 turn MFMA rows 0..3 into the region's score and store
// it; the tile's largest key is reduced over those 16 lanes and stored too.
template <bool PAGED, int RANGE>
__global__ __launch_bounds__(256) void k_score_dec(ScoreArgs a) {
  const int g = blockIdx.y;
  const int qi = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kb = lane >> 4;

  constexpr int kWaveRegions = RANGE / 4;
  const int64_t w0 = (int64_t)blockIdx.x * RANGE + (int64_t)wave * kWaveRegions;
  int32_t seq = query_seq(a.qseq, qi);
  seq = seq < 0 ? 0 : (seq >= a.n_seqs ? a.n_seqs - 1 : seq);
  const int64_t c = current_region(query_pos(a.qpos, a.slen, qi), a.cm.R, a.max_regions);
  // paged caches: lane l holds the page id of the wave's tile l (clamped when
  // used)
  const int64_t ntile_all = a.cm.R / kTile;
  int32_t pgv = 0;
  if constexpr (PAGED) {
    const int64_t tl = (w0 >> 4) + lane;
    pgv = a.cm.bt[(int64_t)seq * a.cm.bt_stride + (tl < ntile_all ? tl : ntile_all - 1)];
  }
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

  u32x4 buf[kDecDepth][4];
  float bsc[kDecDepth];
  static_assert(RANGE / 4 / kTile <= 64 && RANGE % (4 * kTile) == 0, "a lane per tile of the wave");
  auto issue = [&](int t, int slot) {
    int64_t tt = (w0 >> 4) + t;  // tile index (uniform)
    tt = tt < ntile_all ? tt : ntile_all - 1;
    const int64_t ts = PAGED ? ((int64_t)clamp_page(a.cm, __builtin_amdgcn_readlane(pgv, t)) * kGroups + g)
                             : ((int64_t)seq * kGroups + g) * ntile_all + tt;  // tile slot
    const uint8_t* rp = a.summ + ts * 4096 + 16 * lane;
    buf[slot][0] = ldg16(rp);
    buf[slot][1] = ldg16(rp + 1024);
    buf[slot][2] = ldg16(rp + 2048);
    buf[slot][3] = ldg16(rp + 3072);
    bsc[slot] = a.scale[ts * kTile + n];
  };
  // The first tiles are issued before the query operand and the position
  // are waited for (their slots do not depend on them; tiles past the wave's
  // last are loaded and never used).  Paged caches wait for the page ids
  // here, once.
#pragma unroll
  for (int t = 0; t < kDecDepth - 1; ++t) issue(t, t);

  // this wave's tiles: contiguous quarter of the block's range
  int64_t w1 = w0 + kWaveRegions;
  if (w1 > c) w1 = c;
  const int ntile = w0 < w1 ? (int)((w1 - w0 + kTile - 1) / kTile) : 0;
  const int64_t pq = (int64_t)qi * kGroups + g;
  float* scores = a.scores + pq * a.ws_stride;
  float* scores_out = a.scores_out ? a.scores_out + pq * a.max_regions : nullptr;
  uint32_t* tmax = a.tilemax ? a.tilemax + pq * a.tm_stride + w0 / kTile : nullptr;
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
      uint32_t key = 0;
      if (kb == 0 && r < w1) {
        float sv = zz[0] * relu(acc[0]);
        sv = fmaf(zz[1], relu(acc[1]), sv);
        sv = fmaf(zz[2], relu(acc[2]), sv);
        sv = fmaf(zz[3], relu(acc[3]), sv);
        sv *= bsc[u];
        scores[r] = sv;
        if (scores_out) scores_out[r] = sv;
        key = score_key(sv);
      }
      if (tmax) {
        key = max(key, (uint32_t)__shfl_xor((int)key, 8));
        key = max(key, (uint32_t)__shfl_xor((int)key, 4));
        key = max(key, (uint32_t)__shfl_xor((int)key, 2));
        key = max(key, (uint32_t)__shfl_xor((int)key, 1));
        if (lane == 0) tmax[t] = key;
      }
    }
  }
}

// Prefill scoring: 16 queries per wave as four MFMA row-sets (4 queries x
// 4 heads each), so every summary tile feeds 4 MFMAs per k-step.  Block = 4
// waves = 64 queries sharing (region range of kScoreRange, group); the
// block's summary tiles stream through one LDS ring (each wave copies a
// quarter of each tile), so every tile read from L2 feeds 64 queries.
// Queries of one block that belong to different sequences are handled one
// sequence at a time.  TILEMAX also stores each tile's largest key; OUT
// also writes the caller's score array.
//
// The copies are the DMA form of the loads (global -> LDS), issued kPreDepth
// - 1 tiles ahead.  A wave learns that its own copies of tile k landed from
// its count of outstanding memory operations, which complete in order: every
// operation of the loop is issued unconditionally (stores of invalid lanes
// go to an out-of-range buffer offset and are dropped), so the number issued
// after tile k's copies is known exactly.  A barrier then makes all four
// quarters visible, and also shows that every wave is done with the slot the
// next copy overwrites.
template <bool TILEMAX, bool OUT>
struct PreScoreCfg {
  static constexpr int S = 4 * (1 + (TILEMAX ? 1 : 0) + (OUT ? 1 : 0));  // stores per tile
  static constexpr int D = S == 4 ? 8 : (S == 8 ? 6 : 4);                // ring depth
  static constexpr int W_EARLY = 2 * (D - 2);                            // wait counts
  static constexpr int W_FULL = 2 * (D - 2) + (D - 1) * S;
  static_assert(W_FULL + 2 + S <= 63, "the outstanding-operation counter holds 63");
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  // the immediate must be a literal: dispatch over the counts in use
  if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if constexpr (N == 40) asm volatile("s_waitcnt vmcnt(40)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else static_assert(N < 0, "add this count");
}

// Buffer view of rows [first row of the wave, +16 queries) of a [Nq][G][stride]
// array for group g: offsets are bytes from the wave's first row; rows past
// the last query are outside the view.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(void* base, int64_t qw, int g, int64_t stride,
                                                           int32_t nq) {
  int64_t rows = nq - qw;
  rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
  const int64_t bytes = rows ? ((rows - 1) * kGroups + 1) * stride * 4 : 0;
  char* p = (char*)base + ((qw < nq ? qw : 0) * kGroups + g) * stride * 4;
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfView = 0x80000000u;  // byte offset past every view (views stay below 2 GiB)

template <bool TILEMAX, bool OUT, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DSA_PRE_WAVES, DSA_PRE_WAVES))) void k_score_pre(ScoreArgs a) {
  using Cfg = PreScoreCfg<TILEMAX, OUT>;
  constexpr int NRS = 4, D = Cfg::D;
  constexpr bool kPipelined = !TILEMAX && !OUT && !PAGED;
  // Block -> (query block, group, region range).  Consecutive blocks go to
  // the 8 XCDs in turn, so XCD x takes the query blocks x, x + 8, ..., each
  // as all (group, range) blocks in a row: the ones resident together read
  // the same few query operands (128 KB per query block and group), which
  // then come from that XCD's L2, while the summary tiles, copied well ahead
  // of their use, stream from the Infinity Cache.
  const int nranges = (a.max_regions + kScoreRange - 1) / kScoreRange;
  const int per_qblock = nranges * kGroups;
  const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int qblk = xcd + 8 * (jb / per_qblock);
  if (qblk * kPreQ >= a.nq) return;  // (uniform) past the last query block
  const int g = (jb % per_qblock) / nranges;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: buffer views in scalars
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kb = lane >> 4;
  const int qb = qblk * kPreQ;         // the block's first query
  const int qw = qb + 16 * wave;       // the wave's first query
  const int64_t range0 = (int64_t)((jb % per_qblock) % nranges) * kScoreRange;
  __shared__ __attribute__((aligned(16))) uint8_t ring[D][kPreSlot];

  // Query metadata, one round of loads: lane l holds query qb + l (clamped
  // into range); bit l of `remaining` says whether it exists and is still
  // to process.  Every wave computes the same passes.
  const int64_t qm = (qb + lane < a.nq) ? qb + lane : a.nq - 1;
  int32_t sq = query_seq(a.qseq, qm);
  sq = sq < 0 ? 0 : (sq >= a.n_seqs ? a.n_seqs - 1 : sq);
  const int32_t cqm = (int32_t)current_region(query_pos(a.qpos, a.slen, qm), a.cm.R, a.max_regions);
  uint64_t remaining = __ballot(qb + lane < a.nq);

  const __amdgpu_buffer_rsrc_t ws_view = rows_rsrc(a.scores, qw, g, a.ws_stride, a.nq);
  const __amdgpu_buffer_rsrc_t out_view = rows_rsrc(OUT ? (void*)a.scores_out : (void*)a.scores, qw, g,
                                                    OUT ? a.max_regions : a.ws_stride, a.nq);
  const __amdgpu_buffer_rsrc_t tm_view = rows_rsrc(TILEMAX ? (void*)a.tilemax : (void*)a.scores, qw, g,
                                                   TILEMAX ? a.tm_stride : a.ws_stride, a.nq);

  while (remaining) {
    // one pass per sequence among the block's queries
    const int lead = __builtin_ctzll(remaining);
    const int32_t seq = __builtin_amdgcn_readlane(sq, lead);
    const uint64_t active = __ballot(sq == seq) & remaining;
    remaining &= ~active;
    int32_t cm = (active >> lane & 1ull) ? cqm : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cm = max(cm, __shfl_xor(cm, o));
    // uniform: the tile loop's bounds and copy addresses then live in scalars
    cm = __builtin_amdgcn_readfirstlane(cm);

    // A operand: rows = (query, head) pairs of group g; channel permutation
    // pi(s, kb, e) = 64*(s/2) + 16*kb + 8*(s%2) + e.  Rows of queries outside
    // this pass (or past the end, clamped) are loaded too and never stored.
    bf16x8 A[NRS][8];
    // epilogue data of the lane's output query in each row-set: z of the
    // group's 4 heads and the current region (-1: not in this pass)
    f32x4 zq[NRS];
    int32_t cq[NRS];
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      const int jout = 16 * wave + 4 * rs + kb;
      const int64_t qo = (qb + jout < a.nq) ? qb + jout : a.nq - 1;
      zq[rs] = *(const f32x4*)(a.z + qo * kIdxHeads + 4 * g);
      const int32_t cj = __shfl(cqm, jout);
      cq[rs] = (active >> jout & 1ull) ? cj : -1;
    }
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      const int jrow = 4 * rs + (n >> 2);  // query of A row n
      const int64_t qr = (qw + jrow < a.nq) ? qw + jrow : a.nq - 1;
      const int hh = 4 * g + (n & 3);
      const uint16_t* qp = a.iq + (qr * kIdxHeads + hh) * kProxy + 16 * kb;
#pragma unroll
      for (int s = 0; s < 8; ++s) A[rs][s] = as_bf16x8(ld16(qp + 64 * (s >> 1) + 8 * (s & 1)));
    }
    // The operand and epilogue loads are waited for here, before any copy
    // is in flight: a first use inside the tile loop would otherwise wait
    // for every copy issued ahead of it.
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) {
      asm volatile("" ::"v"(zq[rs]));
#pragma unroll
      for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, A[rs][s])));
    }

    const int64_t rend = (range0 + kScoreRange < cm) ? range0 + kScoreRange : (int64_t)cm;
    const int nk = rend > range0 ? (int)((rend - range0 + kTile - 1) / kTile) : 0;  // tiles of the block
    // page ids of the block's tiles (paged caches): lane l holds tile l's
    static_assert(kScoreRange / kTile <= 64, "a lane per tile of the block");
    const int64_t ntile_all = a.cm.R / kTile;
    int32_t pgv = 0;  // (clamped when used)
    if constexpr (PAGED) {
      const int64_t tl = (range0 >> 4) + lane;
      pgv = a.cm.bt[(int64_t)seq * a.cm.bt_stride + (tl < ntile_all ? tl : ntile_all - 1)];
      asm volatile("" ::"v"(pgv));  // waited for here, once, so that no copy below waits for it
    }
    // tile k = regions range0 + 16k ..; wave w copies its codes' quarter w
    // and its own copy of the 16 scales (copies past the end re-read the
    // last tile so every iteration issues the same operations)
    auto issue = [&](int k) {
      const int kk = k < nk ? k : nk - 1;
      const int64_t ts = PAGED ? ((int64_t)clamp_page(a.cm, __builtin_amdgcn_readlane(pgv, kk)) * kGroups + g)
                               : ((int64_t)seq * kGroups + g) * ntile_all + (range0 >> 4) + kk;  // tile slot
      LdsPtr dst = (LdsPtr)&ring[k % D][0];
      __builtin_amdgcn_global_load_lds((const void*)(a.summ + ts * 4096 + 1024 * wave + 16 * lane),
                                       dst + 1024 * wave, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(a.scale + ts * kTile + n), dst + 4096 + 256 * wave, 4, 0, 0);
    };
    if (nk > 0)
#pragma unroll
      for (int k = 0; k < D - 1; ++k) issue(k);
    // Store offsets: the lane's part (row 4rs+kb of the wave, region t0+n) is
    // (kb*G*stride + n)*4, the rest ((4rs*G*stride + t0)*4) is uniform and
    // goes in the scalar offset, so no per-tile offsets stay live in vector
    // registers.
    const uint32_t v_ws = ((uint32_t)(kb * kGroups) * (uint32_t)a.ws_stride + (uint32_t)n) * 4u;
    const uint32_t v_out = OUT ? ((uint32_t)(kb * kGroups) * (uint32_t)a.max_regions + (uint32_t)n) * 4u : 0u;
    const uint32_t v_tm = TILEMAX ? (uint32_t)(kb * kGroups) * (uint32_t)a.tm_stride * 4u : 0u;
    // Scores of tile k: four row-sets of 4 queries x 4 heads; lane (kb, n)
    // turns rows 4kb..4kb+3 of row-set rs (query qw + 4rs + kb, the group's
    // 4 heads) into the score of region t0 + n.  In the plain instance the
    // epilogue is software-pipelined: tile k's runs in iteration k + 1,
    // among tile k + 1's MFMAs (one wave can issue independent VALU work
    // while its MFMAs run), and after the loop for the last tile (3%; the
    // other instances have no registers left for the previous tile's
    // accumulators).  Every call issues the same stores (out of the view
    // when `valid` is false), so the wait counts stay exact.
    auto epilogue = [&](const f32x4 (&accs)[NRS], float sc, int t0, bool valid) {
      const int r = t0 + n;
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        const f32x4 acc = accs[rs];
        const f32x4 zz = zq[rs];
        float sv = zz[0] * relu(acc[0]);
        sv = fmaf(zz[1], relu(acc[1]), sv);
        sv = fmaf(zz[2], relu(acc[2]), sv);
        sv = fmaf(zz[3], relu(acc[3]), sv);
        sv *= sc;
        const bool ok = valid && r < cq[rs];  // cq = -1 outside the pass
        const uint32_t srow = (uint32_t)(4 * rs * kGroups);
        const uint32_t s_ws = (srow * (uint32_t)a.ws_stride + (uint32_t)t0) * 4u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), ws_view, ok ? v_ws : kOutOfView, s_ws, 0);
        if (OUT) {
          const uint32_t s_out = (srow * (uint32_t)a.max_regions + (uint32_t)t0) * 4u;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), out_view, ok ? v_out : kOutOfView, s_out, 0);
        }
        if (TILEMAX) {  // lanes 16kb..16kb+15 hold one query's tile
          uint32_t key = ok ? score_key(sv) : 0u;
          key = max(key, (uint32_t)__shfl_xor((int)key, 8));
          key = max(key, (uint32_t)__shfl_xor((int)key, 4));
          key = max(key, (uint32_t)__shfl_xor((int)key, 2));
          key = max(key, (uint32_t)__shfl_xor((int)key, 1));
          const bool tok = valid && n == 0 && t0 < cq[rs];
          const uint32_t s_tm = (srow * (uint32_t)a.tm_stride + (uint32_t)(t0 >= 0 ? t0 / kTile : 0)) * 4u;
          __builtin_amdgcn_raw_buffer_store_b32(key, tm_view, tok ? v_tm : kOutOfView, s_tm, 0);
        }
      }
    };
    f32x4 pacc[NRS];  // the previous tile's accumulators, scale and first region
#pragma unroll
    for (int rs = 0; rs < NRS; ++rs) pacc[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
    float psc = 0.0f;
    int pt0 = (int)range0;
    for (int k = 0; k < nk; ++k) {
      if (k < D - 1) wait_vm<Cfg::W_EARLY>();
      else wait_vm<Cfg::W_FULL>();
      lds_barrier();  // (a workgroup fence here would drain every copy in flight)
      issue(k + D - 1);
      const int t0 = (int)range0 + k * kTile;  // region indices fit 32 bits (max_regions is int32)
      const uint8_t* src = &ring[k % D][0];
      const u32x4 c0 = *(const u32x4*)(src + 16 * lane), c1 = *(const u32x4*)(src + 1024 + 16 * lane),
                  c2 = *(const u32x4*)(src + 2048 + 16 * lane), c3 = *(const u32x4*)(src + 3072 + 16 * lane);
      const float sc = *(const float*)(src + 4096 + 256 * wave + 4 * n);
      // k-steps outer, row-sets inner: one converted pair of B operands is
      // live at a time (the four accumulators instead of eight B operands)
      f32x4 accs[NRS];
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) accs[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
      const u32x4 cc[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x8 B0, B1;
        codes_to_bf16(cc[q4], B0, B1);
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) {
          accs[rs] = mfma16x16x32(A[rs][2 * q4], B0, accs[rs]);
          accs[rs] = mfma16x16x32(A[rs][2 * q4 + 1], B1, accs[rs]);
        }
      }
      if constexpr (kPipelined) {
        epilogue(pacc, psc, pt0, k > 0);
#pragma unroll
        for (int rs = 0; rs < NRS; ++rs) pacc[rs] = accs[rs];
        psc = sc;
        pt0 = t0;
      } else {
        epilogue(accs, sc, t0, true);
      }
    }
    if (kPipelined && nk > 0) epilogue(pacc, psc, pt0, true);
    // the copies issued past the last tile must land before the ring is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------

struct SelectArgs {
  const float* scores;      // [Nq][G][ws_stride]
  const int32_t* slen;      // [Nq] sequence lengths when qpos is nullptr
  const uint16_t* ik;       // decode step: index_k of the sequences (folded compression), or nullptr
  uint8_t* csumm;           // decode step: summaries written by the folded compression
  float* cscale;
  int32_t n_seqs;
  const uint32_t* tilemax;  // [Nq][G][tm_stride] largest key per 16-region tile, or nullptr
  const int32_t* qpos;
  int32_t* sel;             // [Nq][G][topk]
  int32_t* nsel;            // [Nq][G]
  CacheMap cm;              // the sequences' caches (the folded compression's index_k and summaries)
  int32_t nq, max_regions, ws_stride, tm_stride, topk;
};

__device__ __forceinline__ uint64_t cand_key(const float* sc, int64_t r) {
  return ((uint64_t)score_key(sc[r]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)r);
}

// ---------------------------------------------------------------------------
// Ordered selection on keys held in registers.  Entry e of thread t is the
// (e*NT + t)-th entry of an index-ordered candidate sequence (coalesced
// loads); absent entries carry key 0 and come last.  The need-th largest key
// T is found by bisection on its bits with block-wide counts; keys above T
// are all taken, keys equal to T lowest index first, and the selection is
// written in ascending index order.
// ---------------------------------------------------------------------------

// Shared memory of one selection block.
template <int NT, int KPT>
struct alignas(16) SelectSmem {
  static constexpr int NW = NT / 64;
  uint32_t red[2][NW];     // per-wave partial counts, alternating
  uint32_t tgt[KPT * NW];  // per-(entry slot, wave) counts of keys above the boundary, then their scan
  uint32_t teq[KPT * NW];  // same for keys on the boundary
};

// Sum over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

// Number of keys >= trial held by this wave (ballot + scalar popcount).
template <int KPT>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&key)[KPT], uint32_t trial) {
  uint32_t n = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) n += (uint32_t)__popcll(__ballot(key[e] >= trial));
  return n;
}

// Block-wide number of keys >= trial; `slot` alternates between calls so one
// barrier per call suffices.
template <int NT, int KPT>
__device__ __forceinline__ uint32_t block_count_ge(const uint32_t (&key)[KPT], uint32_t trial,
                                                   SelectSmem<NT, KPT>& sm, int slot) {
  const uint32_t n = wave_count_ge<KPT>(key, trial);
  if ((threadIdx.x & 63) == 0) sm.red[slot][threadIdx.x >> 6] = n;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += sm.red[slot][i];
  return t;
}

// Boundary of the need best keys: every key above T is taken and `need -
// above` keys equal to T, lowest index first.
struct Boundary {
  uint32_t T, above;
};

// The need-th largest key (1 <= need <= number of present entries) by
// bisection on its 32 bits.
template <int NT, int KPT>
__device__ Boundary block_boundary(const uint32_t (&key)[KPT], uint32_t need, SelectSmem<NT, KPT>& sm) {
  uint32_t T = 0;
#pragma unroll 1
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = T | (1u << bit);
    if (block_count_ge<NT, KPT>(key, trial, sm, bit & 1) >= need) T = trial;
  }
  const uint32_t above = (T == 0xFFFFFFFFu) ? 0u : block_count_ge<NT, KPT>(key, T + 1, sm, 1);
  return Boundary{T, above};
}

// Exclusive scan, in place, of two tables of n <= 512 counts by wave 0,
// between block barriers.
template <int NT>
__device__ __forceinline__ void scan_tables(uint32_t* ta, uint32_t* tb, int n) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (n + 63) / 64;
    const int i0 = lane * per;
    uint32_t sa = 0, sb = 0;
    for (int i = 0; i < per; ++i)
      if (i0 + i < n) {
        sa += ta[i0 + i];
        sb += tb[i0 + i];
      }
    uint32_t ra = wave_incl_scan(sa) - sa, rb = wave_incl_scan(sb) - sb;
    for (int i = 0; i < per; ++i)
      if (i0 + i < n) {
        const uint32_t va = ta[i0 + i], vb = tb[i0 + i];
        ta[i0 + i] = ra;
        tb[i0 + i] = rb;
        ra += va;
        rb += vb;
      }
  }
  __syncthreads();
}

// Writes the idx of the need best entries to out[0..need) in index order.
// An entry's position is the number of taken entries before it: entries
// above T before it plus min(entries equal to T before it, need - above).
template <int NT, int KPT>
__device__ void emit_top(const uint32_t (&key)[KPT], const int32_t (&idx)[KPT], const Boundary& bd, uint32_t need,
                         int32_t* out, SelectSmem<NT, KPT>& sm) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  const uint32_t need_eq = need - bd.above;
  uint64_t mgt[KPT], meq[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    mgt[e] = __ballot(key[e] > bd.T);
    meq[e] = __ballot(key[e] == bd.T);
    if (lane == 0) {
      sm.tgt[e * NW + w] = (uint32_t)__popcll(mgt[e]);
      sm.teq[e * NW + w] = (uint32_t)__popcll(meq[e]);
    }
  }
  scan_tables<NT>(sm.tgt, sm.teq, KPT * NW);
  // absent entries (key 0) come after every present entry, and at least need
  // present entries are >= T, so an absent entry is never taken
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const uint32_t gt = sm.tgt[e * NW + w] + (uint32_t)__popcll(mgt[e] & lt);
    const uint32_t eq = sm.teq[e * NW + w] + (uint32_t)__popcll(meq[e] & lt);
    uint32_t pos = need;  // need = not taken
    if ((mgt[e] >> lane) & 1ull) pos = gt + (eq < need_eq ? eq : need_eq);
    else if (((meq[e] >> lane) & 1ull) && eq < need_eq) pos = gt + eq;
    if (pos < need) out[pos] = idx[e];
  }
}

// The selection of one problem: the need best candidates in ascending index
// order, then the forced current region c, then -1 padding.
template <int NT, int KPT>
__device__ void select_strided(const uint32_t (&key)[KPT], const int32_t (&idx)[KPT], uint32_t need, int64_t c,
                               int32_t* sel, int32_t* nsel_out, int topk, SelectSmem<NT, KPT>& sm) {
  const Boundary bd = block_boundary<NT, KPT>(key, need, sm);
  emit_top<NT, KPT>(key, idx, bd, need, sel, sm);
  for (int i = (int)need + 1 + threadIdx.x; i < topk; i += NT) sel[i] = -1;
  if (threadIdx.x == 0) {
    sel[need] = (int32_t)c;
    *nsel_out = (int32_t)need + 1;
  }
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

// Problems beyond the register capacity of the tile selection: exact
// selection by radix narrowing over the scores in global memory (12-bit digits) until the
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
  const int64_t c = current_region(query_pos(a.qpos, a.slen, qi), a.cm.R, a.max_regions);
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

  // ---- level 0: 12-bit digit of the score key (bits 63..52 of the 64-bit key)
  uint32_t above, inbin;
  int d;
  for (int i = tid; i < kHistBins; i += NT) hist[i] = 0;
  __syncthreads();
  for (int64_t r = tid; r < c; r += NT) atomicAdd(&hist[score_key(sc[r]) >> 20], 1u);
  __syncthreads();
  d = find_digit<NT>(hist, kHistBins, need, &above, wsum, &sh_d, &sh_above);
  inbin = hist[d];
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


// Long problems: one block per (query, group).  Pass 1 ranks the tiles of 16
// regions by their largest key and keeps the best need of them (all tiles
// when there are at most need).  Every selected region lies in a kept tile:
// a region in a dropped tile ranks below that tile's maximum, which ranks
// below the maxima of need kept tiles, so need regions rank above it.
// Pass 2 ranks the <= need*16 regions of the kept tiles exactly.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void k_select_tiles(SelectArgs a) {
  static_assert(NT * KPT >= kMaxTopk * kTile, "kept tiles must fit in registers");
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  __shared__ SelectSmem<NT, KPT> sm;
  __shared__ int32_t tiles[kMaxTopk];
  const int64_t c = current_region(query_pos(a.qpos, a.slen, qi), a.cm.R, a.max_regions);
  const uint32_t need = (uint32_t)((c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1));
  int32_t* sel = a.sel + pq * a.topk;
  if (select_trivial(c, need, sel, a.nsel + pq, a.topk, NT)) return;
  const int64_t ntiles = (c + kTile - 1) / kTile;
  if (ntiles > (int64_t)NT * KPT) {
    select_fallback<NT>(a, pq);
    return;
  }
  uint32_t kept;
  if (ntiles <= (int64_t)need) {
    for (int j = threadIdx.x; j < ntiles; j += NT) tiles[j] = j;
    kept = (uint32_t)ntiles;
  } else {
    const uint32_t* tm = a.tilemax + pq * a.tm_stride;
    uint32_t tk[KPT];
    int32_t ti[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = e * NT + threadIdx.x;
      tk[e] = tm[j < ntiles ? j : 0];
    }
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = e * NT + threadIdx.x;
      if (j >= ntiles) tk[e] = 0u;
      ti[e] = j;
    }
    const Boundary bd = block_boundary<NT, KPT>(tk, need, sm);
    emit_top<NT, KPT>(tk, ti, bd, need, tiles, sm);
    kept = need;
  }
  __syncthreads();
  const float* sc = a.scores + pq * a.ws_stride;
  const uint32_t m = kept * kTile;
  uint32_t key[KPT];
  int32_t idx[KPT];
  float v[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const uint32_t i = (uint32_t)e * NT + threadIdx.x;
    const int64_t r = (int64_t)tiles[i < m ? i / kTile : 0] * kTile + (i % kTile);
    idx[e] = (int32_t)r;
    v[e] = sc[r < c ? r : 0];
  }
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const uint32_t i = (uint32_t)e * NT + threadIdx.x;
    key[e] = (i < m && idx[e] < c) ? score_key(v[e]) : 0u;
    if (i >= m) idx[e] = 0;
  }
  select_strided<NT, KPT>(key, idx, need, c, sel, a.nsel + pq, a.topk, sm);
}

// Ordered compaction over a block: the entries (e, thread) with flag set get
// consecutive positions in sequence order e*NT + thread.  tab needs
// KPT*NT/64 + 1 entries; returns the number of flagged entries.
template <int NT, int KPT>
__device__ uint32_t ordered_positions(const bool (&flag)[KPT], uint32_t (&pos)[KPT], uint32_t* tab) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint64_t m[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    m[e] = __ballot(flag[e]);
    if (lane == 0) tab[e * NW + w] = (uint32_t)__popcll(m[e]);
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // exclusive scan of the table by wave 0, total at tab[n]
    constexpr int n = KPT * NW, per = (n + 63) / 64;
    const int i0 = lane * per;
    uint32_t v[per], sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      v[i] = (i0 + i < n) ? tab[i0 + i] : 0u;
      sum += v[i];
    }
    const uint32_t incl = wave_incl_scan(sum);
    uint32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (i0 + i < n) tab[i0 + i] = run;
      run += v[i];
    }
    if (lane == 63) tab[n] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < KPT; ++e) pos[e] = tab[e * NW + w] + (uint32_t)__popcll(m[e] & lt);
  return tab[KPT * NW];
}

// Two flag sets at once (tab needs 2*(KPT*NT/64) + 2 entries); totals in
// *na, *nb.
template <int NT, int KPT>
__device__ void ordered_positions2(const bool (&fa)[KPT], const bool (&fb)[KPT], uint32_t (&pa)[KPT],
                                   uint32_t (&pb)[KPT], uint32_t* tab, uint32_t* na, uint32_t* nb) {
  constexpr int NW = NT / 64, n = KPT * NW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t* ta = tab;
  uint32_t* tb = tab + n + 1;
  uint64_t ma[KPT], mb[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    ma[e] = __ballot(fa[e]);
    mb[e] = __ballot(fb[e]);
    if (lane == 0) {
      ta[e * NW + w] = (uint32_t)__popcll(ma[e]);
      tb[e * NW + w] = (uint32_t)__popcll(mb[e]);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    constexpr int per = (n + 63) / 64;
    const int i0 = lane * per;
    uint32_t va[per], vb[per], sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      va[i] = (i0 + i < n) ? ta[i0 + i] : 0u;
      vb[i] = (i0 + i < n) ? tb[i0 + i] : 0u;
      sa += va[i];
      sb += vb[i];
    }
    const uint32_t ia = wave_incl_scan(sa), ib = wave_incl_scan(sb);
    uint32_t ra = ia - sa, rb = ib - sb;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (i0 + i < n) {
        ta[i0 + i] = ra;
        tb[i0 + i] = rb;
      }
      ra += va[i];
      rb += vb[i];
    }
    if (lane == 63) {
      ta[n] = ia;
      tb[n] = ib;
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    pa[e] = ta[e * NW + w] + (uint32_t)__popcll(ma[e] & lt);
    pb[e] = tb[e * NW + w] + (uint32_t)__popcll(mb[e] & lt);
  }
  *na = ta[n];
  *nb = tb[n];
}

// Folded compression (decode step): query qi's token completes region p/8
// when (p+1) is a multiple of 8; that region is summarised here.  Selection
// and the scoring before it read only regions before the query's current
// region, so they never touch the summary being written.
__device__ __forceinline__ void folded_compress(const SelectArgs& a, int64_t qi, int g) {
  const int64_t p = query_pos(a.qpos, a.slen, qi);
  if (p < 0 || (p + 1) % kRegion != 0 || (p + 1) / kRegion > a.cm.R) return;
  int32_t seq = (int32_t)qi;
  seq = seq >= a.n_seqs ? a.n_seqs - 1 : seq;
  compress_region_wave(a.ik, a.cm, seq, p / kRegion, g, a.csumm, a.cscale);
}

// Standalone form for the selection paths without folded blocks: one wave per
// (query, group).
__global__ __launch_bounds__(256) void k_fold_compress(SelectArgs a) {
  const int64_t qi = blockIdx.x;
  folded_compress(a, qi, threadIdx.x >> 6);
}

constexpr int kDecNT = 1024;
constexpr int kDecTilesPT = 8;                          // tile keys per thread (8192 tiles)
static_assert(kDecTilesPT * (kDecNT / 64) + 1 >= 2 * (kDecNT / 64 + 1), "table holds both passes");

struct alignas(16) DecSmem {
  uint32_t wtot[kDecNT / 64];
  uint32_t res[4];
  uint32_t tab[kDecTilesPT * (kDecNT / 64) + 1];  // ordered positions of the tiles, then of the final pass
  union alignas(16) {
    int32_t tiles[kCandCap];  // kept tiles (step 2)
    uint32_t hh[1024];        // 10-bit digit histogram of the finishing wave (step 3)
  };
  uint32_t ck[kCandCap];      // candidate keys, index order
  int32_t ci[kCandCap];       // candidate regions
  union alignas(16) {
    uint32_t hdig[kHistBins];  // level-0 digit counts: tile maxima (step 1), candidates (step 2)
    uint32_t kin[kCandCap];    // keys in the boundary digit, any order (step 3)
  };
  uint32_t n_in;
  uint32_t stage[kTile][kDecNT];  // each thread's 16 tile keys (a column per thread)
};

// One wave: the digit (of `bits` bits at `shift`) holding the rem-th largest
// of the keys kin[0..n) whose bits above shift+bits equal `hi`; counts of the
// keys in higher digits go to *above.  LDS operations of one wave complete in
// order, so no barrier is needed.
__device__ __forceinline__ uint32_t wave_digit(const uint32_t* kin, uint32_t n, uint32_t hi, int shift, uint32_t rem,
                                               uint32_t* hh, uint32_t* above) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)&hh[16 * lane + 4 * i] = u32x4{0u, 0u, 0u, 0u};
  for (uint32_t q = lane; q < n; q += 64) {
    const uint32_t k = kin[q];
    if ((k >> (shift + 10)) == hi) atomicAdd(&hh[(k >> shift) & 1023u], 1u);
  }
  // lane l owns digits 1023-16l down to 1008-16l
  uint32_t cnt[16], mine = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = *(const u32x4*)&hh[1008 - 16 * lane + 4 * i];
    cnt[15 - 4 * i] = v.x;
    cnt[14 - 4 * i] = v.y;
    cnt[13 - 4 * i] = v.z;
    cnt[12 - 4 * i] = v.w;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) mine += cnt[j];
  const uint32_t incl = wave_incl_scan(mine);
  uint32_t run = incl - mine, dig = 0, ab = 0;
  bool hit = false;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (run < rem && run + cnt[j] >= rem) {
      hit = true;
      dig = (uint32_t)(1023 - 16 * lane - j);
      ab = run;
    }
    run += cnt[j];
  }
  const uint64_t hm = __ballot(hit);
  const int src = hm ? __ffsll((long long)hm) - 1 : 0;
  *above = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
  return (uint32_t)__builtin_amdgcn_readlane((int)dig, src);
}

// Decode selection, one block per (query, group), on what k_score_dec left:
// the scores and each 16-region tile's largest key.
//  1. A histogram of the tile maxima's level-0 digits (12 bits) gives the
//     digit d0 of the need-th largest tile maximum.  The need largest tile
//     maxima are need different scores, so the need-th largest score is at
//     least T0 = d0 << 20, the lowest key of that digit: every region to
//     select lies in a tile whose maximum reaches T0, with a key >= T0.
//  2. Those tiles are compacted in index order, and their regions with keys
//     >= T0 (the candidates) too, while the candidates' digits are counted;
//     the counts give the digit d holding the need-th largest candidate, the
//     number of candidates above it and in it.
//  3. One wave finds the need-th largest key from the keys inside digit d
//     (two 10-bit rounds) and writes the selection in index order.
// Problems with more kept tiles or candidates than kCandCap, or more tiles
// than the block holds, use the radix fallback.
__global__ __launch_bounds__(kDecNT) void k_select_dec(SelectArgs a) {
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ DecSmem sm;
  if (pq >= (int64_t)a.nq * kGroups) {  // folded compression: wave w -> (query, group)
    const int64_t fq = (pq - (int64_t)a.nq * kGroups) * (kDecNT / 64 / kGroups) + w / kGroups;
    if (fq < a.nq) folded_compress(a, fq, w % kGroups);
    return;
  }
  // Every load that needs only the block index is issued before any of them
  // is waited for: the query's position first (so that waiting for it leaves
  // the others in flight), then every tile maximum the block can hold (tiles
  // past the problem are masked below).
  const int32_t qraw = *(a.qpos ? a.qpos + qi : a.slen + qi);  // (one load, no branch)
  const uint32_t* tm = a.tilemax + pq * a.tm_stride;
  uint32_t tk[kDecTilesPT];
#pragma unroll
  for (int e = 0; e < kDecTilesPT; ++e) {
    const int64_t j = (int64_t)e * kDecNT + tid;
    tk[e] = tm[j < a.tm_stride ? j : 0];
  }
  static_assert(kHistBins == 4 * kDecNT, "thread t owns digits 4095-4t .. 4092-4t");
  *(u32x4*)&sm.hdig[4 * tid] = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) sm.n_in = 0;
  // The digit holding the need-th largest of the counted keys (digits from
  // the top, thread t owning digits 4095-4t .. 4092-4t): its value, the count
  // of keys above it and in it in sm.res[0..2] (res[0] = ~0 when fewer than
  // need keys were counted).  Ends with a barrier; sm.res[0] must be ~0 on
  // entry, and sm.wtot is overwritten.
  auto boundary_digit = [&](uint32_t need_) {
    const u32x4 h = *(const u32x4*)&sm.hdig[kHistBins - 4 - 4 * tid];
    const uint32_t cnt[4] = {h.w, h.z, h.y, h.x};
    const uint32_t mine = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    const uint32_t wi = wave_incl_scan(mine);
    if (lane == 63) sm.wtot[w] = wi;
    lds_barrier();
    uint32_t run = wi - mine;
#pragma unroll
    for (int i = 0; i < kDecNT / 256; ++i) {
      const u32x4 v = *(const u32x4*)&sm.wtot[4 * i];
      run += (4 * i < w ? v.x : 0u) + (4 * i + 1 < w ? v.y : 0u) + (4 * i + 2 < w ? v.z : 0u) +
             (4 * i + 3 < w ? v.w : 0u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run < need_ && run + cnt[j] >= need_) {
        sm.res[0] = (uint32_t)(kHistBins - 1 - 4 * tid - j);
        sm.res[1] = run;
        sm.res[2] = cnt[j];
      }
      run += cnt[j];
    }
    lds_barrier();
  };
  if (tid == 0) sm.res[0] = 0xFFFFFFFFu;
  lds_barrier();  // (the histogram cleared)
  const int64_t c = current_region(a.qpos ? qraw : qraw - 1, a.cm.R, a.max_regions);
  const uint32_t need = (uint32_t)((c < (int64_t)(a.topk - 1)) ? c : (int64_t)(a.topk - 1));
  int32_t* sel = a.sel + pq * a.topk;
  if (select_trivial(c, need, sel, a.nsel + pq, a.topk, kDecNT)) return;
  const int64_t ntiles = (c + kTile - 1) / kTile;
  if (ntiles > (int64_t)kDecNT * kDecTilesPT) {
    select_fallback<kDecNT>(a, pq);
    return;
  }
#pragma unroll
  for (int e = 0; e < kDecTilesPT; ++e) {
    if ((int64_t)e * kDecNT + tid >= ntiles) tk[e] = 0u;
    else atomicAdd(&sm.hdig[tk[e] >> 20], 1u);
  }
  lds_barrier();
  // 1. the digit of the need-th largest tile maximum
  boundary_digit(need);
  const uint32_t d0 = sm.res[0];
  if (d0 == 0xFFFFFFFFu) {  // (fewer than need tiles hold a score: not on the tile path)
    select_fallback<kDecNT>(a, pq);
    return;
  }
  const uint32_t T0 = d0 << 20;
  // the histogram again, for the candidates' digits (the kept-tile
  // compaction below passes barriers before any candidate is counted)
  *(u32x4*)&sm.hdig[4 * tid] = u32x4{0u, 0u, 0u, 0u};
  // 2. kept tiles, then the candidates in them
  {
    bool f[kDecTilesPT];
    uint32_t pos[kDecTilesPT];
#pragma unroll
    for (int e = 0; e < kDecTilesPT; ++e) f[e] = tk[e] >= T0 && (int64_t)e * kDecNT + tid < ntiles;
    ordered_positions<kDecNT, kDecTilesPT>(f, pos, sm.tab);
#pragma unroll
    for (int e = 0; e < kDecTilesPT; ++e)
      if (f[e] && pos[e] < (uint32_t)kCandCap) sm.tiles[pos[e]] = e * kDecNT + tid;
  }
  const uint32_t ntl_all = sm.tab[kDecTilesPT * (kDecNT / 64)];
  const uint32_t ntl = min(ntl_all, (uint32_t)kCandCap);
  lds_barrier();
  if (tid == 0) sm.res[0] = 0xFFFFFFFFu;  // (d0 was read before the barriers above)
  // The kept tiles in rounds of one tile per thread (round rd: kept tiles
  // rd*kDecNT + tid, so the rounds follow index order): a tile's 16 scores in
  // one 64-byte row, the candidates among them counted, a block scan of the
  // counts in thread order (= index order), and the candidates written to
  // LDS in index order after those of earlier rounds.
  constexpr int kCandRounds = kCandCap / kDecNT;
  static_assert(kCandCap == kCandRounds * kDecNT, "whole rounds of one kept tile per thread");
  uint32_t ncand = 0;
  for (int rd = 0; rd < kCandRounds; ++rd) {
    if ((uint32_t)rd * kDecNT >= ntl) break;  // (uniform: ntl is the same for every thread)
    const uint32_t ti = (uint32_t)rd * kDecNT + tid;
    const bool have = ti < ntl;
    const int64_t t = have ? sm.tiles[ti] : 0;
    const u32x4* tp = (const u32x4*)(a.scores + pq * a.ws_stride + t * kTile);
    u32x4 q4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q4[j] = tp[j];
    uint32_t key[kTile], fa = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      key[4 * j + 0] = score_key(__uint_as_float(q4[j].x));
      key[4 * j + 1] = score_key(__uint_as_float(q4[j].y));
      key[4 * j + 2] = score_key(__uint_as_float(q4[j].z));
      key[4 * j + 3] = score_key(__uint_as_float(q4[j].w));
    }
#pragma unroll
    for (int i = 0; i < kTile; ++i) sm.stage[i][tid] = key[i];
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
      const bool ok = have && t * kTile + i < c && key[i] >= T0;
      fa |= (ok ? 1u : 0u) << i;
    }
    const uint32_t cntc = (uint32_t)__popc(fa);
    const uint32_t incl = wave_incl_scan(cntc);
    if (lane == 63) sm.wtot[w] = incl;
    lds_barrier();
    uint32_t base = incl - cntc, total = 0;
#pragma unroll
    for (int i = 0; i < kDecNT / 256; ++i) {
      const u32x4 v = *(const u32x4*)&sm.wtot[4 * i];
      base += (4 * i < w ? v.x : 0u) + (4 * i + 1 < w ? v.y : 0u) + (4 * i + 2 < w ? v.z : 0u) +
              (4 * i + 3 < w ? v.w : 0u);
      total += v.x + v.y + v.z + v.w;
    }
    // the thread's keys go through its own LDS column so that the loop over
    // its candidates (about one) can index them
    uint32_t oa = ncand + base;
    for (uint32_t m = fa; m; m &= m - 1u, ++oa) {
      const int i = __ffs((int)m) - 1;
      const uint32_t k = sm.stage[i][tid];
      if (oa < (uint32_t)kCandCap) {
        sm.ck[oa] = k;
        sm.ci[oa] = (int32_t)(t * kTile + i);
        atomicAdd(&sm.hdig[k >> 20], 1u);
      }
    }
    ncand += total;
    lds_barrier();  // (the next round rewrites sm.wtot)
  }
  if (ntl_all > (uint32_t)kCandCap || ncand > (uint32_t)kCandCap || ncand < need) {
    select_fallback<kDecNT>(a, pq);
    return;
  }
  // the candidates' boundary digit, then the keys inside it gathered for
  // the finishing wave (two per thread)
  boundary_digit(need);
  const uint32_t d = sm.res[0], above = sm.res[1];
  static_assert(kCandCap == 2 * kDecNT, "two candidates per thread");
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t j = (uint32_t)e * kDecNT + tid;
    if (j < ncand) {
      const uint32_t k = sm.ck[j];
      if ((k >> 20) == d) sm.kin[atomicAdd(&sm.n_in, 1u)] = k;
    }
  }
  lds_barrier();
  const uint32_t nin = sm.n_in;
  // 3. wave 0: the need-th largest key T lies in digit d; its next 10 bits,
  // then its last 10, from histograms of the in-digit keys
  const uint32_t M = min(ncand, (uint32_t)kCandCap);
  if (w == 0) {
    const uint32_t n_in = min(nin, (uint32_t)kCandCap);
    uint32_t ab1, ab2;
    const uint32_t d1 = wave_digit(sm.kin, n_in, d, 10, need - above, sm.hh, &ab1);
    const uint32_t d2 = wave_digit(sm.kin, n_in, (d << 10) | d1, 0, need - above - ab1, sm.hh, &ab2);
    if (lane == 0) {
      sm.res[0] = (((d << 10) | d1) << 10) | d2;
      sm.res[1] = need - above - ab1 - ab2;  // keys equal to T to take
    }
  }
  __syncthreads();
  const uint32_t T = sm.res[0], need_eq = sm.res[1];
  // 4. every thread places candidates tid and tid + kDecNT: taken entries
  // before one are the keys above T before it plus min(keys equal to T before
  // it, need_eq)
  static_assert(kCandCap == 2 * kDecNT, "two candidates per thread");
  bool fg[2], fe[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t j = (uint32_t)e * kDecNT + tid;
    const uint32_t k = j < M ? sm.ck[j] : 0u;
    fg[e] = j < M && k > T;
    fe[e] = j < M && k == T;
  }
  uint32_t pg[2], pe[2], ng, ne;
  ordered_positions2<kDecNT, 2>(fg, fe, pg, pe, sm.tab, &ng, &ne);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t pos = need;
    if (fg[e]) pos = pg[e] + (pe[e] < need_eq ? pe[e] : need_eq);
    else if (fe[e] && pe[e] < need_eq) pos = pg[e] + pe[e];
    if (pos < need) sel[pos] = sm.ci[(uint32_t)e * kDecNT + tid];
  }
  // the forced current region, the padding and the count
  for (int i = (int)need + 1 + tid; i < a.topk; i += kDecNT) sel[i] = -1;
  if (tid == 0) {
    sel[need] = (int32_t)c;
    a.nsel[pq] = (int32_t)need + 1;
  }
}


#ifndef DSA_PRE_SELECT_NT
#define DSA_PRE_SELECT_NT 256
#endif
constexpr int kPreNT = DSA_PRE_SELECT_NT;  // threads of the prefill selection block (<= 8192 regions)
constexpr int kPreFin = kPreNT;            // bin sizes the prefill selection finishes by ranking

template <int NT, int KPT>
struct alignas(16) PreSmem {
  SelectSmem<NT, KPT> s;           // bisection fallback and tie-aware output
  uint32_t wred[NT / 64];          // per-wave maxima, then per-wave totals
  uint32_t res[4];
  uint32_t n_in;
  alignas(16) uint32_t tab[KPT * (NT / 64)];  // output offsets, [wave][entry]
  alignas(16) uint32_t hist[kHistBins];       // value histogram
  uint32_t kin[kPreFin];           // keys of the boundary bin, any order
  int32_t out[kMaxTopk];           // the selection, staged for a coalesced store
};

// Largest value over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}

// Bin of a key in the prefill histogram: keys of positive scores map
// linearly in score value onto 0..4095 (inv = 4096 / largest score), every
// other key to bin 0.  The map never decreases as the key grows, so the bins
// split the ranking into contiguous runs.
__device__ __forceinline__ uint32_t value_bin(uint32_t key, float inv) {
  const float s = __uint_as_float(key & 0x7FFFFFFFu);
  return key > 0x80000000u ? (uint32_t)fminf(s * inv, (float)(kHistBins - 1)) : 0u;
}

// Prefill: one block per (query, group); the problem's scores (c <= NT*KPT)
// are loaded straight into registers in index order.
//  1. A histogram of the scores on a linear scale up to the block's largest
//     score gives the bin holding the need-th largest key and the count of
//     keys in higher bins.  Scores are spread over many bins, so the LDS
//     increments rarely collide and the boundary bin holds a handful of keys.
//  2. The boundary bin's keys are ranked against each other, which gives the
//     need-th largest key T.
//  3. Keys above T are taken, keys equal to T lowest index first, and the
//     selection is written in ascending index order.
// A boundary bin holding more than kPreFin keys (many equal scores) falls
// back to bisection on the keys in registers.  The phases are short and
// separated by barriers, so blocks overlap each other's waits: seven
// resident per CU (72 registers, 21 KB of LDS each) beat five (96
// registers) by 11%, and eight (64 registers, the histogram overlaid with the
// later buffers) by 4%.
static_assert(kHistBins == kPreNT * 16, "each thread owns 16 histogram bins");
template <int NT, int KPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(7))) void k_select_pre(SelectArgs a) {
  constexpr int NW = NT / 64;
  static_assert(NW == kGroups, "a folded block compresses one query's 4 groups");
  const int64_t pq = blockIdx.x;
  const int qi = (int)(pq / kGroups);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (pq >= (int64_t)a.nq * kGroups) {  // folded compression of a decode step: query pq - nq G, wave w -> group w
    const int64_t fq = pq - (int64_t)a.nq * kGroups;
    if (fq < a.nq) folded_compress(a, fq, w);
    return;
  }
  __shared__ PreSmem<NT, KPT> sm;
  const int64_t c64 = current_region(query_pos(a.qpos, a.slen, qi), a.cm.R, a.max_regions);
  const uint32_t need = (uint32_t)((c64 < (int64_t)(a.topk - 1)) ? c64 : (int64_t)(a.topk - 1));
  int32_t* sel = a.sel + pq * a.topk;
  if (select_trivial(c64, need, sel, a.nsel + pq, a.topk, NT)) return;
  const int c = (int)c64;             // candidates 0..c-1, c < NT*KPT
  const int ne = (c + NT - 1) / NT;   // entries holding a candidate in some thread
  // Loads through a buffer view of the c scores: every one is issued at
  // once, with a scalar offset per entry, and entries past c read 0 (their
  // keys are cleared below).
  const __amdgpu_buffer_rsrc_t view =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.scores + pq * a.ws_stride), 0, c * 4, 0x00020000);
  float v[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(view, tid * 4, e * NT * 4, 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)&sm.hist[16 * tid + 4 * i] = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) {
    sm.res[0] = 0xFFFFFFFFu;
    sm.n_in = 0;
  }
  // Present keys are >= 1 (a NaN score, the lowest, gets 1) and absent
  // entries 0, so no later step needs the entry's index to tell them apart.
  uint32_t key[KPT], kmax = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const uint32_t k = max(score_key(v[e]), 1u);  // converted unconditionally: no branch per entry
    key[e] = k & (0u - (uint32_t)(e * NT + tid < c));
    kmax = max(kmax, key[e]);
  }
  kmax = wave_max(kmax);
  if (lane == 0) sm.wred[w] = kmax;
  __syncthreads();
  // 1. histogram and the bin holding the need-th largest key; absent entries
  // of the last partly filled entry land in bin 0 and are taken out again
#pragma unroll
  for (int i = 0; i < NW; ++i) kmax = max(kmax, sm.wred[i]);
  const float smax = __uint_as_float(kmax & 0x7FFFFFFFu);
  const float inv = kmax > 0x80000000u ? (float)kHistBins / smax : 0.0f;
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if (e < ne) atomicAdd(&sm.hist[value_bin(key[e], inv)], 1u);
  __syncthreads();
  {
    // thread t owns bins 4095-16t down to 4080-16t
    uint32_t cnt[16], mine = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 h = *(const u32x4*)&sm.hist[kHistBins - 16 - 16 * tid + 4 * i];
      cnt[15 - 4 * i] = h.x;
      cnt[14 - 4 * i] = h.y;
      cnt[13 - 4 * i] = h.z;
      cnt[12 - 4 * i] = h.w;
    }
    if (tid == NT - 1) cnt[15] -= (uint32_t)(ne * NT - c);
#pragma unroll
    for (int j = 0; j < 16; ++j) mine += cnt[j];
    const uint32_t wi = wave_incl_scan(mine);
    if (lane == 63) sm.wred[w] = wi;
    __syncthreads();
    uint32_t run = wi - mine;
#pragma unroll
    for (int i = 0; i < NW; ++i) run += i < w ? sm.wred[i] : 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (run < need && run + cnt[j] >= need) {
        sm.res[0] = (uint32_t)(kHistBins - 1 - 16 * tid - j);
        sm.res[1] = run;
        sm.res[2] = cnt[j];
      }
      run += cnt[j];
    }
  }
  __syncthreads();
  const uint32_t d = sm.res[0], above = sm.res[1], inbin = sm.res[2];
  Boundary bd;
  uint32_t n_eq = 0;  // keys equal to T (known on the ranking path)
  if (d == 0xFFFFFFFFu || inbin > (uint32_t)kPreFin) {
    bd = block_boundary<NT, KPT>(key, need, sm.s);
  } else {
    // 2. gather the boundary bin and rank its keys
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      if (key[e] != 0u && value_bin(key[e], inv) == d) {
        const uint32_t slot = atomicAdd(&sm.n_in, 1u);
        if (slot < (uint32_t)kPreFin) sm.kin[slot] = key[e];
      }
    }
    __syncthreads();
    const uint32_t n = min(sm.n_in, (uint32_t)kPreFin);
    const uint32_t rem = need - above;  // 1 <= rem <= n
    if ((uint32_t)tid < n) {
      const uint32_t k = sm.kin[tid];
      uint32_t gt = 0, ge = 0;
      for (uint32_t j = 0; j < n; ++j) {
        const uint32_t o = sm.kin[j];
        gt += o > k ? 1u : 0u;
        ge += o >= k ? 1u : 0u;
      }
      if (gt < rem && rem <= ge) {  // every lane holding T writes the same values
        sm.res[3] = k;
        sm.res[1] = above + gt;
        sm.res[2] = ge - gt;
      }
    }
    __syncthreads();
    bd = Boundary{sm.res[3], sm.res[1]};
    n_eq = sm.res[2];
  }
  // 3. ordered output
  for (int i = (int)need + 1 + tid; i < a.topk; i += NT) sel[i] = -1;
  if (tid == 0) {
    sel[need] = c;
    a.nsel[pq] = (int32_t)need + 1;
  }
  if (n_eq != need - bd.above) {  // only some keys equal to T are taken (or not known)
    int32_t idx[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) idx[e] = e * NT + tid;
    emit_top<NT, KPT>(key, idx, bd, need, sel, sm.s);
    return;
  }
  // every key >= T is taken (T >= 1, so no absent entry): one flag per
  // entry, offsets from a scanned table of per-(entry, wave) counts; the
  // flags are taken again after the scan rather than held in scalar registers
  const uint32_t T = bd.T;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const uint64_t m = __ballot(key[e] >= T);
    if (lane == 0) sm.tab[w * KPT + e] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  if (w == 0) {  // exclusive scan in index order (entry-major, then wave)
    constexpr int n = KPT * NW, per = (n + 63) / 64;
    uint32_t val[per], sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int o = lane * per + i;  // position o in index order = (entry o / NW, wave o % NW)
      val[i] = o < n ? sm.tab[(o % NW) * KPT + o / NW] : 0u;
      sum += val[i];
    }
    uint32_t run = wave_incl_scan(sum) - sum;  // each lane rewrites only the entries it read
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int o = lane * per + i;
      if (o < n) sm.tab[(o % NW) * KPT + o / NW] = run;
      run += val[i];
    }
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < KPT; e += 4) {
    const u32x4 off = *(const u32x4*)&sm.tab[w * KPT + e];
    const uint32_t o4[4] = {off.x, off.y, off.z, off.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool f = key[e + j] >= T;
      const uint64_t m = __ballot(f);
      if (f) sm.out[o4[j] + (uint32_t)__popcll(m & lt)] = (e + j) * NT + tid;
    }
  }
  __syncthreads();
  for (int i = tid; i < (int)need; i += NT) sel[i] = sm.out[i];
}

#ifndef DSA_TILE_SELECT_NT
#define DSA_TILE_SELECT_NT 1024
#endif
constexpr int kTileNT = DSA_TILE_SELECT_NT;

static int64_t ws_stride_of(int32_t max_regions) { return ((int64_t)max_regions + 63) / 64 * 64; }
static bool decode_shaped(int32_t n_queries) { return n_queries < 64; }

// Problems with more candidate regions than kDirectMax go through the tile
// maxima.
static bool tiled_select(int32_t max_regions) { return max_regions > kDirectMax; }
static int64_t tm_stride_of(int32_t max_regions) { return ((int64_t)max_regions / kTile + 1 + 63) / 64 * 64; }

// Decode-shaped problems long enough for the tile path: one selection block
// of kDecNT threads per (query, group).
static bool dec_select(int32_t n_queries, int32_t max_regions) {
  return decode_shaped(n_queries) && tiled_select(max_regions);
}

struct ScoreWs {
  uint32_t* tilemax;
  float* scores;
  size_t bytes;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static ScoreWs score_ws_layout(void* base, int32_t nq, int32_t max_regions) {
  ScoreWs w;
  char* p = (char*)base;
  const size_t np = (size_t)nq * kGroups;
  size_t off = 0;
  w.tilemax = nullptr;
  if (tiled_select(max_regions)) {
    w.tilemax = (uint32_t*)(p + off);
    off += align256(np * (size_t)tm_stride_of(max_regions) * 4);
  }
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

// Score + select launches shared by dsa_score_topk and dsa_decode_step (which
// passes q_seq = q_pos = nullptr with seq_len, and index_k for the folded
// compression).
static dsa_status launch_score_topk(const dsa_geometry* geom, int32_t n_queries, const uint16_t* index_q,
                                    const float* z, const int32_t* q_seq, const int32_t* q_pos,
                                    const int32_t* seq_len, int32_t n_seqs, const uint8_t* summ,
                                    const float* scale, const CacheMap& cm, int32_t max_regions, int32_t* sel,
                                    int32_t* n_sel, float* scores_out, const uint16_t* index_k,
                                    uint8_t* csumm, float* cscale, void* workspace, hipStream_t s) {
  const ScoreWs w = score_ws_layout(workspace, n_queries, max_regions);
  const int32_t stride = (int32_t)ws_stride_of(max_regions);
  ScoreArgs sa;
  sa.iq = index_q; sa.z = z; sa.qseq = q_seq; sa.qpos = q_pos; sa.slen = seq_len; sa.summ = summ; sa.scale = scale;
  sa.scores = w.scores; sa.scores_out = scores_out; sa.tilemax = w.tilemax;
  sa.cm = cm; sa.nq = n_queries; sa.n_seqs = n_seqs; sa.max_regions = max_regions;
  sa.ws_stride = stride; sa.tm_stride = (int32_t)tm_stride_of(max_regions); sa.topk = geom->topk;
  SelectArgs se;
  se.scores = w.scores; se.slen = seq_len; se.tilemax = w.tilemax; se.qpos = q_pos;
  se.ik = index_k; se.csumm = csumm; se.cscale = cscale; se.n_seqs = n_seqs;
  se.sel = sel; se.nsel = n_sel; se.cm = cm; se.nq = n_queries; se.max_regions = max_regions;
  se.ws_stride = stride; se.tm_stride = sa.tm_stride; se.topk = geom->topk;
  // the decode step's compression runs as extra blocks of the selection
  // launch (the decode one, or the short-context one), or as its own small
  // launch before the tile selection
  const bool fold_in_select = index_k && (dec_select(n_queries, max_regions) || !tiled_select(max_regions));
  if (index_k && !fold_in_select) {
    ProfScope prof_("k_compress", s);
    hipLaunchKernelGGL(k_fold_compress, dim3((unsigned)n_queries), dim3(256), 0, s, se);
  }
  // Decode-shaped calls (few queries, many regions) score one query per block
  // over long contiguous tile runs; prefill-shaped calls score 16 queries per
  // wave so each summary tile feeds 4 MFMA row-sets.
  if (decode_shaped(n_queries)) {
    ProfScope prof_("k_score_decode", s);
    // short contexts: ranges of kDecRangeShort regions, so that even one
    // query's few thousand regions spread over tens of blocks
    if (max_regions <= kDirectMax) {
      const dim3 grid((max_regions + kDecRangeShort - 1) / kDecRangeShort, kGroups, n_queries);
      if (cm.bt) hipLaunchKernelGGL((k_score_dec<true, kDecRangeShort>), grid, dim3(256), 0, s, sa);
      else hipLaunchKernelGGL((k_score_dec<false, kDecRangeShort>), grid, dim3(256), 0, s, sa);
    } else {
      const dim3 grid((max_regions + kDecRange - 1) / kDecRange, kGroups, n_queries);
      if (cm.bt) hipLaunchKernelGGL((k_score_dec<true, kDecRange>), grid, dim3(256), 0, s, sa);
      else hipLaunchKernelGGL((k_score_dec<false, kDecRange>), grid, dim3(256), 0, s, sa);
    }
  } else {
    ProfScope prof_("k_score_prefill", s);
    const int ranges = (max_regions + kScoreRange - 1) / kScoreRange;
    const int qblocks = (n_queries + kPreQ - 1) / kPreQ;
    const dim3 grid((unsigned)(8 * ranges * kGroups * ((qblocks + 7) / 8)));  // (see k_score_pre)
    const bool tm = tiled_select(max_regions), out = scores_out != nullptr;
    // (paged and contiguous caches are separate instantiations: the page-id
    // loads stay out of the contiguous kernels)
    if (cm.bt) {
      if (tm && out) hipLaunchKernelGGL((k_score_pre<true, true, true>), grid, dim3(256), 0, s, sa);
      else if (tm) hipLaunchKernelGGL((k_score_pre<true, false, true>), grid, dim3(256), 0, s, sa);
      else if (out) hipLaunchKernelGGL((k_score_pre<false, true, true>), grid, dim3(256), 0, s, sa);
      else hipLaunchKernelGGL((k_score_pre<false, false, true>), grid, dim3(256), 0, s, sa);
    } else {
      if (tm && out) hipLaunchKernelGGL((k_score_pre<true, true, false>), grid, dim3(256), 0, s, sa);
      else if (tm) hipLaunchKernelGGL((k_score_pre<true, false, false>), grid, dim3(256), 0, s, sa);
      else if (out) hipLaunchKernelGGL((k_score_pre<false, true, false>), grid, dim3(256), 0, s, sa);
      else hipLaunchKernelGGL((k_score_pre<false, false, false>), grid, dim3(256), 0, s, sa);
    }
  }
  dsa_status st = check_launch("dsa_score_topk: score");
  if (st != DSA_OK) return st;
  {
    ProfScope prof_("k_select", s);
    const dim3 grid((unsigned)((int64_t)n_queries * kGroups));
    if (!tiled_select(max_regions)) {  // (+ one block per query for the folded compression)
      const dim3 g2((unsigned)((int64_t)n_queries * (kGroups + (fold_in_select ? 1 : 0))));
      if (max_regions <= 4 * kPreNT)  // short problems: 4 score slots per thread instead of 32
        hipLaunchKernelGGL((k_select_pre<kPreNT, 4>), g2, dim3(kPreNT), 0, s, se);
      else
        hipLaunchKernelGGL((k_select_pre<kPreNT, kDirectMax / kPreNT>), g2, dim3(kPreNT), 0, s, se);
    }
    else if (dec_select(n_queries, max_regions)) {
      const int64_t folds = fold_in_select ? ((int64_t)n_queries * kGroups + kDecNT / 64 - 1) / (kDecNT / 64) : 0;
      hipLaunchKernelGGL(k_select_dec, dim3((unsigned)((int64_t)n_queries * kGroups + folds)), dim3(kDecNT), 0, s,
                         se);
    }
    else
      hipLaunchKernelGGL((k_select_tiles<kTileNT, kMaxTopk * kTile / kTileNT>), grid, dim3(kTileNT), 0, s, se);
  }
  return check_launch("dsa_score_topk: select");
}

static dsa_status score_topk(const char* who, const dsa_geometry* geom, int32_t n_queries, const uint16_t* index_q,
                             const float* z, const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                             const uint8_t* summ, const float* scale, const CacheMap& cm, int32_t max_regions,
                             int32_t* sel, int32_t* n_sel, float* scores_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const std::string w(who);
  if (n_queries < 0 || n_seqs < 0 || max_regions < 0) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": bad sizes");
  if (n_queries == 0) return DSA_OK;
  if (n_seqs == 0 || max_regions == 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, w + ": n_seqs and max_regions must be positive");
  if (!index_q || !z || !q_seq || !q_pos || !summ || !scale || !sel || !n_sel || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, w + ": NULL pointer");
  if ((size_t)workspace & 255) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": workspace must be 256-byte aligned");
  if (workspace_bytes < dsa_score_topk_workspace_size(geom, n_queries, max_regions))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, w + ": workspace too small");
  if (n_queries > 65535 * 16) return fail(DSA_ERR_UNSUPPORTED, w + ": too many queries");
  return launch_score_topk(geom, n_queries, index_q, z, q_seq, q_pos, nullptr, n_seqs, summ, scale, cm,
                           max_regions, sel, n_sel, scores_out, nullptr, nullptr, nullptr, workspace,
                           as_stream(stream));
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
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_score_topk: tcap must be a positive multiple of 128");
  return score_topk("dsa_score_topk", geom, n_queries, index_q, z, q_seq, q_pos, n_seqs, summ, scale,
                    contiguous_map(tcap), max_regions, sel, n_sel, scores_out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_score_topk_paged(const dsa_geometry* geom, int32_t n_queries,
                                           const uint16_t* index_q, const float* z, const int32_t* q_seq,
                                           const int32_t* q_pos, int32_t n_seqs, const dsa_page_table* pages,
                                           const uint8_t* summ_pool, const float* scale_pool,
                                           int32_t max_regions, int32_t* sel, int32_t* n_sel, float* scores_out,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_score_topk_paged", pages, &cm);
  if (st != DSA_OK) return st;
  return score_topk("dsa_score_topk_paged", geom, n_queries, index_q, z, q_seq, q_pos, n_seqs, summ_pool,
                    scale_pool, cm, max_regions, sel, n_sel, scores_out, workspace, workspace_bytes, stream);
}

extern "C" size_t dsa_decode_step_workspace_size(const dsa_geometry* geom, int32_t batch, int32_t max_regions) {
  if (batch <= 0 || max_regions <= 0) return 256;
  return align256(dsa_score_topk_workspace_size(geom, batch, max_regions)) +
         align256(dsa_sparse_gqa_workspace_size(geom, batch));
}

static dsa_status decode_step(const char* who, const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                              const uint16_t* index_q, const float* z, const uint16_t* index_k,
                              const uint16_t* k_cache, const uint16_t* v_cache, const CacheMap& cm,
                              const int32_t* seq_len, uint8_t* summ, float* scale, int32_t max_regions,
                              int32_t* sel, int32_t* n_sel, uint16_t* out, void* workspace,
                              size_t workspace_bytes, void* stream, const Fp8Kv* f8 = nullptr) {
  const std::string w(who);
  if (batch < 0 || max_regions < 0) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": bad sizes");
  if (batch == 0) return DSA_OK;
  if (max_regions == 0) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": max_regions must be positive");
  const bool kv_ok = f8 ? (f8->k8 && f8->v8 && f8->kvs) : (k_cache && v_cache);
  if (!q || !index_q || !z || !index_k || !kv_ok || !seq_len || !summ || !scale || !sel || !n_sel || !out ||
      !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, w + ": NULL pointer");
  if ((size_t)workspace & 255) return fail(DSA_ERR_INVALID_ARGUMENT, w + ": workspace must be 256-byte aligned");
  if (workspace_bytes < dsa_decode_step_workspace_size(geom, batch, max_regions))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, w + ": workspace too small");
  if (batch > 65535) return fail(DSA_ERR_UNSUPPORTED, w + ": batch > 65535");
  hipStream_t s = as_stream(stream);
  const size_t ws1 = align256(dsa_score_topk_workspace_size(geom, batch, max_regions));
  dsa_status st = launch_score_topk(geom, batch, index_q, z, nullptr, nullptr, seq_len, batch, summ, scale, cm,
                                    max_regions, sel, n_sel, nullptr, index_k, summ, scale, workspace, s);
  if (st != DSA_OK) return st;
  return sparse_gqa_decode(who, geom, batch, q, k_cache, v_cache, cm, seq_len, sel, n_sel, out,
                           (char*)workspace + ws1, workspace_bytes - ws1, stream, f8);
}

extern "C" dsa_status dsa_decode_step(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                      const uint16_t* index_q, const float* z, const uint16_t* index_k,
                                      const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                      const int32_t* seq_len, uint8_t* summ, float* scale,
                                      int32_t max_regions, int32_t* sel, int32_t* n_sel, uint16_t* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_decode_step: tcap must be a positive multiple of 128");
  return decode_step("dsa_decode_step", geom, batch, q, index_q, z, index_k, k_cache, v_cache, contiguous_map(tcap),
                     seq_len, summ, scale, max_regions, sel, n_sel, out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_decode_step_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                            const uint16_t* index_q, const float* z, const dsa_page_table* pages,
                                            const uint16_t* ik_pool, const uint16_t* k_pool, const uint16_t* v_pool,
                                            const int32_t* seq_len, uint8_t* summ_pool, float* scale_pool,
                                            int32_t max_regions, int32_t* sel, int32_t* n_sel, uint16_t* out,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_decode_step_paged", pages, &cm);
  if (st != DSA_OK) return st;
  return decode_step("dsa_decode_step_paged", geom, batch, q, index_q, z, ik_pool, k_pool, v_pool, cm, seq_len,
                     summ_pool, scale_pool, max_regions, sel, n_sel, out, workspace, workspace_bytes, stream);
}

extern "C" dsa_status dsa_decode_step_fp8(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                          const uint16_t* index_q, const float* z, const uint16_t* index_k,
                                          const uint8_t* k8_cache, const uint8_t* v8_cache, const float* kv_scale,
                                          int64_t tcap, const int32_t* seq_len, uint8_t* summ, float* scale,
                                          int32_t max_regions, int32_t* sel, int32_t* n_sel, uint16_t* out,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_decode_step_fp8: tcap must be a positive multiple of 128");
  const Fp8Kv f8{k8_cache, v8_cache, kv_scale};
  return decode_step("dsa_decode_step_fp8", geom, batch, q, index_q, z, index_k, nullptr, nullptr, contiguous_map(tcap),
                     seq_len, summ, scale, max_regions, sel, n_sel, out, workspace, workspace_bytes, stream, &f8);
}

extern "C" dsa_status dsa_decode_step_fp8_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                                const uint16_t* index_q, const float* z, const dsa_page_table* pages,
                                                const uint16_t* ik_pool, const uint8_t* k8_pool, const uint8_t* v8_pool,
                                                const float* kvs_pool, const int32_t* seq_len, uint8_t* summ_pool,
                                                float* scale_pool, int32_t max_regions, int32_t* sel, int32_t* n_sel,
                                                uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  CacheMap cm;
  st = paged_map("dsa_decode_step_fp8_paged", pages, &cm);
  if (st != DSA_OK) return st;
  const Fp8Kv f8{k8_pool, v8_pool, kvs_pool};
  return decode_step("dsa_decode_step_fp8_paged", geom, batch, q, index_q, z, ik_pool, nullptr, nullptr, cm, seq_len,
                     summ_pool, scale_pool, max_regions, sel, n_sel, out, workspace, workspace_bytes, stream, &f8);
}

// ---------------------------------------------------------------------------
// dsa_decode_step without a caller workspace, for callers that cannot
// allocate device memory (code under stream capture, serving loops that
// forbid it).  The workspace is a static device array of fixed size: each
// GPU the library runs on holds its own copy at its own address, found once
// per device with hipGetSymbolAddress and kept; the array's name is never
// used as a device address on the host.  The decode step's workspace holds no
// state that must start at zero: every partial result in it is written
// before it is read.  Calls that overlap on one GPU share
// the array and race.
// ---------------------------------------------------------------------------
namespace dsa {
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the device that runs `stream` (which must be
// the current device); nullptr with the message in *err on failure.
static void* static_scratch(hipStream_t stream, std::string* err) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    *err = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return nullptr;
  }
  hipDevice_t sdev = cur;
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) {
    *err = std::string("hipStreamGetDevice: ") + hipGetErrorString(e);
    return nullptr;
  }
  if ((int)sdev != cur) {
    *err = "the stream belongs to another device than the current one";
    return nullptr;
  }
  if (cur < 0 || cur >= kMaxScratchDevices) {
    *err = "device index beyond the supported range";
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = std::string("hipGetSymbolAddress: ") + hipGetErrorString(e);
      return nullptr;
    }
    g_scratch_ptr[cur] = p;
  }
  return g_scratch_ptr[cur];
}
}  // namespace dsa

extern "C" dsa_status dsa_decode_step_noalloc(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                              const uint16_t* index_q, const float* z, const uint16_t* index_k,
                                              const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                              const int32_t* seq_len, uint8_t* summ, float* scale,
                                              int32_t max_regions, int32_t* sel, int32_t* n_sel, uint16_t* out,
                                              void* stream) {
  dsa_status st = check_geometry(geom);
  if (st != DSA_OK) return st;
  if (tcap <= 0 || tcap % kTcapAlign)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_decode_step_noalloc: tcap must be a positive multiple of 128");
  if (batch < 0 || max_regions < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_decode_step_noalloc: bad sizes");
  if (batch == 0) return DSA_OK;
  const size_t need = dsa_decode_step_workspace_size(geom, batch, max_regions);
  if (need > kStaticScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_decode_step_noalloc: batch and max_regions need " + std::to_string(need) +
                                         " bytes of scratch; the static area holds " +
                                         std::to_string(kStaticScratchBytes) + " (use dsa_decode_step)");
  std::string err;
  void* ws = static_scratch(as_stream(stream), &err);
  if (!ws) return fail(DSA_ERR_HIP, "dsa_decode_step_noalloc: " + err);
  return decode_step("dsa_decode_step_noalloc", geom, batch, q, index_q, z, index_k, k_cache, v_cache,
                     contiguous_map(tcap), seq_len, summ, scale, max_regions, sel, n_sel, out, ws,
                     kStaticScratchBytes, stream);
}
