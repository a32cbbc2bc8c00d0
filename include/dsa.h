/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA sparse-attention library.
 *
 * The layer is the one Step-5-Preview uses in its full-attention layers, as
 * described on these pages (cited by title and section):
 *  [P1] Step-5-Preview long-context explainer (no title in the extract),
 *       kwkr.cn/news/601179, section DSA 稀疏注意力 (four-step list ①-④) and
 *       section 滑窗注意力只读最近 512 个 token.
 *  [P2] "Step-5-Preview 如何实现1M长上下文？滑窗+DSA稀疏注意力混合机制完整揭秘",
 *       yfxerp.com/news/376439: sparse_config table, sections 区域压缩（CSA）,
 *       索引器打分 + Top-K 选择, 512 Token 的环形缓冲区, 给预填充做的小优化.
 *  [P3] "100 万 token 上下文实测：Step 5 Preview 一次能吞下多大的工程",
 *       kwkr.cn/news/593658, section 一 (config table, kernel list).
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *    row-major and contiguous in the layout documented below.  bf16 values are
 *    passed as uint16_t bit patterns, E4M3 (OCP e4m3fn) codes as uint8_t.
 *  - `geom` is HOST memory.  The library is compiled for one geometry:
 *    region 8, proxy 256, 4 KV groups, 16 indexer heads, 64 query heads,
 *    head_dim 192, 1 <= topk <= 512; anything else returns DSA_ERR_UNSUPPORTED.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work and returns; it never synchronises.
 *  - Ownership: the caller allocates and owns every buffer, caches and
 *    workspaces included.  The library allocates no device memory, keeps no
 *    pointer after a call returns, and holds no global device state (the
 *    optional instrumentation below keeps host-side event records only).
 *  - Errors: argument checks run on the host before any launch and return a
 *    status without touching memory; a failed launch returns DSA_ERR_HIP.
 *    dsa_last_error() gives a message for the calling thread's last failure.
 *    Index arrays that live on the device (positions, region lists, ranges)
 *    are the caller's contract; kernels clamp them so that every access stays
 *    inside the buffers described by the host-side sizes, but results for
 *    out-of-contract indices are unspecified.
 *  - Outputs are bitwise reproducible from run to run (no floating-point
 *    atomics on any result path).
 *
 * Cache layouts (per sequence b of a batch, capacity tcap tokens, tcap a
 * multiple of 128; region r = tokens 8r..8r+7; R = tcap/8):
 *   index_k  [B][G][tcap][P]    bf16   indexer keys
 *   K        [B][G][R][1536]    bf16   keys (post-RoPE), region-tiled: key
 *                                      channel d of token 8r+p is element
 *                                      ((((p/4)*6 + (d%48)/8)*4 + d/48)*4
 *                                      + p%4)*8 + d%8 of region r's 1536
 *   V        [B][G][R][D][8]    bf16   values, "region-transposed": the 8
 *                                      tokens of one region are contiguous
 *                                      for each channel
 *   summ     [B][G][R/16][4096] uint8  E4M3 region summaries, tiled: byte j
 *                                      (channel j) of region r of (b, g) is at
 *                                      (r/16)*4096 + (j/64)*1024
 *                                      + ((j%64)/16)*256 + (r%16)*16 + j%16
 *                                      within that (b, g)'s R*256 bytes
 *   scale    [B][G][R]          fp32   per-(region, group) summary scale
 * Sliding-window ring (window W = 512, slot of position t = t mod W):
 *   k_ring   [S][G][W/8][1536]  bf16   region-tiled like K (8-slot regions)
 *   v_ring   [S][G][W/8][D][8]  bf16   region-transposed like V
 *
 * Paged caches ([P3] section 一, kernel list: prefill_sparse_meta and
 * decode_sparse_meta pack the selected tokens over a PagedAttention block
 * table).  A page holds 128 consecutive positions (16 regions, one summary
 * tile) of one sequence for every tensor above, in pools that share the page
 * numbering:
 *   ik_pool    [n_pages][G][128][P]   bf16
 *   k_pool     [n_pages][G][16][1536] bf16   (region-tiled as K)
 *   v_pool     [n_pages][G][16][D][8] bf16   (region-transposed as V)
 *   summ_pool  [n_pages][G][4096]     uint8  (one summary tile)
 *   scale_pool [n_pages][G][16]       fp32
 * Position t of sequence s lives in page block_table[s*max_pages + t/128],
 * at t%128 within it; a sequence's capacity is max_pages*128 positions.
 * Pages may be shared or reused by the caller in any way; page ids are
 * clamped into [0, n_pages), so a bad id reads or writes a wrong page of the
 * pools, never memory outside them.
 *
 * FP8 K/V caches ([P3] section 一: an FP8 KV cache halves it; the per-row
 * rule is the summary stand-in applied to each cached row): every (token,
 * group) row of K and of V is stored as E4M3 codes of x/s with one fp32
 * scale s = amax/448 of the row (fp32 IEEE division, one rounding to nearest
 * even, saturating; s = 0 gives zero codes).  Per region slot (contiguous
 * order [B][G][R] as above):
 *   k8_cache [B][G][R][1536] uint8 region-tiled: the 16-byte unit
 *            ((t*3 + s2)*4 + kb)*4 + p%4 holds token p (t = p/4), channels
 *            48kb + 16s2 .. +15
 *   v8_cache [B][G][R][D][8] uint8 region-transposed
 *   kv_scale [B][G][R][16]   fp32: the K scales of tokens 0..7, then their
 *            V scales
 * In paged form the same per-slot blocks live in pools sharing the page
 * numbering above: k8_pool [n_pages][G][16][1536], v8_pool
 * [n_pages][G][16][D][8] (uint8), kvs_pool [n_pages][G][16][16] (fp32).
 */
#ifndef DSA_MI355X_H
#define DSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4
} dsa_status;

/* Geometry of the layer ([P2] sparse_config table: topk 512, region_block_size
 * 8, proxy_dim 256; [P1] step ③: 16-head indexer; [P3] section 一: 64 query
 * heads in 4 groups; head_dim 192 per [P3]'s KV arithmetic).  softmax_scale
 * is 1/sqrt(head_dim) by default; any finite positive value is accepted. */
typedef struct {
  int32_t region_size; /* 8   */
  int32_t proxy_dim;   /* 256 */
  int32_t n_groups;    /* 4   */
  int32_t n_idx_heads; /* 16  */
  int32_t n_q_heads;   /* 64  */
  int32_t head_dim;    /* 192 */
  int32_t topk;        /* 512 */
  float softmax_scale; /* 1/sqrt(192) */
} dsa_geometry;

/* Block table of paged caches (HOST struct; the table itself is device
 * memory, [n_seqs][max_pages] int32 page ids).  n_pages <= 2^25 and
 * max_pages*128 <= 2^31. */
typedef struct {
  const int32_t* block_table;
  int32_t max_pages; /* pages per sequence (row length of the table) */
  int32_t n_pages;   /* pages in every pool */
} dsa_page_table;

/* Fills the default geometry.  Never fails for a non-NULL pointer. */
dsa_status dsa_geometry_default(dsa_geometry* geom);
/* Static English text for a status code. */
const char* dsa_status_string(int status);
/* Message of the calling thread's last failing call ("" if none). */
const char* dsa_last_error(void);

/*
 * Writes the K/V (and optionally index_k) rows of new tokens into the caches,
 * converting to the cache layouts above (the DSA layer cache keeps the full
 * K/V for exact attention: [P2] section 区域压缩（CSA）, DSALayerCache).
 *   n_tokens        number of new token rows
 *   tok_seq/tok_pos [n_tokens] int32 device: sequence index in [0, n_seqs)
 *                   and absolute position in [0, tcap); rows with either out
 *                   of range are skipped
 *   k_new, v_new    [n_tokens][G][D] bf16; ik_new [n_tokens][G][P] or NULL
 *   k_cache, v_cache, ik_cache (NULL iff ik_new is NULL): caches of n_seqs
 *                   sequences with capacity tcap
 */
dsa_status dsa_cache_write(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                           const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                           const uint16_t* ik_new, uint16_t* k_cache, uint16_t* v_cache,
                           uint16_t* ik_cache, int32_t n_seqs, int64_t tcap, void* stream);

/*
 * dsa_cache_write into paged pools (layouts above): the same rows, written at
 * the page the block table gives for each token's position.  Rows whose
 * sequence is outside [0, n_seqs) or whose position is outside the
 * sequence's capacity (max_pages*128) are skipped.
 */
dsa_status dsa_cache_write_paged(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                                 const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                                 const uint16_t* ik_new, const dsa_page_table* pages, int32_t n_seqs,
                                 uint16_t* k_pool, uint16_t* v_pool, uint16_t* ik_pool, void* stream);

/*
 * dsa_cache_write for FP8 K/V caches: the K and V rows of the new tokens are
 * quantised (rule above; bit-exact) and stored in k8_cache, v8_cache and
 * kv_scale of n_seqs sequences with capacity tcap.  index_k stays bf16
 * (write it with dsa_cache_write).  Rows out of range are skipped.
 */
dsa_status dsa_cache_write_fp8(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                               const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                               uint8_t* k8_cache, uint8_t* v8_cache, float* kv_scale, int32_t n_seqs,
                               int64_t tcap, void* stream);

/* dsa_cache_write_fp8 into paged FP8 pools (page of each position from the
 * block table). */
dsa_status dsa_cache_write_fp8_paged(const dsa_geometry* geom, int32_t n_tokens, const int32_t* tok_seq,
                                     const int32_t* tok_pos, const uint16_t* k_new, const uint16_t* v_new,
                                     const dsa_page_table* pages, int32_t n_seqs, uint8_t* k8_pool,
                                     uint8_t* v8_pool, float* kvs_pool, void* stream);

/*
 * Region compression ([P1] steps ①②; [P2] section 区域压缩（CSA）; [P3] kernel
 * list: csa_compress_regions).  For every sequence b and region r in
 * [region_begin[b], region_end[b]) (clamped to [0, tcap/8) and to at most
 * max_span regions), and every group g: the mean of index_k rows 8r..8r+7 of
 * group g (fp32, summed in token order, times 0.125) is quantised to E4M3
 * with scale = amax/448 (fp32 IEEE division m/scale, round to nearest even,
 * saturating at +-448; scale 0 gives all-zero codes).  The pages do not give
 * the summary maths; this is the stand-in rule.  Only complete regions are
 * summarised: the caller passes region_end <= (tokens written)/8, keeping the
 * partial tail region back until it fills.
 *   batch           number of sequences
 *   index_k         [batch][G][tcap][P] bf16
 *   region_begin/end [batch] int32 device
 *   max_span        host bound on region_end - region_begin (grid size), >= 0
 *   summ, scale     summaries (tiled layout above) and scales of `batch`
 *                   sequences with capacity tcap
 * Output is bit-exact with the stated rule.
 */
dsa_status dsa_compress_regions(const dsa_geometry* geom, int32_t batch, const uint16_t* index_k,
                                int64_t tcap, const int32_t* region_begin,
                                const int32_t* region_end, int32_t max_span, uint8_t* summ,
                                float* scale, void* stream);

/* dsa_compress_regions over paged pools: index_k rows are read from ik_pool
 * and the summaries and scales written to summ_pool and scale_pool, all at
 * the pages of sequence b's block-table row (b < batch).  Bit-exact with the
 * contiguous call on the same data. */
dsa_status dsa_compress_regions_paged(const dsa_geometry* geom, int32_t batch,
                                      const dsa_page_table* pages, const uint16_t* ik_pool,
                                      const int32_t* region_begin, const int32_t* region_end,
                                      int32_t max_span, uint8_t* summ_pool, float* scale_pool,
                                      void* stream);

/* Workspace bytes dsa_score_topk needs for n_queries and max_regions. */
size_t dsa_score_topk_workspace_size(const dsa_geometry* geom, int32_t n_queries,
                                     int32_t max_regions);

/*
 * Indexer scoring + top-k region selection ([P2] section 索引器打分 + Top-K
 * 选择: score_regions, radix-style top-k, prefill/decode_metadata, current
 * region always kept; [P3] kernel list: indexer_logits_radix_topk_threshold).
 * For query i at position p = q_pos[i] of sequence q_seq[i], current region
 * c = p/8, and each group g:
 *   score(r) = sum_{h=4g..4g+3} z[i][h] * ReLU(index_q[i][h] . S_g[r]),
 *   S_g[r] = E4M3 value of summ[...][g][r][:] * scale[...][g][r],
 * for the complete regions r < c (stand-in maths; the pages give none).  The
 * selection is region c plus the min(topk-1, c) best of 0..c-1 ranked by
 * score descending, lower index first on ties; it is written ascending.
 *   index_q   [n_queries][16][P] bf16;  z [n_queries][16] fp32
 *   q_seq, q_pos [n_queries] int32 device; q_seq in [0, n_seqs)
 *   summ, scale  summaries of n_seqs sequences with capacity tcap (layout above)
 *   max_regions  host bound: p/8 <= max_regions for every query (grid,
 *             workspace; the candidates r < p/8 must have r < max_regions)
 *   sel       [n_queries][G][topk] int32, ascending region ids, -1 padded
 *   n_sel     [n_queries][G] int32 = min(topk, c+1)
 *   scores_out NULL or [n_queries][G][max_regions] fp32: score(r) for r < c
 *             (entries r >= c are left untouched)
 *   workspace device buffer of at least dsa_score_topk_workspace_size() bytes
 * Scores are fp32 (bf16 x E4M3 products, fp32 accumulation); on equal fp32
 * scores the lower index wins; a NaN score ranks below every number.
 * The workspace holds the fp32 scores and, when max_regions > 8192, the
 * largest score of every 16-region tile.  Every byte of it is written before
 * it is read, so results never depend on its contents on entry.  Calls
 * sharing a workspace must not overlap.
 */
dsa_status dsa_score_topk(const dsa_geometry* geom, int32_t n_queries, const uint16_t* index_q,
                          const float* z, const int32_t* q_seq, const int32_t* q_pos,
                          int32_t n_seqs, const uint8_t* summ, const float* scale, int64_t tcap,
                          int32_t max_regions, int32_t* sel, int32_t* n_sel, float* scores_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* dsa_score_topk over paged summaries: the summary tiles and scales of query
 * i's sequence are read from summ_pool/scale_pool at the pages of its
 * block-table row.  Bit-identical to the contiguous call on the same data
 * (same workspace rules). */
dsa_status dsa_score_topk_paged(const dsa_geometry* geom, int32_t n_queries, const uint16_t* index_q,
                                const float* z, const int32_t* q_seq, const int32_t* q_pos,
                                int32_t n_seqs, const dsa_page_table* pages, const uint8_t* summ_pool,
                                const float* scale_pool, int32_t max_regions, int32_t* sel,
                                int32_t* n_sel, float* scores_out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Workspace bytes dsa_sparse_gqa_decode needs for `batch` queries. */
size_t dsa_sparse_gqa_workspace_size(const dsa_geometry* geom, int32_t batch);

/*
 * Sparse GQA decode ([P1] step ④; [P3] kernel list: sparse_attention_decode;
 * attention_impl sparse_gqa in [P2]'s sparse_config table).  Query b sits at
 * position p = seq_len[b]-1 of sequence b.  Head h (group g = h/16) attends
 * to the tokens 8r..min(8r+7, p) of every region r in sel[b][g][0..n_sel):
 *   out[b][h] = sum_j softmax_j(softmax_scale * q[b][h] . K_j) V_j
 * (fp32 softmax and accumulation, bf16 MFMA products, bf16 output).  Region
 * ids outside [0, p/8] are ignored.
 *   q   [batch][64][D] bf16 (post-RoPE);  out [batch][64][D] bf16
 *   k_cache, v_cache: caches of `batch` sequences with capacity tcap
 *   seq_len [batch] int32 device (1 <= seq_len <= tcap)
 *   sel, n_sel as produced by dsa_score_topk
 */
dsa_status dsa_sparse_gqa_decode(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                 const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                 const int32_t* seq_len, const int32_t* sel, const int32_t* n_sel,
                                 uint16_t* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* dsa_sparse_gqa_decode over paged K/V pools (sequence b's block-table row,
 * capacity max_pages*128).  Bit-identical to the contiguous call on the same
 * data. */
dsa_status dsa_sparse_gqa_decode_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                       const dsa_page_table* pages, const uint16_t* k_pool,
                                       const uint16_t* v_pool, const int32_t* seq_len,
                                       const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* dsa_sparse_gqa_decode over FP8 K/V caches: each K and V value is the E4M3
 * value of its code times its row's scale; the codes enter bf16 MFMAs
 * exactly, K scales multiply the scores and V scales the softmax weights
 * (fp32), weights rounded to bf16 for P.V.  Same workspace. */
dsa_status dsa_sparse_gqa_decode_fp8(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                     const uint8_t* k8_cache, const uint8_t* v8_cache,
                                     const float* kv_scale, int64_t tcap, const int32_t* seq_len,
                                     const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* dsa_sparse_gqa_decode_fp8 over paged FP8 pools; bit-identical to the
 * contiguous call on the same data. */
dsa_status dsa_sparse_gqa_decode_fp8_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                           const dsa_page_table* pages, const uint8_t* k8_pool,
                                           const uint8_t* v8_pool, const float* kvs_pool,
                                           const int32_t* seq_len, const int32_t* sel,
                                           const int32_t* n_sel, uint16_t* out, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Workspace bytes dsa_decode_step needs. */
size_t dsa_decode_step_workspace_size(const dsa_geometry* geom, int32_t batch, int32_t max_regions);

/*
 * One decode step of the DSA layer for `batch` sequences, one query token per
 * sequence ([P1] steps ①-④ in order; [P3] kernel list): the region the
 * query token completes is compressed, every earlier complete region is
 * scored, the top-k plus the current region are selected, and sparse GQA runs
 * over them.  Results are identical to dsa_compress_regions (of region
 * seq_len/8 - 1 when seq_len is a multiple of 8) + dsa_score_topk (q_seq = b,
 * q_pos = seq_len[b] - 1) + dsa_sparse_gqa_decode; the compression is folded
 * into the scoring launch (its region is never scored in the same step).
 *   q [batch][64][D], index_q [batch][16][P] bf16; z [batch][16] fp32
 *   index_k, k_cache, v_cache, summ, scale: caches of `batch` sequences with
 *             capacity tcap (layouts above); summaries of all complete regions
 *             before the query's region must be present
 *   seq_len   [batch] int32 device, 1 <= seq_len <= tcap, including the token
 *   max_regions host bound: seq_len/8 <= max_regions (grid, workspace); a
 *             query in a partial region (seq_len not a multiple of 8) has
 *             current region seq_len/8 and candidates below it, so this bound
 *             covers it
 *   sel, n_sel, out as for dsa_score_topk and dsa_sparse_gqa_decode
 *   workspace >= dsa_decode_step_workspace_size() bytes, 256-byte aligned;
 *             the same contents rules as dsa_score_topk's workspace apply
 */
dsa_status dsa_decode_step(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                           const uint16_t* index_q, const float* z, const uint16_t* index_k,
                           const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                           const int32_t* seq_len, uint8_t* summ, float* scale, int32_t max_regions,
                           int32_t* sel, int32_t* n_sel, uint16_t* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * dsa_decode_step for callers that cannot allocate device memory (code under
 * HIP graph / stream capture, serving loops or harnesses that forbid
 * hipMalloc): the same arguments without the workspace, and results
 * bit-identical to dsa_decode_step.  Its workspace is a static 64 MiB device
 * area of the library; each GPU holds its own copy until the process ends.
 * Shapes whose dsa_decode_step_workspace_size() exceeds 64 MiB (e.g. batch 4
 * at 1M tokens needs 14.6 MiB, batch 16 at 128K 28.8 MiB) return
 * DSA_ERR_UNSUPPORTED.  `stream` must belong to the current device; the
 * first call on a device resolves the area's address there (make it outside
 * stream capture).  The call allocates and frees nothing.  Every call on one
 * GPU shares that GPU's area, so calls that overlap on one GPU race: issue
 * them on one stream or order them.
 */
dsa_status dsa_decode_step_noalloc(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                   const uint16_t* index_q, const float* z, const uint16_t* index_k,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                   const int32_t* seq_len, uint8_t* summ, float* scale, int32_t max_regions,
                                   int32_t* sel, int32_t* n_sel, uint16_t* out, void* stream);

/* dsa_decode_step over paged pools (sequence b = block-table row b): the
 * folded compression reads ik_pool and writes summ_pool/scale_pool; scoring
 * and attention read the pools.  Bit-identical to the contiguous call on the
 * same data. */
dsa_status dsa_decode_step_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                 const uint16_t* index_q, const float* z, const dsa_page_table* pages,
                                 const uint16_t* ik_pool, const uint16_t* k_pool,
                                 const uint16_t* v_pool, const int32_t* seq_len, uint8_t* summ_pool,
                                 float* scale_pool, int32_t max_regions, int32_t* sel, int32_t* n_sel,
                                 uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* dsa_decode_step with FP8 K/V caches (index_k, summaries and scales as in
 * dsa_decode_step); the attention is dsa_sparse_gqa_decode_fp8's. */
dsa_status dsa_decode_step_fp8(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                               const uint16_t* index_q, const float* z, const uint16_t* index_k,
                               const uint8_t* k8_cache, const uint8_t* v8_cache, const float* kv_scale,
                               int64_t tcap, const int32_t* seq_len, uint8_t* summ, float* scale,
                               int32_t max_regions, int32_t* sel, int32_t* n_sel, uint16_t* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* dsa_decode_step_fp8 over paged pools (index_k, summaries and scales as in
 * dsa_decode_step_paged, K/V in FP8 pools). */
dsa_status dsa_decode_step_fp8_paged(const dsa_geometry* geom, int32_t batch, const uint16_t* q,
                                     const uint16_t* index_q, const float* z, const dsa_page_table* pages,
                                     const uint16_t* ik_pool, const uint8_t* k8_pool,
                                     const uint8_t* v8_pool, const float* kvs_pool,
                                     const int32_t* seq_len, uint8_t* summ_pool, float* scale_pool,
                                     int32_t max_regions, int32_t* sel, int32_t* n_sel, uint16_t* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dsa_sparse_gqa_prefill needs for n_queries queries. */
size_t dsa_sparse_gqa_prefill_workspace_size(const dsa_geometry* geom, int32_t n_queries);

/*
 * Sparse GQA for a chunk of prefill queries ([P3] kernel list:
 * sparse_attention_prefill).  Same maths as decode, per query i of sequence
 * q_seq[i] at position q_pos[i] (the current region may be partial; tokens
 * after p are masked).  The chunk's own K/V must already be in the caches.
 * The list entries need not be sorted; a list is a set (a repeated id counts
 * once), and ids outside [0, p/8] are ignored.
 *   q, out [n_queries][64][D] bf16;  caches of n_seqs sequences, capacity tcap
 *   workspace >= dsa_sparse_gqa_prefill_workspace_size() bytes, 256-byte
 *             aligned: per-(query, group) partial results over 8 ranges of
 *             regions, merged into out by the same call
 */
dsa_status dsa_sparse_gqa_prefill(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                  const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                  const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                  const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* dsa_sparse_gqa_prefill over paged K/V pools (query i reads its sequence's
 * block-table row).  Bit-identical to the contiguous call on the same data. */
dsa_status dsa_sparse_gqa_prefill_paged(const dsa_geometry* geom, int32_t n_queries,
                                        const uint16_t* q, const int32_t* q_seq, const int32_t* q_pos,
                                        int32_t n_seqs, const dsa_page_table* pages,
                                        const uint16_t* k_pool, const uint16_t* v_pool,
                                        const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Neighbour-merged prefill ([P5], Sparse GQA paragraph: similar selections of
 * neighbouring tokens are merged to use the GPU better).  Same arguments,
 * workspace and result as dsa_sparse_gqa_prefill, computed differently:
 * every 2 consecutive queries of the call walk the union of their
 * selections once per KV group, each region's K/V read once and applied to
 * the queries that selected it, so a chunk whose neighbouring queries
 * select overlapping regions gathers less.  Each query still attends
 * exactly its own selection (here a list is a set: repeated ids count
 * once).  Neighbours of different sequences are allowed (one pass per
 * sequence).  Pays off when neighbouring selections overlap; with
 * unrelated selections the per-query call is faster.
 */
dsa_status dsa_sparse_gqa_prefill_merged(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                         const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                         const uint16_t* k_cache, const uint16_t* v_cache, int64_t tcap,
                                         const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* dsa_sparse_gqa_prefill_merged over paged K/V pools; bit-identical to the
 * contiguous merged call on the same data. */
dsa_status dsa_sparse_gqa_prefill_merged_paged(const dsa_geometry* geom, int32_t n_queries,
                                               const uint16_t* q, const int32_t* q_seq,
                                               const int32_t* q_pos, int32_t n_seqs,
                                               const dsa_page_table* pages, const uint16_t* k_pool,
                                               const uint16_t* v_pool, const int32_t* sel,
                                               const int32_t* n_sel, uint16_t* out, void* workspace,
                                               size_t workspace_bytes, void* stream);

/* dsa_sparse_gqa_prefill over FP8 K/V caches (maths as in
 * dsa_sparse_gqa_decode_fp8). */
dsa_status dsa_sparse_gqa_prefill_fp8(const dsa_geometry* geom, int32_t n_queries, const uint16_t* q,
                                      const int32_t* q_seq, const int32_t* q_pos, int32_t n_seqs,
                                      const uint8_t* k8_cache, const uint8_t* v8_cache,
                                      const float* kv_scale, int64_t tcap, const int32_t* sel,
                                      const int32_t* n_sel, uint16_t* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* dsa_sparse_gqa_prefill_fp8 over paged FP8 pools; bit-identical to the
 * contiguous call on the same data. */
dsa_status dsa_sparse_gqa_prefill_fp8_paged(const dsa_geometry* geom, int32_t n_queries,
                                            const uint16_t* q, const int32_t* q_seq,
                                            const int32_t* q_pos, int32_t n_seqs,
                                            const dsa_page_table* pages, const uint8_t* k8_pool,
                                            const uint8_t* v8_pool, const float* kvs_pool,
                                            const int32_t* sel, const int32_t* n_sel, uint16_t* out,
                                            void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes swa_attention needs. */
size_t swa_attention_workspace_size(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                                    int32_t max_new_per_seq);

/*
 * Sliding-window attention of the other layers ([P1] section 滑窗注意力只读最近
 * 512 个 token; [P2] sections 512 Token 的环形缓冲区 and 给预填充做的小优化):
 * the query at position p attends to positions max(0, p-W+1)..p.  Decode is
 * the case of one new token per sequence; chunked prefill passes a chunk of
 * new tokens (any length: the band mask is applied per query, so the result
 * does not depend on how a prompt is cut into chunks).
 *   window           512 (the only supported value)
 *   n_seqs           sequences in this call; sequence s has new tokens at
 *                    positions seq_pos0[s] .. seq_pos0[s]+n_s-1 stored in rows
 *                    seq_row0[s] .. seq_row0[s+1]-1 (n_s = the difference)
 *   max_new_per_seq  host bound on n_s (grid, workspace)
 *   seq_pos0 [n_seqs], seq_row0 [n_seqs+1] int32 device
 *   q [rows][64][D], k_new/v_new [rows][G][D] bf16, out [rows][64][D] bf16,
 *                    rows <= n_seqs*max_new_per_seq (kernels clamp row indices
 *                    to that bound, so the arrays must hold that many rows)
 *   k_ring, v_ring   the ring of each sequence BEFORE this call's tokens are
 *                    appended: it holds positions seq_pos0[s]-W .. seq_pos0[s]-1
 *                    (those >= 0) in slots t mod W
 *   workspace        >= swa_attention_workspace_size() bytes
 * Call swa_ring_append afterwards to advance the rings.
 */
dsa_status swa_attention(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                         int32_t max_new_per_seq, const int32_t* seq_pos0,
                         const int32_t* seq_row0, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, const uint16_t* k_ring, const uint16_t* v_ring,
                         uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ring-buffer append ([P2] section 512 Token 的环形缓冲区: DenseLayerCache.write
 * puts each token in slot position mod window): writes the last min(n_s, W)
 * new rows of every sequence into slots t mod W of k_ring/v_ring.  Arguments
 * as for swa_attention.
 */
dsa_status swa_ring_append(const dsa_geometry* geom, int32_t window, int32_t n_seqs,
                           int32_t max_new_per_seq, const int32_t* seq_pos0,
                           const int32_t* seq_row0, const uint16_t* k_new, const uint16_t* v_new,
                           uint16_t* k_ring, uint16_t* v_ring, void* stream);

/*
 * One decode step of a sliding-window layer ([P1] section 滑窗注意力只读最近
 * 512 个 token; [P2] section 512 Token 的环形缓冲区: attention over the last W
 * positions, the new token written at slot position mod W): sequence s has one
 * new token at position p = seq_pos[s], in row s of q, k_new and v_new; it
 * attends to positions max(0, p-W+1)..p, and its K/V are then written into
 * ring slot p mod W.  The output equals swa_attention with one new token per
 * sequence (seq_row0 = 0, 1, .., n_seqs) and the rings equal a following
 * swa_ring_append.  One launch, no workspace: the window is exactly the
 * ring's 64 region slots (the slot shared by the window's first and current
 * regions holds the first region's tokens above offset p mod 8 and the
 * current region's up to it), each (sequence, group) is served by 6 blocks
 * owning 32 output channels each, and one of them writes the token into
 * ring slot p mod W, which held position p - W (no value this step reads).
 *   window   512
 *   seq_pos  [n_seqs] int32 device (>= 0)
 *   q, out   [n_seqs][64][D] bf16;  k_new, v_new [n_seqs][G][D] bf16
 *   k_ring, v_ring  rings holding positions p-W .. p-1 (those >= 0), layouts as
 *            for swa_attention; updated in place.  Calls updating one ring
 *            must not overlap.
 */
dsa_status swa_decode_step(const dsa_geometry* geom, int32_t window, int32_t n_seqs, const int32_t* seq_pos,
                           const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_ring,
                           uint16_t* v_ring, uint16_t* out, void* stream);

/*
 * Indexer front-end ([P2] section 索引器打分 + Top-K 选择: the indexer projects
 * the hidden state into index_q / index_k / index_z, then normalises them and
 * rotates part of their dimensions; [P1] paragraph after step ④ and [P3]
 * section 一: llama3-style rope_scaling with low_freq_factor 1.0,
 * high_freq_factor 32.0, original_max_position_embeddings 1048576, partial
 * rotary factor 1/3, i.e. 64 of the 192 head dimensions rotate).
 *
 * Rotation: pair (i, i + 32) of the first 64 dimensions of a vector turns by
 * pos * f_i, f_i = llama3(theta^(-2i/64)): frequencies whose wavelength
 * 2*pi/f is below original_max_pos / high_freq_factor stay, those above
 * original_max_pos / low_freq_factor are divided by `factor`, and in between
 * f moves linearly in original_max_pos / wavelength from f/factor to f.
 * theta and factor are not on the pages: dsa_rope_config_default fills
 * theta 10000 and factor 8 beside the pages' values.  rot_dims must be 64.
 */
typedef struct dsa_rope_config {
  int32_t rot_dims;
  float theta;
  float factor;
  float low_freq_factor;
  float high_freq_factor;
  int32_t original_max_pos;
} dsa_rope_config;

dsa_status dsa_rope_config_default(dsa_rope_config* rope);

/* Workspace bytes of dsa_indexer_project (hidden size `hidden`) and of
 * dsa_rope_qk (hidden 0) for n_tokens tokens: a cos/sin table of 32 pairs
 * per token, plus the fp32 projection (n_tokens x 5136; for up to 64 tokens
 * one such block per split of the hidden dimension, hidden/256 or
 * hidden/128 splits). */
size_t dsa_indexer_workspace_size(int32_t n_tokens, int32_t hidden);

/*
 * Hidden states -> the indexer's inputs: y = x . W^T (bf16 MFMA, fp32
 * accumulation); each 256-d index vector is RMS-normalised (eps 1e-6, gain
 * gamma_q for the 16 query heads, gamma_k for the 4 key groups) and its
 * first 64 dimensions rotated by the token's position; z is the plain
 * projection (fp32).
 *   x        [n_tokens][hidden] bf16, 16-byte aligned; hidden a multiple of 128
 *   w        [16*256 + 4*256 + 16][hidden] bf16 (rows: index_q heads,
 *            index_k groups, z heads), 16-byte aligned
 *   gamma_q, gamma_k  [256] fp32;  pos [n_tokens] int32 (>= 0)
 *   index_q  [n_tokens][16][256] bf16;  index_k [n_tokens][4][256] bf16
 *            (the layouts dsa_score_topk and dsa_cache_write read)
 *   z        [n_tokens][16] fp32
 *   workspace >= dsa_indexer_workspace_size(n_tokens), 256-byte aligned
 */
dsa_status dsa_indexer_project(const dsa_rope_config* rope, int32_t n_tokens, int32_t hidden,
                               const uint16_t* x, const uint16_t* w, const float* gamma_q,
                               const float* gamma_k, const int32_t* pos, uint16_t* index_q,
                               uint16_t* index_k, float* z, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The same rotation applied in place to the attention's projected q
 * [n_tokens][64][192] and k [n_tokens][4][192] (bf16, token-major): the first
 * 64 dimensions of every head turn by the token's position (the full-attention
 * layers' partial RoPE).  Workspace as for dsa_indexer_project.
 */
dsa_status dsa_rope_qk(const dsa_rope_config* rope, int32_t n_tokens, const int32_t* pos, uint16_t* q,
                       uint16_t* k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Instrumentation (not part of the layer's maths).  While enabled, every
 * kernel the library launches outside stream capture is bracketed by two
 * hipEvents recorded on its launch stream.  dsa_profile_enable(on) drops
 * earlier records (waiting for them) and switches recording on or off;
 * dsa_profile_kernel_stats waits for the recorded events of one kernel and
 * returns the summed interval (ms) and the number of launches.  Kernel
 * names: k_compress, k_cache_write, k_score_decode,
 * k_score_prefill, k_select, k_sgqa_decode, k_sgqa_merge, k_sgqa_prefill,
 * k_swa_stage, k_swa_band (chunks of 16 or more tokens), k_swa_attend (shorter
 * ones), k_swa_decode (swa_decode_step), k_ring_append,
 * k_sgqa_prefill_merged, k_rope_table,
 * k_indexer_proj, k_indexer_finish, k_rope_qk.  Host-side state only, guarded
 * by a mutex; at most 8192 launches are recorded between resets.
 */
dsa_status dsa_profile_enable(int on);
dsa_status dsa_profile_kernel_stats(const char* kernel, double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* DSA_MI355X_H */
