// Indexer front-end and the partial rotary embedding of the attention's Q/K.
//
// [P2] yfxerp.com/news/376439, section 索引器打分 + Top-K 选择: the indexer
// projects the hidden state into index_q / index_k / index_z, normalises them
// and rotates part of their dimensions (RoPE); same page, closing paragraph,
// and [P1] kwkr.cn/news/601179 (paragraph after step ④): llama3-style
// rope_scaling (low_freq_factor 1.0, high_freq_factor 32.0) on the
// full-attention layers, partial rotary factor 1/3; [P3] kwkr.cn/news/593658,
// section 一: original_max_position_embeddings 1048576, about 64 of the 192
// head dimensions rotate.
//
// The projection is one GEMM, y = x . W^T in fp32, W holding the 4096
// index_q, 1024 index_k and 16 z rows: for many tokens k_indexer_gemm
// (128 x 128 tiles through LDS, XCD-aware tile order), for up to 64 tokens
// (decode) k_indexer_proj_splitk (split over the hidden dimension, so the
// weights stream once over the whole GPU).  k_indexer_finish then sums the
// partials of each token, RMS-normalises each 256-d vector, applies the
// gain, rotates dimensions 0..63 (rotate-half) and rounds to bf16; z is
// the plain sum.  k_rope_qk rotates the attention's q [T][64][192] and
// k [T][4][192] in place.  Angles are pos * freq in double, reduced to
// [-pi, pi] before sincos, so positions up to 2^31 keep full fp32 accuracy.
#include <math.h>

#include "common.hpp"

namespace dsa {

constexpr int kRotDims = 64;               // rotated dimensions of every vector
constexpr int kRotPairs = kRotDims / 2;    // pairs (i, i + 32)
constexpr int kVecs = kIdxHeads + kGroups;  // 20 normalised 256-d outputs per token
constexpr int kProjN = kVecs * kProxy + kIdxHeads;  // 5136 weight rows
constexpr float kNormEps = 1e-6f;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct RopeFreqs {
  double f[kRotPairs];
};

// (cos, sin) of the angle pos * f: the product in double, reduced to
// [-pi, pi] before sincos.
__device__ __forceinline__ float2 rope_cs(int32_t pos, double f) {
  const double a = (double)pos * f;
  const double two_pi = 6.283185307179586476925286766559;
  const double r = a - two_pi * rint(a / two_pi);
  double s, c;
  sincos(r, &s, &c);
  return make_float2((float)c, (float)s);
}

// cos/sin of pair i at the token's position; one block of 64 threads per
// 2 tokens.
__global__ __launch_bounds__(64) void k_rope_table(const int32_t* __restrict__ pos, int32_t n, RopeFreqs fr,
                                                   float2* __restrict__ cs) {
  const int64_t t = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 5);
  const int i = threadIdx.x & 31;
  if (t >= n) return;
  cs[t * kRotPairs + i] = rope_cs(pos[t], fr.f[i]);
}

// Few tokens (decode): the weights are the cost (5136 x hidden bf16), and
// 20 blocks of the tiled kernel would leave most CUs idle.  Split-K instead:
// wave = (64 output columns, one k range), all (<= 64) tokens as row tiles,
// fp32 partials to the workspace; k_indexer_finish sums them in split order
// and applies the epilogue.  Column group 80 holds the 16 z columns.
constexpr int kSmallT = 64;                 // token counts up to this take the split-K path
constexpr int kColGroups = kVecs * 4 + 1;   // 81 groups of 64 columns

__global__ __launch_bounds__(64) void k_indexer_proj_splitk(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w,
                                                            float* __restrict__ part, int32_t T, int32_t H,
                                                            int32_t kper) {
  const int lane = threadIdx.x, n = lane & 15, kb = lane >> 4;
  const int cg = blockIdx.x, sp = blockIdx.y;
  const int64_t k0 = (int64_t)sp * kper + 8 * kb;
  const int nrt = (T + 15) / 16;
  const uint16_t* xr[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int t = 16 * rt + n < T ? 16 * rt + n : T - 1;
    xr[rt] = x + (int64_t)t * H + k0;
  }
  const uint16_t* wr[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int col = 64 * cg + 16 * ct + n;
    wr[ct] = w + (int64_t)(col < kProjN ? col : kProjN - 1) * H + k0;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k = 0; k < kper; k += 32) {
    u32x4 b[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) b[ct] = ld16(wr[ct] + k);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt >= nrt) break;
      const bf16x8 af = as_bf16x8(ld16(xr[rt] + k));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = mfma16x16x32(af, as_bf16x8(b[ct]), acc[rt][ct]);
    }
  }
  // D[row 4kb + i][column n] of each tile
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * rt + 4 * kb + i, col = 64 * cg + 16 * ct + n;
        if (t < T && col < kProjN) part[((int64_t)sp * T + t) * kProjN + col] = acc[rt][ct][i];
      }
}

// block (t, b) = token t; wave w of it takes vectors 4b + w, 4b + w + 4B,
// ... (B = gridDim.y: 5 for few tokens, which spreads the split sums over
// more CUs, 1 for many).  Lane owns columns lane + 64k, k = 0..3: sum of the
// split partials in split order, RMS by wave reduction, gain, rotation of
// columns 0..63 (the partner of column c < 32 is lane c + 32 of the same
// slot), bf16 store; block (t, 0) also sums the z columns.  No barrier.
__global__ __launch_bounds__(256) void k_indexer_finish(const float* __restrict__ part, int32_t ks,
                                                        const float* __restrict__ gq, const float* __restrict__ gk,
                                                        const int32_t* __restrict__ pos, RopeFreqs fr,
                                                        uint16_t* __restrict__ iq, uint16_t* __restrict__ ik,
                                                        float* __restrict__ z, int32_t T) {
  const int64_t t = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pstride = (int64_t)T * kProjN;
  const float* pt = part + t * kProjN;
  if (blockIdx.y == 0 && wave == 0 && lane < kIdxHeads) {
    float acc = 0.f;
    for (int sp = 0; sp < ks; ++sp) acc += pt[sp * pstride + kVecs * kProxy + lane];
    z[t * kIdxHeads + lane] = acc;
  }
  const float2 cc = rope_cs(pos[t], fr.f[lane & (kRotPairs - 1)]);
  for (int h = 4 * blockIdx.y + wave; h < kVecs; h += 4 * gridDim.y) {
    float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int sp = 0; sp < ks; ++sp) {
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] += pt[sp * pstride + h * kProxy + 64 * k + lane];
    }
    float ss = (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kProxy) + kNormEps);
    const float* g = h < kIdxHeads ? gq : gk;
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] *= inv * g[64 * k + lane];
    const float other = __shfl_xor(y[0], kRotPairs);  // column lane ^ 32 of slot 0
    y[0] = lane < kRotPairs ? y[0] * cc.x - other * cc.y : y[0] * cc.x + other * cc.y;
    uint16_t* o = h < kIdxHeads ? iq + (t * kIdxHeads + h) * kProxy : ik + (t * kGroups + h - kIdxHeads) * kProxy;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[64 * k + lane] = (uint16_t)(pack_bf16x2(y[k], 0.f) & 0xffffu);
  }
}

static int32_t splitk_kper(int32_t hidden) { return hidden % 256 == 0 ? 256 : 128; }

// Many tokens: y[T][5136] = x . W^T in fp32 (the finishing kernel then
// normalises, rotates and converts).  Block = 128 tokens x 128 weight rows,
// both tiles staged through LDS (double buffered, padded rows) and shared:
// wave (wm, wn) computes rows 64wm.. x columns 64wn.. as 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, so each 16-byte fragment read from LDS feeds 2
// MFMAs of 32K flops.  Two blocks fit a CU (72 KB of LDS, 186 VGPRs).
constexpr int kGM = 128, kGN = 128, kGK = 64, kGPitch = kGK + 8;

// Tile order: consecutive blocks go to the 8 XCDs in turn, so block b runs
// on XCD b % 8; XCD x takes the x-th eighth of the tiles, ordered column
// tile by column tile, so the blocks one XCD runs together share a few
// weight tiles and every token tile through its own L2.
__global__ __launch_bounds__(256, 2) void k_indexer_gemm(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, float* __restrict__ y,
                                                         int32_t T, int32_t H) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int nrow = (T + kGM - 1) / kGM;
  const int ntile = nrow * ((kProjN + kGN - 1) / kGN);
  const int per_xcd = (ntile + 7) / 8;
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= ntile) return;
  const int64_t c0 = (int64_t)(tile / nrow) * kGN, t0 = (int64_t)(tile % nrow) * kGM;
  __shared__ __attribute__((aligned(16))) uint16_t as[2][kGM * kGPitch];
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][kGN * kGPitch];
  // tile copies: thread t moves rows t/8 + 32r (r = 0..3) of each tile, 8 elements at (t%8)*8
  const int lr = threadIdx.x >> 3, lk = (threadIdx.x & 7) * 8;
  const uint16_t* ar[4];
  const uint16_t* br[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = t0 + lr + 32 * r, c = c0 + lr + 32 * r;
    ar[r] = x + (t < T ? t : T - 1) * H + lk;             // rows past the end: re-reads, never stored
    br[r] = w + (c < kProjN ? c : kProjN - 1) * H + lk;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // two stages of tile copies in flight: the registers of stage st + 2 are
  // requested while stage st computes from LDS (stage st + 1 already sits in
  // the other LDS buffer), which covers the memory latency at 2 blocks per CU
  const int nst = H / kGK;
  u32x4 ra[2][4], rb[2][4];
  auto fetch = [&](u32x4 (&a)[4], u32x4 (&b)[4], int stage) {
    const int64_t k = (int64_t)(stage < nst ? stage : nst - 1) * kGK;  // past the end: a re-read, unused
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = ld16(ar[r] + k);
      b[r] = ld16(br[r] + k);
    }
  };
  auto stash = [&](const u32x4 (&a)[4], const u32x4 (&b)[4], int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *(u32x4*)&as[buf][(lr + 32 * r) * kGPitch + lk] = a[r];
      *(u32x4*)&bs[buf][(lr + 32 * r) * kGPitch + lk] = b[r];
    }
  };
  auto compute = [&](int buf) {
    // v_mfma_f32_32x32x16_bf16: lane l holds row l % 32, k 8(l / 32) .. +7 of
    // A (and column l % 32 of B); half the fragment reads per flop of 16x16x32
    const int r32 = lane & 31, k8 = 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = as_bf16x8(*(const u32x4*)&as[buf][(64 * wm + 32 * i + r32) * kGPitch + 16 * ks + k8]);
        bf[i] = as_bf16x8(*(const u32x4*)&bs[buf][(64 * wn + 32 * i + r32) * kGPitch + 16 * ks + k8]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  fetch(ra[0], rb[0], 0);
  fetch(ra[1], rb[1], 1);
  stash(ra[0], rb[0], 0);
  fetch(ra[0], rb[0], 2);
  __syncthreads();
  // nst is even (H is a multiple of 128): stages go in pairs with static register sets
  for (int st = 0; st < nst; st += 2) {
    compute(0);
    stash(ra[1], rb[1], 1);  // stage st + 1
    fetch(ra[1], rb[1], st + 3);
    __syncthreads();
    compute(1);
    stash(ra[0], rb[0], 0);  // stage st + 2
    fetch(ra[0], rb[0], st + 4);
    __syncthreads();
  }
  // 32 x 32 tile (i, j): element e of lane l is row 8(e/4) + 4(l/32) + e%4, column l % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t c = c0 + 64 * wn + 32 * j + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = t0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (t < T && c < kProjN) y[t * kProjN + c] = acc[i][j][e];
      }
    }
}

// In-place rotation of the first 64 dimensions of every head of q and k:
// block = one token; its 32 (cos, sin) pairs come from the table.
__global__ __launch_bounds__(256) void k_rope_qk(const float2* __restrict__ cs, uint16_t* __restrict__ q,
                                                 uint16_t* __restrict__ k, int32_t T) {
  const int64_t t = blockIdx.x;
  // 68 heads x 32 pairs; thread handles pairs p = threadIdx.x + 256 j
  for (int p = threadIdx.x; p < (kQHeads + kGroups) * kRotPairs; p += 256) {
    const int hd = p / kRotPairs, i = p % kRotPairs;
    uint16_t* v = hd < kQHeads ? q + (t * kQHeads + hd) * kHeadDim : k + (t * kGroups + hd - kQHeads) * kHeadDim;
    const float2 c = cs[t * kRotPairs + i];
    const float a = bf16_to_f32(v[i]), b = bf16_to_f32(v[i + kRotPairs]);
    v[i] = (uint16_t)(pack_bf16x2(a * c.x - b * c.y, 0.f) & 0xffffu);
    v[i + kRotPairs] = (uint16_t)(pack_bf16x2(b * c.x + a * c.y, 0.f) & 0xffffu);
  }
}

// llama3 scaling of base frequency theta^(-2i/64): wavelengths below
// orig/high keep their frequency, above orig/low are slowed by `factor`,
// and in between the frequency moves linearly in orig/wavelength.
static RopeFreqs rope_freqs(const dsa_rope_config& c) {
  RopeFreqs r;
  const double pi = 3.14159265358979323846;
  for (int i = 0; i < kRotPairs; ++i) {
    const double f = pow((double)c.theta, -2.0 * i / kRotDims);
    const double wl = 2.0 * pi / f;
    const double hi_wl = c.original_max_pos / (double)c.high_freq_factor;
    const double lo_wl = c.original_max_pos / (double)c.low_freq_factor;
    double g;
    if (wl < hi_wl) g = f;
    else if (wl > lo_wl) g = f / c.factor;
    else {
      const double s = (c.original_max_pos / wl - c.low_freq_factor) / ((double)c.high_freq_factor - c.low_freq_factor);
      g = (1.0 - s) * f / c.factor + s * f;
    }
    r.f[i] = g;
  }
  return r;
}

static dsa_status check_rope(const char* who, const dsa_rope_config* c) {
  if (!c) return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": NULL rope config");
  if (c->rot_dims != kRotDims)
    return fail(DSA_ERR_UNSUPPORTED, std::string(who) + ": rot_dims must be 64");
  if (!(c->theta > 1.0f) || !(c->factor >= 1.0f) || !(c->low_freq_factor > 0.0f) ||
      !(c->high_freq_factor > c->low_freq_factor) || c->original_max_pos <= 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, std::string(who) + ": bad rope config");
  return DSA_OK;
}

static size_t table_bytes(int32_t n) { return ((size_t)n * kRotPairs * sizeof(float2) + 255) / 256 * 256; }
static size_t splitk_bytes(int32_t n, int32_t hidden) {
  if (hidden <= 0) return 0;
  if (n > kSmallT) return (size_t)n * kProjN * sizeof(float);  // the fp32 projection
  return (size_t)(hidden / splitk_kper(hidden)) * n * kProjN * sizeof(float);
}

}  // namespace dsa

using namespace dsa;

extern "C" dsa_status dsa_rope_config_default(dsa_rope_config* c) {
  if (!c) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_rope_config_default: NULL");
  c->rot_dims = kRotDims;
  c->theta = 10000.0f;
  c->factor = 8.0f;
  c->low_freq_factor = 1.0f;
  c->high_freq_factor = 32.0f;
  c->original_max_pos = 1048576;
  return DSA_OK;
}

extern "C" size_t dsa_indexer_workspace_size(int32_t n_tokens, int32_t hidden) {
  return n_tokens <= 0 ? 256 : table_bytes(n_tokens) + splitk_bytes(n_tokens, hidden);
}

extern "C" dsa_status dsa_indexer_project(const dsa_rope_config* rope, int32_t n_tokens, int32_t hidden,
                                          const uint16_t* x, const uint16_t* w, const float* gamma_q,
                                          const float* gamma_k, const int32_t* pos, uint16_t* index_q,
                                          uint16_t* index_k, float* z, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  const char* who = "dsa_indexer_project";
  dsa_status st = check_rope(who, rope);
  if (st != DSA_OK) return st;
  if (n_tokens < 0 || hidden <= 0 || hidden % 128)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_indexer_project: hidden must be a positive multiple of 128");
  if (n_tokens == 0) return DSA_OK;
  if (!x || !w || !gamma_q || !gamma_k || !pos || !index_q || !index_k || !z || !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_indexer_project: NULL pointer");
  if (((uintptr_t)x | (uintptr_t)w) & 15)
    return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_indexer_project: x and w must be 16-byte aligned");
  if ((size_t)workspace & 255) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_indexer_project: workspace alignment");
  if (workspace_bytes < dsa_indexer_workspace_size(n_tokens, hidden))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_indexer_project: workspace too small");
  hipStream_t s = as_stream(stream);
  const RopeFreqs fr = rope_freqs(*rope);
  if (n_tokens <= kSmallT) {
    const int32_t kper = splitk_kper(hidden), ks = hidden / kper;
    float* part = (float*)((char*)workspace + table_bytes(n_tokens));
    {
      ProfScope prof_("k_indexer_proj", s);
      hipLaunchKernelGGL(k_indexer_proj_splitk, dim3(kColGroups, (unsigned)ks), dim3(64), 0, s, x, w, part, n_tokens,
                         hidden, kper);
    }
    st = check_launch(who);
    if (st != DSA_OK) return st;
    {
      ProfScope prof_("k_indexer_finish", s);
      hipLaunchKernelGGL(k_indexer_finish, dim3((unsigned)n_tokens, kVecs / 4), dim3(256), 0, s, (const float*)part, ks,
                         gamma_q, gamma_k, pos, fr, index_q, index_k, z, n_tokens);
    }
    return check_launch(who);
  }
  {
    float* yv = (float*)((char*)workspace + table_bytes(n_tokens));
    {
      ProfScope prof_("k_indexer_proj", s);
      const int ntile = ((n_tokens + kGM - 1) / kGM) * ((kProjN + kGN - 1) / kGN);
      hipLaunchKernelGGL(k_indexer_gemm, dim3((unsigned)(8 * ((ntile + 7) / 8))), dim3(256), 0, s, x, w, yv,
                         n_tokens, hidden);
    }
    st = check_launch(who);
    if (st != DSA_OK) return st;
    {
      ProfScope prof_("k_indexer_finish", s);
      hipLaunchKernelGGL(k_indexer_finish, dim3((unsigned)n_tokens, 1), dim3(256), 0, s, (const float*)yv, 1, gamma_q,
                         gamma_k, pos, fr, index_q, index_k, z, n_tokens);
    }
    return check_launch(who);
  }
}

extern "C" dsa_status dsa_rope_qk(const dsa_rope_config* rope, int32_t n_tokens, const int32_t* pos, uint16_t* q,
                                  uint16_t* k, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "dsa_rope_qk";
  dsa_status st = check_rope(who, rope);
  if (st != DSA_OK) return st;
  if (n_tokens < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_rope_qk: bad sizes");
  if (n_tokens == 0) return DSA_OK;
  if (!pos || !q || !k || !workspace) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_rope_qk: NULL pointer");
  if ((size_t)workspace & 255) return fail(DSA_ERR_INVALID_ARGUMENT, "dsa_rope_qk: workspace alignment");
  if (workspace_bytes < dsa_indexer_workspace_size(n_tokens, 0))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_rope_qk: workspace too small");
  hipStream_t s = as_stream(stream);
  float2* cs = (float2*)workspace;
  {
    ProfScope prof_("k_rope_table", s);
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n_tokens + 1) / 2)), dim3(64), 0, s, pos, n_tokens,
                       rope_freqs(*rope), cs);
  }
  st = check_launch(who);
  if (st != DSA_OK) return st;
  {
    ProfScope prof_("k_rope_qk", s);
    hipLaunchKernelGGL(k_rope_qk, dim3((unsigned)n_tokens), dim3(256), 0, s, (const float2*)cs, q, k, n_tokens);
  }
  return check_launch(who);
}
