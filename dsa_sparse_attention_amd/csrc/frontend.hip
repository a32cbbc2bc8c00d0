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
// k_indexer_proj: one fused MFMA GEMM + epilogue per (128 tokens, 256-wide
// output vector).  The 20 vectors are the 16 index_q heads and the 4 index_k
// groups; a block computes x[128 x H] . W_h^T[H x 256] with 4 waves of 64
// columns each (8 x 4 tiles of v_mfma_f32_16x16x32_bf16 per wave, 128 fp32
// accumulators), the x tile staged in LDS (shared by the 4 waves, double
// buffered, padded rows), the weight fragments read straight from memory
// (each wave reads its own 64 rows of W).  The epilogue never leaves
// registers except for the RMS: per-token sums of squares of the 4 waves
// meet in LDS, then x * rsqrt(mean + eps) * gamma, the rotate-half rotation
// of dimensions 0..63 (wave 0 holds both halves of every pair in one lane),
// bf16 rounding and the store.
// k_indexer_z: the 16 z columns (x . W_z^T, fp32 out), 4 waves splitting H.
// k_rope_qk: the rotation applied in place to q [T][64][192], k [T][4][192].
// Angles are pos * freq in double, reduced to [-pi, pi] before sincos, so
// positions up to 2^31 keep full fp32 accuracy.
#include <math.h>

#include "common.hpp"

namespace dsa {

constexpr int kRotDims = 64;               // rotated dimensions of every vector
constexpr int kRotPairs = kRotDims / 2;    // pairs (i, i + 32)
constexpr int kVecs = kIdxHeads + kGroups;  // 20 normalised 256-d outputs per token
constexpr int kProjN = kVecs * kProxy + kIdxHeads;  // 5136 weight rows
constexpr float kNormEps = 1e-6f;

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

#ifndef DSA_FE_PM
#define DSA_FE_PM 128
#endif
constexpr int kPM = DSA_FE_PM;  // tokens per block
constexpr int kPRT = kPM / 16;  // row tiles per wave
constexpr int kPLR = kPM / 32;  // x-tile rows each thread copies per stage
constexpr int kPK = 64;        // k per LDS stage
constexpr int kPPitch = kPK + 8;  // padded row (elements): 144 bytes, conflict-free fragment reads

struct ProjArgs {
  const uint16_t* x;   // [T][H]
  const uint16_t* w;   // [kProjN][H]
  const float* gq;     // [256]
  const float* gk;     // [256]
  const float2* cs;    // [T][32] (cos, sin)
  uint16_t* iq;        // [T][16][256]
  uint16_t* ik;        // [T][4][256]
  int32_t T, H;
};

__global__ __launch_bounds__(256) void k_indexer_proj(ProjArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kPM;
  const int h = blockIdx.y;  // output vector 0..19
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kPM * kPPitch];
  __shared__ float red[4][kPM];

  // x tile loads: thread t copies rows t/8 + 32r, 8 elements at (t%8)*8
  const int lr = threadIdx.x >> 3, lk = (threadIdx.x & 7) * 8;
  const uint16_t* xrow[kPLR];
#pragma unroll
  for (int r = 0; r < kPLR; ++r) {
    int64_t t = t0 + lr + 32 * r;
    t = t < a.T ? t : a.T - 1;  // rows past the end re-read the last token; never stored
    xrow[r] = a.x + t * a.H + lk;
  }
  // weight fragments: column (64*wave + 16*ct + n) of vector h, k = 8*kb .. +7 of each 32-step
  const uint16_t* wrow[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) wrow[ct] = a.w + ((int64_t)h * kProxy + 64 * wave + 16 * ct + n) * a.H + 8 * kb;

  f32x4 acc[kPRT][4];
#pragma unroll
  for (int rt = 0; rt < kPRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nst = a.H / kPK;
  u32x4 xr[kPLR];
#pragma unroll
  for (int r = 0; r < kPLR; ++r) xr[r] = ld16(xrow[r]);
#pragma unroll
  for (int r = 0; r < kPLR; ++r) *(u32x4*)&xs[0][(lr + 32 * r) * kPPitch + lk] = xr[r];
  // weight fragments run one stage ahead of their use
  u32x4 wn[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) wn[ks][ct] = ld16(wrow[ct] + 32 * ks);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const int64_t k0 = (int64_t)st * kPK;
    // next stage's x rows and weight fragments while this stage computes
    // (past the last stage: a re-read of the last one, never used)
    const int64_t kn = st + 1 < nst ? k0 + kPK : k0;
#pragma unroll
    for (int r = 0; r < kPLR; ++r) xr[r] = ld16(xrow[r] + kn);
    u32x4 wf[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        wf[ks][ct] = wn[ks][ct];
        wn[ks][ct] = ld16(wrow[ct] + kn + 32 * ks);
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) {
        const bf16x8 af = as_bf16x8(*(const u32x4*)&xs[buf][(16 * rt + n) * kPPitch + 32 * ks + 8 * kb]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = mfma16x16x32(af, as_bf16x8(wf[ks][ct]), acc[rt][ct]);
      }
    }
#pragma unroll
    for (int r = 0; r < kPLR; ++r) *(u32x4*)&xs[buf ^ 1][(lr + 32 * r) * kPPitch + lk] = xr[r];
    __syncthreads();
  }

  // RMS over the vector's 256 columns: lane holds rows 16rt + 4kb + i, columns 64wave + 16ct + n
#pragma unroll
  for (int rt = 0; rt < kPRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float ss = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) ss += acc[rt][ct][i] * acc[rt][ct][i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off);
      if (n == 0) red[wave][16 * rt + 4 * kb + i] = ss;
    }
  __syncthreads();
  const float* gam = h < kIdxHeads ? a.gq : a.gk;
  float g[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) g[ct] = gam[64 * wave + 16 * ct + n];
  uint16_t* out = h < kIdxHeads ? a.iq + (int64_t)h * kProxy : a.ik + (int64_t)(h - kIdxHeads) * kProxy;
  const int64_t tstride = (h < kIdxHeads ? kIdxHeads : kGroups) * kProxy;
#pragma unroll
  for (int rt = 0; rt < kPRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * kb + i;
      const int64_t t = t0 + row;
      const float ms = (red[0][row] + red[1][row] + red[2][row] + red[3][row]) * (1.0f / kProxy);
      const float inv = 1.0f / sqrtf(ms + kNormEps);
      float y[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) y[ct] = acc[rt][ct][i] * inv * g[ct];
      if (wave == 0) {  // columns 0..63: pairs (n, n + 32) and (16 + n, 48 + n)
        const int64_t tc = t < a.T ? t : a.T - 1;
        const float2 c0 = a.cs[tc * kRotPairs + n], c1 = a.cs[tc * kRotPairs + 16 + n];
        const float y0 = y[0] * c0.x - y[2] * c0.y, y2 = y[2] * c0.x + y[0] * c0.y;
        const float y1 = y[1] * c1.x - y[3] * c1.y, y3 = y[3] * c1.x + y[1] * c1.y;
        y[0] = y0;
        y[1] = y1;
        y[2] = y2;
        y[3] = y3;
      }
      if (t < a.T) {
        uint16_t* o = out + t * tstride + 64 * wave + n;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) o[16 * ct] = (uint16_t)(pack_bf16x2(y[ct], 0.f) & 0xffffu);
      }
    }
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

// block = (token, output vector 0..19, or 20 = z); thread = column.
__global__ __launch_bounds__(256) void k_indexer_finish(const float* __restrict__ part, int32_t ks,
                                                        const float* __restrict__ gq, const float* __restrict__ gk,
                                                        const int32_t* __restrict__ pos, RopeFreqs fr,
                                                        uint16_t* __restrict__ iq, uint16_t* __restrict__ ik,
                                                        float* __restrict__ z, int32_t T) {
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y, c = threadIdx.x, lane = c & 63, wave = c >> 6;
  __shared__ float red[4];
  __shared__ float ys[kRotDims];
  if (h == kVecs) {
    if (c < kIdxHeads) {
      float acc = 0.f;
      for (int sp = 0; sp < ks; ++sp) acc += part[((int64_t)sp * T + t) * kProjN + kVecs * kProxy + c];
      z[t * kIdxHeads + c] = acc;
    }
    return;
  }
  // the rotation's (cos, sin) for this column's pair, while the partials load
  const float2 cc = c < kRotDims ? rope_cs(pos[t], fr.f[c & (kRotPairs - 1)]) : make_float2(1.f, 0.f);
  float y = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < ks; ++sp) y += part[((int64_t)sp * T + t) * kProjN + h * kProxy + c];
  float ss = y * y;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float ms = (red[0] + red[1] + red[2] + red[3]) * (1.0f / kProxy);
  y = y * (1.0f / sqrtf(ms + kNormEps)) * (h < kIdxHeads ? gq : gk)[c];
  if (c < kRotDims) ys[c] = y;
  __syncthreads();
  if (c < kRotDims) {
    y = c < kRotPairs ? ys[c] * cc.x - ys[c + kRotPairs] * cc.y : ys[c] * cc.x + ys[c - kRotPairs] * cc.y;
  }
  uint16_t* o = h < kIdxHeads ? iq + (t * kIdxHeads + h) * kProxy : ik + (t * kGroups + h - kIdxHeads) * kProxy;
  o[c] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xffffu);
}

static int32_t splitk_kper(int32_t hidden) { return hidden % 256 == 0 ? 256 : 128; }

// z = x . W_z^T: block = 16 tokens, wave w takes k in [w*H/4, (w+1)*H/4).
__global__ __launch_bounds__(256) void k_indexer_z(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                   float* __restrict__ z, int32_t T, int32_t H) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  __shared__ f32x4 part[4][64];
  int64_t t = t0 + n;
  t = t < T ? t : T - 1;
  const uint16_t* xr = x + t * H + 8 * kb;
  const uint16_t* wr = w + ((int64_t)kVecs * kProxy + n) * H + 8 * kb;
  const int kq = H / 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = wave * kq; k < (wave + 1) * kq; k += 32)
    acc = mfma16x16x32(as_bf16x8(ld16(xr + k)), as_bf16x8(ld16(wr + k)), acc);
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4 s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tt = t0 + 4 * kb + i;  // row 4kb + i, column n
      if (tt < T) z[tt * kIdxHeads + n] = s[i];
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
  if (n > kSmallT || hidden <= 0) return 0;
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
      hipLaunchKernelGGL(k_indexer_finish, dim3((unsigned)n_tokens, kVecs + 1), dim3(256), 0, s, (const float*)part,
                         ks, gamma_q, gamma_k, pos, fr, index_q, index_k, z, n_tokens);
    }
    return check_launch(who);
  }
  float2* cs = (float2*)workspace;
  {
    ProfScope prof_("k_rope_table", s);
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n_tokens + 1) / 2)), dim3(64), 0, s, pos, n_tokens, fr, cs);
  }
  st = check_launch(who);
  if (st != DSA_OK) return st;
  ProjArgs a;
  a.x = x; a.w = w; a.gq = gamma_q; a.gk = gamma_k; a.cs = cs; a.iq = index_q; a.ik = index_k;
  a.T = n_tokens; a.H = hidden;
  {
    ProfScope prof_("k_indexer_proj", s);
    hipLaunchKernelGGL(k_indexer_proj, dim3((unsigned)((n_tokens + kPM - 1) / kPM), kVecs), dim3(256), 0, s, a);
  }
  st = check_launch(who);
  if (st != DSA_OK) return st;
  {
    ProfScope prof_("k_indexer_z", s);
    hipLaunchKernelGGL(k_indexer_z, dim3((unsigned)((n_tokens + 15) / 16)), dim3(256), 0, s, x, w, z, n_tokens,
                       hidden);
  }
  return check_launch(who);
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
