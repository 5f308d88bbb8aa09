// Standalone and helper kernels: RMSNorm (wavefront reduction), RoPE and its
// cos/sin tables, attention operand packing, embedding gather, dtype
// conversion, and the plain fp32 path used by fp32 workloads (VALU kernels).
//
// RMSNorm with gain: paperfordummies.in LLaMA page "RMSNorm: LayerNorm minus the
// mean" (rms_norm in "The code") and the chenyuan1125.github.io page's RMSNorm
// equation. RoPE: the same pages' "RoPE: rotate Q and K, leave V alone" /
// rope() and the RoPE equation: interleaved channel pairs (2i, 2i+1) of each
// head rotate by pos * theta^(-2i/head_dim).
#include "common.h"
#include "internal.h"

namespace llama {

// ------------------------------------------------------------------ RoPE tables
// tab[p * hd/2 + i] = (cos, sin)(p * theta^(-2i/hd)), angles in fp64.
DEV float2 rope_entry(int p, int i, int hd, double theta) {
  const double ang = (double)p * pow(theta, -(2.0 * i) / hd);
  double sn, cs;
  sincos(ang, &sn, &cs);
  return make_float2((float)cs, (float)sn);
}

__global__ void rope_table_kernel(float2 *tab, int positions, int hd, double theta) {
  const int half = hd >> 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)positions * half) return;
  tab[idx] = rope_entry((int)(idx / half), (int)(idx % half), hd, theta);
}

__global__ void rope_table_pos_kernel(float2 *tab, const int32_t *pos, int n, int hd, double theta) {
  const int half = hd >> 1;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * half) return;
  const int b = idx / half, i = idx % half;
  const double ang = (double)pos[b] * pow(theta, -(2.0 * i) / hd);
  double sn, cs;
  sincos(ang, &sn, &cs);
  tab[idx] = make_float2((float)cs, (float)sn);
}

hipError_t rope_table_launch(float2 *tab, int positions, int head_dim, float theta, hipStream_t s) {
  const int64_t n = (int64_t)positions * (head_dim / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tab,
                     positions, head_dim, (double)theta);
  return hipGetLastError();
}

hipError_t rope_table_pos_launch(float2 *tab, const int32_t *pos, int n, int head_dim, float theta,
                                 int max_seq, hipStream_t s) {
  (void)max_seq;
  const int tot = n * (head_dim / 2);
  if (tot == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_pos_kernel, dim3((tot + 255) / 256), dim3(256), 0, s, tab, pos, n,
                     head_dim, (double)theta);
  return hipGetLastError();
}

// ------------------------------------------------------------------ norm prep
// One 64-lane wavefront per row, 8 consecutive channels per lane and 512-wide
// chunk. It writes the GEMM operand x * g (bf16, a bf16 hi/lo pair, or IEEE
// fp16 by OUT) and the row multiplier rmul that the consumer applies to its
// fp32 accumulator; x * g times rmul is RMSNorm(x; g) (RMSNorm with gain, as
// in the chenyuan1125.github.io page's equation), so the product
// (x * g) W^T * rmul completes RMSNorm(x; g) W^T. With g == nullptr the
// operand is x itself (a block without a norm before the projection) and
// rmul only undoes the operand's scale below.
//
// RMSNorm puts every row on the same scale ("RMSNorm: LayerNorm minus the
// mean" on the paperfordummies.in page), so the operand must not depend on
// the row's own scale. fp16 holds magnitudes from 2^-14 to 65504 only: the
// fp16 operand is x * g * 2^k with 2^k the largest power of two at most
// 4 rstd, which puts the row's RMS in (2, 4] and every element below
// 4 sqrt(dim) |g|, and rmul = rstd * 2^-k. Scaling by 2^k is exact, so inside
// fp16's range the products and the accumulator are exactly 2^k times those
// of the unscaled operand and the result bits do not change. bf16 and bf16
// pairs have fp32's range and stay unscaled (rmul = rstd). The statistics are
// fp32: a row whose sum of squares overflows fp32 is out of range.
//
// NC > 0: the row stays in registers between the statistics and the operand
// (NC chunks per lane, dim <= 512 NC; every load issues before the first
// use); NC == 0: two passes over memory.
// PARTS: the row is h = x + part[0] + ... (split-K partial products, added in
// split order), written to h_out in fp32.
template <bool IN_F32, int OUT, bool PARTS, int NC>
__global__ __launch_bounds__(256) void norm_prep_kernel(const void *__restrict__ x, const u16 *__restrict__ g,
                                                        int64_t rows, int dim, float eps, float *__restrict__ rmul,
                                                        u16 *__restrict__ xg_hi, u16 *__restrict__ xg_lo,
                                                        const float *__restrict__ part, int n_parts,
                                                        float *__restrict__ h_out, const RopeRows rope,
                                                        int *__restrict__ zero, int n_zero) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  if (row >= rows) return;
  // table row p = row for the first rope.positions rows: the RoPE table is
  // built by this launch instead of one of its own
  if (row < rope.positions)
    for (int i = lane; i < rope.hd / 2; i += 64) rope.tab[row * (rope.hd / 2) + i] = rope_entry((int)row, i, rope.hd, rope.theta);
  const int64_t base = row * dim;
  const int64_t pstride = rows * dim;
  // channels c .. c+7 of the row (c is a multiple of 8 below dim)
  auto load = [&](int c, float *f) {
    if (IN_F32) {
      const f32x4 a0 = *(const f32x4 *)((const float *)x + base + c);
      const f32x4 a1 = *(const f32x4 *)((const float *)x + base + c + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = a0[i];
        f[4 + i] = a1[i];
      }
    } else {
      unpack8(*(const u32x4 *)((const u16 *)x + base + c), f);
    }
    if (PARTS) {
      for (int z = 0; z < n_parts; ++z) {
        const float *pp = part + z * pstride + base + c;
        const f32x4 p0 = *(const f32x4 *)pp, p1 = *(const f32x4 *)(pp + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] += p0[i];
          f[4 + i] += p1[i];
        }
      }
    }
  };
  auto put_h = [&](int c, const float *f) {
    *(f32x4 *)(h_out + base + c) = f32x4{f[0], f[1], f[2], f[3]};
    *(f32x4 *)(h_out + base + c + 4) = f32x4{f[4], f[5], f[6], f[7]};
  };
  auto put_operand = [&](int c, const float *f, float scale) {
    float v[8], gf[8];
    if (g) {
      unpack8(*(const u32x4 *)(g + c), gf);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) gf[i] = 1.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f[i] * gf[i] * scale;
    if (OUT == 1) {
      u32x4 hi, lo;
      pack8_pair(v, hi, lo);
      *(u32x4 *)(xg_hi + base + c) = hi;
      *(u32x4 *)(xg_lo + base + c) = lo;
    } else {
      *(u32x4 *)(xg_hi + base + c) = OUT == 2 ? pack8h(v) : pack8(v);
    }
  };
  // operand scale 2^k and row multiplier from the statistics
  auto scales = [&](float ss, float &scale, float &mul) {
    const float r = rstd_of(ss, dim, eps);
    const float keep = g ? r : 1.0f;   // no norm: the multiplier only undoes the scale
    scale = 1.0f;
    mul = keep;
    const int e = (int)((__float_as_uint(r) >> 23) & 0xff);
    if (OUT == 2 && e != 0 && e != 0xff) {   // finite nonzero rstd; otherwise unscaled (0 * inf stays NaN)
      const int k = min(max(e - 127 + 2, -126), 126);
      scale = __uint_as_float((uint32_t)(k + 127) << 23);
      mul = keep * __uint_as_float((uint32_t)(127 - k) << 23);
    }
  };

  float ss = 0.f, scale, mul;
  if (NC > 0) {
    float f[NC > 0 ? NC : 1][8];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = 8 * lane + 512 * u;
      const bool in = c < dim;     // chunks past dim (and the tail of a dim not a multiple of 512)
      float t[8];
      load(in ? c : dim - 8, t);   // every load issues before the first use
#pragma unroll
      for (int i = 0; i < 8; ++i) f[u][i] = in ? t[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = 8 * lane + 512 * u;
      if (PARTS && c < dim) put_h(c, f[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += f[u][i] * f[u][i];
    }
    ss = wave_sum(ss);
    scales(ss, scale, mul);
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = 8 * lane + 512 * u;
      if (c < dim) put_operand(c, f[u], scale);
    }
  } else {
    for (int c = 8 * lane; c < dim; c += 512) {
      float f[8];
      load(c, f);
      if (PARTS) put_h(c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
    }
    ss = wave_sum(ss);
    scales(ss, scale, mul);
    for (int c = 8 * lane; c < dim; c += 512) {
      float f[8];
      if (PARTS) {   // h as this lane wrote it
        const f32x4 a0 = *(const f32x4 *)(h_out + base + c), a1 = *(const f32x4 *)(h_out + base + c + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = a0[i];
          f[4 + i] = a1[i];
        }
      } else {
        load(c, f);
      }
      put_operand(c, f, scale);
    }
  }
  if (lane == 0) rmul[row] = mul;
}

hipError_t norm_prep_launch(int in_f32, const void *x, const uint16_t *g, int64_t rows, int dim, float eps,
                            float *rmul, uint16_t *xg_hi, uint16_t *xg_lo, hipStream_t s, const float *part,
                            int n_parts, float *h_out, int out_f16, RopeRows rope, int *zero, int n_zero) {
  if (rows == 0) return hipSuccess;
  if (n_zero < 0 || (n_zero > 0 && !zero)) return hipErrorInvalidValue;
  if (rope.positions > rows || (rope.positions > 0 && (!rope.tab || rope.hd <= 0))) return hipErrorInvalidValue;
  if (dim % 8) return hipErrorInvalidValue;
  const bool parts = part != nullptr && n_parts > 0;
  if (parts && h_out == nullptr) return hipErrorInvalidValue;
  if (out_f16 && xg_lo) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 3) / 4));
  const int out = out_f16 ? 2 : (xg_lo ? 1 : 0);
  const int nc = dim <= 2048 ? 4 : (dim <= 4096 ? 8 : (dim <= 8192 ? 16 : 0));
#define NP_CASE(F, O_, R, NC_)                                                                                    \
  if (!!in_f32 == F && out == O_ && parts == R && nc == NC_) {                                                   \
    hipLaunchKernelGGL((norm_prep_kernel<F, O_, R, NC_>), grid, dim3(256), 0, s, x, g, rows, dim, eps, rmul, xg_hi, \
                       xg_lo, part, n_parts, h_out, rope, zero, n_zero);                                          \
    return hipGetLastError();                                                                                   \
  }
#define NP_CASES(NC_)                                                                                   \
  NP_CASE(true, 0, false, NC_) NP_CASE(true, 1, false, NC_) NP_CASE(true, 2, false, NC_)                \
  NP_CASE(false, 0, false, NC_) NP_CASE(false, 1, false, NC_) NP_CASE(false, 2, false, NC_)             \
  NP_CASE(true, 0, true, NC_) NP_CASE(true, 1, true, NC_) NP_CASE(true, 2, true, NC_)                   \
  NP_CASE(false, 0, true, NC_) NP_CASE(false, 1, true, NC_) NP_CASE(false, 2, true, NC_)
  NP_CASES(4)
  NP_CASES(8)
  NP_CASES(16)
  NP_CASES(0)
#undef NP_CASES
#undef NP_CASE
  return hipErrorInvalidValue;
}

// NaN logits rows of the sequences whose prefill chunk does not fit the cache.
__global__ void nan_unplaced_rows_kernel(const int32_t *start_pos, int seq, int max_seq, float *logits,
                                         int64_t per_seq) {
  const int b = blockIdx.y;
  if (chunk_start(start_pos, b, seq, max_seq) >= 0) return;
  float *row = logits + (int64_t)b * per_seq;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < per_seq; i += (int64_t)gridDim.x * blockDim.x)
    row[i] = __builtin_nanf("");
}

hipError_t nan_unplaced_rows_launch(const int32_t *start_pos, int batch, int seq, int max_seq, float *logits,
                                    int vocab, hipStream_t s) {
  if (batch == 0 || seq == 0 || !start_pos) return hipSuccess;
  hipLaunchKernelGGL(nan_unplaced_rows_kernel, dim3(64, batch), dim3(256), 0, s, start_pos, seq, max_seq, logits,
                     (int64_t)seq * vocab);
  return hipGetLastError();
}

// y = r + part[0] + ... + part[n_parts-1] (fp32, split order), 4 floats per thread.
__global__ void resid_sum_kernel(const float *r, const float *part, int n_parts, int64_t n, float *y) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 v = *(const f32x4 *)(r + i);
  for (int z = 0; z < n_parts; ++z) v += *(const f32x4 *)(part + z * n + i);
  *(f32x4 *)(y + i) = v;
}

hipError_t resid_sum_launch(const float *r, const float *part, int n_parts, int64_t n, float *y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(resid_sum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, r, part, n_parts, n,
                     y);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// One 64-lane wavefront per row; the sum of squares is reduced across lanes.
// In place (y == x) is allowed: each lane rereads only the elements it writes.
template <bool IN_F32, bool OUT_F32, bool G_F32>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void *x, const void *g, void *y, int64_t rows,
                                                      int dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  auto ld = [&](const void *p, int64_t i) -> float {
    return IN_F32 ? ((const float *)p)[i] : bf2f(((const u16 *)p)[i]);
  };
  const int64_t base = row * dim;
  float ss = 0.f;
  for (int c = lane; c < dim; c += 64) {
    const float v = ld(x, base + c);
    ss += v * v;
  }
  ss = wave_sum(ss);
  const float r = rstd_of(ss, dim, eps);
  for (int c = lane; c < dim; c += 64) {
    float v = ld(x, base + c) * r;
    if (g) v *= G_F32 ? ((const float *)g)[c] : bf2f(((const u16 *)g)[c]);
    if (OUT_F32)
      ((float *)y)[base + c] = v;
    else
      ((u16 *)y)[base + c] = f2bf(v);
  }
}

hipError_t rmsnorm_launch(int in_f32, int out_f32, const void *x, const void *g, void *y, int64_t rows,
                          int dim, float eps, hipStream_t s, int g_f32) {
  if (rows == 0) return hipSuccess;
  if (g_f32 < 0) g_f32 = in_f32;
  dim3 grid((unsigned)((rows + 3) / 4));
#define RMS_CASE(I, O, G)                                                                       \
  if (!!in_f32 == I && !!out_f32 == O && !!g_f32 == G) {                                        \
    hipLaunchKernelGGL((rmsnorm_kernel<I, O, G>), grid, dim3(256), 0, s, x, g, y, rows, dim, eps); \
    return hipGetLastError();                                                                   \
  }
  RMS_CASE(true, true, true)
  RMS_CASE(true, false, true)
  RMS_CASE(false, true, false)
  RMS_CASE(false, false, false)
  RMS_CASE(true, true, false)
#undef RMS_CASE
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ RoPE
template <bool F32>
__global__ void rope_kernel(const void *x, void *y, const int32_t *pos, int64_t tokens, int n_heads,
                            int hd, double theta, int seq_mod, double sign) {
  const int half = hd >> 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)n_heads * half;
  if (idx >= tokens * per_tok) return;
  const int64_t t = idx / per_tok;
  const int rem = (int)(idx % per_tok);
  const int h = rem / half, i = rem % half;
  const int p = pos ? pos[t] : (int)(t % seq_mod);
  const double ang = sign * (double)p * pow(theta, -(2.0 * i) / hd);   // sign -1: the inverse rotation
  double sn, cs;
  sincos(ang, &sn, &cs);
  const float c = (float)cs, sv = (float)sn;
  const int64_t o = t * (int64_t)n_heads * hd + h * hd + 2 * i;
  float a, b;
  if (F32) {
    a = ((const float *)x)[o];
    b = ((const float *)x)[o + 1];
  } else {
    a = bf2f(((const u16 *)x)[o]);
    b = bf2f(((const u16 *)x)[o + 1]);
  }
  const float ra = a * c - b * sv, rb = a * sv + b * c;
  if (F32) {
    ((float *)y)[o] = ra;
    ((float *)y)[o + 1] = rb;
  } else {
    ((u16 *)y)[o] = f2bf(ra);
    ((u16 *)y)[o + 1] = f2bf(rb);
  }
}

hipError_t rope_launch(int f32, const void *x, void *y, const int32_t *pos, int64_t tokens, int n_heads,
                       int head_dim, float theta, int seq_mod, hipStream_t s, int inverse) {
  const double sign = inverse ? -1.0 : 1.0;
  const int64_t n = tokens * n_heads * (head_dim / 2);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (f32)
    hipLaunchKernelGGL(rope_kernel<true>, grid, dim3(256), 0, s, x, y, pos, tokens, n_heads, head_dim,
                       (double)theta, seq_mod, sign);
  else
    hipLaunchKernelGGL(rope_kernel<false>, grid, dim3(256), 0, s, x, y, pos, tokens, n_heads, head_dim,
                       (double)theta, seq_mod, sign);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention operand packing
// q, k -> hi/lo bf16 [n, d]; v -> hi/lo bf16 transposed [b, h, hd, vt_stride].
template <bool F32>
__global__ void attn_pack_kernel(const void *q, const void *k, const void *v, u16 *qh, u16 *ql, u16 *kh,
                                 u16 *kl, u16 *vth, u16 *vtl, int batch, int seq, int n_heads, int hd,
                                 int vt_stride) {
  const int d = n_heads * hd;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * seq * d) return;
  auto ld = [&](const void *p) -> float { return F32 ? ((const float *)p)[idx] : bf2f(((const u16 *)p)[idx]); };
  u16 hi, lo;
  split_pair(ld(q), hi, lo);
  qh[idx] = hi;
  ql[idx] = lo;
  split_pair(ld(k), hi, lo);
  kh[idx] = hi;
  kl[idx] = lo;
  split_pair(ld(v), hi, lo);
  const int64_t tok = idx / d;
  const int c = (int)(idx % d);
  const int b = (int)(tok / seq), s = (int)(tok % seq);
  const int h = c / hd, e = c % hd;
  const int64_t o = (((int64_t)b * n_heads + h) * hd + e) * vt_stride + s;
  vth[o] = hi;
  vtl[o] = lo;
}

hipError_t attn_pack_launch(int in_f32, const void *q, const void *k, const void *v, uint16_t *qh,
                            uint16_t *ql, uint16_t *kh, uint16_t *kl, uint16_t *vth, uint16_t *vtl,
                            int batch, int seq, int n_heads, int head_dim, int vt_stride, hipStream_t s) {
  const int64_t n = (int64_t)batch * seq * n_heads * head_dim;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (in_f32)
    hipLaunchKernelGGL(attn_pack_kernel<true>, grid, dim3(256), 0, s, q, k, v, qh, ql, kh, kl, vth, vtl,
                       batch, seq, n_heads, head_dim, vt_stride);
  else
    hipLaunchKernelGGL(attn_pack_kernel<false>, grid, dim3(256), 0, s, q, k, v, qh, ql, kh, kl, vth, vtl,
                       batch, seq, n_heads, head_dim, vt_stride);
  return hipGetLastError();
}

// ------------------------------------------------------------------ embedding gather
// x[t] = emb[tokens[t]] widened to f32; an id outside [0, vocab) gives a NaN row.
template <bool F32>
__global__ void embed_kernel(const void *emb, const int32_t *tokens, int64_t n, int dim, int vocab,
                             float *x) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * dim) return;
  const int64_t t = idx / dim;
  const int c = (int)(idx % dim);
  const int tok = tokens[t];
  float v = __builtin_nanf("");
  if (tok >= 0 && tok < vocab) {
    const int64_t o = (int64_t)tok * dim + c;
    v = F32 ? ((const float *)emb)[o] : bf2f(((const u16 *)emb)[o]);
  }
  x[idx] = v;
}

hipError_t embed_launch(int w_f32, const void *emb, const int32_t *tokens, int64_t n, int dim, int vocab,
                        float *x, hipStream_t s) {
  const int64_t tot = n * dim;
  if (tot == 0) return hipSuccess;
  const dim3 grid((unsigned)((tot + 255) / 256));
  if (w_f32)
    hipLaunchKernelGGL(embed_kernel<true>, grid, dim3(256), 0, s, emb, tokens, n, dim, vocab, x);
  else
    hipLaunchKernelGGL(embed_kernel<false>, grid, dim3(256), 0, s, emb, tokens, n, dim, vocab, x);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dtype conversion
__global__ void convert_kernel(int in_f32, int out_f32, const void *x, void *y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = in_f32 ? ((const float *)x)[i] : bf2f(((const u16 *)x)[i]);
  if (out_f32)
    ((float *)y)[i] = v;
  else
    ((u16 *)y)[i] = f2bf(v);
}

hipError_t convert_launch(int in_f32, int out_f32, const void *x, void *y, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in_f32, out_f32,
                     x, y, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32 path
// C[M, N] = A[M, K] B[N, K]^T (+ R), 64x64 tiles through LDS, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *A, const float *B, float *C,
                                                       const float *R, int M, int N, int K) {
  __shared__ float As[16][65], Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      const int r = i / 16, c = i % 16;
      As[c][r] = (m0 + r < M && k0 + c < K) ? A[(int64_t)(m0 + r) * K + k0 + c] : 0.f;
      Bs[c][r] = (n0 + r < N && k0 + c < K) ? B[(int64_t)(n0 + r) * K + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) {
        const int64_t o = (int64_t)m * N + n;
        C[o] = acc[i][j] + (R ? R[o] : 0.f);
      }
    }
}

hipError_t gemm_f32_launch(const float *A, const float *B, float *C, const float *R, int M, int N, int K,
                           hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  // C = A B^T: A(m, k) = A[m K + k], B(k, n) = B[n K + k]
  const hipError_t e = gemm_f32_mfma_launch(A, K, 1, B, 1, K, C, R, M, N, K, 0, s);
  if (e != hipErrorNotSupported) return e;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, A, B, C, R, M,
                     N, K);
  return hipGetLastError();
}

__global__ void silu_mul_kernel(const float *g, const float *u, float *out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = silu(g[i]) * u[i];
}

hipError_t silu_mul_f32_launch(const float *g, const float *u, float *out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, u, out, n);
  return hipGetLastError();
}

// Causal attention in fp32 on the matrix cores (v_mfma_f32_32x32x2_f32:
// fp32 products and sums). One workgroup per (32-query tile, sequence, head);
// its four wavefronts take the 32-key tiles at or before the diagonal in turn
// (wavefront w: tiles w, w + 4, ...), each keeping the running (max, sum,
// output) of its keys, and the four states of a query are merged in
// wavefront order at the end, so the result does not depend on timing. lse
// (optional) gets max + log(sum).
// Per key tile a wavefront computes S^T = K Q^T (32 keys x 32 queries): a lane
// holds 16 keys of one query, so the softmax of a query reduces over the
// lane and its partner half-wave. O^T += V^T P^T then contracts over the keys
// in the order the accumulator holds them, so P enters the product straight
// from the lane's registers. K and V tiles go through a wavefront-private LDS
// region (rows padded so the half-waves' reads fall on distinct banks); the
// next tile is loaded into registers while the current one is multiplied.
template <int HD>
__global__ __launch_bounds__(256, 1) void attn_f32_mfma_kernel(const float *q, const float *k, const float *v,
                                                               float *o, float *lse, int batch, int seq,
                                                               int n_heads) {
  constexpr int KS = HD + 4, VS = HD + 8;   // LDS row strides (floats) of the K and V tiles
  constexpr int TILE = 32 * KS + 32 * VS;   // floats per wavefront
  constexpr int NEB = HD / 32;              // 32-wide blocks of the head dimension
  constexpr int HH = HD / 2;                // head-dimension entries each half-wave contracts
  constexpr int NV4 = 32 * HD / 4 / 64;     // 16-byte pieces per lane of one K (or V) tile
  __shared__ float lds[4 * TILE];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y, b = bh / n_heads, h = bh % n_heads;
  const int q0 = blockIdx.x * 32, qi = q0 + l32;
  const int d = n_heads * HD;
  float *sk = lds + w * TILE, *sv = sk + 32 * KS;
  const float sc = 1.0f / sqrtf((float)HD);

  // this lane's query, head-dimension entries g*HH .. g*HH+HH-1 (the B operand of S^T)
  float qr[HH];
  {
    const float *qp = q + ((int64_t)b * seq + min(qi, seq - 1)) * d + h * HD + g * HH;
#pragma unroll
    for (int i = 0; i < HH; i += 4) *(f32x4 *)&qr[i] = *(const f32x4 *)(qp + i);
  }
  f32x16 acc[NEB];
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[e][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int nkt = min(q0 + 31, seq - 1) / 32 + 1;   // key tiles a query of the tile sees
  // piece i of a tile: row i / (HD/4), 4 columns at 4 (i % (HD/4)); rows past seq load the last key
  f32x4 kr[NV4], vr[NV4];
  auto load = [&](int kt) {
#pragma unroll
    for (int it = 0; it < NV4; ++it) {
      const int i = lane + 64 * it, row = i / (HD / 4), c = 4 * (i % (HD / 4));
      const int64_t src = ((int64_t)b * seq + min(kt * 32 + row, seq - 1)) * d + h * HD + c;
      kr[it] = *(const f32x4 *)(k + src);
      vr[it] = *(const f32x4 *)(v + src);
    }
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (w < nkt) load(w);
  for (int kt = w; kt < nkt; kt += 4) {
#pragma unroll
    for (int it = 0; it < NV4; ++it) {
      const int i = lane + 64 * it, row = i / (HD / 4), c = 4 * (i % (HD / 4));
      *(f32x4 *)&sk[row * KS + c] = kr[it];
      *(f32x4 *)&sv[row * VS + c] = vr[it];
    }
    wave_sync();
    load(min(kt + 4, nkt - 1));   // the next tile (past the end: the last one again, unused)

    // S^T[key][query]: A = K[key l32][g*HH + kk], B = Q[query l32][g*HH + kk]
    f32x16 st[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) st[0][r] = st[1][r] = 0.f;
#pragma unroll
    for (int j = 0; j < HH / 4; ++j) {
      const f32x4 ka = *(const f32x4 *)&sk[l32 * KS + g * HH + 4 * j];
#pragma unroll
      for (int u = 0; u < 4; ++u)   // two independent chains
        st[u & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[u], qr[4 * j + u], st[u & 1], 0, 0, 0);
    }
    // online softmax of query qi over the tile's keys 8*(r/4) + 4g + r%4
    float p[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      p[r] = key <= qi && key < seq ? (st[0][r] + st[1][r]) * sc : -INFINITY;
      mx = fmaxf(mx, p[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);   // finite: key kt*32 <= q0 <= qi is always seen
    const float al = expf(m - mn);   // m = -inf before the first tile: 0
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = expf(p[r] - mn);        // masked keys: exp(-inf) = 0
      ps += p[r];
    }
    ps += __shfl_xor(ps, 32, 64);
    l = l * al + ps;
    m = mn;
    // O^T[e][query] += V^T P^T: step kk contracts keys 8*(kk/4) + 4g + kk%4
#pragma unroll
    for (int e = 0; e < NEB; ++e) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[e][r] *= al;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const int key = 8 * (kk >> 2) + 4 * g + (kk & 3);
        acc[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(sv[key * VS + 32 * e + l32], p[kk], acc[e], 0, 0, 0);
      }
    }
    wave_sync();   // this tile's LDS reads are done before the next store
  }

  // merge wavefronts 1, 2, 3 into wavefront 0, in that order (same layout:
  // element (e-block, r) of lane `lane`)
  __syncthreads();
  if (w > 0) {
    float *buf = lds + w * TILE;
#pragma unroll
    for (int e = 0; e < NEB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) buf[(e * 16 + r) * 64 + lane] = acc[e][r];
    buf[NEB * 16 * 64 + lane] = m;
    buf[(NEB * 16 + 1) * 64 + lane] = l;
  }
  __syncthreads();
  if (w != 0) return;
  for (int src = 1; src < 4; ++src) {
    const float *buf = lds + src * TILE;
    const float m1 = buf[NEB * 16 * 64 + lane], l1 = buf[(NEB * 16 + 1) * 64 + lane];
    const float mn = fmaxf(m, m1);
    const float a0 = expf(m - mn), a1 = expf(m1 - mn);   // m1 = -inf (no tiles): a1 = 0
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int e = 0; e < NEB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[e][r] = acc[e][r] * a0 + buf[(e * 16 + r) * 64 + lane] * a1;
    m = mn;
  }
  if (qi >= seq) return;
  float *op = o + ((int64_t)b * seq + qi) * d + h * HD;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int e0 = 32 * e + 8 * rq + 4 * g;
      *(f32x4 *)(op + e0) = f32x4{acc[e][4 * rq] * inv, acc[e][4 * rq + 1] * inv, acc[e][4 * rq + 2] * inv,
                                  acc[e][4 * rq + 3] * inv};
    }
  if (lse && g == 0) lse[((int64_t)b * n_heads + h) * seq + qi] = m + logf(l);   // [batch][n_heads][seq]
}

hipError_t attn_f32_launch(const float *q, const float *k, const float *v, float *o, int batch, int seq,
                           int n_heads, int head_dim, hipStream_t s, float *lse) {
  if (batch * n_heads * seq == 0) return hipSuccess;
  const dim3 grid((seq + 31) / 32, batch * n_heads);
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_f32_mfma_kernel<64>, grid, dim3(256), 0, s, q, k, v, o, lse, batch, seq, n_heads);
  else if (head_dim == 128)
    hipLaunchKernelGGL(attn_f32_mfma_kernel<128>, grid, dim3(256), 0, s, q, k, v, o, lse, batch, seq, n_heads);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ argmax
// One workgroup per row: each thread scans a strided share of the row keeping
// the largest value and its lowest index, then a tree over the block picks
// (larger value, else lower index). Any NaN in the row gives -1.
__global__ __launch_bounds__(256) void argmax_kernel(const float *logits, int vocab, int32_t *out) {
  const int64_t row = blockIdx.x;
  const float *p = logits + row * vocab;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  bool nan = false;
  for (int i = threadIdx.x; i < vocab; i += 256) {
    const float v = p[i];
    nan |= v != v;
    if (v > best || (v == best && i < idx)) {
      best = v;
      idx = i;
    }
  }
  __shared__ float sv[256];
  __shared__ int si[256];
  __shared__ int sn;
  if (threadIdx.x == 0) sn = 0;
  __syncthreads();
  if (nan) sn = 1;   // benign race: every writer stores 1
  sv[threadIdx.x] = best;
  si[threadIdx.x] = idx;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
      const float v = sv[threadIdx.x + h];
      const int j = si[threadIdx.x + h];
      if (v > sv[threadIdx.x] || (v == sv[threadIdx.x] && j < si[threadIdx.x])) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = j;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[row] = (sn || si[0] >= vocab) ? -1 : si[0];
}

hipError_t argmax_launch(const float *logits, int64_t rows, int vocab, int32_t *out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)rows), dim3(256), 0, s, logits, vocab, out);
  return hipGetLastError();
}

// Weights bf16 -> IEEE fp16 ahead of time, by the conversion the GEMM applies
// to bf16 B fragments in registers (bf16x8_to_f16x8: the value widened to fp32,
// then rounded toward zero to fp16), so that a product over converted weights
// sees the same bits. Eight values per lane when both pointers are 16-byte
// aligned (VEC), else one. In place (src == dst) is safe: a lane reads its
// values before it writes them and no lane touches another's.
template <bool VEC>
__global__ void bf16_to_f16_kernel(const uint16_t *src, uint16_t *dst, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (VEC) {
    const int64_t i = t * 8;
    if (i + 8 <= n) {
      const u32x4 v = *(const u32x4 *)(src + i);
      *(u32x4 *)(dst + i) = bf16x8_to_f16x8(v);
      return;
    }
    for (int64_t j = i; j < n; ++j) {   // the last lane: fewer than 8 left
      const float f = __uint_as_float((uint32_t)src[j] << 16);
      dst[j] = (uint16_t)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f, 0.f));
    }
  } else if (t < n) {
    const float f = __uint_as_float((uint32_t)src[t] << 16);
    dst[t] = (uint16_t)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f, 0.f));
  }
}

hipError_t bf16_to_f16_launch(const uint16_t *src, uint16_t *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool vec = (((uintptr_t)src | (uintptr_t)dst) & 15) == 0;
  const int64_t lanes = vec ? (n + 7) / 8 : n;
  const int64_t blocks = (lanes + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL(bf16_to_f16_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  else
    hipLaunchKernelGGL(bf16_to_f16_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace llama
