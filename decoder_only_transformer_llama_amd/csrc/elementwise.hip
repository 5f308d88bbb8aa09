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
__global__ void rope_table_kernel(float2 *tab, int positions, int hd, double theta) {
  const int half = hd >> 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)positions * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double ang = (double)p * pow(theta, -(2.0 * i) / hd);
  double sn, cs;
  sincos(ang, &sn, &cs);
  tab[idx] = make_float2((float)cs, (float)sn);
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
// One 64-lane wavefront per row, 8 consecutive channels per lane and step:
// rstd = 1/sqrt(mean(x^2) + eps) (sum reduced across the wavefront) and the
// GEMM operand x * g as bf16 hi (+ lo), or as IEEE fp16 (H). The product's
// consumer multiplies its
// fp32 accumulator by rstd, which completes RMSNorm(x; g) W^T. dim % 8 == 0.
// g == nullptr: the operand is x itself (a block without a norm before the
// projection; rstd is then written but not used).
// U consecutive 512-channel chunks per step (dim a multiple of 512 * U when
// U > 1): all their loads issue before any is used, and __restrict__ lets the
// compiler move the next step's loads above this step's stores.
template <bool IN_F32, bool PAIR, bool PARTS, int U, bool H = false>
__global__ __launch_bounds__(256) void norm_prep_kernel(const void *__restrict__ x, const u16 *__restrict__ g,
                                                        int64_t rows, int dim, float eps, float *__restrict__ rstd,
                                                        u16 *__restrict__ xg_hi, u16 *__restrict__ xg_lo,
                                                        const float *__restrict__ part, int n_parts,
                                                        float *__restrict__ h_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = row * dim;
  const int64_t pstride = rows * dim;
  float ss = 0.f;
  for (int c0 = 8 * lane; c0 < dim; c0 += 512 * U) {
    float f[U][8], gf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 512 * u;
      if (IN_F32) {
        const f32x4 a0 = *(const f32x4 *)((const float *)x + base + c);
        const f32x4 a1 = *(const f32x4 *)((const float *)x + base + c + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[u][i] = a0[i];
          f[u][4 + i] = a1[i];
        }
      } else {
        unpack8(*(const u32x4 *)((const u16 *)x + base + c), f[u]);
      }
      if (PARTS) {
        // h = x + the split-K partial products, added in split order
        for (int z = 0; z < n_parts; ++z) {
          const float *pp = part + z * pstride + base + c;
          const f32x4 p0 = *(const f32x4 *)pp, p1 = *(const f32x4 *)(pp + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[u][i] += p0[i];
            f[u][4 + i] += p1[i];
          }
        }
      }
      if (g) {
        unpack8(*(const u32x4 *)(g + c), gf[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) gf[u][i] = 1.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 512 * u;
      if (PARTS) {
        *(f32x4 *)(h_out + base + c) = f32x4{f[u][0], f[u][1], f[u][2], f[u][3]};
        *(f32x4 *)(h_out + base + c + 4) = f32x4{f[u][4], f[u][5], f[u][6], f[u][7]};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss += f[u][i] * f[u][i];
        f[u][i] *= gf[u][i];
      }
      if (PAIR) {
        u32x4 hi, lo;
        pack8_pair(f[u], hi, lo);
        *(u32x4 *)(xg_hi + base + c) = hi;
        *(u32x4 *)(xg_lo + base + c) = lo;
      } else {
        *(u32x4 *)(xg_hi + base + c) = H ? pack8h(f[u]) : pack8(f[u]);   // H: IEEE fp16 operand
      }
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) rstd[row] = rstd_of(ss, dim, eps);
}

hipError_t norm_prep_launch(int in_f32, const void *x, const uint16_t *g, int64_t rows, int dim, float eps,
                            float *rstd, uint16_t *xg_hi, uint16_t *xg_lo, hipStream_t s, const float *part,
                            int n_parts, float *h_out, int out_f16) {
  if (rows == 0) return hipSuccess;
  if (dim % 8) return hipErrorInvalidValue;
  const bool parts = part != nullptr && n_parts > 0;
  if (parts && h_out == nullptr) return hipErrorInvalidValue;
  if (out_f16 && xg_lo) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 3) / 4));
  const int u = dim % 2048 == 0 ? 4 : (dim % 1024 == 0 ? 2 : 1);
  if (out_f16) {
#define NPH_CASE(F, R, U_)                                                                                      \
  if (!!in_f32 == F && parts == R && u == U_) {                                                                 \
    hipLaunchKernelGGL((norm_prep_kernel<F, false, R, U_, true>), grid, dim3(256), 0, s, x, g, rows, dim, eps, rstd, \
                       xg_hi, xg_lo, part, n_parts, h_out);                                                     \
    return hipGetLastError();                                                                                   \
  }
    NPH_CASE(true, false, 4) NPH_CASE(true, true, 4) NPH_CASE(false, false, 4) NPH_CASE(false, true, 4)
    NPH_CASE(true, false, 2) NPH_CASE(true, true, 2) NPH_CASE(false, false, 2) NPH_CASE(false, true, 2)
    NPH_CASE(true, false, 1) NPH_CASE(true, true, 1) NPH_CASE(false, false, 1) NPH_CASE(false, true, 1)
#undef NPH_CASE
    return hipErrorInvalidValue;
  }
#define NP_CASE(F, P, R, U_)                                                                                     \
  if (!!in_f32 == F && (xg_lo != nullptr) == P && parts == R && u == U_) {                                      \
    hipLaunchKernelGGL((norm_prep_kernel<F, P, R, U_>), grid, dim3(256), 0, s, x, g, rows, dim, eps, rstd, xg_hi, \
                       xg_lo, part, n_parts, h_out);                                                             \
    return hipGetLastError();                                                                                  \
  }
#define NP_CASES(U_)              \
  NP_CASE(true, true, false, U_)  \
  NP_CASE(true, false, false, U_) \
  NP_CASE(false, true, false, U_) \
  NP_CASE(false, false, false, U_) \
  NP_CASE(true, true, true, U_)   \
  NP_CASE(true, false, true, U_)  \
  NP_CASE(false, true, true, U_)  \
  NP_CASE(false, false, true, U_)
  NP_CASES(4)
  NP_CASES(2)
  NP_CASES(1)
#undef NP_CASES
#undef NP_CASE
  return hipErrorInvalidValue;
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

// Causal attention in fp32 with online softmax. One workgroup per (query
// tile of 32, sequence, head): 8 key groups of 32 lanes (two per wavefront),
// all on the same 32 queries (one per lane), group g taking the keys
// j = g mod 8 of every 64-key tile of K and V staged in LDS (the lanes of a
// group read the same key row: broadcast). Each lane keeps the running (max,
// sum, output) of its keys; the eight partial states of a query are merged in
// group order at the end, so the result does not depend on timing. lse
// (optional) gets max + log(sum).
constexpr int kAttnQ = 32, kAttnK = 64, kAttnG = 8;
template <int HD>
__global__ __launch_bounds__(kAttnQ * kAttnG) void attn_f32_kernel(const float *q, const float *k, const float *v,
                                                                   float *o, float *lse, int batch, int seq,
                                                                   int n_heads) {
  __shared__ float kv[2][kAttnK][HD];   // K and V tiles; after the loop, the merge buffer
  const int lq = threadIdx.x % kAttnQ, grp = threadIdx.x / kAttnQ;
  const int bh = blockIdx.y, b = bh / n_heads, h = bh % n_heads;
  const int q0 = blockIdx.x * kAttnQ, qi = q0 + lq;
  const int d = n_heads * HD;
  float qr[HD], acc[HD];
  {
    const float *qp = q + ((int64_t)b * seq + min(qi, seq - 1)) * d + h * HD;
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      qr[e] = qp[e];
      acc[e] = 0.f;
    }
  }
  const float sc = 1.0f / sqrtf((float)HD);
  float m = -INFINITY, l = 0.f;
  const int kend = min(seq, q0 + kAttnQ);   // keys any query of the tile sees
  for (int j0 = 0; j0 < kend; j0 += kAttnK) {
    __syncthreads();   // everyone is done with the previous tile
    for (int i = threadIdx.x; i < kAttnK * HD; i += kAttnQ * kAttnG) {   // rows past seq: zeros
      const int r = i / HD, c = i % HD;
      const int j = j0 + r;
      const int64_t src = ((int64_t)b * seq + j) * d + h * HD + c;
      kv[0][r][c] = j < seq ? k[src] : 0.f;
      kv[1][r][c] = j < seq ? v[src] : 0.f;
    }
    __syncthreads();
    for (int u = 0; u < kAttnK / kAttnG; ++u) {
      const int jl = grp + kAttnG * u, j = j0 + jl;
      if (j > qi || j >= seq) break;   // keys ascend: past the diagonal (or the end) for this lane
      float sdot = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) sdot = fmaf(qr[e], kv[0][jl][e], sdot);
      const float s = sdot * sc;
      const float mn = fmaxf(m, s);
      const float al = expf(m - mn), p = expf(s - mn);
      l = l * al + p;
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = acc[e] * al + p * kv[1][jl][e];
      m = mn;
    }
  }
  // merge group g = 1, 2, 3 into group 0, in that order
  float *xb = &kv[0][0][0];   // [32 queries][HD + 2]
  for (int gsrc = 1; gsrc < kAttnG; ++gsrc) {
    __syncthreads();
    if (grp == gsrc) {
      float *row = xb + lq * (HD + 2);
#pragma unroll
      for (int e = 0; e < HD; ++e) row[e] = acc[e];
      row[HD] = m;
      row[HD + 1] = l;
    }
    __syncthreads();
    if (grp == 0) {
      const float *row = xb + lq * (HD + 2);
      const float m1 = row[HD], l1 = row[HD + 1];
      const float mn = fmaxf(m, m1);
      const float a0 = expf(m - mn), a1 = expf(m1 - mn);   // m1 = -inf (no keys): a1 = 0
      l = l * a0 + l1 * a1;
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = acc[e] * a0 + row[e] * a1;
      m = mn;
    }
  }
  if (grp != 0 || qi >= seq) return;
  float *op = o + ((int64_t)b * seq + qi) * d + h * HD;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < HD; ++e) op[e] = acc[e] * inv;
  if (lse) lse[((int64_t)b * n_heads + h) * seq + qi] = m + logf(l);   // [batch][n_heads][seq]: the backward's statistic
}

hipError_t attn_f32_launch(const float *q, const float *k, const float *v, float *o, int batch, int seq,
                           int n_heads, int head_dim, hipStream_t s, float *lse) {
  if (batch * n_heads * seq == 0) return hipSuccess;
  const dim3 grid((seq + kAttnQ - 1) / kAttnQ, batch * n_heads);
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kAttnQ * kAttnG), 0, s, q, k, v, o, lse, batch, seq, n_heads);
  else if (head_dim == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kAttnQ * kAttnG), 0, s, q, k, v, o, lse, batch, seq,
                       n_heads);
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
