// Backward pass of the pre-norm block in fp32: the kernels behind
// llama_causal_attn_backward, llama_block_train_forward / llama_block_backward
// and llama_axpby.
//
// What is computed is the chain rule of the forward (the manual backward of
// the training note's "Efficient Training Implementation"; attention backward
// after its FlashAttention-inspired variant: the S x S probabilities are
// recomputed tile by tile from q, k and the forward's per-row log-sum-exp,
// never stored):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_e dO_ie O_ie,
//   dQ = dS K / sqrt(hd),  dK = dS^T Q / sqrt(hd)
// Two kernels share the recomputation: one workgroup per 64-key tile
// accumulates dK, dV over the query tiles at or after it (causal), one per
// 32-query tile accumulates dQ over the key tiles at or before it. Neither
// uses atomics, so the gradients are deterministic.
#include "common.h"
#include "internal.h"

namespace llama {

// ------------------------------------------------------------------ strided fp32 GEMM
// C[m, n] = (accumulate ? C[m, n] : 0) + sum_k A(m, k) B(k, n) with
// A(m, k) = A[m * sam + k * sak] and B(k, n) = B[k * sbk + n * sbn]: the
// plain, transposed-left and transposed-right products of a backward pass.
// 64 x 64 tiles through LDS, 4 x 4 outputs per thread; the tile loads walk the
// unit-stride index fastest.
__global__ __launch_bounds__(256) void gemm_f32_strided_kernel(const float *A, int64_t sam, int64_t sak,
                                                               const float *B, int64_t sbk, int64_t sbn,
                                                               float *C, int M, int N, int K, int accumulate) {
  __shared__ float As[16][65], Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      int r, c;
      if (sam == 1) {
        r = i % 64;
        c = i / 64;
      } else {
        r = i / 16;
        c = i % 16;
      }
      As[c][r] = (m0 + r < M && k0 + c < K) ? A[(int64_t)(m0 + r) * sam + (int64_t)(k0 + c) * sak] : 0.f;
      if (sbn == 1) {
        r = i % 64;
        c = i / 64;
      } else {
        r = i / 16;
        c = i % 16;
      }
      Bs[c][r] = (n0 + r < N && k0 + c < K) ? B[(int64_t)(k0 + c) * sbk + (int64_t)(n0 + r) * sbn] : 0.f;
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
        C[o] = acc[i][j] + (accumulate ? C[o] : 0.f);
      }
    }
}

hipError_t gemm_f32_strided_launch(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk,
                                   int64_t sbn, float *C, int M, int N, int K, int accumulate, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_f32_strided_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, A, sam, sak, B,
                     sbk, sbn, C, M, N, K, accumulate);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention backward
// D[(b * H + h) * seq + i] = sum_e dO[b, i, h, e] * O[b, i, h, e]
__global__ void attn_bwd_delta_kernel(const float *o, const float *dout, float *delta, int batch, int seq,
                                      int n_heads, int hd) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * n_heads * seq) return;
  const int i = (int)(idx % seq), h = (int)((idx / seq) % n_heads), b = (int)(idx / ((int64_t)seq * n_heads));
  const int64_t base = ((int64_t)b * seq + i) * n_heads * hd + (int64_t)h * hd;
  float acc = 0.f;
  for (int e = 0; e < hd; ++e) acc = fmaf(dout[base + e], o[base + e], acc);
  delta[idx] = acc;
}

constexpr int kBwdBK = 64;   // keys per tile
constexpr int kBwdBQ = 32;   // queries per tile

// Rows [r0, r0 + n) of head h of sequence b into an LDS tile [n][HD + 1];
// rows past seq are zero.
template <int HD>
DEV void bwd_load_rows(float (*dst)[HD + 1], const float *src, int b, int h, int r0, int n, int seq,
                       int n_heads) {
  const int d = n_heads * HD;
  for (int i = threadIdx.x; i < n * HD; i += 256) {
    const int r = i / HD, e = i % HD;
    const int row = r0 + r;
    dst[r][e] = row < seq ? src[((int64_t)b * seq + row) * d + (int64_t)h * HD + e] : 0.f;
  }
}

// Scores, probabilities and dS of 2 queries (rows 2*tq, 2*tq+1 of the query
// tile) x 4 keys (rows 4*tk .. 4*tk+3 of the key tile), written to sP / sdS.
template <int HD>
DEV void bwd_scores(const float (*sQ)[HD + 1], const float (*sdO)[HD + 1], const float (*sK)[HD + 1],
                    const float (*sV)[HD + 1], const float *sL, const float *sD, int q0, int k0, int seq,
                    float scale, float (*sP)[kBwdBK + 1], float (*sdS)[kBwdBK + 1]) {
  const int tq = threadIdx.x / 16, tk = threadIdx.x % 16;
  float s[2][4] = {}, dp[2][4] = {};
  for (int e = 0; e < HD; ++e) {
    const float q0v = sQ[2 * tq][e], q1v = sQ[2 * tq + 1][e];
    const float o0v = sdO[2 * tq][e], o1v = sdO[2 * tq + 1][e];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float kv = sK[4 * tk + j][e], vv = sV[4 * tk + j][e];
      s[0][j] = fmaf(q0v, kv, s[0][j]);
      s[1][j] = fmaf(q1v, kv, s[1][j]);
      dp[0][j] = fmaf(o0v, vv, dp[0][j]);
      dp[1][j] = fmaf(o1v, vv, dp[1][j]);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = 2 * tq + a, qi = q0 + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * tk + j, kj = k0 + c;
      const bool ok = qi < seq && kj <= qi;   // kj < seq follows
      const float p = ok ? expf(s[a][j] * scale - sL[r]) : 0.f;
      if (sP) sP[r][c] = p;
      sdS[r][c] = p * (dp[a][j] - sD[r]);
    }
  }
}

template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const float *q, const float *k, const float *v,
                                                            const float *dout, const float *lse,
                                                            const float *delta, float *dk, float *dv, int seq,
                                                            int n_heads, float scale) {
  constexpr int CW = HD / 16;
  __shared__ float sK[kBwdBK][HD + 1], sV[kBwdBK][HD + 1];
  __shared__ float sQ[kBwdBQ][HD + 1], sdO[kBwdBQ][HD + 1];
  __shared__ float sP[kBwdBQ][kBwdBK + 1], sdS[kBwdBQ][kBwdBK + 1];
  __shared__ float sL[kBwdBQ], sD[kBwdBQ];
  const int bh = blockIdx.y, b = bh / n_heads, h = bh % n_heads;
  const int k0 = blockIdx.x * kBwdBK;
  bwd_load_rows<HD>(sK, k, b, h, k0, kBwdBK, seq, n_heads);
  bwd_load_rows<HD>(sV, v, b, h, k0, kBwdBK, seq, n_heads);
  const int kq = threadIdx.x / 16, ce = threadIdx.x % 16;   // keys 4*kq.., channels ce*CW..
  float accK[4][CW] = {}, accV[4][CW] = {};
  const int nqt = (seq + kBwdBQ - 1) / kBwdBQ;
  for (int it = k0 / kBwdBQ; it < nqt; ++it) {   // causal: queries at or after the key tile
    const int q0 = it * kBwdBQ;
    __syncthreads();   // the previous tile's readers are done (and sK/sV are loaded)
    bwd_load_rows<HD>(sQ, q, b, h, q0, kBwdBQ, seq, n_heads);
    bwd_load_rows<HD>(sdO, dout, b, h, q0, kBwdBQ, seq, n_heads);
    if (threadIdx.x < kBwdBQ) {
      const int qi = q0 + threadIdx.x;
      sL[threadIdx.x] = qi < seq ? lse[(int64_t)bh * seq + qi] : 0.f;
      sD[threadIdx.x] = qi < seq ? delta[(int64_t)bh * seq + qi] : 0.f;
    }
    __syncthreads();
    bwd_scores<HD>(sQ, sdO, sK, sV, sL, sD, q0, k0, seq, scale, sP, sdS);
    __syncthreads();
    for (int r = 0; r < kBwdBQ; ++r) {
      float pr[4], dsr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pr[j] = sP[r][4 * kq + j];
        dsr[j] = sdS[r][4 * kq + j];
      }
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const float ov = sdO[r][ce * CW + c], qv = sQ[r][ce * CW + c];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accV[j][c] = fmaf(pr[j], ov, accV[j][c]);
          accK[j][c] = fmaf(dsr[j], qv, accK[j][c]);
        }
      }
    }
  }
  const int d = n_heads * HD;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kj = k0 + 4 * kq + j;
    if (kj >= seq) continue;
    const int64_t o = ((int64_t)b * seq + kj) * d + (int64_t)h * HD + ce * CW;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      dk[o + c] = accK[j][c] * scale;
      dv[o + c] = accV[j][c];
    }
  }
}

template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const float *q, const float *k, const float *v,
                                                          const float *dout, const float *lse, const float *delta,
                                                          float *dq, int seq, int n_heads, float scale) {
  constexpr int CW = HD / 16;
  __shared__ float sK[kBwdBK][HD + 1], sV[kBwdBK][HD + 1];
  __shared__ float sQ[kBwdBQ][HD + 1], sdO[kBwdBQ][HD + 1];
  __shared__ float sdS[kBwdBQ][kBwdBK + 1];
  __shared__ float sL[kBwdBQ], sD[kBwdBQ];
  const int bh = blockIdx.y, b = bh / n_heads, h = bh % n_heads;
  const int q0 = blockIdx.x * kBwdBQ;
  bwd_load_rows<HD>(sQ, q, b, h, q0, kBwdBQ, seq, n_heads);
  bwd_load_rows<HD>(sdO, dout, b, h, q0, kBwdBQ, seq, n_heads);
  if (threadIdx.x < kBwdBQ) {
    const int qi = q0 + threadIdx.x;
    sL[threadIdx.x] = qi < seq ? lse[(int64_t)bh * seq + qi] : 0.f;
    sD[threadIdx.x] = qi < seq ? delta[(int64_t)bh * seq + qi] : 0.f;
  }
  const int tq = threadIdx.x / 16, tk = threadIdx.x % 16;   // queries 2*tq.., channels tk*CW..
  float acc[2][CW] = {};
  const int last = min(q0 + kBwdBQ, seq) - 1;                // causal: keys up to the last query
  const int nkt = last / kBwdBK + 1;
  for (int jt = 0; jt < nkt; ++jt) {
    const int k0 = jt * kBwdBK;
    __syncthreads();   // the previous tile's readers are done (and sQ/sdO/sL/sD are loaded)
    bwd_load_rows<HD>(sK, k, b, h, k0, kBwdBK, seq, n_heads);
    bwd_load_rows<HD>(sV, v, b, h, k0, kBwdBK, seq, n_heads);
    __syncthreads();
    bwd_scores<HD>(sQ, sdO, sK, sV, sL, sD, q0, k0, seq, scale, nullptr, sdS);
    __syncthreads();
    for (int kk = 0; kk < kBwdBK; ++kk) {
      const float d0 = sdS[2 * tq][kk], d1 = sdS[2 * tq + 1][kk];
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const float kv = sK[kk][tk * CW + c];
        acc[0][c] = fmaf(d0, kv, acc[0][c]);
        acc[1][c] = fmaf(d1, kv, acc[1][c]);
      }
    }
  }
  const int d = n_heads * HD;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int qi = q0 + 2 * tq + a;
    if (qi >= seq) continue;
    const int64_t o = ((int64_t)b * seq + qi) * d + (int64_t)h * HD + tk * CW;
#pragma unroll
    for (int c = 0; c < CW; ++c) dq[o + c] = acc[a][c] * scale;
  }
}

hipError_t attn_bwd_launch(const float *q, const float *k, const float *v, const float *o, const float *dout,
                           const float *lse, float *delta, float *dq, float *dk, float *dv, int batch, int seq,
                           int n_heads, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)batch * n_heads * seq;
  if (rows == 0) return hipSuccess;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bwd_delta_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, o, dout, delta,
                     batch, seq, n_heads, head_dim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale = 1.0f / sqrtf((float)head_dim);
  const dim3 gkv((seq + kBwdBK - 1) / kBwdBK, batch * n_heads), gq((seq + kBwdBQ - 1) / kBwdBQ, batch * n_heads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, gkv, dim3(256), 0, s, q, k, v, dout, lse, delta, dk, dv, seq,
                       n_heads, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gq, dim3(256), 0, s, q, k, v, dout, lse, delta, dq, seq, n_heads,
                       scale);
  } else {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, gkv, dim3(256), 0, s, q, k, v, dout, lse, delta, dk, dv, seq,
                       n_heads, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gq, dim3(256), 0, s, q, k, v, dout, lse, delta, dq, seq, n_heads,
                       scale);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm, SwiGLU, elementwise
// One wavefront per row: r = 1/sqrt(mean(x^2) + eps), n = x r, dn = dy g;
// dx = (add ? add : 0) + r (dn - n mean(dn n)); rstd[row] = r.
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float *x, const float *g, const float *dy,
                                                          const float *add, float *dx, float *rstd, int64_t rows,
                                                          int dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = row * dim;
  float ss = 0.f;
  for (int c = lane; c < dim; c += 64) ss = fmaf(x[base + c], x[base + c], ss);
  const float r = rstd_of(wave_sum(ss), dim, eps);
  float t = 0.f;
  for (int c = lane; c < dim; c += 64) t = fmaf(dy[base + c] * g[c], x[base + c] * r, t);
  const float mean = wave_sum(t) / (float)dim;
  for (int c = lane; c < dim; c += 64) {
    const float n = x[base + c] * r;
    dx[base + c] = (add ? add[base + c] : 0.f) + r * (dy[base + c] * g[c] - n * mean);
  }
  if (lane == 0) rstd[row] = r;
}

// dg[c] = sum over rows of dy[row, c] x[row, c] rstd[row] (one thread per column, rows in order).
__global__ void rmsnorm_bwd_gain_kernel(const float *x, const float *dy, const float *rstd, float *dg, int64_t rows,
                                        int dim) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= dim) return;
  float acc = 0.f;
  for (int64_t r = 0; r < rows; ++r) acc = fmaf(dy[r * dim + c], x[r * dim + c] * rstd[r], acc);
  dg[c] = acc;
}

hipError_t rmsnorm_bwd_launch(const float *x, const float *g, const float *dy, const float *add, float *dx,
                              float *dg, float *rstd, int64_t rows, int dim, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, g, dy, add, dx, rstd,
                     rows, dim, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rmsnorm_bwd_gain_kernel, dim3((dim + 255) / 256), dim3(256), 0, s, x, dy, rstd, dg, rows, dim);
  return hipGetLastError();
}

// u = SiLU(gate) up: d_gate = du up SiLU'(gate), d_up = du SiLU(gate), with
// SiLU'(t) = s (1 + t (1 - s)), s = 1 / (1 + e^-t). d_gate may alias du.
__global__ void swiglu_bwd_kernel(const float *gate, const float *up, const float *du, float *d_gate, float *d_up,
                                  int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float t = gate[i], g = du[i];
  const float sg = 1.0f / (1.0f + expf(-t));
  d_up[i] = g * (t * sg);
  d_gate[i] = g * up[i] * sg * (1.0f + t * (1.0f - sg));
}

hipError_t swiglu_bwd_launch(const float *gate, const float *up, const float *du, float *d_gate, float *d_up,
                             int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gate, up, du, d_gate,
                     d_up, n);
  return hipGetLastError();
}

// z = a x + b y (z may alias x or y).
__global__ void axpby_kernel(float *z, const float *x, const float *y, float a, float b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) z[i] = a * x[i] + b * y[i];
}

hipError_t axpby_launch(float *z, const float *x, const float *y, float a, float b, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(axpby_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, z, x, y, a, b, n);
  return hipGetLastError();
}

}  // namespace llama
