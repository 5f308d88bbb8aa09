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

// fp32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32: fp32 products,
// fp32 accumulation): C[m][n] = sum_k A(m, k) B(k, n) (+ R[m][n]) (+ C[m][n]
// when accumulating), with A(m, k) = A[m sam + k sak] and B(k, n) =
// B[k sbk + n sbn]. A_KC / B_KC: the operand is contiguous along K (sak == 1 /
// sbk == 1), else along M / N (sam == 1 / sbn == 1); tiles arrive as 16-byte
// vectors along the contiguous direction. One workgroup = 4 wavefronts
// computing a 64 x 64 tile (32 x 32 each); K in steps of 16 through a 2-stage
// LDS ring whose rows [k][m] are padded to 96 floats, so the two half-waves of
// an operand read (rows k and k + 1) fall on disjoint banks.
constexpr int kMfT = 64, kMfK = 16, kMfLd = 96;
template <bool KC>
DEV void mf_load(const float *P, int64_t s_row, int64_t s_k, int r0, int rows, int k0, int K, f32x4 &v) {
  const int t = threadIdx.x;
  if (KC) {   // row r = t / 4 holds k0 + 4 (t % 4) .. +3 contiguously
    const int r = r0 + t / 4, k = k0 + 4 * (t % 4);
    if (r < rows && k + 3 < K) {
      v = *(const f32x4 *)(P + (int64_t)r * s_row + k);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (r < rows && k + e < K) ? P[(int64_t)r * s_row + k + e] : 0.f;
    }
  } else {    // k row t / 16 holds rows r0 + 4 (t % 16) .. +3 contiguously
    const int k = k0 + t / 16, r = r0 + 4 * (t % 16);
    if (k < K && r + 3 < rows) {
      v = *(const f32x4 *)(P + (int64_t)k * s_k + r);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k < K && r + e < rows) ? P[(int64_t)k * s_k + r + e] : 0.f;
    }
  }
}
template <bool KC>
DEV void mf_store(float (*S)[kMfLd], const f32x4 &v) {
  const int t = threadIdx.x;
  if (KC) {
#pragma unroll
    for (int e = 0; e < 4; ++e) S[4 * (t % 4) + e][t / 4] = v[e];
  } else {
    *(f32x4 *)&S[t / 16][4 * (t % 16)] = v;
  }
}

template <bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void gemm_f32_mfma_kernel(const float *A, int64_t sam, int64_t sak, const float *B,
                                                            int64_t sbk, int64_t sbn, float *C, const float *R, int M,
                                                            int N, int K, int accumulate) {
  __shared__ float As[2][kMfK][kMfLd], Bs[2][kMfK][kMfLd];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.y * kMfT, n0 = blockIdx.x * kMfT;
  const int mw = 32 * (w >> 1), nw = 32 * (w & 1);   // this wavefront's 32 x 32 block of the tile
  const int nk = (K + kMfK - 1) / kMfK;
  f32x4 va, vb;
  mf_load<A_KC>(A, sam, sak, m0, M, 0, K, va);
  mf_load<B_KC>(B, sbn, sbk, n0, N, 0, K, vb);
  mf_store<A_KC>(As[0], va);
  mf_store<B_KC>(Bs[0], vb);
  __syncthreads();
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {   // next tile: global -> registers while this one is multiplied
      mf_load<A_KC>(A, sam, sak, m0, M, (kt + 1) * kMfK, K, va);
      mf_load<B_KC>(B, sbn, sbk, n0, N, (kt + 1) * kMfK, K, vb);
    }
#pragma unroll
    for (int kk = 0; kk < kMfK / 2; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[st][2 * kk + g][mw + l32], Bs[st][2 * kk + g][nw + l32], acc, 0,
                                                 0, 0);
    if (more) {   // the other stage was last read before the previous barrier
      mf_store<A_KC>(As[st ^ 1], va);
      mf_store<B_KC>(Bs[st ^ 1], vb);
    }
    __syncthreads();
  }
  const int n = n0 + nw + l32;
  if (n >= N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + mw + 8 * (r >> 2) + 4 * g + (r & 3);
    if (m >= M) continue;
    const int64_t o = (int64_t)m * N + n;
    C[o] = acc[r] + (R ? R[o] : 0.f) + (accumulate ? C[o] : 0.f);
  }
}

// The matrix-core path when the contiguous strides allow 16-byte vectors;
// hipErrorNotSupported otherwise (the caller then uses the VALU kernel).
hipError_t gemm_f32_mfma_launch(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk, int64_t sbn,
                                float *C, const float *R, int M, int N, int K, int accumulate, hipStream_t s) {
  const bool a_kc = sak == 1, b_kc = sbk == 1;
  const int64_t sa = a_kc ? sam : sak, sb = b_kc ? sbn : sbk;   // strides between the 16-byte runs
  if ((!a_kc && sam != 1) || (!b_kc && sbn != 1) || sa % 4 || sb % 4 || ((uintptr_t)A | (uintptr_t)B) % 16)
    return hipErrorNotSupported;
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((N + kMfT - 1) / kMfT, (M + kMfT - 1) / kMfT);
#define MF_CASE(AK, BK)                                                                                          \
  if (a_kc == AK && b_kc == BK) {                                                                                \
    hipLaunchKernelGGL((gemm_f32_mfma_kernel<AK, BK>), grid, dim3(256), 0, s, A, sam, sak, B, sbk, sbn, C, R, M, \
                       N, K, accumulate);                                                                        \
    return hipGetLastError();                                                                                    \
  }
  MF_CASE(true, true) MF_CASE(true, false) MF_CASE(false, true) MF_CASE(false, false)
#undef MF_CASE
  return hipErrorNotSupported;
}

hipError_t gemm_f32_strided_launch(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk,
                                   int64_t sbn, float *C, int M, int N, int K, int accumulate, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const hipError_t e = gemm_f32_mfma_launch(A, sam, sak, B, sbk, sbn, C, nullptr, M, N, K, accumulate, s);
  if (e != hipErrorNotSupported) return e;
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

// Key/value gradients of one 64-key tile. The causal loop over query tiles
// (those at or after the key tile) is split into gridDim.z contiguous ranges,
// one per workgroup: with one range the tile's dk (scaled) and dv are stored;
// with several, range z stores its unscaled sums to part[z] ([2][rows][d]:
// dk then dv) and attn_bwd_kv_sum_kernel adds the ranges in order.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const float *q, const float *k, const float *v,
                                                            const float *dout, const float *lse,
                                                            const float *delta, float *dk, float *dv, int seq,
                                                            int n_heads, float scale, float *part) {
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
  const int it0 = k0 / kBwdBQ, nit = nqt - it0, nz = gridDim.z, z = blockIdx.z;
  const int ib = it0 + (int)((int64_t)nit * z / nz), ie = it0 + (int)((int64_t)nit * (z + 1) / nz);
  for (int it = ib; it < ie; ++it) {   // causal: queries at or after the key tile, this range
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
  const int64_t rd = (int64_t)gridDim.y / n_heads * seq * d;   // rows x d of one gradient
  float *pk = part + (int64_t)z * 2 * rd, *pv = pk + rd;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kj = k0 + 4 * kq + j;
    if (kj >= seq) continue;
    const int64_t o = ((int64_t)b * seq + kj) * d + (int64_t)h * HD + ce * CW;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      if (nz == 1) {
        dk[o + c] = accK[j][c] * scale;
        dv[o + c] = accV[j][c];
      } else {
        pk[o + c] = accK[j][c];
        pv[o + c] = accV[j][c];
      }
    }
  }
}

// dk = scale * (part[0].k + part[1].k + ...), dv = part[0].v + ..., ranges in order.
__global__ void attn_bwd_kv_sum_kernel(const float *part, int nz, int64_t rd, float scale, float *dk, float *dv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rd) return;
  float sk = 0.f, sv = 0.f;
  for (int z = 0; z < nz; ++z) {
    sk += part[(int64_t)z * 2 * rd + i];
    sv += part[(int64_t)z * 2 * rd + rd + i];
  }
  dk[i] = sk * scale;
  dv[i] = sv;
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
                           int n_heads, int head_dim, hipStream_t s, float *kv_part) {
  const int64_t rows = (int64_t)batch * n_heads * seq;
  if (rows == 0) return hipSuccess;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bwd_delta_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, o, dout, delta,
                     batch, seq, n_heads, head_dim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale = 1.0f / sqrtf((float)head_dim);
  const int nz = kv_part ? kAttnBwdKvRanges : 1;
  const dim3 gkv((seq + kBwdBK - 1) / kBwdBK, batch * n_heads, nz), gq((seq + kBwdBQ - 1) / kBwdBQ, batch * n_heads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, gkv, dim3(256), 0, s, q, k, v, dout, lse, delta, dk, dv, seq,
                       n_heads, scale, kv_part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gq, dim3(256), 0, s, q, k, v, dout, lse, delta, dq, seq, n_heads,
                       scale);
  } else {
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, gkv, dim3(256), 0, s, q, k, v, dout, lse, delta, dk, dv, seq,
                       n_heads, scale, kv_part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gq, dim3(256), 0, s, q, k, v, dout, lse, delta, dq, seq, n_heads,
                       scale);
  }
  if ((e = hipGetLastError()) != hipSuccess || nz == 1) return e;
  const int64_t rd = rows * head_dim;
  hipLaunchKernelGGL(attn_bwd_kv_sum_kernel, dim3((unsigned)((rd + 255) / 256)), dim3(256), 0, s, kv_part, nz, rd,
                     scale, dk, dv);
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
// dg[c] = sum_r dy[r][c] x[r][c] rstd[r]: one workgroup per 64 columns,
// 16 row phases (rows p, p + 16, ...) summed per thread, then the phases
// added in a fixed order through LDS (deterministic, no atomics).
constexpr int kGainCols = 64, kGainPhases = 16;
__global__ __launch_bounds__(kGainCols * kGainPhases) void rmsnorm_bwd_gain_kernel(
    const float *x, const float *dy, const float *rstd, float *dg, int64_t rows, int dim) {
  __shared__ float part[kGainPhases][kGainCols];
  const int cl = threadIdx.x % kGainCols, ph = threadIdx.x / kGainCols;
  const int c = blockIdx.x * kGainCols + cl;
  float acc = 0.f;
  if (c < dim) {
#pragma unroll 8
    for (int64_t r = ph; r < rows; r += kGainPhases) acc = fmaf(dy[r * dim + c], x[r * dim + c] * rstd[r], acc);
  }
  part[ph][cl] = acc;
  __syncthreads();
  if (ph == 0 && c < dim) {
    float t = 0.f;
    for (int p = 0; p < kGainPhases; ++p) t += part[p][cl];
    dg[c] = t;
  }
}

hipError_t rmsnorm_bwd_launch(const float *x, const float *g, const float *dy, const float *add, float *dx,
                              float *dg, float *rstd, int64_t rows, int dim, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, g, dy, add, dx, rstd,
                     rows, dim, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rmsnorm_bwd_gain_kernel, dim3((dim + kGainCols - 1) / kGainCols), dim3(kGainCols * kGainPhases),
                     0, s, x, dy, rstd, dg, rows, dim);
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
