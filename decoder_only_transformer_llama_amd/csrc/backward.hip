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

// Both gradient kernels run on the matrix cores (v_mfma_f32_32x32x2_f32)
// over 32 x 32 tiles. A workgroup owns one 32-query tile (dQ) or one 32-key
// tile (dK, dV); its four wavefronts take the other side's tiles in turn and
// their sums are added in wavefront order at the end (deterministic). Each
// wavefront stages its tiles in a private LDS region, rows padded by 4
// floats so that the row-wise 16-byte operand reads of the 32 lanes of a
// half-wave fall on distinct banks. The score-side products contract the head
// dimension with half-wave g taking entries g*HD/2 .. g*HD/2 + HD/2 - 1; the
// gradient products contract keys (or queries) in the order the accumulators
// hold them (8*(kk/4) + 4g + kk%4 at step kk), so P and dS enter them straight
// from the lane's registers.
constexpr int kBwdT = 32;   // keys or queries per tile

DEV void bwd_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16-byte piece it of rows [r0, r0 + 32) of head h (row past seq: the last row).
template <int HD>
DEV f32x4 bwd_piece(const float *src, int b, int h, int r0, int seq, int n_heads, int it) {
  const int i = (threadIdx.x & 63) + 64 * it, row = i / (HD / 4), c = 4 * (i % (HD / 4));
  return *(const f32x4 *)(src + ((int64_t)b * seq + min(r0 + row, seq - 1)) * n_heads * HD + (int64_t)h * HD + c);
}
template <int HD>
DEV void bwd_put(float *dst, const f32x4 &v, int it) {
  const int i = (threadIdx.x & 63) + 64 * it, row = i / (HD / 4), c = 4 * (i % (HD / 4));
  *(f32x4 *)&dst[row * (HD + 4) + c] = v;
}

// Score-side product of one 32 x 32 tile: C[m][n] = sum_e A[m][e] B[n][e], A
// rows m from the LDS tile (row l32), B as the lane's own HD/2 entries.
template <int HD>
DEV f32x16 bwd_rows_product(const float *tile, const float *breg) {
  constexpr int HH = HD / 2;
  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  f32x16 c0, c1;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = 0.f;
#pragma unroll
  for (int j = 0; j < HH / 4; ++j) {
    const f32x4 a = *(const f32x4 *)&tile[l32 * (HD + 4) + g * HH + 4 * j];
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], breg[4 * j], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], breg[4 * j + 1], c1, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], breg[4 * j + 2], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], breg[4 * j + 3], c1, 0, 0, 0);
  }
  return c0 + c1;
}

// Gradient-side product: acc[e-block][...] += tile^T[e][row] * w[row][col],
// contracting the 32 rows of the LDS tile in accumulator order, w[kk] from
// the lane's registers.
template <int HD, int NA, int OFF>
DEV void bwd_cols_product(f32x16 (&acc)[NA], const float *tile, const float (&wv)[16]) {
  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int e = 0; e < HD / 32; ++e)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int row = 8 * (kk >> 2) + 4 * g + (kk & 3);
      acc[OFF + e] =
          __builtin_amdgcn_mfma_f32_32x32x2f32(tile[row * (HD + 4) + 32 * e + l32], wv[kk], acc[OFF + e], 0, 0, 0);
    }
}

// Adds wavefronts 1..3's accumulators (NA of them, 16 floats per lane each)
// into wavefront 0's, in order; returns false on wavefronts 1..3.
template <int NA>
DEV bool bwd_merge(f32x16 (&acc)[NA], float *lds, int stride) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (w > 0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) lds[w * stride + (a * 16 + r) * 64 + lane] = acc[a][r];
  }
  __syncthreads();
  if (w > 0) return false;
  for (int src = 1; src < 4; ++src)
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][r] += lds[src * stride + (a * 16 + r) * 64 + lane];
  return true;
}

// Key/value gradients of one 32-key tile: dV^T = dO^T P and dK^T = Q^T dS over
// the query tiles at or after it (causal). The query tiles are split into
// gridDim.z contiguous ranges, one per workgroup: with one range the tile's
// dk (scaled) and dv are stored; with several, range z stores its unscaled
// sums to part[z] ([2][rows][d]: dk then dv) and attn_bwd_kv_sum_kernel adds
// the ranges in order. Per query tile: S = Q K^T and dP = dO V^T (query rows,
// a lane holds 16 queries of one key), P = exp(S scale - lse), dS = P (dP - D).
template <int HD>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(const float *q, const float *k, const float *v,
                                                               const float *dout, const float *lse,
                                                               const float *delta, float *dk, float *dv, int seq,
                                                               int n_heads, float scale, float *part) {
  constexpr int HH = HD / 2, NEB = HD / 32, NV4 = kBwdT * HD / 4 / 64;
  constexpr int TS = kBwdT * (HD + 4);   // floats of one staged tile
  constexpr int WS = 2 * TS + 2 * kBwdT;  // per wavefront: Q, dO, lse, D
  static_assert(2 * NEB * 16 * 64 <= WS, "merge buffer fits a wavefront's region");
  __shared__ float lds[4 * WS];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y, b = bh / n_heads, h = bh % n_heads;
  const int k0 = blockIdx.x * kBwdT, kj = k0 + l32;
  const int d = n_heads * HD;
  float *sq = lds + w * WS, *so = sq + TS, *sl = so + TS, *sd = sl + kBwdT;
  // this lane's key and value rows, entries g*HH .. (B operands of S and dP)
  float kr[HH], vr[HH];
  {
    const int64_t base = ((int64_t)b * seq + min(kj, seq - 1)) * d + (int64_t)h * HD + g * HH;
#pragma unroll
    for (int i = 0; i < HH; i += 4) {
      *(f32x4 *)&kr[i] = *(const f32x4 *)(k + base + i);
      *(f32x4 *)&vr[i] = *(const f32x4 *)(v + base + i);
    }
  }
  f32x16 acc[2 * NEB];   // dK^T blocks, then dV^T blocks
#pragma unroll
  for (int a = 0; a < 2 * NEB; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[a][r] = 0.f;
  const int nqt = (seq + kBwdT - 1) / kBwdT;
  const int it0 = k0 / kBwdT, nit = nqt - it0, nz = gridDim.z, z = blockIdx.z;
  const int ib = it0 + (int)((int64_t)nit * z / nz), ie = it0 + (int)((int64_t)nit * (z + 1) / nz);
  f32x4 qn[NV4], on[NV4];
  float ln = 0.f, dn = 0.f;
  auto load = [&](int it) {
    const int q0 = it * kBwdT;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      qn[i] = bwd_piece<HD>(q, b, h, q0, seq, n_heads, i);
      on[i] = bwd_piece<HD>(dout, b, h, q0, seq, n_heads, i);
    }
    const int qi = min(q0 + l32, seq - 1);
    ln = lse[(int64_t)bh * seq + qi];
    dn = delta[(int64_t)bh * seq + qi];
  };
  // hd 128 keeps 2 x 64 key/value entries and 2 x 64 accumulators per lane:
  // the next tile is then loaded after the current one is multiplied, not
  // during (prefetching it as well spills)
  constexpr bool kPrefetch = HD <= 64;
  if (kPrefetch && ib + w < ie) load(ib + w);
  for (int it = ib + w; it < ie; it += 4) {
    const int q0 = it * kBwdT;
    if (!kPrefetch) load(it);
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      bwd_put<HD>(sq, qn[i], i);
      bwd_put<HD>(so, on[i], i);
    }
    if (g == 0) {
      sl[l32] = ln;
      sd[l32] = dn;
    }
    bwd_wave_sync();
    if (kPrefetch) load(min(it + 4, ie - 1));
    const f32x16 st = bwd_rows_product<HD>(sq, kr);   // S[query][key]
    const f32x16 dp = bwd_rows_product<HD>(so, vr);   // dP[query][key]
    float pw[16], dsw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = 8 * (r >> 2) + 4 * g + (r & 3), qi = q0 + ql;
      const bool ok = qi < seq && kj <= qi;
      pw[r] = ok ? expf(st[r] * scale - sl[ql]) : 0.f;
      dsw[r] = pw[r] * (dp[r] - sd[ql]);
    }
    bwd_cols_product<HD, 2 * NEB, NEB>(acc, so, pw);   // dV^T[e][key] += dO^T P
    bwd_cols_product<HD, 2 * NEB, 0>(acc, sq, dsw);    // dK^T[e][key] += Q^T dS
    bwd_wave_sync();
  }
  if (!bwd_merge<2 * NEB>(acc, lds, WS)) return;
  if (kj >= seq) return;
  const int64_t rd = (int64_t)gridDim.y / n_heads * seq * d;   // rows x d of one gradient
  float *pk = part + (int64_t)z * 2 * rd, *pv = pk + rd;
  const int64_t o = ((int64_t)b * seq + kj) * d + (int64_t)h * HD;
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int e0 = 32 * e + 8 * rq + 4 * g;
      const f32x4 vk = {acc[e][4 * rq], acc[e][4 * rq + 1], acc[e][4 * rq + 2], acc[e][4 * rq + 3]};
      const f32x4 vv = {acc[NEB + e][4 * rq], acc[NEB + e][4 * rq + 1], acc[NEB + e][4 * rq + 2],
                        acc[NEB + e][4 * rq + 3]};
      if (nz == 1) {
        *(f32x4 *)(dk + o + e0) = vk * scale;
        *(f32x4 *)(dv + o + e0) = vv;
      } else {
        *(f32x4 *)(pk + o + e0) = vk;
        *(f32x4 *)(pv + o + e0) = vv;
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

// Query gradients of one 32-query tile: dQ^T = K^T dS^T over the key tiles at
// or before it. Per key tile: S^T = K Q^T and dP^T = V dO^T (key rows, a lane
// holds 16 keys of one query), P^T = exp(S^T scale - lse), dS^T = P^T (dP^T - D).
template <int HD>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(const float *q, const float *k, const float *v,
                                                             const float *dout, const float *lse, const float *delta,
                                                             float *dq, int seq, int n_heads, float scale) {
  constexpr int HH = HD / 2, NEB = HD / 32, NV4 = kBwdT * HD / 4 / 64;
  constexpr int TS = kBwdT * (HD + 4);
  constexpr int WS = 2 * TS;   // per wavefront: K, V
  static_assert(NEB * 16 * 64 <= WS, "merge buffer fits a wavefront's region");
  __shared__ float lds[4 * WS];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y, b = bh / n_heads, h = bh % n_heads;
  const int q0 = blockIdx.x * kBwdT, qi = q0 + l32;
  const int d = n_heads * HD;
  float *sk = lds + w * WS, *sv = sk + TS;
  float qr[HH], dor[HH];
  {
    const int64_t base = ((int64_t)b * seq + min(qi, seq - 1)) * d + (int64_t)h * HD + g * HH;
#pragma unroll
    for (int i = 0; i < HH; i += 4) {
      *(f32x4 *)&qr[i] = *(const f32x4 *)(q + base + i);
      *(f32x4 *)&dor[i] = *(const f32x4 *)(dout + base + i);
    }
  }
  const float lq = lse[(int64_t)bh * seq + min(qi, seq - 1)], dq_d = delta[(int64_t)bh * seq + min(qi, seq - 1)];
  f32x16 acc[NEB];
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[e][r] = 0.f;
  const int nkt = (min(q0 + kBwdT, seq) - 1) / kBwdT + 1;   // key tiles up to the tile's last query
  f32x4 kn[NV4], vn[NV4];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      kn[i] = bwd_piece<HD>(k, b, h, kt * kBwdT, seq, n_heads, i);
      vn[i] = bwd_piece<HD>(v, b, h, kt * kBwdT, seq, n_heads, i);
    }
  };
  if (w < nkt) load(w);
  for (int kt = w; kt < nkt; kt += 4) {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      bwd_put<HD>(sk, kn[i], i);
      bwd_put<HD>(sv, vn[i], i);
    }
    bwd_wave_sync();
    load(min(kt + 4, nkt - 1));
    const f32x16 st = bwd_rows_product<HD>(sk, qr);    // S^T[key][query]
    const f32x16 dp = bwd_rows_product<HD>(sv, dor);   // dP^T[key][query]
    float dsw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * kBwdT + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool ok = qi < seq && key <= qi;
      const float p = ok ? expf(st[r] * scale - lq) : 0.f;
      dsw[r] = p * (dp[r] - dq_d);
    }
    bwd_cols_product<HD, NEB, 0>(acc, sk, dsw);   // dQ^T[e][query] += K^T dS^T
    bwd_wave_sync();
  }
  if (!bwd_merge<NEB>(acc, lds, WS)) return;
  if (qi >= seq) return;
  float *op = dq + ((int64_t)b * seq + qi) * d + (int64_t)h * HD;
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int e0 = 32 * e + 8 * rq + 4 * g;
      *(f32x4 *)(op + e0) = f32x4{acc[e][4 * rq], acc[e][4 * rq + 1], acc[e][4 * rq + 2], acc[e][4 * rq + 3]} * scale;
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
  // key-tile workgroups; split their query loops into ranges (when a partial
  // buffer is given) only while there are fewer than one per compute unit
  const int tiles = (seq + kBwdT - 1) / kBwdT;
  int nz = 1;
  if (kv_part)
    while (nz < kAttnBwdKvRanges && (int64_t)tiles * batch * n_heads * nz < 256) nz *= 2;
  const dim3 gkv(tiles, batch * n_heads, nz), gq(tiles, batch * n_heads);
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
