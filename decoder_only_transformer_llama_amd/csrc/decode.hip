// Decode-step kernels (one new token per sequence, batch <= 32). The step is
// bound by HBM: every weight byte and every cached K/V byte is read once.
//
//  - gemv_kernel: skinny split-K product part[s][m][n] = sum_{k in split s}
//    A[m][k] B[n][k] with the batch as the 32 rows of one v_mfma_f32_32x32x16
//    tile. Weights stream from HBM straight into the B-operand registers (each
//    lane reads 64 contiguous bytes of one weight row per step, register
//    double-buffered); the activation operand is a bf16 hi/lo pair so the
//    product is fp32-accurate at bf16 matrix-core rate. K order inside a step
//    is permuted identically for A and B, which leaves the sum unchanged.
//  - the *_combine / resid_norm kernels reduce the split-K partials in a fixed
//    order (deterministic, no atomics) and apply the elementwise work: RMSNorm
//    statistics and gain, RoPE at pos[b], the KV-cache append, SiLU(gate)*up,
//    and the residual adds of the pre-norm block.
//  - dec_attn_kernel: split-sequence attention of one fp32 query over the
//    cached bf16 keys/values (chunks of the cache in parallel, each with its
//    own max and sum), followed by a fixed-order merge of the chunks.
//
// The per-layer formula is the pre-norm block of the paperfordummies.in LLaMA
// page ("The one formula"); the cache of keys and values of earlier tokens is
// the one described on the chenyuan1125.github.io page ("GQA Was Not an
// Original LLaMA Feature"; LLaMA-1 has one K/V head per query head).
#include "common.h"
#include "internal.h"

namespace llama {

DEV bool pos_ok(int p, int max_seq) { return p >= 0 && p < max_seq; }

// ------------------------------------------------------------------ skinny GEMM
// Workgroup = 4 wavefronts x (NTW x 32) output columns over one K range of at
// most KC_MAX. The activation pair for that K range sits in LDS (loaded once,
// rows XOR-swizzled); weights stream from HBM into a DEPTH-deep ring of
// B-operand registers, so DEPTH steps of 64 K are in flight per wavefront.
constexpr int KC_MAX = 512;

template <int NTW, int DEPTH>
__global__ __launch_bounds__(256, 2) void gemv_kernel(const GemvArgs a) {
  __shared__ u32x4 sA[2][32][KC_MAX / 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ks = blockIdx.y * a.k_chunk;
  const int ke = min(a.K, ks + a.k_chunk);
  const int kc8 = (ke - ks) >> 3;

  // activation pair of this K range -> LDS (rows past M are zero)
  for (int idx = tid; idx < 2 * 32 * kc8; idx += 256) {
    const int part = idx / (32 * kc8), rem = idx % (32 * kc8);
    const int m = rem / kc8, c = rem % kc8;
    u32x4 v = {0, 0, 0, 0};
    if (m < a.M) v = *(const u32x4 *)((part ? a.A_lo : a.A_hi) + (int64_t)m * a.K + ks + 8 * c);
    sA[part][m][c ^ (m & 15)] = v;
  }
  __syncthreads();

  const int nw0 = (blockIdx.x * 4 + w) * 32 * NTW;
  if (nw0 >= a.N) return;
  const u16 *brow[NTW];
  bool bok[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = nw0 + 32 * j + l32;
    bok[j] = n < a.N;
    const int nn = bok[j] ? n : 0;
    const u16 *p;
    if (a.b_mode == BMODE_GATEUP) {
      const int blk = nn >> 5;
      p = ((blk & 1) ? a.B1 : a.B0) + (int64_t)((blk >> 1) * 32 + (nn & 31)) * a.K;
    } else if (a.b_mode == BMODE_CONCAT3) {
      const int seg = nn / a.n_seg;
      p = (seg == 0 ? a.B0 : (seg == 1 ? a.B1 : a.B2)) + (int64_t)(nn - seg * a.n_seg) * a.K;
    } else {
      p = a.B0 + (int64_t)nn * a.K;
    }
    brow[j] = p + ks + 32 * g;
  }

  f32x16 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // K order inside a 64-step: lane group g supplies k = 32 g + 8 q + (0..7) at
  // matrix-core step q, identically for the activation and the weights.
  u32x4 ring[DEPTH][NTW][4];
  const int nit = (ke - ks) >> 6;
  auto load = [&](u32x4 (&B)[NTW][4], int it) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        B[j][q] = bok[j] ? *(const u32x4 *)(brow[j] + 64 * it + 8 * q) : u32x4{0, 0, 0, 0};
  };
  auto compute = [&](u32x4 (&B)[NTW][4], int it) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = (8 * it + 4 * g + q) ^ (l32 & 15);
      const bf16x8 ah = as_bf16x8(sA[0][l32][c]);
      const bf16x8 al = as_bf16x8(sA[1][l32][c]);
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        acc[j] = mfma32(ah, as_bf16x8(B[j][q]), acc[j]);
        acc[j] = mfma32(al, as_bf16x8(B[j][q]), acc[j]);
      }
    }
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (d < nit) load(ring[d], d);
  for (int it0 = 0; it0 < nit; it0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int it = it0 + d;
      if (it < nit) {
        compute(ring[d], it);
        if (it + DEPTH < nit) load(ring[d], it + DEPTH);
      }
    }
  }

  float *out = a.part + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = nw0 + 32 * j + l32;
    if (!bok[j]) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * g + (r & 3);
      if (m < a.M) out[(int64_t)m * a.N + n] = acc[j][r];
    }
  }
}

int gemv_ntw(int N) { return N > 8192 ? 2 : 1; }

hipError_t gemv_launch(const GemvArgs &a, hipStream_t s) {
  if (a.k_chunk > KC_MAX || a.k_chunk % 64 || a.K % 64 || a.M > 32) return hipErrorInvalidValue;
  const int ntw = gemv_ntw(a.N);
  const int per_wg = 4 * 32 * ntw;
  dim3 grid((a.N + per_wg - 1) / per_wg, a.splits);
  if (ntw == 2)
    hipLaunchKernelGGL((gemv_kernel<2, 4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<1, 4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ row kernels
DEV float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}

// Row statistics are kept as partial sums of squares, one per 1024-channel
// chunk of the row (ss[b][chunk]); consumers finish rstd in a fixed order.
DEV float rstd_from_parts(const float *ss, int b, int nss, int dim, float eps) {
  float t = 0.f;
  for (int i = 0; i < nss; ++i) t += ss[b * nss + i];
  return rstd_of(t, dim, eps);
}

DEV void chunk_sumsq_store(float v, float *ss, int b, int nss) {
  __shared__ float red[4];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) ss[b * nss + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// grid (dim/1024, batch): x = emb[tok] (f32), pair of x*g, partial sums of squares.
__global__ __launch_bounds__(256) void dec_embed_norm_kernel(const DecodeArgs d, const u16 *emb,
                                                             const int32_t *tok, const u16 *g, float *x,
                                                             float *ss, u16 *xg_hi, u16 *xg_lo) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * 1024 + threadIdx.x * 4;
  const int t = tok[b];
  const bool ok = t >= 0 && t < d.vocab;
  float q = 0.f;
  if (c < d.dim) {
    const int64_t o = (int64_t)b * d.dim + c;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = ok ? bf2f(emb[(int64_t)t * d.dim + c + i]) : __builtin_nanf("");
      q += v[i] * v[i];
    }
    *(f32x4 *)(x + o) = f32x4{v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u16 hi, lo;
      split_pair(v[i] * bf2f(g[c + i]), hi, lo);
      xg_hi[o + i] = hi;
      xg_lo[o + i] = lo;
    }
  }
  chunk_sumsq_store(q, ss, b, gridDim.x);
}

hipError_t dec_embed_norm_launch(const DecodeArgs &d, const uint16_t *emb, const int32_t *tok,
                                 const uint16_t *g, float *x, float *ss, uint16_t *xg_hi, uint16_t *xg_lo,
                                 hipStream_t s) {
  hipLaunchKernelGGL(dec_embed_norm_kernel, dim3((d.dim + 1023) / 1024, d.batch), dim3(256), 0, s, d, emb, tok,
                     g, x, ss, xg_hi, xg_lo);
  return hipGetLastError();
}

// grid (dim/1024, batch): out = res + sum_s part[s] (fixed split order),
// pair of out*g, partial sums of squares of out.
__global__ __launch_bounds__(256) void dec_resid_norm_kernel(const DecodeArgs d, const float *res,
                                                             const float *part, int splits, const u16 *g,
                                                             float *out, float *ss, u16 *og_hi, u16 *og_lo) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * 1024 + threadIdx.x * 4;
  const int64_t stride = (int64_t)d.batch * d.dim;
  float q = 0.f;
  if (c < d.dim) {
    const int64_t o = (int64_t)b * d.dim + c;
    f32x4 v = *(const f32x4 *)(res + o);
    for (int sp = 0; sp < splits; ++sp) v += *(const f32x4 *)(part + sp * stride + o);
    *(f32x4 *)(out + o) = v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q += v[i] * v[i];
      u16 hi, lo;
      split_pair(v[i] * bf2f(g[c + i]), hi, lo);
      og_hi[o + i] = hi;
      og_lo[o + i] = lo;
    }
  }
  chunk_sumsq_store(q, ss, b, gridDim.x);
}

hipError_t dec_resid_norm_launch(const DecodeArgs &d, const float *res, const float *part, int splits,
                                 const uint16_t *g, float *out, float *ss, uint16_t *og_hi, uint16_t *og_lo,
                                 hipStream_t s) {
  hipLaunchKernelGGL(dec_resid_norm_kernel, dim3((d.dim + 1023) / 1024, d.batch), dim3(256), 0, s, d, res, part,
                     splits, g, out, ss, og_hi, og_lo);
  return hipGetLastError();
}

// q = RoPE(rstd * sum part[:, :, 0:d]); k = RoPE(rstd * ...[d:2d]); v = rstd * ...[2d:3d].
// One thread per channel pair; k and v go to cache slot pos[b] (bf16).
__global__ void dec_qkv_combine_kernel(const DecodeArgs d, const float *part, int splits,
                                       const float *ss, float *q, u16 *kc, u16 *vc) {
  const int pairs = 3 * d.dim / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d.batch * pairs) return;
  const int b = idx / pairs, pc = idx % pairs;
  const int n = 2 * pc;
  const int N = 3 * d.dim;
  const int64_t stride = (int64_t)d.batch * N;
  float v0 = 0.f, v1 = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const float2 p2 = *(const float2 *)(part + sp * stride + (int64_t)b * N + n);
    v0 += p2.x;
    v1 += p2.y;
  }
  const float r = rstd_from_parts(ss, b, (d.dim + 1023) / 1024, d.dim, d.eps);
  v0 *= r;
  v1 *= r;
  const int seg = n / d.dim, c = n - seg * d.dim;
  const int hh = c / d.head_dim, e = c % d.head_dim;
  if (seg < 2) {
    const float2 cs = d.rope_tab[b * (d.head_dim / 2) + (e >> 1)];
    const float a0 = v0 * cs.x - v1 * cs.y, a1 = v0 * cs.y + v1 * cs.x;
    v0 = a0;
    v1 = a1;
  }
  if (seg == 0) {
    q[(int64_t)b * d.dim + c] = v0;
    q[(int64_t)b * d.dim + c + 1] = v1;
    return;
  }
  const int p = d.pos[b];
  if (!pos_ok(p, d.max_seq)) return;
  u16 *cache = seg == 1 ? kc : vc;
  const int64_t o = (((int64_t)b * d.n_heads + hh) * d.max_seq + p) * d.head_dim + e;
  *(uint32_t *)(cache + o) = pack2(v0, v1);
}

hipError_t dec_qkv_combine_launch(const DecodeArgs &d, const float *part, int splits, const float *rstd,
                                  float *q, uint16_t *kc, uint16_t *vc, hipStream_t s) {
  const int n = d.batch * 3 * d.dim / 2;
  hipLaunchKernelGGL(dec_qkv_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, d, part, splits, rstd,
                     q, kc, vc);
  return hipGetLastError();
}

// u = SiLU(rstd * gate) * (rstd * up); gate/up partials are interleaved in blocks of 32.
__global__ void dec_gateup_combine_kernel(const DecodeArgs d, const float *part, int splits,
                                          const float *ss, u16 *u_hi, u16 *u_lo) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d.batch * d.hidden) return;
  const int b = idx / d.hidden, j = idx % d.hidden;
  const int N = 2 * d.hidden;
  const int ng = (j >> 5) * 64 + (j & 31);
  const int64_t stride = (int64_t)d.batch * N;
  float gt = 0.f, up = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const float *pp = part + sp * stride + (int64_t)b * N;
    gt += pp[ng];
    up += pp[ng + 32];
  }
  const float r = rstd_from_parts(ss, b, (d.dim + 1023) / 1024, d.dim, d.eps);
  const float u = silu(gt * r) * (up * r);
  u16 hi, lo;
  split_pair(u, hi, lo);
  u_hi[idx] = hi;
  u_lo[idx] = lo;
}

hipError_t dec_gateup_combine_launch(const DecodeArgs &d, const float *part, int splits,
                                     const float *rstd, uint16_t *u_hi, uint16_t *u_lo, hipStream_t s) {
  const int n = d.batch * d.hidden;
  hipLaunchKernelGGL(dec_gateup_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, d, part, splits,
                     rstd, u_hi, u_lo);
  return hipGetLastError();
}

__global__ void dec_head_combine_kernel(const DecodeArgs d, const float *part, int splits,
                                        const float *ss, float *logits) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d.batch * d.vocab) return;
  const int b = idx / d.vocab;
  const int64_t stride = (int64_t)d.batch * d.vocab;
  float v = 0.f;
  for (int sp = 0; sp < splits; ++sp) v += part[sp * stride + idx];
  const float r = rstd_from_parts(ss, b, (d.dim + 1023) / 1024, d.dim, d.eps);
  logits[idx] = pos_ok(d.pos[b], d.max_seq) ? v * r : __builtin_nanf("");
}

hipError_t dec_head_combine_launch(const DecodeArgs &d, const float *part, int splits, const float *rstd,
                                   float *logits, hipStream_t s) {
  const int n = d.batch * d.vocab;
  hipLaunchKernelGGL(dec_head_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, d, part, splits, rstd,
                     logits);
  return hipGetLastError();
}

// ------------------------------------------------------------------ cache attention
// grid (chunk, head, sequence). 16 lanes share one cached key (8 channels
// each), a wavefront covers 4 keys per step. Partial result of the chunk:
// o_part = sum_j e^(s_j - m) v_j, ml_part = (m, sum_j e^(s_j - m)).
template <int HD>
__global__ __launch_bounds__(256) void dec_attn_kernel(const DecodeArgs d, const float *q, const u16 *kc,
                                                       const u16 *vc, int chunk, int n_chunks,
                                                       float *o_part, float *ml_part) {
  constexpr int LPK = HD / 8;          // lanes per key
  constexpr int KPW = 64 / LPK;        // keys per wavefront step
  __shared__ float sc[1024];
  __shared__ float red[8];
  __shared__ float osum[4][KPW][HD];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = lane / LPK, d8 = lane % LPK;
  const int p = d.pos[b];
  const int n_keys = pos_ok(p, d.max_seq) ? p + 1 : 0;
  const int k0 = c * chunk;
  const int k1 = min(n_keys, k0 + chunk);
  const int64_t cbase = ((int64_t)b * d.n_heads + h) * d.max_seq * HD;
  const int64_t slot = (int64_t)((b * d.n_heads + h) * n_chunks + c);

  float qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = q[(int64_t)b * d.dim + h * HD + d8 * 8 + i];
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  // scores (log2 domain)
  for (int kb = k0 + w * KPW; kb < k1; kb += 4 * KPW) {
    const int key = kb + kg;
    float s = 0.f;
    if (key < k1) {
      float kv[8];
      unpack8(*(const u32x4 *)(kc + cbase + (int64_t)key * HD + d8 * 8), kv);
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(qv[i], kv[i], s);
    }
#pragma unroll
    for (int o = 1; o < LPK; o <<= 1) s += __shfl_xor(s, o, 64);
    if (d8 == 0 && key < k1) sc[key - k0] = s * scale;
  }
  __syncthreads();
  const int nk = max(k1 - k0, 0);
  float mx = -INFINITY;
  for (int i = tid; i < nk; i += 256) mx = fmaxf(mx, sc[i]);
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float ls = 0.f;
  for (int i = tid; i < nk; i += 256) {
    const float e = exp2f(sc[i] - mx);
    sc[i] = e;
    ls += e;
  }
  ls = block_sum(ls, red);  // block_sum syncs before use of sc below

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int kb = k0 + w * KPW; kb < k1; kb += 4 * KPW) {
    const int key = kb + kg;
    if (key < k1) {
      float vv[8];
      unpack8(*(const u32x4 *)(vc + cbase + (int64_t)key * HD + d8 * 8), vv);
      const float pr = sc[key - k0];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(pr, vv[i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) osum[w][kg][d8 * 8 + i] = acc[i];
  __syncthreads();
  for (int e = tid; e < HD; e += 256) {
    float t = 0.f;
    for (int ww = 0; ww < 4; ++ww)
      for (int g2 = 0; g2 < KPW; ++g2) t += osum[ww][g2][e];
    o_part[slot * HD + e] = t;
  }
  if (tid == 0) {
    ml_part[slot * 2] = nk > 0 ? mx : -INFINITY;
    ml_part[slot * 2 + 1] = nk > 0 ? ls : 0.f;
  }
}

hipError_t dec_attn_launch(const DecodeArgs &d, const float *q, const uint16_t *kc, const uint16_t *vc,
                           int chunk, int n_chunks, float *o_part, float *ml_part, hipStream_t s) {
  if (chunk > 1024) return hipErrorInvalidValue;
  dim3 grid(n_chunks, d.n_heads, d.batch);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(dec_attn_kernel<128>, grid, dim3(256), 0, s, d, q, kc, vc, chunk, n_chunks, o_part,
                       ml_part);
  else if (d.head_dim == 64)
    hipLaunchKernelGGL(dec_attn_kernel<64>, grid, dim3(256), 0, s, d, q, kc, vc, chunk, n_chunks, o_part,
                       ml_part);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Merge the chunks of one (sequence, head) in chunk order; output as bf16 pair.
__global__ void dec_attn_combine_kernel(const DecodeArgs d, const float *o_part, const float *ml_part,
                                        int n_chunks, u16 *a_hi, u16 *a_lo) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t slot0 = (int64_t)(b * d.n_heads + h) * n_chunks;
  float m = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) m = fmaxf(m, ml_part[(slot0 + c) * 2]);
  for (int e = threadIdx.x; e < d.head_dim; e += blockDim.x) {
    float l = 0.f, o = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
      const float mc = ml_part[(slot0 + c) * 2];
      if (mc == -INFINITY) continue;
      const float f = exp2f(mc - m);
      l += ml_part[(slot0 + c) * 2 + 1] * f;
      o += o_part[(slot0 + c) * d.head_dim + e] * f;
    }
    const float v = o / l;  // no keys (invalid position): 0/0 = NaN
    u16 hi, lo;
    split_pair(v, hi, lo);
    const int64_t oo = (int64_t)b * d.dim + h * d.head_dim + e;
    a_hi[oo] = hi;
    a_lo[oo] = lo;
  }
}

hipError_t dec_attn_combine_launch(const DecodeArgs &d, const float *o_part, const float *ml_part,
                                   int n_chunks, uint16_t *a_hi, uint16_t *a_lo, hipStream_t s) {
  hipLaunchKernelGGL(dec_attn_combine_kernel, dim3(d.n_heads, d.batch), dim3(128), 0, s, d, o_part,
                     ml_part, n_chunks, a_hi, a_lo);
  return hipGetLastError();
}

}  // namespace llama
