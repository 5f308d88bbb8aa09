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
// most KC_MAX. The activation pair for that K range is dropped into LDS with
// global_load_lds_dwordx4 (rows XOR-swizzled) while the first DEPTH steps of
// weights are already streaming from HBM into a ring of B-operand registers,
// so the two latencies overlap; afterwards DEPTH steps of 64 K stay in flight
// per wavefront.
#ifndef GEMV_KC_MAX
#define GEMV_KC_MAX 512
#endif
constexpr int KC_MAX = GEMV_KC_MAX;

#define GEMV_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#define GEMV_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

template <int NTW, int DEPTH>
__global__ __launch_bounds__(256, KC_MAX > 512 ? 1 : 2) void gemv_kernel(const GemvArgs a) {
  __shared__ u32x4 sA[2][32][KC_MAX / 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ks = blockIdx.y * a.k_chunk;
  const int ke = min(a.K, ks + a.k_chunk);
  const int nit = (ke - ks) >> 6;

  const int nw0 = (blockIdx.x * 4 + w) * 32 * NTW;
  const u16 *brow[NTW];
  bool bok[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = nw0 + 32 * j + l32;
    if (a.packed) {
      // tile t = nw0/32 + j: 4 KB per 64-wide K step, this lane's 16 bytes at 16 * lane
      const int t = (nw0 >> 5) + j;
      bok[j] = 32 * t < a.N;   // wavefront-uniform
      brow[j] = a.packed + ((int64_t)t * (a.K >> 6) + (ks >> 6)) * 2048 + lane * 8;
      continue;
    }
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

  // activation pair -> LDS: one 1 KB load per (part, row); lane i lands in
  // chunk i of the row and fetches logical chunk i ^ (row & 15). Rows past M
  // and chunks past the range load valid addresses whose results are never used.
  constexpr int SEGS = KC_MAX / 512;   // 1 KB segments per staged row
#pragma unroll
  for (int q = 0; q < 16 * SEGS; ++q) {
    const int rr = w * 16 + q % 16;     // 0..63 = part * 32 + row
    const int seg = q / 16;
    const int part = rr >> 5, m = rr & 31;
    const int c = (seg * 64 + lane) ^ (m & 15);
    const int k = ks + min(8 * c, (ke - ks) - 8);
    const int mm = m < a.M ? m : 0;
    const u16 *src = (part ? a.A_lo : a.A_hi) + (int64_t)mm * a.K + k;
    __builtin_amdgcn_global_load_lds((const void *)src, GEMV_LDS(&sA[part][m][seg * 64]), 16, 0, 0);
  }

  f32x16 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // K order inside a 64-step: lane group g supplies k = 32 g + 8 q + (0..7) at
  // matrix-core step q, identically for the activation and the weights.
  u32x4 ring[DEPTH][NTW][4];
  auto load = [&](u32x4 (&B)[NTW][4], int it) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        B[j][q] = bok[j] ? *(const u32x4 *)(brow[j] + (a.packed ? 2048 * it + 512 * q : 64 * it + 8 * q))
                         : u32x4{0, 0, 0, 0};
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
  // wait for this wavefront's loads (the activation rows it staged, and the
  // ring prologue the first step needs anyway), then for everyone's rows
  GEMV_WAIT_VMCNT(0);
  __syncthreads();

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
  if (nw0 >= a.N) return;

  float *out = a.part + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = nw0 + 32 * j + l32;
    if (!bok[j] || n >= a.N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * g + (r & 3);
      if (m < a.M) out[(int64_t)m * a.N + n] = acc[j][r];
    }
  }
}

int gemv_ntw(int N) { return N > 8192 ? 2 : 1; }

// One thread per 16-byte piece of the tile-ordered copy.
__global__ void pack_tiles_kernel(int b_mode, const u16 *B0, const u16 *B1, const u16 *B2, int n_seg, int N,
                                  int K, u16 *dst, int64_t pieces) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= pieces) return;
  const int lane = (int)(idx & 63), q = (int)((idx >> 6) & 3);
  const int64_t blk = idx >> 8;               // (tile, step)
  const int ksteps = K >> 6;
  const int t = (int)(blk / ksteps), st = (int)(blk % ksteps);
  const int n = 32 * t + (lane & 31);
  const int k = 64 * st + 32 * (lane >> 5) + 8 * q;
  u32x4 v = {0, 0, 0, 0};
  if (n < N) {
    const u16 *row;
    if (b_mode == BMODE_GATEUP) {
      const int b32 = n >> 5;
      row = ((b32 & 1) ? B1 : B0) + (int64_t)((b32 >> 1) * 32 + (n & 31)) * K;
    } else if (b_mode == BMODE_CONCAT3) {
      const int seg = n / n_seg;
      row = (seg == 0 ? B0 : (seg == 1 ? B1 : B2)) + (int64_t)(n - seg * n_seg) * K;
    } else {
      row = B0 + (int64_t)n * K;
    }
    v = *(const u32x4 *)(row + k);
  }
  *(u32x4 *)(dst + idx * 8) = v;
}

hipError_t pack_tiles_launch(int b_mode, const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int n_seg,
                             int N, int K, uint16_t *dst, hipStream_t s) {
  if (K % 64) return hipErrorInvalidValue;
  const int64_t pieces = (int64_t)((N + 31) / 32) * (K / 64) * 256;
  hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, b_mode, B0, B1,
                     B2, n_seg, N, K, dst, pieces);
  return hipGetLastError();
}

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
// One workgroup per (head, sequence), fused with the Q/K/V split-K finish:
//  1. q, k, v of the new token for this head: rstd * (sum of the projection
//     partials in split order), RoPE on q and k at pos[b]; k and v (bf16) go to
//     cache slot pos[b] and stay in LDS for the new key's own term;
//  2. scores of the fp32 query against cached bf16 keys 0..pos-1 (16 lanes per
//     key, 4 keys per wavefront instruction) plus the new key;
//  3. softmax in fp32 (exp2, log2(e)/sqrt(hd) prescale), weighted sum of the
//     cached values plus the new value;
//  4. the normalised head output is written as the bf16 hi/lo pair the Wo
//     projection consumes.
// An invalid position writes nothing to the cache and yields NaN outputs.
template <int HD>
__global__ __launch_bounds__(256) void dec_attn_kernel(const DecodeArgs d, const float *part, int splits,
                                                       const float *ss, u16 *kc, u16 *vc, u16 *a_hi,
                                                       u16 *a_lo) {
  constexpr int LPK = HD / 8;          // lanes per key
  constexpr int KPW = 64 / LPK;        // keys per wavefront instruction
#ifndef DEC_ATTN_UNROLL
#define DEC_ATTN_UNROLL 4
#endif
  constexpr int UNR = DEC_ATTN_UNROLL; // instructions in flight per wavefront
  __shared__ float sq[HD], sknew[HD], svnew[HD];
  __shared__ float sc[2048 + 1];
  __shared__ float red[8];
  __shared__ float osum[4][KPW][HD];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int p = d.pos[b];
  const bool ok = pos_ok(p, d.max_seq) && p <= 2048;
  const int64_t cbase = ((int64_t)b * d.n_heads + h) * d.max_seq * HD;
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  // ---- 1. q, k, v of the new token (threads 0..HD-1: channel e)
  if (tid < HD) {
    const int e = tid;
    const int N = 3 * d.dim;
    const int64_t stride = (int64_t)d.batch * N;
    const float *pp = part + (int64_t)b * N + h * HD + e;
    float q = 0.f, k = 0.f, v = 0.f;
    for (int sp = 0; sp < splits; ++sp) {
      q += pp[sp * stride];
      k += pp[sp * stride + d.dim];
      v += pp[sp * stride + 2 * d.dim];
    }
    const float r = rstd_from_parts(ss, b, (d.dim + 1023) / 1024, d.dim, d.eps);
    q *= r;
    k *= r;
    v *= r;
    const float qp = __shfl_xor(q, 1, 64), kp = __shfl_xor(k, 1, 64);
    const float2 cs = d.rope_tab[b * (HD / 2) + (e >> 1)];
    q = (e & 1) ? qp * cs.y + q * cs.x : q * cs.x - qp * cs.y;
    k = (e & 1) ? kp * cs.y + k * cs.x : k * cs.x - kp * cs.y;
    // the cache holds bf16: the new key/value enter attention as stored
    const u16 kb = f2bf(k), vb = f2bf(v);
    sq[e] = q;
    sknew[e] = bf2f(kb);
    svnew[e] = bf2f(vb);
    if (ok) {
      kc[cbase + (int64_t)p * HD + e] = kb;
      vc[cbase + (int64_t)p * HD + e] = vb;
    }
  }
  __syncthreads();
  const int nk = ok ? p : 0;    // cached keys 0..p-1; key p is the new one

  // ---- 2. scores (log2 domain) of cached keys
  const int kg = lane / LPK, d8 = lane % LPK;
  float qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = sq[d8 * 8 + i];
  for (int kb0 = w * KPW * UNR; kb0 < nk; kb0 += 4 * KPW * UNR) {
    u32x4 kr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = kb0 + u * KPW + kg;
      kr[u] = key < nk ? *(const u32x4 *)(kc + cbase + (int64_t)key * HD + d8 * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = kb0 + u * KPW + kg;
      float kv[8];
      unpack8(kr[u], kv);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(qv[i], kv[i], s);
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) s += __shfl_xor(s, o, 64);
      if (d8 == 0 && key < nk) sc[key] = s * scale;
    }
  }
  if (tid < 64) {   // the new key's score (one wavefront)
    float s = 0.f;
    for (int e = lane; e < HD; e += 64) s += sq[e] * sknew[e];
    s = wave_sum(s);
    if (lane == 0) sc[nk] = s * scale;
  }
  __syncthreads();

  // ---- 3. softmax over nk + 1 scores
  const int tot = nk + 1;
  float mx = -INFINITY;
  for (int i = tid; i < tot; i += 256) mx = fmaxf(mx, sc[i]);
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float ls = 0.f;
  for (int i = tid; i < tot; i += 256) {
    const float e = exp2f(sc[i] - mx);
    sc[i] = e;
    ls += e;
  }
  ls = block_sum(ls, red);   // contains barriers: sc is complete afterwards

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int kb0 = w * KPW * UNR; kb0 < nk; kb0 += 4 * KPW * UNR) {
    u32x4 vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = kb0 + u * KPW + kg;
      vr[u] = key < nk ? *(const u32x4 *)(vc + cbase + (int64_t)key * HD + d8 * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = kb0 + u * KPW + kg;
      if (key < nk) {
        float vv[8];
        unpack8(vr[u], vv);
        const float pr = sc[key];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(pr, vv[i], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) osum[w][kg][d8 * 8 + i] = acc[i];
  __syncthreads();

  // ---- 4. normalised output (+ the new value's term) as a bf16 pair
  if (tid < HD) {
    const int e = tid;
    float o = sc[nk] * svnew[e];
    for (int ww = 0; ww < 4; ++ww)
      for (int g2 = 0; g2 < KPW; ++g2) o += osum[ww][g2][e];
    const float v = ok ? o / ls : __builtin_nanf("");
    u16 hi, lo;
    split_pair(v, hi, lo);
    const int64_t oo = (int64_t)b * d.dim + h * HD + e;
    a_hi[oo] = hi;
    a_lo[oo] = lo;
  }
}

hipError_t dec_attn_launch(const DecodeArgs &d, const float *part, int splits, const float *ss, uint16_t *kc,
                           uint16_t *vc, uint16_t *a_hi, uint16_t *a_lo, hipStream_t s) {
  if (d.max_seq > 2048 + 1) return hipErrorInvalidValue;
  dim3 grid(d.n_heads, d.batch);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(dec_attn_kernel<128>, grid, dim3(256), 0, s, d, part, splits, ss, kc, vc, a_hi, a_lo);
  else if (d.head_dim == 64)
    hipLaunchKernelGGL(dec_attn_kernel<64>, grid, dim3(256), 0, s, d, part, splits, ss, kc, vc, a_hi, a_lo);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace llama
