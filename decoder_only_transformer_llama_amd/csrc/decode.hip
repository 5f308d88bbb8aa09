// Decode-step kernels (one new token per sequence, batch <= 32). The step is
// bound by HBM: every weight byte and every cached K/V byte is read once.
//
//  - gemv_kernel: skinny split-K product part[s][m][n] = sum_{k in split s}
//    A[m][k] B[n][k] with the batch as the 32 rows of one v_mfma_f32_32x32x16
//    tile. Weights stream from HBM (tile-packed: one contiguous 4 KB block per
//    32 columns x 64 K) into a ring of B-operand registers, DEPTH steps deep;
//    the activation operand is a bf16 hi/lo pair staged in LDS, so the product
//    is fp32-accurate at bf16 matrix-core rate. K order inside a step is
//    permuted identically for A and B, which leaves the sum unchanged.
//  - the *_combine / resid_norm kernels reduce the split-K partials in a fixed
//    order (deterministic, no atomics) and apply the elementwise work: RMSNorm
//    statistics and gain, SiLU(gate)*up, the residual adds of the pre-norm
//    block, the head's row scale.
//  - dec_attn_kernel: per (head, sequence) the Q/K/V split-K finish, RoPE at
//    pos, the cache append, and one pass of online-softmax attention over the
//    cached keys and values.
//
// Loads in the streaming loops are never placed under a branch and their
// loops unroll into straight-line code: at a control-flow join the compiler
// waits for every outstanding load, which would serialise the stream.
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
constexpr int KC_MAX = kGemvMaxChunk;

#define GEMV_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#define GEMV_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

constexpr int kGemvOcc = 2;   // workgroups per CU the register budget is sized for

template <int NTW, int DEPTH>
__global__ __launch_bounds__(256, kGemvOcc) void gemv_kernel(const GemvArgs a) {
  __shared__ u32x4 sA[2][32][KC_MAX / 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ks = blockIdx.y * a.k_chunk;
  const int ke = min(a.K, ks + a.k_chunk);
  const int nit = (ke - ks) >> 6;
  const int n_tiles = (a.N + 31) >> 5;

  // Every load below is unconditional: columns past N read the last valid
  // tile (or row) and their results are never stored. Loads under branches
  // would make the compiler wait for all outstanding loads at each join,
  // which serialises the weight stream.
  const int nw0 = (blockIdx.x * 4 + w) * 32 * NTW;
  const u16 *brow[NTW];
  bool bok[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = nw0 + 32 * j + l32;
    if (a.packed) {
      // tile t: 4 KB per 64-wide K step, this lane's 16 bytes at 16 * lane
      const int t = (nw0 >> 5) + j;
      bok[j] = t < n_tiles;   // wavefront-uniform
      brow[j] = a.packed + pack_block(min(t, n_tiles - 1), ks >> 6, n_tiles, a.K >> 6, a.k_chunk >> 6) * 2048 +
                lane * 8;
      continue;
    }
    bok[j] = n < a.N;
    const int nn = bok[j] ? n : a.N - 1;
    const u16 *p;
    if (a.b_mode == BMODE_GATEUP) {
      const int blk = nn >> 5;
      p = ((blk & 1) ? a.B1 : a.B0) + (int64_t)((blk >> 1) * 32 + (nn & 31)) * a.K;
    } else if (a.b_mode == BMODE_CONCAT3) {
      p = concat3_row(a.B0, a.B1, a.B2, a.n_seg, a.n_seg_kv > 0 ? a.n_seg_kv : a.n_seg, nn, a.K);
    } else {
      p = a.B0 + (int64_t)nn * a.K;
    }
    brow[j] = p + ks + 32 * g;
  }

  // activation pair -> LDS: one 1 KB load per (part, row); lane i lands in
  // chunk i of the row and fetches logical chunk i ^ (row & 15). Rows past M
  // and chunks past the range load valid addresses, so the whole staged
  // region holds finite values.
  constexpr int SEGS = KC_MAX / 512;   // 1 KB segments per staged row
#pragma unroll
  for (int q = 0; q < 16 * SEGS; ++q) {
    const int rr = w * 16 + q % 16;     // 0..63 = part * 32 + row
    const int seg = q / 16;
    const int part = rr >> 5, m = rr & 31;
    const int c = (seg * 64 + lane) ^ (m & 15);
    const int mm = m < a.M ? m : 0;
    // buffer form of the load: the global form would make the compiler wait
    // for every load in flight (the weight ring too) before the first LDS read
    buf_load_lds16((part ? a.A_lo : a.A_hi) + (int64_t)mm * a.K + ks, (uint32_t)(min(8 * c, (ke - ks) - 8) * 2), 0,
                   &sA[part][m][seg * 64]);
  }

  f32x16 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // K order inside a 64-step: lane group g supplies k = 32 g + 8 q + (0..7) at
  // matrix-core step q, identically for the activation and the weights.
  u32x4 ring[DEPTH][NTW][4];
  auto load = [&](u32x4 (&B)[NTW][4], int it) {   // it is clamped to the range by the caller
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        B[j][q] = *(const u32x4 *)(brow[j] + (a.packed ? 2048 * it + 512 * q : 64 * it + 8 * q));
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
  for (int d = 0; d < DEPTH; ++d) {
    load(ring[d], min(d, nit - 1));
    __builtin_amdgcn_sched_barrier(0);   // issue order = the loop's refill order
  }
  // the activation rows were issued first: once at most the ring's loads are
  // outstanding, this wavefront's rows are in LDS; the barrier covers the others
  GEMV_WAIT_VMCNT(DEPTH * NTW * 4);
  __builtin_amdgcn_s_barrier();

  // The K range has at most KC_MAX / 64 steps, so the step loop unrolls into
  // straight-line code whose only branches leave it: with no join inside,
  // each step waits for exactly its own weights while the next DEPTH - 1
  // steps stay in flight. Refills past the range re-read the last step (never
  // used) rather than branching around the load.
  constexpr int NSTEP = KC_MAX / 64;
#pragma unroll
  for (int it = 0; it < NSTEP; ++it) {
    if (it >= nit) break;
    compute(ring[it % DEPTH], it);
    if (it + DEPTH < NSTEP) load(ring[it % DEPTH], min(it + DEPTH, nit - 1));
    // keep each refill right behind the step that frees its registers (the
    // scheduler would otherwise sink all refills together)
    __builtin_amdgcn_sched_barrier(0);
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

constexpr int kGemvDepth = 4;   // 64-deep weight steps in flight per wavefront
// three tiles per wavefront keep three steps in flight (four would spill);
// the bytes in flight per wavefront stay about the same
constexpr int kGemvDepth3 = 3;

// The K ranges aim at about 256 workgroups and hold at most KC_MAX (the
// activation pair of a range is staged in LDS). Wavefronts take one 32-column
// tile, two above 8192 columns and three above 16384: measured on the 7B
// shapes, gate/up (22016 columns) is 3% faster with three than with two,
// while the down projection (4096 columns, 22 K ranges) is 15% slower with two
// than with one, so the count follows the width rather than the number of
// workgroups. The K ranges, and so the packed weight layout, do not depend on
// the tile count.
GemvShape gemv_shape(int N, int K) {
  constexpr int kTargetWgs = 256;
  const int ksteps = K / 64;
  GemvShape g;
  g.ntw = N > 16384 ? 3 : (N > 8192 ? 2 : 1);
  const int n_wg = (N + 128 * g.ntw - 1) / (128 * g.ntw);
  const int s = max(1, min(ksteps, (kTargetWgs + n_wg - 1) / n_wg));
  const int per = min((ksteps + s - 1) / s, KC_MAX / 64);
  g.k_chunk = per * 64;
  g.splits = (ksteps + per - 1) / per;
  return g;
}

// One thread per 16-byte piece: source block (tile, step) in tile-major order,
// written to its chunk-major position.
__global__ void pack_tiles_kernel(int b_mode, const u16 *B0, const u16 *B1, const u16 *B2, int n_seg, int n_seg_kv,
                                  int N, int K, int kcs, u16 *dst, int64_t pieces) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= pieces) return;
  const int lane = (int)(idx & 63), q = (int)((idx >> 6) & 3);
  const int64_t blk = idx >> 8;               // (tile, step)
  const int ksteps = K >> 6, n_tiles = (N + 31) >> 5;
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
      row = concat3_row(B0, B1, B2, n_seg, n_seg_kv > 0 ? n_seg_kv : n_seg, n, K);
    } else {
      row = B0 + (int64_t)n * K;
    }
    v = *(const u32x4 *)(row + k);
  }
  const int64_t o = pack_block(t, st, n_tiles, ksteps, kcs) * 2048 + q * 512 + lane * 8;
  *(u32x4 *)(dst + o) = v;
}

hipError_t pack_tiles_launch(int b_mode, const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int n_seg,
                             int n_seg_kv, int N, int K, int k_chunk, uint16_t *dst, hipStream_t s) {
  if (K % 64 || k_chunk % 64 || k_chunk <= 0) return hipErrorInvalidValue;
  const int64_t pieces = (int64_t)((N + 31) / 32) * (K / 64) * 256;
  hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, b_mode, B0, B1,
                     B2, n_seg, n_seg_kv, N, K, k_chunk / 64, dst, pieces);
  return hipGetLastError();
}

hipError_t gemv_launch(const GemvArgs &a, hipStream_t s) {
  if (a.k_chunk > KC_MAX || a.k_chunk % 64 || a.K % 64 || a.M > 32) return hipErrorInvalidValue;
  const int ntw = gemv_shape(a.N, a.K).ntw;
  const int per_wg = 4 * 32 * ntw;
  dim3 grid((a.N + per_wg - 1) / per_wg, a.splits);
  if (ntw == 3)
    hipLaunchKernelGGL((gemv_kernel<3, kGemvDepth3>), grid, dim3(256), 0, s, a);
  else if (ntw == 2)
    hipLaunchKernelGGL((gemv_kernel<2, kGemvDepth>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<1, kGemvDepth>), grid, dim3(256), 0, s, a);
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

// init + p[0] + p[stride] + ... + p[(n-1) stride], added in that order. The
// loads go out eight at a time (indices past n re-read the last element and
// add zero), so a long split-K reduction costs a few memory round trips, not
// one per split.
DEV float sum_parts(float init, const float *p, int64_t stride, int n) {
  float t = init;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(int64_t)min(s0 + i, n - 1) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) t += s0 + i < n ? v[i] : 0.f;
  }
  return t;
}

DEV f32x4 sum_parts4(f32x4 init, const float *p, int64_t stride, int n) {
  f32x4 t = init;
  for (int s0 = 0; s0 < n; s0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *(const f32x4 *)(p + (int64_t)min(s0 + i, n - 1) * stride);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < n) t += v[i];
  }
  return t;
}

// Row statistics are kept as partial sums of squares, one per 1024-channel
// chunk of the row (ss[b][chunk]); consumers finish rstd in a fixed order.
DEV float rstd_from_parts(const float *ss, int b, int nss, int dim, float eps) {
  return rstd_of(sum_parts(0.f, ss + b * nss, 1, nss), dim, eps);
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
    const f32x4 v = sum_parts4(*(const f32x4 *)(res + o), part + o, stride, splits);
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
  const float *pp = part + (int64_t)b * N + ng;
  const float gt = sum_parts(0.f, pp, stride, splits);
  const float up = sum_parts(0.f, pp + 32, stride, splits);
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
  const float v = sum_parts(0.f, part + idx, stride, splits);
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
// One workgroup per (key/value head, sequence, key range), fused with the
// Q/K/V split-K finish:
//  1. q, k, v of the new token for this head: rstd * (sum of the projection
//     partials in split order), RoPE on q and k at pos[b]; k and v (bf16) go to
//     cache slot pos[b] (written by the first key range only) and stay in LDS
//     for the new key's own term;
//  2. one pass over the range's share of the cached keys 0..pos-1 (NS equal
//     ranges, multiples of one step) and their values: a lane group of
//     HD/8 lanes owns one key per instruction (4 keys per wavefront
//     instruction, UNR instructions per step), keeps a running max, sum and
//     weighted value sum in fp32 (online softmax, exp2 with log2(e)/sqrt(hd)
//     folded into q); keys and values of the next step are in flight while
//     one step is processed;
//  3. the lane groups' partial softmax states and (first range only) the new
//     key's term are merged in a fixed order. With one range the normalised
//     head output is written as the bf16 hi/lo pair the Wo projection
//     consumes; with NS ranges each writes (max, sum, unnormalised output) and
//     dec_attn_combine_kernel merges the NS states in range order.
// Splitting the keys gives NS times more workgroups: grouped heads leave only
// n_kv_heads * batch (key/value head, sequence) pairs, too few to keep enough
// loads in flight on 256 compute units.
// An invalid position writes nothing to the cache and yields NaN outputs.
// Sum over aligned groups of G lanes (G = 2..16), every lane getting its
// group's total, with DPP lane moves inside each 16-lane row: swap
// neighbours, swap pairs, mirror within 8, mirror within 16. Each step adds a
// permutation of the partial sums, so after log2(G) steps all G lanes hold
// the same sum.
template <int G>
DEV float lane_group_sum(float v) {
  static_assert(G >= 2 && G <= 16 && (G & (G - 1)) == 0, "group of 2..16 lanes");
#define LLAMA_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, false))
  v += LLAMA_DPP(v, 0xB1);                  // quad_perm [1,0,3,2]
  if (G >= 4) v += LLAMA_DPP(v, 0x4E);      // quad_perm [2,3,0,1]
  if (G >= 8) v += LLAMA_DPP(v, 0x141);     // row_half_mirror
  if (G >= 16) v += LLAMA_DPP(v, 0x140);    // row_mirror
#undef LLAMA_DPP
  return v;
}

constexpr int kMaxSeq = 2048;   // cache positions one set of key ranges unrolls for (longer caches: more ranges)

// The new token's part of a decode attention workgroup (key/value head hk,
// sequence b, key range rs): q of the G query heads hk*G .. hk*G+G-1, k and
// v, each the sum of the Q/K/V split-K partials times rstd, RoPE on q and k;
// q scaled by log2(e)/sqrt(hd) into sq, k and v (fp32) into sknew / svnew,
// the bf16 cache copy at position p (first range only), and the new key's
// score per query head into snew (log2 domain). Ends synchronised.
template <int HD, int G, int NT = 256>
DEV void dec_attn_new_token(const DecodeArgs &d, const float *part, int splits, const float *ss, u16 *kc, u16 *vc,
                            int hk, int b, int rs, int p, bool ok, int64_t cbase, float (*sq)[HD], float *sknew,
                            float *svnew, float *snew) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kvd = d.n_kv_heads * HD;
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  {
    const int N = d.dim + 2 * kvd;
    const int64_t stride = (int64_t)d.batch * N;
    const float r = rstd_from_parts(ss, b, (d.dim + 1023) / 1024, d.dim, d.eps);
    for (int c = tid; c < (G + 2) * HD; c += NT) {   // an even stride: pairs (e, e^1) stay in one pass
      const int gq = c / HD, e = c % HD;
      const int col = gq < G ? (hk * G + gq) * HD + e : d.dim + (gq - G) * kvd + hk * HD + e;
      float x = sum_parts(0.f, part + (int64_t)b * N + col, stride, splits) * r;
      const float xp = __shfl_xor(x, 1, 64);   // RoPE partner (channel e ^ 1)
      if (gq <= G) {                           // q heads and k are rotated, v is not
        const float2 cs = d.rope_tab[b * (HD / 2) + (e >> 1)];
        x = (e & 1) ? xp * cs.y + x * cs.x : x * cs.x - xp * cs.y;
      }
      if (gq < G) {
        sq[gq][e] = x * scale;
      } else {
        // the cache stores bf16 for later steps; this step's own key and
        // value enter its attention unrounded (fp32), as in the definition:
        // attending to them after the storage rounding made the decode of
        // some 7B-shape sequences drift up to 4e-2 from the exact logits over
        // 32 layers, against 1.5e-4 with fp32 values
        (gq == G ? sknew : svnew)[e] = x;
        if (ok && rs == 0) (gq == G ? kc : vc)[cbase + (int64_t)p * HD + e] = f2bf(x);
      }
    }
  }
  __syncthreads();
  if (w == 0) {                 // the new key's scores (log2 domain)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
      for (int e = lane; e < HD; e += 64) s += sq[g][e] * sknew[e];
      s = wave_sum(s);
      if (lane == 0) snew[g] = s;
    }
  }
}

// Launch bounds at head dim 128: four workgroups per compute unit (at most 128
// registers; the grouped-query instances would otherwise take 129 and fit
// only three). At head dim 64 that bound would spill, so two.
template <int HD, int G, int NS>
__global__ __launch_bounds__(256, HD == 128 ? 4 : 2) void dec_attn_kernel(const DecodeArgs d, const float *part, int splits,
                                                       const float *ss, u16 *kc, u16 *vc, u16 *a_hi,
                                                       u16 *a_lo, float *opart) {
  constexpr int LPK = HD / 8;          // lanes per key
  constexpr int KPW = 64 / LPK;        // keys per wavefront instruction
  constexpr int UNR = 2;               // key instructions per wavefront per step
  constexpr int KPS = 4 * KPW * UNR;   // keys per workgroup step
  constexpr int NG = 4 * KPW;          // lane groups per workgroup
  constexpr float kLazyRescale = 8.0f;   // log2 units a running maximum may lag the true one
  // One workgroup per (key/value head hk, sequence b): the G query heads
  // hk*G .. hk*G+G-1 share its cached keys and values, which are read once.
  __shared__ float sq[G][HD], sknew[HD], svnew[HD];
  __shared__ float gm[NG][G], gl[NG][G], snew[G];
  __shared__ float osum[NG][G][HD];
  // nr key ranges (gridDim.z): NS, or a multiple of it for caches longer
  // than kMaxSeq, so that no range holds more than the unrolled ceil(kMaxSeq / NS) keys
  const int hk = blockIdx.x, b = blockIdx.y, rs = blockIdx.z, nr = gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int p = d.pos[b];
  const bool ok = pos_ok(p, d.max_seq);
  const int64_t cbase = ((int64_t)b * d.n_kv_heads + hk) * d.max_seq * HD;

  // cached keys 0..p-1 (key p is the new one); this range covers keys
  // k0 .. k0+nk-1, a multiple of KPS long except at the end
  const int nk_all = ok ? p : 0;
  const int chunk = nr == 1 ? nk_all : ((nk_all + nr - 1) / nr + KPS - 1) / KPS * KPS;
  const int k0 = min(rs * chunk, nk_all);
  const int nk = min(k0 + chunk, nk_all) - k0;

  // ---- 2. one pass over the cached keys and values
  const int kg = lane / LPK, d8 = lane % LPK;
  float qv[G][8];   // this lane's channels of the G queries (after the new token's part below)
  float m_run[G], l_run[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }
  const int nsteps = (nk + KPS - 1) / KPS;
  const int kbase = w * KPW * UNR + kg;          // + st * KPS + u * KPW
  // Loads are unconditional: keys past the range read key max(nk-1, 0) (a
  // valid row) and get probability 0.
  auto load = [&](u32x4 (&kr)[UNR], u32x4 (&vr)[UNR], int st) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int key = k0 + max(min(st * KPS + kbase + u * KPW, nk - 1), 0);
      const int64_t o = cbase + (int64_t)key * HD + d8 * 8;
      kr[u] = *(const u32x4 *)(kc + o);
      vr[u] = *(const u32x4 *)(vc + o);
    }
  };
  auto step = [&](const u32x4 (&kr)[UNR], const u32x4 (&vr)[UNR], int st) {
    float kv[UNR][8], vv[UNR][8];
    bool live[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      unpack8(kr[u], kv[u]);
      unpack8(vr[u], vv[u]);
      live[u] = st * KPS + kbase + u * KPW < nk;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float sc[UNR];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float sdot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sdot = fmaf(qv[g][i], kv[u][i], sdot);
        sdot = lane_group_sum<LPK>(sdot);
        sc[u] = live[u] ? sdot : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      // Lazy rescaling: the reference maximum m_run moves (and the running
      // sum and output are rescaled) only when some lane's new maximum
      // exceeds it by more than kLazyRescale (scores are in log2 units), so
      // probabilities up to 2^kLazyRescale enter the sums; the merge below
      // works from each group's reference. m_run = -inf always takes it.
      if (!__all(mx <= m_run[g] + kLazyRescale)) {
        const float m_new = fmaxf(m_run[g], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[g] - (m_new == -INFINITY ? 0.f : m_new));   // -inf -> 0
        m_run[g] = m_new;
        l_run[g] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] *= alpha;
      }
      const float m_use = m_run[g] == -INFINITY ? 0.f : m_run[g];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float pr = __builtin_amdgcn_exp2f(sc[u] - m_use);   // raw v_exp_f32; exp2(-inf) = 0
        l_run[g] += pr;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(pr, vv[u][i], acc[g][i]);
      }
    }
  };
  // The step loop unrolls fully (a cache holds at most kMaxSeq positions) and
  // no load sits under a branch, so each step waits for exactly its own keys
  // and values while the next step's are in flight; steps past the range are
  // skipped (a uniform branch around arithmetic only) and their loads re-read
  // one valid row. The fences keep each refill right behind the step that
  // frees its registers.
  // a range holds at most ceil(kMaxSeq / NS) keys rounded up to a step
  constexpr int MAXSTEPS = ((kMaxSeq + NS - 1) / NS + KPS - 1) / KPS;
  const int last = max(nsteps - 1, 0);
  u32x4 kb[2][UNR], vb[2][UNR];
  load(kb[0], vb[0], 0);
  load(kb[1], vb[1], min(1, last));

  // ---- 1. q (G heads), k, v of the new token (its latency overlaps the
  // first two steps' loads, which read only cached rows below p)
  dec_attn_new_token<HD, G>(d, part, splits, ss, kc, vc, hk, b, rs, p, ok, cbase, sq, sknew, svnew, snew);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[g][i] = sq[g][d8 * 8 + i];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < MAXSTEPS; ++st) {
    if (st < nsteps) step(kb[st & 1], vb[st & 1], st);
    if (st + 2 < MAXSTEPS) load(kb[st & 1], vb[st & 1], min(st + 2, last));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (d8 == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      gm[w * KPW + kg][g] = m_run[g];
      gl[w * KPW + kg][g] = l_run[g];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) osum[w * KPW + kg][g][d8 * 8 + i] = acc[g][i];
  __syncthreads();

  // ---- 3. per query head: merge the lane groups and the new key (fixed
  // order); one range: normalise and write the bf16 hi/lo pair the Wo
  // projection consumes; several: store this range's softmax state
  for (int c = tid; c < G * HD; c += 256) {
    const int g = c / HD, e = c % HD;
    const float sn = rs == 0 ? snew[g] : -INFINITY;   // the new key belongs to the first range
    float M = sn;
    for (int gi = 0; gi < NG; ++gi) M = fmaxf(M, gm[gi][g]);
    const float Mu = M == -INFINITY ? 0.f : M;        // a later range may see no key at all
    const float pn = exp2f(sn - Mu);
    float L = pn, o = pn * svnew[e];
    for (int gi = 0; gi < NG; ++gi) {
      const float f = exp2f(gm[gi][g] - Mu);   // 0 for a group that saw no key
      L += f * gl[gi][g];
      o += f * osum[gi][g][e];
    }
    if (nr == 1) {
      const float v = ok ? o / L : __builtin_nanf("");
      u16 hi, lo;
      split_pair(v, hi, lo);
      const int64_t oo = (int64_t)b * d.dim + (hk * G + g) * HD + e;
      a_hi[oo] = hi;
      a_lo[oo] = lo;
    } else {
      float *st = opart + (((int64_t)b * d.n_heads + hk * G + g) * nr + rs) * (HD + 2);
      st[2 + e] = o;
      if (e == 0) {
        st[0] = M;
        st[1] = L;
      }
    }
  }
}

// Grouped-query decode attention on the matrix cores (head dim 128, G = 2..8
// query heads per key/value head), for the same workgroups as dec_attn_kernel
// (key/value head, sequence, key range). Each wavefront takes 32-key chunks
// of the range in turn (chunk c to wavefront c mod 4):
//  - S = K Q^T with v_mfma_f32_16x16x32_bf16, two 16-key blocks: K rows go
//    from the cache straight into the A operand (a lane holds 8 channels of
//    one key), q (fp32) enters as a bf16 hi/lo pair (two products, ~2^-17
//    relative), G of the 16 columns used. The keys of block b, row r are
//    chunk keys 8 (r / 4) + 4 b + r % 4, so that a lane's four scores of
//    each block are the eight consecutive keys the P operand wants.
//  - online softmax in fp32 against a per-head reference maximum that moves
//    only when some score exceeds it by more than 2^8 (no cross-lane step in
//    the common case); P as a bf16 hi/lo pair.
//  - O = P V with the same instruction over the 32 keys: V (row-major in the
//    cache) is staged in a per-wavefront LDS tile by direct loads and read
//    with ds_read_b64_tr_b16, which hands each lane four consecutive keys of
//    one channel. Tile rows are 256 bytes with the 16-byte chunks XOR-ed by
//    2 f(row), f(row) = (row & 3) + 4 ((row >> 3) & 1), so the 16 rows one
//    transposing read touches fall on distinct chunks per half-wavefront.
// The next chunk's keys and value tile are in flight while one is processed.
// The four wavefronts' states and the new key merge in a fixed order (as in
// dec_attn_kernel); results are deterministic.
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <int G, int NS>
__global__ __launch_bounds__(512, 1) void dec_attn_mfma_kernel(const DecodeArgs d, const float *part, int splits,
                                                               const float *ss, u16 *kc, u16 *vc, u16 *a_hi,
                                                               u16 *a_lo, float *opart) {
  static_assert(G >= 2 && G <= 8, "grouped heads, 2 to 8 per key/value head");
  constexpr int HD = 128;
  constexpr int CK = 32;                   // keys per chunk
  constexpr int NB = HD / 16;              // 16-channel blocks of O
  constexpr int VT = CK * HD / 8;          // u32x4 per value tile (8 KB)
  constexpr float kLazyRescale = 8.0f;     // log2 units the reference maximum may lag
  constexpr int NWV = 8;                   // wavefronts (two per SIMD)
  __shared__ float sq[G][HD], sknew[HD], svnew[HD];
  __shared__ float gm[NWV][G], gl[NWV][G], snew[G];
  // two value tiles per wavefront; after the key loop the same memory holds
  // the wavefronts' output sums for the merge
  __shared__ u32x4 vtile[NWV * 2 * VT];
  static_assert(NWV * G * HD * 4 <= (int)sizeof(vtile), "output sums fit the value tiles");
  float(*osum)[G][HD] = (float(*)[G][HD])vtile;

  // nr key ranges (gridDim.z): NS, or a multiple of it for caches longer
  // than kMaxSeq, so that no range holds more than the unrolled ceil(kMaxSeq / NS) keys
  const int hk = blockIdx.x, b = blockIdx.y, rs = blockIdx.z, nr = gridDim.z;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g4 = lane >> 4;   // operand column / row-block of the 16 x 16 products
  const int p = d.pos[b];
  const bool ok = pos_ok(p, d.max_seq);
  const int64_t cbase = ((int64_t)b * d.n_kv_heads + hk) * d.max_seq * HD;

  // cached keys 0..p-1: this range covers k0 .. k0+nk-1 (a multiple of NWV
  // chunks long except at the end), chunk c of it to wavefront c % NWV
  const int nk_all = ok ? p : 0;
  const int chunk = nr == 1 ? nk_all : ((nk_all + nr - 1) / nr + NWV * CK - 1) / (NWV * CK) * (NWV * CK);
  const int k0 = min(rs * chunk, nk_all);
  const int nk = min(k0 + chunk, nk_all) - k0;
  const int nch = (nk + CK - 1) / CK;
  const int my_n = nch > w ? (nch - w + NWV - 1) / NWV : 0;

  const u16 *kbase = kc + cbase;
  const u16 *vbase = wave_uniform(vc + cbase);
  u32x4 *const myv = vtile + w * (2 * VT);
  auto tile_f = [](int row) { return (row & 3) + 4 * ((row >> 3) & 1); };
  // keys of chunk c into kf (past the range: the range's last key, masked;
  // an empty range reads its first position, never used)
  auto load_k = [&](u32x4 (&kf)[2][4], int c) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int key = k0 + max(min(c * CK + 8 * (j >> 2) + 4 * bb + (j & 3), nk - 1), 0);
      const u16 *row = kbase + (int64_t)key * HD + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kf[bb][kk] = *(const u32x4 *)(row + 32 * kk);
    }
  };
  // values of chunk c into tile slot `slot` (8 direct loads of 4 rows each)
  auto load_v = [&](int slot, int c) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 4 * q + (lane >> 4);
      const int lc = (lane & 15) ^ (2 * tile_f(row));
      const int key = k0 + max(min(c * CK + row, nk - 1), 0);
      buf_load_lds16(vbase, (uint32_t)((key * HD + 8 * lc) * 2), 0, myv + slot * VT + q * 64);
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float my_ref = -INFINITY, lpart = 0.f;   // this lane's head j: reference maximum, partial sum

  // The chunk loop unrolls fully (at most MAXIT chunks per wavefront for a
  // cache of kMaxSeq positions), so the two buffers are indexed at compile
  // time; loads are unconditional (the next chunk's, clamped to valid rows
  // past the range) and only the arithmetic of chunks past this
  // wavefront's share is skipped: a load under a branch would make the
  // compiler wait for every load in flight at the join.
  constexpr int MAXIT = ((kMaxSeq + NS - 1) / NS + NWV * CK - 1) / (NWV * CK);
  u32x4 kf[2][2][4];
  load_k(kf[0], w);
  load_v(0, w);

  // ---- 1. the new token (its latency overlaps the first chunk's loads)
  dec_attn_new_token<HD, G, NWV * 64>(d, part, splits, ss, kc, vc, hk, b, rs, p, ok, cbase, sq, sknew, svnew, snew);

  // q as the B operand of S = K Q^T: column j (query head j < G), channels
  // 32 kk + 8 g4 .. +7, as a bf16 hi/lo pair
  u32x4 qhi[4], qlo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    float qf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[i] = j < G ? sq[j][32 * kk + 8 * g4 + i] : 0.f;
    pack8_pair(qf, qhi[kk], qlo[kk]);
  }

  // ---- 2. the cached keys
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int c = w + NWV * it, cur = it & 1;
    if (it + 1 < MAXIT) {
      load_k(kf[cur ^ 1], c + NWV);
      load_v(cur ^ 1, c + NWV);
    }
    if (it >= my_n) continue;
    // scores of the two 16-key blocks
    f32x4 sc[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[cur][bb][kk]), as_bf16x8(qhi[kk]), sc[bb], 0, 0, 0);
        sc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[cur][bb][kk]), as_bf16x8(qlo[kk]), sc[bb], 0, 0, 0);
      }
    }
    // lane (g4, j): head j, chunk keys 8 g4 + 4 bb + u
    float mx = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool live = j < G && c * CK + 8 * g4 + 4 * bb + u < nk;
        sc[bb][u] = live ? sc[bb][u] : -INFINITY;
        mx = fmaxf(mx, sc[bb][u]);
      }
    if (__any(mx > my_ref + kLazyRescale)) {
      // a head's maximum moved: over the four lanes of each head, the new
      // reference, and every accumulator of that head rescaled
      float hm = fmaxf(mx, __shfl_xor(mx, 16, 64));
      hm = fmaxf(hm, __shfl_xor(hm, 32, 64));
      const float m_new = fmaxf(my_ref, hm);
      const float alpha = __builtin_amdgcn_exp2f(my_ref - (m_new == -INFINITY ? 0.f : m_new));   // -inf -> 0
      my_ref = m_new;
      lpart *= alpha;
      // O rows of this lane are heads 4 g4 + u; their factors sit in lanes 4 g4 + u
      float af[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) af[u] = __shfl(alpha, 4 * g4 + u, 64);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[nb][u] *= af[u];
    }
    const float m_use = my_ref == -INFINITY ? 0.f : my_ref;
    float pr[8];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pr[4 * bb + u] = __builtin_amdgcn_exp2f(sc[bb][u] - m_use);   // exp2(-inf) = 0
        lpart += pr[4 * bb + u];
      }
    u32x4 phi, plo;
    pack8_pair(pr, phi, plo);   // P operand: row j (head), keys 8 g4 .. +7
    // this chunk's value tile is in LDS once its direct loads are done (the
    // next chunk's 16 loads may still be in flight)
    if (it + 1 < MAXIT) {
      GEMV_WAIT_VMCNT(16);
    } else {
      GEMV_WAIT_VMCNT(0);
    }
    const u32x4 *tile = myv + cur * VT;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // B operand: channel 16 nb + j of keys 8 g4 .. +7, two transposing reads
      // of four keys; lane j of a 16-lane group points at row kb + j / 4,
      // channels 16 nb + 4 (j % 4) .. +3
      u32x2 vv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g4 + 4 * h + (j >> 2);
        const int ch = 2 * nb + ((j & 3) >> 1);            // logical 16-byte chunk
        const int byte = (row * 16 + (ch ^ (2 * tile_f(row)))) * 16 + 8 * (j & 1);
        const auto t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)((char *)tile + byte));
        vv[h] = __builtin_bit_cast(u32x2, t);
      }
      const u32x4 vb = u32x4{vv[0][0], vv[0][1], vv[1][0], vv[1][1]};
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(phi), as_bf16x8(vb), acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(plo), as_bf16x8(vb), acc[nb], 0, 0, 0);
    }
  }
  GEMV_WAIT_VMCNT(0);   // the last prefetch (unused) is in LDS before the tiles are reused

  // ---- per wavefront: head references and sums (lanes j < G of the first
  // row block), output sums (rows 4 g4 + u < G)
  {
    float ls = lpart + __shfl_xor(lpart, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (g4 == 0 && j < G) {
      gm[w][j] = my_ref;
      gl[w][j] = ls;
    }
  }
  __syncthreads();   // every wavefront is done with its value tiles
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (4 * g4 + u < G) osum[w][4 * g4 + u][16 * nb + j] = acc[nb][u];
  __syncthreads();

  // ---- 3. per query head: merge the wavefronts and the new key (fixed
  // order), as in dec_attn_kernel
  for (int c = tid; c < G * HD; c += NWV * 64) {
    const int g = c / HD, e = c % HD;
    const float sn = rs == 0 ? snew[g] : -INFINITY;   // the new key belongs to the first range
    float M = sn;
    for (int gi = 0; gi < NWV; ++gi) M = fmaxf(M, gm[gi][g]);
    const float Mu = M == -INFINITY ? 0.f : M;        // a later range may see no key at all
    const float pn = exp2f(sn - Mu);
    float L = pn, o = pn * svnew[e];
    for (int gi = 0; gi < NWV; ++gi) {
      const float f = exp2f(gm[gi][g] - Mu);   // 0 for a wavefront that saw no key
      L += f * gl[gi][g];
      o += f * osum[gi][g][e];
    }
    if (nr == 1) {
      const float v = ok ? o / L : __builtin_nanf("");
      u16 hi, lo;
      split_pair(v, hi, lo);
      const int64_t oo = (int64_t)b * d.dim + (hk * G + g) * HD + e;
      a_hi[oo] = hi;
      a_lo[oo] = lo;
    } else {
      float *st = opart + (((int64_t)b * d.n_heads + hk * G + g) * nr + rs) * (HD + 2);
      st[2 + e] = o;
      if (e == 0) {
        st[0] = M;
        st[1] = L;
      }
    }
  }
}

// Merge the NS key-range states of each (sequence, query head) in range
// order; one thread per output channel.
__global__ void dec_attn_combine_kernel(const DecodeArgs d, const float *opart, int ns, u16 *a_hi, u16 *a_lo) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d.batch * d.dim) return;
  const int HD = d.head_dim, b = idx / d.dim, c = idx - b * d.dim, h = c / HD, e = c - h * HD;
  const float *st = opart + ((int64_t)b * d.n_heads + h) * ns * (HD + 2);
  float M = -INFINITY;
  for (int r = 0; r < ns; ++r) M = fmaxf(M, st[r * (HD + 2)]);
  float L = 0.f, o = 0.f;
  for (int r = 0; r < ns; ++r) {
    const float f = exp2f(st[r * (HD + 2)] - M);   // 0 for a range that saw no key
    L += f * st[r * (HD + 2) + 1];
    o += f * st[r * (HD + 2) + 2 + e];
  }
  const float v = pos_ok(d.pos[b], d.max_seq) ? o / L : __builtin_nanf("");
  u16 hi, lo;
  split_pair(v, hi, lo);
  a_hi[idx] = hi;
  a_lo[idx] = lo;
}

// Key ranges per (key/value head, sequence): at least 1024 workgroups (four
// per compute unit; the kernel's launch bounds keep four resident). Measured
// on the 7B-shape decode step (batch 32, 2047 cached positions) with 8
// key/value heads (256 pairs): 2.79 / 2.22 / 2.39 / 2.48 ms per step of
// attention with 1 / 2 / 4 / 8 ranges at three workgroups per compute unit;
// with four resident, 4 ranges take 2.06-2.17 ms against 2.09-2.19 with 2.
// 32 heads (1024 pairs) are fastest unsplit (5.94 ms against 6.15 with 2
// ranges).
int dec_attn_ranges(const DecodeArgs &d) {
  int ns = 1;
  while (ns < kDecAttnMaxRanges && d.n_kv_heads * d.batch * ns < 1024) ns *= 2;
  return ns;
}

// Key ranges per (key/value head, sequence) for a cache of max_seq
// positions: ns (the occupancy choice) times one more per kMaxSeq positions,
// so that a range never holds more keys than the ns-range kernel unrolls for.
int dec_attn_range_factor(int max_seq) { return (max(max_seq, 1) + kMaxSeq - 1) / kMaxSeq; }

template <int HD, int G>
hipError_t dec_attn_launch_g(const DecodeArgs &d, const float *part, int splits, const float *ss, uint16_t *kc,
                             uint16_t *vc, uint16_t *a_hi, uint16_t *a_lo, float *opart, int ns, hipStream_t s) {
  const int nr = ns * dec_attn_range_factor(d.max_seq);
  dim3 grid(d.n_kv_heads, d.batch, nr);
  switch (ns) {
    case 1:
      hipLaunchKernelGGL((dec_attn_kernel<HD, G, 1>), grid, dim3(256), 0, s, d, part, splits, ss, kc, vc, a_hi,
                         a_lo, opart);
      break;
    case 2:
      hipLaunchKernelGGL((dec_attn_kernel<HD, G, 2>), grid, dim3(256), 0, s, d, part, splits, ss, kc, vc, a_hi,
                         a_lo, opart);
      break;
    case 4:
      hipLaunchKernelGGL((dec_attn_kernel<HD, G, 4>), grid, dim3(256), 0, s, d, part, splits, ss, kc, vc, a_hi,
                         a_lo, opart);
      break;
    case 8:
      hipLaunchKernelGGL((dec_attn_kernel<HD, G, 8>), grid, dim3(256), 0, s, d, part, splits, ss, kc, vc, a_hi,
                         a_lo, opart);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nr == 1) return e;
  const int n = d.batch * d.dim;
  hipLaunchKernelGGL(dec_attn_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, d, opart, nr, a_hi, a_lo);
  return hipGetLastError();
}

// Matrix-core kernel for grouped heads at head dim 128: key ranges until there
// are at least 256 workgroups (one per compute unit; each range repeats the
// new token's work, so fewer, longer ranges are faster: on the 7B shape with 8
// key/value heads, 1.84-1.92 ms per step of attention with 256 four-wavefront
// workgroups against 1.92-1.98 with 512 and 2.02-2.14 with 1024).
int dec_attn_mfma_ranges(const DecodeArgs &d) {
  int ns = 1;
  while (ns < kDecAttnMaxRanges && d.n_kv_heads * d.batch * ns < 256) ns *= 2;
  return ns;
}

template <int G>
hipError_t dec_attn_mfma_launch(const DecodeArgs &d, const float *part, int splits, const float *ss, uint16_t *kc,
                                uint16_t *vc, uint16_t *a_hi, uint16_t *a_lo, float *opart, hipStream_t s) {
  const int ns = dec_attn_mfma_ranges(d), nr = ns * dec_attn_range_factor(d.max_seq);
  if (nr > 1 && !opart) return hipErrorInvalidValue;
  dim3 grid(d.n_kv_heads, d.batch, nr);
  switch (ns) {
    case 1:
      hipLaunchKernelGGL((dec_attn_mfma_kernel<G, 1>), grid, dim3(512), 0, s, d, part, splits, ss, kc, vc, a_hi, a_lo,
                         opart);
      break;
    case 2:
      hipLaunchKernelGGL((dec_attn_mfma_kernel<G, 2>), grid, dim3(512), 0, s, d, part, splits, ss, kc, vc, a_hi, a_lo,
                         opart);
      break;
    case 4:
      hipLaunchKernelGGL((dec_attn_mfma_kernel<G, 4>), grid, dim3(512), 0, s, d, part, splits, ss, kc, vc, a_hi, a_lo,
                         opart);
      break;
    case 8:
      hipLaunchKernelGGL((dec_attn_mfma_kernel<G, 8>), grid, dim3(512), 0, s, d, part, splits, ss, kc, vc, a_hi, a_lo,
                         opart);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nr == 1) return e;
  const int n = d.batch * d.dim;
  hipLaunchKernelGGL(dec_attn_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, d, opart, nr, a_hi, a_lo);
  return hipGetLastError();
}

hipError_t dec_attn_launch(const DecodeArgs &d, const float *part, int splits, const float *ss, uint16_t *kc,
                           uint16_t *vc, uint16_t *a_hi, uint16_t *a_lo, float *opart, hipStream_t s) {
  if (d.max_seq > kDecMaxCache) return hipErrorInvalidValue;
  if (d.n_kv_heads <= 0 || d.n_heads % d.n_kv_heads) return hipErrorInvalidValue;
  const int group = d.n_heads / d.n_kv_heads;
  const int ns = dec_attn_ranges(d);
  if (ns * dec_attn_range_factor(d.max_seq) > 1 && !opart) return hipErrorInvalidValue;
  // grouped heads at head dim 128: the matrix-core kernel
  if (d.head_dim == 128 && group == 2) return dec_attn_mfma_launch<2>(d, part, splits, ss, kc, vc, a_hi, a_lo, opart, s);
  if (d.head_dim == 128 && group == 4) return dec_attn_mfma_launch<4>(d, part, splits, ss, kc, vc, a_hi, a_lo, opart, s);
  if (d.head_dim == 128 && group == 8) return dec_attn_mfma_launch<8>(d, part, splits, ss, kc, vc, a_hi, a_lo, opart, s);
#define DEC_ATTN_CASE(HD_, G_)                                                                         \
  if (d.head_dim == HD_ && group == G_)                                                               \
    return dec_attn_launch_g<HD_, G_>(d, part, splits, ss, kc, vc, a_hi, a_lo, opart, ns, s);
  DEC_ATTN_CASE(128, 1)
  DEC_ATTN_CASE(128, 2)
  DEC_ATTN_CASE(128, 4)
  DEC_ATTN_CASE(128, 8)
  DEC_ATTN_CASE(64, 1)
  DEC_ATTN_CASE(64, 2)
  DEC_ATTN_CASE(64, 4)
  DEC_ATTN_CASE(64, 8)
#undef DEC_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace llama
