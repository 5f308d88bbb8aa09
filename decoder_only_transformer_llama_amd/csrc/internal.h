// Host-side internal interface between the C-ABI layer (api.hip) and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/llama_mi355x.h"

namespace llama {

// ---------------------------------------------------------------- GEMM
// C[M, N] = A[M, K] * B[N, K]^T on bf16 matrix cores, fp32 accumulate.
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_QKV = 3, EPI_PARTIAL = 4 };
enum BMode { BMODE_PLAIN = 0, BMODE_CONCAT3 = 1, BMODE_GATEUP = 2 };

struct GemmArgs {
  int M, N, K;                   // K % (32 * k_splits) == 0
  int k_splits;                  // >= 1: grid.y splits K into equal contiguous ranges
  int n_base, n_end;             // columns [n_base, n_end) of C (n_end 0: N); n_base % BN == 0
  float *part;                   // EPI_PARTIAL: fp32 [k_splits][M][N] partial products
  const uint16_t *A;             // [M, lda] bf16 (hi part when A_lo is set)
  const uint16_t *A_lo;          // optional lo part of a bf16 pair, same layout
  int64_t lda;
  const float *rstd;             // optional per-row scale applied to the accumulator
  int b_mode;
  const uint16_t *B0, *B1, *B2;  // weights [rows, K] bf16 (fp16 with key f16 == 2)
  int n_seg;                     // BMODE_CONCAT3: rows of B0 (the query projection)
  int n_seg_kv;                  // BMODE_CONCAT3: rows of B1 and of B2 (0: n_seg)
  // EPI_STORE / EPI_RESID / EPI_SILU outputs
  void *C;            // f32 or bf16 (EPI_SILU: bf16 hi, or fp16 when c_f16)
  uint16_t *C_lo;     // EPI_SILU / EPI_STORE bf16: optional lo part
  int c_f16;          // EPI_SILU: u as IEEE fp16 (the operand of an fp16 down projection)
  int c_f32;          // EPI_STORE: 1 -> f32 output, 0 -> bf16
  int64_t ldc;
  const void *R;      // EPI_RESID residual [M, ldc]
  int r_f32;
  // EPI_QKV
  uint16_t *qh, *ql, *kh, *kl;   // [M, dim] hi/lo of rotated q and k
  uint16_t *vth, *vtl;           // [batch, n_heads, head_dim, vt_stride] hi/lo of v (transposed)
  int attn_f16;                  // 1: qh, kh, vth hold fp16 (no lo parts written)
  float q_mul;                   // with attn_f16: q is written times this factor (the
                                 // attention's log2(e)/sqrt(head_dim)); 0 = none
  const float2 *rope_tab;        // [seq, head_dim/2] (cos, sin)
  int seq, n_heads, head_dim, dim;
  int kv_dim, n_kv_heads;        // width and heads of k and v (0: dim, n_heads)
  int vt_stride;                 // row stride of the transposed v (>= seq, multiple of 64)
  uint16_t *kcache, *vcache;     // optional bf16: [batch, n_kv_heads, max_seq, head_dim] of this layer
  int max_seq;
  // Prefill that continues a cached prefix: sequence b's rows take positions
  // start_pos[b] + s (RoPE angle, cache slot), and k and v^T are stored by
  // position, k at row b * kv_rows + position. nullptr: positions 0..seq-1,
  // k at the token's own row. A sequence whose chunk does not fit the cache
  // (chunk_start < 0) is computed as if it started at 0 and writes no cache.
  const int32_t *start_pos;
  int kv_rows;                   // rows per sequence of k (0: seq)
  // EPI_PARTIAL with k_splits == 2 and tile_flags (one int per output tile,
  // zero before the launch): range 0 stores its partial coherently and sets
  // its tile's flag; range 1 waits for the flag, then writes
  // C = (R + partial 0) + its own product (fp32, R fp32), the order of
  // adding the ranges after the launch. Requires the row-contiguous epilogue
  // (gemm_fused_split_ok).
  int *tile_flags;
};
// The layouts the fused split-K residual runs with (those of the GEMM's
// row-contiguous epilogue): N % 32 == 0, ldc % 16 == 0, 16-byte aligned
// C, C_lo, R and part, and a partial below 4 GiB (32-bit buffer offsets).
inline bool gemm_fused_split_ok(const GemmArgs &a) {
  return a.N % 32 == 0 && a.ldc % 16 == 0 && (int64_t)a.M * a.N < (int64_t(1) << 30) &&   // 32-bit byte offsets
         (((uintptr_t)a.C | (uintptr_t)a.C_lo | (uintptr_t)a.R | (uintptr_t)a.part) % 16) == 0;
}

// Position of the first token of sequence b's chunk of `seq` tokens:
// start_pos[b] when 0 <= start_pos[b] and start_pos[b] + seq <= max_seq, -1
// otherwise; 0 without start_pos.
__host__ __device__ inline int chunk_start(const int32_t *start_pos, int b, int seq, int max_seq) {
  if (!start_pos) return 0;
  const int p = start_pos[b];
  return (p >= 0 && p <= max_seq - seq) ? p : -1;
}

// Row n of the BMODE_CONCAT3 operand [B0 (n_q rows); B1 (n_kv rows); B2 (n_kv rows)]:
// the query, key and value projections stacked (fewer key/value rows under
// grouped-query attention).
__host__ __device__ inline const uint16_t *concat3_row(const uint16_t *B0, const uint16_t *B1, const uint16_t *B2,
                                                       int n_q, int n_kv, int n, int64_t K) {
  if (n < n_q) return B0 + (int64_t)n * K;
  if (n < n_q + n_kv) return B1 + (int64_t)(n - n_q) * K;
  return B2 + (int64_t)(n - n_q - n_kv) * K;
}

struct GemmKey {
  int bn, apair, epi;
  int f16 = 0;   // 1: A operand fp16, B (bf16 weights) converted to fp16 in registers;
                 // 2: A and B (weights converted ahead of time) both fp16
  int bm = 256;  // tile rows: 256, or 192 (256-wide single-operand SiLU tiles)
};

// Returns a hipError_t; hipErrorInvalidValue when no instance matches `key`.
hipError_t gemm_launch(const GemmKey &key, const GemmArgs &a, hipStream_t s);
hipError_t gemm_launch_qkv(const GemmKey &key, const GemmArgs &a, hipStream_t s);
hipError_t gemm_launch_ffn(const GemmKey &key, const GemmArgs &a, hipStream_t s);
hipError_t gemm_launch_misc(const GemmKey &key, const GemmArgs &a, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const uint16_t *qh, *ql, *kh, *kl;   // [batch*seq, dim]
  const uint16_t *vth, *vtl;           // [batch, n_heads, head_dim, seq]
  void *o;                             // [batch*seq, dim] f32, bf16 (hi) or fp16
  uint16_t *o_lo;                      // optional lo part (bf16 output only)
  int o_f32;
  int o_f16;                           // output as IEEE fp16 (no lo part)
  int batch, seq, n_heads, head_dim, dim;
  int kv_dim, n_kv_heads;              // k rows [batch*seq, kv_dim]; v^T [batch, n_kv_heads, head_dim, vt_stride]
  int vt_stride;                       // row stride of v^T (>= keys per sequence, multiple of 64)
  float scale_log2;                    // log2(e) / sqrt(head_dim)
  int q_scaled;                        // q already carries scale_log2 (required with fp16 operands)
  // With start_pos, sequence b's queries are positions p0 .. p0+seq-1
  // (p0 = chunk_start(start_pos, b, seq, max_seq), 0 when negative) and its
  // keys are positions 0 .. p0+seq-1: k rows b * kv_rows + position, v^T
  // columns by position; query s sees keys up to p0 + s.
  const int32_t *start_pos;
  int kv_rows;                         // rows per sequence of k (0: seq)
  int max_seq;
};
// f16: q, k, v^T hold IEEE fp16 (single, no lo parts), q already multiplied
// by scale_log2 (q_scaled = 1, else hipErrorInvalidValue), and the
// probabilities are rounded to fp16; otherwise bf16 with optional hi/lo pairs.
hipError_t attn_prefill_launch(const AttnArgs &a, int qk_pair, int v_pair, int f16, hipStream_t s);
// The cached prefix of a prefill chunk in the attention's operand layout: for
// every sequence b with p0 = chunk_start(...) > 0, cache positions 0..p0-1 of
// this layer (bf16 [batch, n_kv, max_seq, hd]) go to k rows b * kv_rows + j
// and to v^T columns j (IEEE fp16 when f16, else bf16 with zero lo parts when
// kl / vtl are given); v^T columns p0+seq .. up to the next multiple of 32 are
// zeroed (the attention's last key tile multiplies them by zero weights).
hipError_t kv_prefix_launch(const uint16_t *kcache, const uint16_t *vcache, const int32_t *start_pos, int batch,
                            int n_kv, int head_dim, int max_seq, int seq, uint16_t *kh, uint16_t *kl, uint16_t *vth,
                            uint16_t *vtl, int kv_rows, int vt_stride, int f16, hipStream_t s);
// logits rows [b*seq, (b+1)*seq) set to NaN for every sequence whose chunk
// does not fit the cache (chunk_start < 0).
hipError_t nan_unplaced_rows_launch(const int32_t *start_pos, int batch, int seq, int max_seq, float *logits,
                                    int vocab, hipStream_t s);

// ---------------------------------------------------------------- small kernels
hipError_t rope_table_launch(float2 *tab, int positions, int head_dim, float theta, hipStream_t s);
hipError_t rope_table_pos_launch(float2 *tab, const int32_t *pos, int n, int head_dim, float theta,
                                 int max_seq, hipStream_t s);
// Norm prep (one wavefront per row): the GEMM operand x[r] * g (bf16 hi, and
// lo when xg_lo is non-null; IEEE fp16 with out_f16, carrying an exact
// power-of-two row scale that keeps it inside fp16's range) and rmul[r], the
// multiplier the consumer applies to its fp32 accumulator: rstd[r] =
// 1/sqrt(mean(x[r]^2) + eps) times the inverse of that scale. g == nullptr
// gives x[r] itself (no norm: rmul only undoes the scale).
// With `part` (n_parts fp32 [rows, dim] split-K partial products), the row is
// first h = x + part[0] + ... (split order), written to h_out (fp32), and the
// statistics and product are those of h.
// With rope.positions > 0 (at most rows) the same launch also writes the
// RoPE (cos, sin) table of positions 0 .. rope.positions-1, as
// rope_table_launch does.
struct RopeRows {
  float2 *tab = nullptr;
  int positions = 0, hd = 0;
  double theta = 0.0;
};
// zero / n_zero: ints the launch also clears (flags a later kernel of the
// same stream counts on starting at zero).
hipError_t norm_prep_launch(int in_f32, const void *x, const uint16_t *g, int64_t rows, int dim, float eps,
                            float *rmul, uint16_t *xg_hi, uint16_t *xg_lo, hipStream_t s,
                            const float *part = nullptr, int n_parts = 0, float *h_out = nullptr,
                            int out_f16 = 0, RopeRows rope = RopeRows{}, int *zero = nullptr, int n_zero = 0);
// Index of the largest logit per row (lowest among equals; -1 if the row has a NaN).
hipError_t argmax_launch(const float *logits, int64_t rows, int vocab, int32_t *out, hipStream_t s);
// y = r + part[0] + ... + part[n_parts-1], fp32, n elements (n % 4 == 0).
hipError_t resid_sum_launch(const float *r, const float *part, int n_parts, int64_t n, float *y, hipStream_t s);
// y = x / sqrt(mean(x^2) + eps) * g per row; g in fp32 when g_f32 (default:
// the dtype of x); y may alias x.
hipError_t rmsnorm_launch(int in_f32, int out_f32, const void *x, const void *g, void *y, int64_t rows,
                          int dim, float eps, hipStream_t s, int g_f32 = -1);
// pos == nullptr: the position of token t is t % seq_mod.
// inverse: rotate by minus the angle (the transpose of RoPE, for its gradient).
hipError_t rope_launch(int f32, const void *x, void *y, const int32_t *pos, int64_t tokens, int n_heads,
                       int head_dim, float theta, int seq_mod, hipStream_t s, int inverse = 0);
hipError_t attn_pack_launch(int in_f32, const void *q, const void *k, const void *v, uint16_t *qh,
                            uint16_t *ql, uint16_t *kh, uint16_t *kl, uint16_t *vth, uint16_t *vtl,
                            int batch, int seq, int n_heads, int head_dim, int vt_stride, hipStream_t s);
hipError_t embed_launch(int w_f32, const void *emb, const int32_t *tokens, int64_t n, int dim, int vocab,
                        float *x, hipStream_t s);

// fp32 path (small workloads, plain VALU kernels)
hipError_t gemm_f32_launch(const float *A, const float *B, float *C, const float *R, int M, int N, int K,
                           hipStream_t s);
// fp32 GEMM on the matrix cores for operands with a unit stride along K or
// along M / N (16-byte aligned runs); hipErrorNotSupported for other layouts.
hipError_t gemm_f32_mfma_launch(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk, int64_t sbn,
                                float *C, const float *R, int M, int N, int K, int accumulate, hipStream_t s);
hipError_t silu_mul_f32_launch(const float *g, const float *u, float *out, int64_t n, hipStream_t s);
// lse (optional): [batch][n_heads][seq] log-sum-exp of each query's scaled scores.
hipError_t attn_f32_launch(const float *q, const float *k, const float *v, float *o, int batch, int seq,
                           int n_heads, int head_dim, hipStream_t s, float *lse = nullptr);
hipError_t convert_launch(int in_f32, int out_f32, const void *x, void *y, int64_t n, hipStream_t s);

// ---------------------------------------------------------------- decode
struct GemvArgs {
  int M, N, K, k_chunk, splits;
  const uint16_t *A_hi, *A_lo;   // [M, K] bf16 pair
  int b_mode;
  const uint16_t *B0, *B1, *B2;
  int n_seg, n_seg_kv;           // BMODE_CONCAT3 row counts (n_seg_kv 0: n_seg)
  const uint16_t *packed;        // optional: the same matrix in 32-row tile order (see pack_tiles_launch)
  float *part;                   // [splits, M, N]
};
// Tile-packed weights: one 4 KB block per (32-column tile t, 64-wide K step),
// holding the 64 lanes' 16-byte B-operand pieces in lane order. Blocks are
// ordered chunk-major for the split-K chunks of kcs steps (the last chunk may
// be shorter): all tiles' blocks of chunk 0, then chunk 1, ...; within a
// chunk tile-major, step-minor. The blocks one workgroup streams (its
// consecutive tiles over one K chunk) are then one contiguous region.
__host__ __device__ inline int64_t pack_block(int t, int st, int n_tiles, int ksteps, int kcs) {
  const int c = st / kcs, s = st - c * kcs;
  const int len = ksteps - c * kcs < kcs ? ksteps - c * kcs : kcs;
  return (int64_t)c * n_tiles * kcs + (int64_t)t * len + s;
}

hipError_t gemv_launch(const GemvArgs &a, hipStream_t s);
// Copy B (row mapping b_mode as in GemvArgs) into tile order: 4 KB block per
// (32-row tile t, 64-wide K step s), piece (q, lane g*32+j) = B[32t+j][64s+32g+8q..+7];
// rows >= N are zero. dst holds ceil(N/32)*32 x K elements.
// Tile-packed copy of B for the skinny GEMM, ordered for split-K chunks of
// k_chunk (the chunk the skinny GEMM later runs with for this N and K).
hipError_t pack_tiles_launch(int b_mode, const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int n_seg,
                             int n_seg_kv, int N, int K, int k_chunk, uint16_t *dst, hipStream_t s);
// Shape of the skinny product of N columns over K: 32-column tiles per
// wavefront (ntw), K range per workgroup (k_chunk) and number of ranges.
struct GemvShape {
  int ntw, k_chunk, splits;
};
GemvShape gemv_shape(int N, int K);
constexpr int kGemvMaxChunk = 512;  // largest K range of one workgroup

struct DecodeArgs {
  int batch, dim, n_heads, head_dim, hidden, max_seq, vocab;
  int n_kv_heads;                // key/value heads (query heads per group: n_heads / n_kv_heads)
  float eps;
  const int32_t *pos;            // [batch]
  const float2 *rope_tab;        // [batch, head_dim/2] for pos[b]
};
// Row statistics travel as partial sums of squares ss[b][dim/1024 chunks].
// x[b] = emb[tok[b]] (f32), ss, xg pair = x*g
hipError_t dec_embed_norm_launch(const DecodeArgs &d, const uint16_t *emb, const int32_t *tok,
                                 const uint16_t *g, float *x, float *ss, uint16_t *xg_hi,
                                 uint16_t *xg_lo, hipStream_t s);
// Attention of one new token per sequence over the KV cache, fused with the
// finish of the Q/K/V split-K partials (rstd, RoPE, cache append at pos[b]);
// writes the head outputs as a bf16 pair [batch, dim]. max_seq <= kDecMaxCache.
// opart: [batch, n_heads, kDecAttnMaxRanges * dec_attn_range_factor(max_seq),
// head_dim + 2] fp32 states of the key ranges (unused with one range).
constexpr int kDecAttnMaxRanges = 8;
// Longest decode cache: a cache of max_seq positions takes
// dec_attn_range_factor(max_seq) (one per 2048 positions) times the key
// ranges, and opart room for that many.
constexpr int kDecMaxCache = 16384;
int dec_attn_range_factor(int max_seq);
int dec_attn_ranges(const DecodeArgs &d);
hipError_t dec_attn_launch(const DecodeArgs &d, const float *part, int splits, const float *ss, uint16_t *kc,
                           uint16_t *vc, uint16_t *a_hi, uint16_t *a_lo, float *opart, hipStream_t s);
// out = res + sum(part); ss of out; out*g as pair
hipError_t dec_resid_norm_launch(const DecodeArgs &d, const float *res, const float *part, int splits,
                                 const uint16_t *g, float *out, float *ss, uint16_t *og_hi,
                                 uint16_t *og_lo, hipStream_t s);
hipError_t dec_gateup_combine_launch(const DecodeArgs &d, const float *part, int splits,
                                     const float *ss, uint16_t *u_hi, uint16_t *u_lo, hipStream_t s);
hipError_t dec_head_combine_launch(const DecodeArgs &d, const float *part, int splits, const float *ss,
                                   float *logits, hipStream_t s);

// ------------------------------------------------------------------ backward (fp32)
// C[m, n] = (accumulate ? C : 0) + sum_k A[m*sam + k*sak] B[k*sbk + n*sbn]
hipError_t gemm_f32_strided_launch(const float *A, int64_t sam, int64_t sak, const float *B, int64_t sbk,
                                   int64_t sbn, float *C, int M, int N, int K, int accumulate, hipStream_t s);
// dq, dk, dv of causal attention from q, k, v, the forward output o, its
// log-sum-exp lse [batch][n_heads][seq] and dout; delta: scratch of the lse's size.
// kv_part: nullptr, or kAttnBwdKvRanges * 2 * batch * seq * n_heads * head_dim
// floats of scratch, with which the key/value-gradient loop runs split over
// up to that many workgroups per key tile while the key tiles alone make
// fewer than 256 workgroups.
constexpr int kAttnBwdKvRanges = 4;
hipError_t attn_bwd_launch(const float *q, const float *k, const float *v, const float *o, const float *dout,
                           const float *lse, float *delta, float *dq, float *dk, float *dv, int batch, int seq,
                           int n_heads, int head_dim, hipStream_t s, float *kv_part = nullptr);
// dx = add + gradient of RMSNorm(x; g) for dy; dg = its gain gradient; rstd: [rows] scratch.
hipError_t rmsnorm_bwd_launch(const float *x, const float *g, const float *dy, const float *add, float *dx,
                              float *dg, float *rstd, int64_t rows, int dim, float eps, hipStream_t s);
hipError_t swiglu_bwd_launch(const float *gate, const float *up, const float *du, float *d_gate, float *d_up,
                             int64_t n, hipStream_t s);
hipError_t axpby_launch(float *z, const float *x, const float *y, float a, float b, int64_t n, hipStream_t s);
// dst[i] = IEEE fp16 of the bf16 value src[i], by the GEMM's in-register
// weight conversion (round toward zero). src == dst allowed.
hipError_t bf16_to_f16_launch(const uint16_t *src, uint16_t *dst, int64_t n, hipStream_t s);


}  // namespace llama
