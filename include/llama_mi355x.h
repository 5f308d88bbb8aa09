/*
 * llama_mi355x.h — C ABI of the MI355X (gfx950) LLaMA pre-norm decoder block
 * forward library (libllama_mi355x.so).
 *
 * What is computed follows these pages:
 *  [P1] paperfordummies.in, "LLaMA: Open and Efficient Foundation Language
 *       Models" (explained as a diff): sections "The one formula",
 *       "RMSNorm: LayerNorm minus the mean", "SwiGLU: a gate in the FFN, paid
 *       for with a narrower hidden layer", "RoPE: rotate Q and K, leave V
 *       alone", "6.7B parameters, 1T tokens: the arithmetic", "The code".
 *  [P4] chenyuan1125.github.io, "LLaMA: No Architecture Revolution, Yet It
 *       Became the Open-Model Foundation": section "An Architecture Recipe
 *       Without an Invention Myth" (RMSNorm with gain g, SwiGLU, RoPE
 *       equations) and "GQA Was Not an Original LLaMA Feature" (KV cache).
 *
 * Conventions shared by every entry point
 *  - Pointers named in the argument list are DEVICE pointers (memory the
 *    caller allocated on the current HIP device) unless marked "host".
 *    The library never allocates, frees or synchronises: scratch memory comes
 *    from a caller-provided workspace whose size llama_workspace_size reports
 *    (llama_model_decode_static instead uses a device array the library
 *    owns).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream). Buffers must stay valid until the stream passes the call.
 *  - Activations are [tokens, dim] row-major with token = b*seq + s. Head h
 *    owns columns [h*head_dim, (h+1)*head_dim). Weights are [out, in]
 *    row-major, so a projection is y = x W^T ([P1] writes x @ W with W
 *    [in, out]: the same map). Norm gains are [dim] in the weight dtype.
 *  - bf16 is IEEE binary32 truncated to its top 16 bits (round to nearest
 *    even when the library narrows). Accumulation, softmax, norm statistics
 *    and RoPE run in fp32.
 *  - Every entry point returns a llama_status. Arguments are validated on the
 *    host before anything is enqueued; a failed validation enqueues nothing.
 *    A HIP launch error returns LLAMA_ERR_HIP and its text is kept for
 *    llama_last_error() (per thread). No C++ exception crosses the ABI.
 *  - Floating-point special values in the data are data: eps = 0 on an
 *    all-zero row gives NaN, as the mathematics says ([P1] "RMSNorm ...").
 */
#ifndef LLAMA_MI355X_H
#define LLAMA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLAMA_F32 = 0, LLAMA_BF16 = 1 } llama_dtype;

typedef enum {
  LLAMA_OK = 0,
  LLAMA_ERR_NULL = -1,        /* a required pointer is NULL */
  LLAMA_ERR_SHAPE = -2,       /* a size is <= 0, inconsistent, or does not fit the kernels' tiling */
  LLAMA_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination */
  LLAMA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than llama_workspace_size */
  LLAMA_ERR_POSITION = -5,    /* a position or sequence length exceeds max_seq */
  LLAMA_ERR_UNSUPPORTED = -6, /* valid request outside what this build implements */
  LLAMA_ERR_HIP = -7          /* the HIP runtime reported an error; see llama_last_error */
} llama_status;

/* Operations for llama_workspace_size. */
typedef enum {
  LLAMA_OP_CAUSAL_ATTN = 1,
  LLAMA_OP_SWIGLU_FFN = 2,
  LLAMA_OP_BLOCK_FORWARD = 3,
  LLAMA_OP_MODEL_FORWARD = 4,
  LLAMA_OP_MODEL_DECODE = 5,
  LLAMA_OP_CAUSAL_ATTN_BACKWARD = 6,
  LLAMA_OP_BLOCK_BACKWARD = 7 /* also the workspace of llama_block_train_forward */
} llama_op;

/* Numerics options of the bf16 path (llama_config.numerics). Weights are
 * exact bf16 inputs; an activation operand of a bf16 matrix-core product is
 * either rounded to bf16 or carried as an exact-to-2^-16 pair hi + lo of two
 * bf16 values (two products, same fp32 accumulator). Other bits use IEEE fp16
 * operands instead (11 significant bits against bf16's 8, one pass per
 * product, values below 65504 in magnitude):
 *  - LLAMA_NUM_ATTN_F16: q, k, v and the probabilities inside attention;
 *  - LLAMA_NUM_{QKV,O,FFN,DOWN}_A_F16: the activation operand of that block
 *    projection (x*g1, the attention output, h*g2, SiLU(gate)*up); the bf16
 *    weights are converted to fp16 in registers, exactly for magnitudes in
 *    [2^-14, 65504] (smaller ones become fp16 subnormals, within 2^-24).
 *    LLAMA_NUM_GEMM_F16 is all four.
 *  - LLAMA_NUM_W_F16: the weights of every projection whose activation
 *    operand is fp16 arrive as IEEE fp16 instead of bf16, made once by
 *    llama_convert_weights_f16 (wq, wk, wv with QKV_A_F16, and the output head
 *    of llama_model_forward with it; wo with O_A_F16; w_gate, w_up with
 *    FFN_A_F16; w_down with DOWN_A_F16). That is the conversion the matrix
 *    cores' operand otherwise gets in registers, so results are bit-identical
 *    to the same set without this bit; it only moves the conversion out of the
 *    GEMM loop. Gains, embeddings and the other projections stay bf16.
 *    llama_pack_decode_weights rejects it (the pack is built from bf16
 *    weights), and llama_model_decode accepts it only with a decode pack.
 * LLAMA_NUM_DEFAULT (0) selects the library's default set,
 * LLAMA_NUM_ATTN_F16 | LLAMA_NUM_QKV_A_F16 | LLAMA_NUM_O_A_F16 |
 * LLAMA_NUM_FFN_A_F16 (SiLU(gate)*up stays a single bf16 value), and
 * LLAMA_NUM_W_F16 alone that set with fp16 weights;
 * LLAMA_NUM_EXPLICIT plus any of the
 * bits selects exactly those (ATTN_F16 excludes QK_PAIR and V_PAIR; an
 * operand is either a pair or fp16). Any other value (option bits without
 * LLAMA_NUM_EXPLICIT, unknown bits) is LLAMA_ERR_UNSUPPORTED. The KV cache is
 * bf16 in every mode. */
#define LLAMA_NUM_DEFAULT 0u
#define LLAMA_NUM_EXPLICIT (1u << 31)
#define LLAMA_NUM_QKV_A_PAIR (1u << 0)  /* x*g1 operand of the Q/K/V projection */
#define LLAMA_NUM_QK_PAIR (1u << 1)     /* q and k of the attention scores (3 products) */
#define LLAMA_NUM_V_PAIR (1u << 2)      /* v of the probability-weighted sum */
#define LLAMA_NUM_O_A_PAIR (1u << 3)    /* attention output into the Wo projection */
#define LLAMA_NUM_FFN_A_PAIR (1u << 4)  /* h*g2 operand of the gate/up projection */
#define LLAMA_NUM_DOWN_A_PAIR (1u << 5) /* SiLU(gate)*up operand of the down projection */
#define LLAMA_NUM_ATTN_F16 (1u << 6)    /* q, k, v and probabilities as fp16 in prefill attention */
#define LLAMA_NUM_QKV_A_F16 (1u << 7)   /* x*g1 operand of the Q/K/V projection as fp16 */
#define LLAMA_NUM_O_A_F16 (1u << 8)     /* attention output into the Wo projection as fp16 */
#define LLAMA_NUM_FFN_A_F16 (1u << 9)   /* h*g2 operand of the gate/up projection as fp16 */
#define LLAMA_NUM_DOWN_A_F16 (1u << 10) /* SiLU(gate)*up operand of the down projection as fp16 */
#define LLAMA_NUM_GEMM_F16 (LLAMA_NUM_QKV_A_F16 | LLAMA_NUM_O_A_F16 | LLAMA_NUM_FFN_A_F16 | LLAMA_NUM_DOWN_A_F16)
#define LLAMA_NUM_W_F16 (1u << 11)      /* weights of the fp16-operand projections supplied as fp16 */

/* Where a block's two RMSNorms sit ([P1] "Pre-norm: the norm goes on the
 * branch, not the trunk" and "Now break it"). With Attn and FFN the two
 * branches of the block:
 *   PRE  (LLaMA): h = x + Attn(RMSNorm(x; g1)),  y = h + FFN(RMSNorm(h; g2))
 *   POST (2017):  h = RMSNorm(x + Attn(x); g1),  y = RMSNorm(h + FFN(h); g2)
 *   NONE:         h = x + Attn(x),               y = h + FFN(h)  (gains unused) */
typedef enum { LLAMA_NORM_PRE = 0, LLAMA_NORM_POST = 1, LLAMA_NORM_NONE = 2 } llama_norm_placement;

/* Model / block configuration. head_dim = dim / n_heads. */
typedef struct llama_config {
  int32_t dim;        /* model width d */
  int32_t n_heads;    /* query heads */
  int32_t hidden;     /* SwiGLU hidden width (llama_hidden_dim(dim, 256) for LLaMA) */
  int32_t n_layers;   /* blocks in the model (model entry points only) */
  int32_t vocab;      /* embedding rows / output-head width (model entry points only) */
  int32_t max_seq;    /* KV-cache positions per sequence (model entry points only) */
  float norm_eps;     /* RMSNorm epsilon, inside the square root */
  float rope_theta;   /* RoPE base (10000 for LLaMA) */
  int32_t dtype;      /* llama_dtype of weights, gains, inputs and KV cache */
  uint32_t numerics;  /* LLAMA_NUM_* (bf16 path only; ignored for LLAMA_F32) */
  int32_t n_kv_heads; /* key/value heads; 0 means n_heads (LLaMA-1: one K/V head per
                       * query head). Fewer divide n_heads: grouped-query attention,
                       * consecutive groups of n_heads / n_kv_heads query heads
                       * sharing one K/V head ([P4] "GQA Was Not an Original LLaMA
                       * Feature"). bf16 block/model entry points only; group size
                       * 1, 2, 4 or 8; n_kv_heads * head_dim a multiple of 128. */
  int32_t norm_placement; /* llama_norm_placement; llama_block_forward only, the model
                           * entry points take LLAMA_NORM_PRE */
} llama_config;

/* Weights of one block, device pointers in config dtype ([P1] "The one
 * formula"; parameter set of [P1] "6.7B parameters ..."): two norm gains
 * [dim], wq/wo [dim, dim], wk/wv [n_kv_heads * head_dim, dim] (= [dim, dim]
 * for LLaMA), w_gate/w_up [hidden, dim], w_down [dim, hidden]. */
typedef struct llama_block_weights {
  const void *attn_norm, *wq, *wk, *wv, *wo;
  const void *ffn_norm, *w_gate, *w_up, *w_down;
} llama_block_weights;

/* Whole-model weights: token embedding [vocab, dim], `layers` is a HOST
 * array of n_layers block-weight structs (holding device pointers), the final
 * norm gain [dim] and the untied output head [vocab, dim]. decode_pack is
 * NULL, or a device buffer filled by llama_pack_decode_weights from these same
 * weights: llama_model_decode then streams the projections from it. */
typedef struct llama_model_weights {
  const void *tok_embeddings;
  const llama_block_weights *layers;
  const void *final_norm;
  const void *output;
  const void *decode_pack;
} llama_model_weights;

/* SwiGLU hidden width: int(2*4*dim/3) rounded up to a multiple of
 * multiple_of ([P1] "SwiGLU ..." and llama_hidden in "The code").
 * Host only. Returns -1 for dim <= 0 or multiple_of <= 0. */
int llama_hidden_dim(int dim, int multiple_of);

/* RMSNorm with gain ([P1] rms_norm; [P4] RMSNorm equation):
 *   y[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * g
 * x [rows, dim] in in_dtype; g [dim] in in_dtype, or NULL for g = 1;
 * y [rows, dim] in out_dtype (may alias x when the dtypes match).
 * Errors: NULL x/y, rows < 0 or dim <= 0, unknown dtypes. rows == 0 is a no-op. */
int llama_rmsnorm(int in_dtype, int out_dtype, const void *x, const void *g, void *y,
                  int64_t rows, int dim, float eps, void *stream);

/* Rotary position embedding on each head ([P1] rope; [P4] RoPE):
 * channels (2i, 2i+1) of every head are rotated by the angle
 * positions[t] * theta^(-2i/head_dim), i < head_dim/2 (interleaved pairs).
 * x, y [tokens, n_heads*head_dim] in dtype (y may alias x);
 * positions [tokens] int32 (device). Angles are formed in fp64.
 * Errors: NULL pointers, tokens < 0, n_heads <= 0, odd head_dim, bad dtype. */
int llama_rope(int dtype, const void *x, void *y, const int32_t *positions, int64_t tokens,
               int n_heads, int head_dim, float theta, void *stream);

/* Projection y = x W^T (the matrix products of [P1] "The code").
 * x [rows, k] and w [n, k] in the same dtype; y [rows, n] in y_dtype.
 * bf16 runs on the matrix cores with fp32 accumulation (y f32 or bf16);
 * f32 runs in fp32 on the vector ALUs (y f32).
 * Errors: NULL pointers, sizes <= 0, k % 64 != 0 for bf16, mixed or bad dtypes. */
int llama_linear(int x_dtype, int w_dtype, int y_dtype, const void *x, const void *w, void *y,
                 int64_t rows, int n, int k, void *stream);

/* Causal scaled-dot-product attention per (sequence, head) ([P1] "LLaMA is a
 * pull request ...": the 2017 attention with a causal mask):
 *   o_i = sum_{j<=i} softmax_j(q_i . k_j / sqrt(head_dim)) v_j
 * q, k, v [batch*seq, n_heads*head_dim] in in_dtype (bf16 or f32);
 * o [batch*seq, n_heads*head_dim] in out_dtype (f32 or bf16).
 * ws / ws_bytes: workspace of at least llama_workspace_size(LLAMA_OP_CAUSAL_ATTN).
 * head_dim must be 64 or 128. Errors: NULL pointers, sizes <= 0,
 * unsupported head_dim, workspace too small, bad dtypes. */
int llama_causal_attn(int in_dtype, int out_dtype, const void *q, const void *k, const void *v,
                      void *o, int batch, int seq, int n_heads, int head_dim, void *ws,
                      size_t ws_bytes, void *stream);

/* SwiGLU feed-forward ([P1] swiglu_ffn; [P4] SwiGLU):
 *   y = (SiLU(z W_gate^T) * (z W_up^T)) W_down^T,  SiLU(t) = t / (1 + e^-t)
 * z [tokens, dim] in in_dtype; w_gate, w_up [hidden, dim] and w_down
 * [dim, hidden] in in_dtype; y [tokens, dim] in out_dtype (f32 or bf16).
 * bf16: dim % 64 == 0, hidden % 128 == 0. ws as llama_workspace_size(LLAMA_OP_SWIGLU_FFN)
 * with config {dim, hidden, dtype = in_dtype} and batch*seq = tokens. */
int llama_swiglu_ffn(int in_dtype, int out_dtype, const void *z, const void *w_gate,
                     const void *w_up, const void *w_down, void *y, int64_t tokens, int dim,
                     int hidden, void *ws, size_t ws_bytes, void *stream);

/* One pre-norm LLaMA block ([P1] "The one formula", pre_norm_block):
 *   h = x + Wo CausalAttn(RoPE(Wq z), RoPE(Wk z), Wv z),  z  = RMSNorm(x; attn_norm)
 *   y = h + W_down (SiLU(W_gate z2) * W_up z2),           z2 = RMSNorm(h; ffn_norm)
 * RoPE positions are 0..seq-1 in every sequence; V is not rotated.
 * x [batch*seq, dim] in x_dtype (config dtype, or f32); y [batch*seq, dim] f32.
 * Requirements: head_dim 64 or 128; bf16: dim % 256 == 0, hidden % 128 == 0.
 * ws: llama_workspace_size(c, LLAMA_OP_BLOCK_FORWARD, batch, seq). */
int llama_block_forward(const llama_config *c, const llama_block_weights *w, int x_dtype,
                        const void *x, float *y, int batch, int seq, void *ws, size_t ws_bytes,
                        void *stream);

/* Whole-model prefill ([P1] "The one formula": embedding, the blocks, one
 * final RMSNorm, then the output head) of tokens [batch, seq] (int32, device).
 * start_pos (int32 [batch], device, or NULL for all zeros): sequence b's
 * tokens take positions start_pos[b] .. start_pos[b]+seq-1 (their RoPE angles
 * and cache slots), and each attends over cache slots 0 .. its own position:
 * the cache keeps the keys and values of every earlier token ([P4] "GQA Was
 * Not an Original LLaMA Feature"), so slots below start_pos[b] must hold the
 * entries an earlier llama_model_forward or llama_model_decode wrote. That
 * allows a prompt to be prefilled in chunks or extended after decoding. Each
 * layer's rotated keys and values of the new tokens are written to their
 * slots. k_cache, v_cache: [n_layers][batch][n_kv_heads][max_seq][head_dim]
 * in config dtype. logits [batch, seq, vocab] f32. The head's operand
 * RMSNorm(x; final_norm) is carried as the Q/K/V projection's operand is
 * (numerics bits QKV_A_F16 / QKV_A_PAIR).
 * The host cannot see start_pos: a sequence with start_pos[b] < 0 or
 * start_pos[b] + seq > max_seq gets NaN logits rows and no cache write; the
 * other sequences are unaffected.
 * bf16 configs only (LLAMA_ERR_UNSUPPORTED for f32). seq <= max_seq
 * (LLAMA_ERR_POSITION otherwise).
 * ws: llama_workspace_size(c, LLAMA_OP_MODEL_FORWARD, batch, seq), which
 * holds keys for max_seq positions per sequence. */
int llama_model_forward(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                        const int32_t *start_pos, int batch, int seq, void *k_cache, void *v_cache,
                        float *logits, void *ws, size_t ws_bytes, void *stream);

/* One decode step ([P4] "GQA Was Not an Original LLaMA Feature": keys and
 * values of earlier tokens are cached; LLaMA-1 has one K/V head per query
 * head): for each sequence b, token tokens[b] at position pos[b] (int32
 * arrays [batch], device) runs through every block, its rotated key and value
 * are written to cache slot pos[b], attention covers slots 0..pos[b], then the
 * final norm and head give logits [batch, vocab] f32. The caches have the
 * layout of llama_model_forward. A pos[b] outside [0, max_seq) cannot be
 * checked on the host: for such a row nothing is written to the cache and
 * its logits are NaN. max_seq <= 16384 (LLAMA_ERR_UNSUPPORTED above); any
 * batch: more than 32 sequences run as consecutive chunks of 32 (the skinny
 * GEMMs carry the batch in one matrix-core tile's 32 rows), each chunk
 * streaming the weights again; the workspace is that of min(batch, 32).
 * bf16 configs only. The cache-slot write is idempotent, so a step can be
 * re-run. */
int llama_model_decode(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                       const int32_t *pos, int batch, void *k_cache, void *v_cache, float *logits,
                       void *ws, size_t ws_bytes, void *stream);

/* llama_model_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Its scratch is a device array owned by
 * the library, LLAMA_DECODE_STATIC_SCRATCH_BYTES (64 MiB) on each GPU it runs
 * on, held until the process ends; the call itself allocates nothing.
 * Arguments, layouts, results and errors are those of llama_model_decode; a
 * step that needs more scratch than the array holds (llama_workspace_size
 * reports the need; 38 MiB for the LLaMA-7B shape at batch 32) returns
 * LLAMA_ERR_WORKSPACE before any launch, with the sizes in llama_last_error.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (streams not ordered against each other, or several host threads) race.
 * The step writes every scratch word before reading it, so nothing carries
 * over from an earlier call. */
#define LLAMA_DECODE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int llama_model_decode_static(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                              const int32_t *pos, int batch, void *k_cache, void *v_cache, float *logits,
                              void *stream);

/* Greedy token choice over logits [rows, vocab] f32 (device): out[r] (int32,
 * device) is the index of the largest logit of row r, the lowest index among
 * equal maxima; a row holding a NaN (as decode gives for an invalid position)
 * yields -1, which the embedding turns back into a NaN row. The logits are
 * those of the output head ([P1] "The one formula"); choosing the most
 * likely next token at each step is the plain reading of generation with
 * them. Errors: NULL pointers, rows < 0, vocab <= 0 (LLAMA_ERR_SHAPE). */
int llama_argmax(const float *logits, int64_t rows, int vocab, int32_t *out, void *stream);

/* Decode weight pack: every projection of every block (Wq|Wk|Wv, Wo,
 * W_gate/W_up interleaved in blocks of 32 rows, W_down) and the output head,
 * copied into matrix-core tile order: for each 32-row tile and each 64-wide
 * K step one 4 KB block whose 16-byte piece for lane (g, j), step q is
 * W[32 t + j][64 s + 32 g + 8 q .. +7]. The blocks are ordered for the
 * split-K chunks the decode step uses (all tiles of one K chunk together), so
 * one decode step reads every weight byte in contiguous runs; the order is
 * internal to this library. This is a load-time transform of the
 * model (the pack costs the size of the weights once more in HBM); it does
 * not change any result. Rows past a matrix's height are zero.
 * llama_decode_pack_size: bytes of the pack for config c (host, *bytes).
 * llama_pack_decode_weights: fill dst (device, dst_bytes >= that size) from
 * w on `stream`. bf16 configs only. Errors as llama_model_decode validates. */
int llama_decode_pack_size(const llama_config *c, size_t *bytes);
/* One past the last byte of the pack that the decode step's skinny GEMMs
 * read (host, *bytes), computed with the launches' own tile, split and block
 * addressing; a pack of llama_decode_pack_size bytes holds it. For checking
 * the layout without a GPU. Errors as llama_decode_pack_size. */
int llama_decode_pack_max_read(const llama_config *c, size_t *bytes);
int llama_pack_decode_weights(const llama_config *c, const llama_model_weights *w, void *dst,
                              size_t dst_bytes, void *stream);

/* Prefill weights as IEEE fp16 (for LLAMA_NUM_W_F16), a load-time transform
 * like the decode pack, not an operation of the pages: dst[i] = the bf16
 * value src[i] widened to fp32 and rounded toward zero to fp16, exactly the
 * conversion the fp16 matrix-core products apply to bf16 weights in
 * registers. Exact for magnitudes in [2^-14, 65504]; smaller ones become fp16
 * subnormals (an absolute change below 2^-24); larger ones are outside the
 * fp16 operand's range. src and dst are device buffers of n 16-bit values,
 * either the same buffer (in place) or disjoint; any alignment. Runs on
 * `stream`. Errors: n < 0 or a partial overlap (LLAMA_ERR_SHAPE), NULL
 * pointers with n > 0. n == 0 is a no-op. */
int llama_convert_weights_f16(const void *src, void *dst, int64_t n, void *stream);

/* Workspace bytes for `op` at the given batch and seq (seq ignored for decode).
 * Writes *bytes (host pointer). Errors as the matching entry point would report
 * for the config and sizes. */
int llama_workspace_size(const llama_config *c, int op, int batch, int seq, size_t *bytes);

/* Static text for a status code. */
const char *llama_status_string(int status);

/* Text of the last LLAMA_ERR_HIP on the calling thread ("" if none). */
const char *llama_last_error(void);

/* ---------------------------------------------------------------- training (fp32)
 * The backward of the pre-norm block written out by hand, with the forward's
 * linear outputs kept and the rest recomputed ([P3] "Efficient Training
 * Implementation": manual backward of the transformer layers, FlashAttention-
 * inspired attention backward, selective activation checkpointing). Gradients
 * follow the chain rule of the forward defined above; the attention backward
 * recomputes the probabilities tile by tile from q, k and the forward's
 * per-row log-sum-exp and never stores an S x S matrix. All three calls take
 * LLAMA_F32 only (bf16 configs: LLAMA_ERR_UNSUPPORTED), pre-norm blocks with
 * one K/V head per query head, head_dim 64 or 128. Results are deterministic
 * (no atomics). */

/* Gradients of llama_causal_attn (fp32 q, k, v, dout [batch*seq, n_heads*head_dim],
 * same layout as the forward) into dq, dk, dv. The forward's output and
 * log-sum-exp are recomputed into the workspace (llama_workspace_size with
 * LLAMA_OP_CAUSAL_ATTN_BACKWARD and a config of dim = n_heads*head_dim,
 * n_heads, dtype). Errors as llama_causal_attn. */
int llama_causal_attn_backward(int dtype, const void *q, const void *k, const void *v, const void *dout,
                               void *dq, void *dk, void *dv, int batch, int seq, int n_heads, int head_dim,
                               void *ws, size_t ws_bytes, void *stream);

/* Bytes of the activation buffer llama_block_train_forward fills: the rotated
 * q and k, v, the attention output, h = x + attention (each [tokens, dim]),
 * the gate and up projections ([tokens, hidden]) and the attention's
 * log-sum-exp ([batch, n_heads, seq]), fp32, 256-byte aligned pieces. */
int llama_block_train_saved_size(const llama_config *cfg, int batch, int seq, size_t *bytes);

/* y = llama_block_forward(x) (fp32), keeping the linear outputs listed above
 * in `saved` for llama_block_backward; RMSNorm outputs and SiLU(gate)*up are
 * not kept. ws: llama_workspace_size(LLAMA_OP_BLOCK_BACKWARD). */
int llama_block_train_forward(const llama_config *cfg, const llama_block_weights *w, const float *x, float *y,
                              void *saved, size_t saved_bytes, int batch, int seq, void *ws, size_t ws_bytes,
                              void *stream);

/* Backward of the block for the upstream gradient dy = dL/dy [tokens, dim]:
 * dx = dL/dx and the gradient of every weight, written through the device
 * pointers of `grads` (same shapes as the weights, fp32; the struct's pointers
 * are outputs here). x and `saved` must be those of the llama_block_train_forward
 * call. The norms and SiLU(gate)*up are recomputed from x, h, gate and up. */
int llama_block_backward(const llama_config *cfg, const llama_block_weights *w, const float *x,
                         const void *saved, size_t saved_bytes, const float *dy, float *dx,
                         const llama_block_weights *grads, int batch, int seq, void *ws, size_t ws_bytes,
                         void *stream);

/* z = a*x + b*y elementwise over n fp32 values (z may alias x or y): the loss
 * gradient y - target and the SGD update w - lr*g of a training step. */
int llama_axpby(float *z, const float *x, const float *y, float a, float b, int64_t n, void *stream);

/* Launch trace for profiling, per calling thread, off by default.
 * llama_trace_begin(events, capacity): after every kernel the library then
 * enqueues, it records events[i] (hipEvent_t handles the caller created;
 * i = 0, 1, ...) on that kernel's stream, until `capacity` are used. The
 * elapsed time between consecutive events is the duration of one kernel plus
 * its launch gap. llama_trace_end() stops tracing and returns the number of
 * events recorded. Errors: NULL events with capacity > 0, capacity < 0. */
int llama_trace_begin(void *const *events, int capacity);
int llama_trace_end(void);
/* Label of the i-th kernel of the last trace (a static string naming the step,
 * e.g. "qkv projection"; one step may launch several kernels, each labelled),
 * valid until the next llama_trace_begin on this thread; NULL when i is out
 * of range. */
const char *llama_trace_label(int i);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_MI355X_H */
