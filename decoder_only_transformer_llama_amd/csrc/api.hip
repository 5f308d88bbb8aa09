// C-ABI entry points: host-side validation, workspace carving and the launch
// sequence of each operation on the caller's stream. No allocation, no
// synchronisation, no global mutable state except the per-thread text of the
// last HIP error and the per-device address of the static decode scratch
// (looked up once per device, under a lock).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

// Scratch of llama_model_decode_static: library-owned device memory, one copy
// per GPU the library runs on, held until the process ends. In host code this
// name is only a stand-in: the memory is reached through the address that
// hipGetSymbolAddress returns on each device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

using namespace llama;

namespace {

thread_local std::string g_last_error;

// Optional launch trace (per thread): an event recorded after every kernel,
// and the launch's label (a string literal) kept until the next trace begins.
thread_local hipEvent_t const *g_trace_ev = nullptr;
thread_local int g_trace_cap = 0, g_trace_n = 0;
thread_local std::vector<const char *> g_trace_labels;

int hip_fail(hipError_t e, const char *where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return LLAMA_ERR_HIP;
}

hipError_t traced(hipError_t e, hipStream_t s, const char *where) {
  if (e == hipSuccess && g_trace_ev && g_trace_n < g_trace_cap) {
    e = hipEventRecord(g_trace_ev[g_trace_n++], s);
    g_trace_labels.push_back(where);
  }
  return e;
}

// Every kernel launch goes through HIP_TRY with the launch stream named `s`;
// `where` is a string literal naming the step.
#define HIP_TRY(expr, where)                              \
  do {                                                    \
    hipError_t e_ = traced((expr), s, where);             \
    if (e_ != hipSuccess) return hip_fail(e_, where);     \
  } while (0)

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};

int static_scratch_of_current_device(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "static scratch: device index out of range";
    return LLAMA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return LLAMA_OK;
}

bool dtype_ok(int d) { return d == LLAMA_F32 || d == LLAMA_BF16; }
size_t dsize(int d) { return d == LLAMA_F32 ? 4 : 2; }

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *b) : base((char *)b) {}
  template <class T>
  T *take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T *p = base ? (T *)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

constexpr uint32_t kNumOptionBits = (LLAMA_NUM_W_F16 << 1) - 1;   // bits 0 .. 11 of the numerics field

uint32_t numerics_of(const llama_config *c) {
  if (c->numerics & LLAMA_NUM_EXPLICIT) return c->numerics;
  return LLAMA_NUM_ATTN_F16 | LLAMA_NUM_QKV_A_F16 | LLAMA_NUM_O_A_F16 | LLAMA_NUM_FFN_A_F16 |
         (c->numerics & LLAMA_NUM_W_F16);
}

int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Compute units of the current device (queried once per process).
int cu_count() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    return cus;
  }();
  return n;
}

// Tile width (256 or 128 output columns) whose tile count fills the last
// round of workgroups best; ties go to the wider tile (less operand re-reading).
// Tile width by estimated time: rounds of workgroups over the CUs, a 256 x 128
// tile costing 0.5 / 0.72 of a 256 x 256 tile (it does half the work at
// ~0.72 of the matrix-core efficiency, measured on the 7B shapes).
constexpr double kHalfTileCost = 0.5 / 0.72;
int choose_bn(int M, int N) {
  const int cus = cu_count();
  auto rounds = [&](int bn) {
    const long tiles = (long)((M + 255) / 256) * ((N + bn - 1) / bn);
    return (double)((tiles + cus - 1) / cus);
  };
  return rounds(128) * kHalfTileCost < rounds(256) ? 128 : 256;
}

// Column ranges and tile widths of the QKV GEMM: whole rounds of 256 x 256
// tiles over the CUs, and when the remainder fills at most half a round, the
// remaining columns as 256 x 128 tiles (twice as many workgroups, each half
// the work, one round) instead of a mostly idle round of 256 x 256 tiles.
struct ColPart {
  int bn, n_base, n_end;
};
int plan_qkv(int M, int d, int kvd, ColPart parts[2]) {
  const int N = d + 2 * kvd;
  if (kvd != d) {   // grouped K/V heads: q in 256-wide tiles, k and v (multiples of 128) in 128-wide tiles
    parts[0] = {256, 0, d};
    parts[1] = {128, d, N};
    return 2;
  }
  const int cus = cu_count();
  const int tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int full_rounds = (tm * tn) / cus;
  const int rem = tm * tn - full_rounds * cus;
  if (N % 256 == 0 && full_rounds > 0 && rem > 0 && rem % tm == 0 && 2 * rem <= cus) {
    const int n1 = N - (rem / tm) * 256;
    parts[0] = {256, 0, n1};
    parts[1] = {128, n1, N};
    return 2;
  }
  parts[0] = {choose_bn(M, N), 0, N};
  return 1;
}

// Column ranges of the gate/up GEMM: whole rounds of 256 x 256 tiles over the
// CUs, and when the columns left over make a partial round whose tiles still
// fit one round as 192 x 256 tiles (three quarters of the work each), those
// columns as 192 x 256 tiles: the last round then takes about three quarters
// of a tile's time instead of a whole one. (7B shape: 688 tiles = 2 rounds
// of 512 + 176; the 22 last column tiles become 11 x 22 = 242 tiles of 192.)
struct FfnPart {
  int bm, n_base, n_end;
};
int plan_ffn(int M, int N, bool apair, FfnPart parts[2]) {
  const int cus = cu_count();
  const int tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int total = tm * tn, full = total / cus, rem = total - full * cus;
  if (!apair && N % 256 == 0 && full > 0 && rem > 0 && rem % tm == 0) {
    const int rem_cols = rem / tm;
    if ((long)((M + 191) / 192) * rem_cols <= cus) {
      const int n1 = N - rem_cols * 256;
      parts[0] = {256, 0, n1};
      parts[1] = {192, n1, N};
      return 2;
    }
  }
  parts[0] = {256, 0, N};
  return 1;
}

// Tiling of a GEMM whose epilogue adds the residual (O and down projections):
// 256 x 128 tiles, 256 x 256 tiles, or 256 x 256 tiles with K split in two
// (partial products added in order by the consumer). The cost model counts
// rounds of workgroups over the CUs in units of one full-K 256 x 256 tile;
// a 256 x 128 tile costs kHalfTileCost; a split pays for writing and reading
// its partials at ~5 TB/s against ~4 TFLOP/s per CU of matrix-core work
// (twice the passes when A is a hi/lo pair).
struct ResidCfg {
  int bn, splits;
};
ResidCfg choose_resid(int M, int N, int K, bool apair) {
  const int cus = cu_count();
  const long tm = (M + 255) / 256;
  auto rounds = [&](long tiles) { return (double)((tiles + cus - 1) / cus); };
  const double c128 = rounds(tm * ((N + 127) / 128)) * kHalfTileCost;
  const double c256 = rounds(tm * ((N + 255) / 256));
  double c256s2 = 1e30;
  if (K % 128 == 0) {   // each half a whole number of 64-deep steps
    const double traffic_us = (double)M * N * 4.0 * 2.0 * 2.0 / 5e6;
    const double round_us = 256.0 * 256.0 * K * 2.0 / 4e6 * (apair ? 2.0 : 1.0);
    c256s2 = rounds(tm * ((N + 255) / 256) * 2) * 0.5 + traffic_us / round_us;
  }
  if (c256s2 < c256 && c256s2 < c128) return {256, 2};
  return c256 <= c128 ? ResidCfg{256, 1} : ResidCfg{128, 1};
}

// ------------------------------------------------------------------ validation
int check_block_cfg(const llama_config *c, int batch, int seq) {
  if (!c) return LLAMA_ERR_NULL;
  if (!dtype_ok(c->dtype)) return LLAMA_ERR_DTYPE;
  if (c->dim <= 0 || c->n_heads <= 0 || c->hidden <= 0 || batch <= 0 || seq <= 0) return LLAMA_ERR_SHAPE;
  if (c->dim % c->n_heads) return LLAMA_ERR_SHAPE;
  const int hd = c->dim / c->n_heads;
  if (hd != 64 && hd != 128) return LLAMA_ERR_UNSUPPORTED;
  if (!(c->norm_eps >= 0.f) || !(c->rope_theta > 0.f)) return LLAMA_ERR_SHAPE;
  if ((int64_t)batch * seq > (1 << 24)) return LLAMA_ERR_SHAPE;
  if (c->dtype == LLAMA_BF16) {
    if (c->dim % 256 || c->hidden % 128) return LLAMA_ERR_UNSUPPORTED;
  }
  if (c->norm_placement < LLAMA_NORM_PRE || c->norm_placement > LLAMA_NORM_NONE) return LLAMA_ERR_UNSUPPORTED;
  // numerics: 0 or LLAMA_NUM_W_F16 (default operands), or LLAMA_NUM_EXPLICIT with known option bits
  if (c->numerics != LLAMA_NUM_DEFAULT && c->numerics != LLAMA_NUM_W_F16 &&
      (!(c->numerics & LLAMA_NUM_EXPLICIT) || (c->numerics & ~(LLAMA_NUM_EXPLICIT | kNumOptionBits))))
    return LLAMA_ERR_UNSUPPORTED;
  // fp16 attention operands are single values: no q/k or v pairs with them
  const uint32_t num = numerics_of(c);
  if ((num & LLAMA_NUM_ATTN_F16) && (num & (LLAMA_NUM_QK_PAIR | LLAMA_NUM_V_PAIR))) return LLAMA_ERR_UNSUPPORTED;
  // fp16 projection operands are single values too
  if (((num & LLAMA_NUM_QKV_A_F16) && (num & LLAMA_NUM_QKV_A_PAIR)) ||
      ((num & LLAMA_NUM_O_A_F16) && (num & LLAMA_NUM_O_A_PAIR)) ||
      ((num & LLAMA_NUM_FFN_A_F16) && (num & LLAMA_NUM_FFN_A_PAIR)) ||
      ((num & LLAMA_NUM_DOWN_A_F16) && (num & LLAMA_NUM_DOWN_A_PAIR)))
    return LLAMA_ERR_UNSUPPORTED;
  // grouped K/V heads: a divisor of n_heads, groups of 1, 2, 4 or 8, K/V
  // width a multiple of the 128-column GEMM tile; bf16 path only
  const int nkv = c->n_kv_heads > 0 ? c->n_kv_heads : c->n_heads;
  if (c->n_kv_heads < 0 || nkv > c->n_heads || c->n_heads % nkv) return LLAMA_ERR_SHAPE;
  const int group = c->n_heads / nkv;
  if (group > 1) {
    if (c->dtype != LLAMA_BF16) return LLAMA_ERR_UNSUPPORTED;
    if ((group & (group - 1)) || group > 8 || (nkv * hd) % 128) return LLAMA_ERR_UNSUPPORTED;
  }
  return LLAMA_OK;
}

int kv_heads(const llama_config *c) { return c->n_kv_heads > 0 ? c->n_kv_heads : c->n_heads; }
int kv_dim(const llama_config *c) { return kv_heads(c) * (c->dim / c->n_heads); }

int check_block_w(const llama_block_weights *w) {
  if (!w) return LLAMA_ERR_NULL;
  if (!w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->ffn_norm || !w->w_gate || !w->w_up ||
      !w->w_down)
    return LLAMA_ERR_NULL;
  return LLAMA_OK;
}

int check_model_cfg(const llama_config *c, int batch, int seq) {
  int st = check_block_cfg(c, batch, seq);
  if (st) return st;
  if (c->n_layers <= 0 || c->vocab <= 0 || c->max_seq <= 0) return LLAMA_ERR_SHAPE;
  if (c->dtype != LLAMA_BF16 || c->norm_placement != LLAMA_NORM_PRE) return LLAMA_ERR_UNSUPPORTED;
  return LLAMA_OK;
}

int check_model_w(const llama_config *c, const llama_model_weights *w) {
  if (!w || !w->tok_embeddings || !w->layers || !w->final_norm || !w->output) return LLAMA_ERR_NULL;
  for (int l = 0; l < c->n_layers; ++l) {
    const int st = check_block_w(&w->layers[l]);
    if (st) return st;
  }
  return LLAMA_OK;
}

// ------------------------------------------------------------------ workspace layouts
struct BlockWs {
  float2 *rope_tab;
  uint16_t *xg_hi, *xg_lo, *qh, *ql, *kh, *kl, *vth, *vtl, *a_hi, *a_lo, *u_hi, *u_lo;
  float *h, *rstd1, *rstd2;
  float *part;   // split-K partials [2][n][d] fp32: aliases qh..kl (dead after attention)
  int *tile_flags;   // one per 256 x 128 output tile of an [n, d] product (fused split-K residual)
  // fp32 path
  float *z, *q, *k, *v, *att, *gate, *up;
};

int vt_stride_of(int seq) { return round_up(seq, 64); }
// flags for the output tiles of an [n, d] product (256-row tiles, at least 128 wide)
int tile_flag_count(int64_t n, int d) { return (int)(((n + 255) / 256) * ((d + 127) / 128)); }

// kv_rows: key rows held per sequence (seq, or max_seq for a prefill that may
// continue a cached prefix); the rope table covers as many positions.
BlockWs carve_block(Carve &cv, const llama_config *c, int batch, int seq, int kv_rows = 0) {
  BlockWs b{};
  const int64_t n = (int64_t)batch * seq;
  const int d = c->dim, hd = d / c->n_heads;
  kv_rows = std::max(kv_rows, seq);
  const int64_t nk = (int64_t)batch * kv_rows;
  if (c->dtype == LLAMA_BF16) {
    b.rope_tab = cv.take<float2>((size_t)kv_rows * hd / 2);
    b.rstd1 = cv.take<float>(n);
    b.rstd2 = cv.take<float>(n);
    b.xg_hi = cv.take<uint16_t>(n * d);
    b.xg_lo = cv.take<uint16_t>(n * d);
    b.qh = cv.take<uint16_t>(n * d);
    b.ql = cv.take<uint16_t>(n * d);
    b.kh = cv.take<uint16_t>(nk * d);
    b.kl = cv.take<uint16_t>(nk * d);
    b.part = (float *)b.qh;   // qh, ql, kh, kl are contiguous: at least 8 n d bytes = 2 n d floats
    const size_t vt = (size_t)batch * kv_dim(c) * vt_stride_of(kv_rows);
    b.vth = cv.take<uint16_t>(vt);
    b.vtl = cv.take<uint16_t>(vt);
    b.a_hi = cv.take<uint16_t>(n * d);
    b.a_lo = cv.take<uint16_t>(n * d);
    b.h = cv.take<float>(n * d);
    b.u_hi = cv.take<uint16_t>(n * c->hidden);
    b.u_lo = cv.take<uint16_t>(n * c->hidden);
    b.tile_flags = cv.take<int>(tile_flag_count(n, d));
  } else {
    b.z = cv.take<float>(n * d);
    b.q = cv.take<float>(n * d);
    b.k = cv.take<float>(n * d);
    b.v = cv.take<float>(n * d);
    b.att = cv.take<float>(n * d);
    b.h = cv.take<float>(n * d);
    b.gate = cv.take<float>(n * c->hidden);
    b.up = cv.take<float>(n * c->hidden);
  }
  return b;
}

struct DecodeWs {
  float *x, *h, *rstd, *part;
  uint16_t *ag_hi, *ag_lo;
  float2 *rope_tab;
  float *attn_part;   // key-range softmax states of the decode attention
};

constexpr int kDecMaxSeq = kDecMaxCache;   // longest cache of the decode path
// The skinny GEMMs carry the batch in the 32 rows of one matrix-core tile: a
// step over more sequences runs in chunks of 32 (each chunk streams the
// weights again).
constexpr int kDecChunk = 32;

void gemv_split(int N, int K, int &splits, int &k_chunk) {
  const GemvShape g = gemv_shape(N, K);
  splits = g.splits;
  k_chunk = g.k_chunk;
}

size_t dec_part_floats(const llama_config *c, int batch) {
  const int d = c->dim, h = c->hidden;
  const int NK[5][2] = {{d + 2 * kv_dim(c), d}, {d, d}, {2 * h, d}, {d, h}, {c->vocab, d}};
  size_t mx = 0;
  for (int i = 0; i < 5; ++i) {
    int sp, kc;
    gemv_split(NK[i][0], NK[i][1], sp, kc);
    mx = std::max(mx, (size_t)sp * batch * NK[i][0]);
  }
  return mx;
}

DecodeWs carve_decode(Carve &cv, const llama_config *c, int batch) {
  DecodeWs w{};
  const int d = c->dim, hd = d / c->n_heads;
  w.x = cv.take<float>((size_t)batch * d);
  w.h = cv.take<float>((size_t)batch * d);
  w.rstd = cv.take<float>((size_t)batch * ((c->dim + 1023) / 1024));
  w.part = cv.take<float>(dec_part_floats(c, batch));
  const int wmax = std::max(d, c->hidden);
  w.ag_hi = cv.take<uint16_t>((size_t)batch * wmax);
  w.ag_lo = cv.take<uint16_t>((size_t)batch * wmax);
  w.rope_tab = cv.take<float2>((size_t)batch * hd / 2);
  w.attn_part = cv.take<float>((size_t)batch * c->n_heads * kDecAttnMaxRanges * dec_attn_range_factor(c->max_seq) *
                                (hd + 2));
  return w;
}

// ------------------------------------------------------------------ training layouts
// Activations kept by the training forward (fp32): the linear outputs and h.
struct TrainSaved {
  float *q, *k, *v, *a, *h, *gate, *up, *lse;
};
TrainSaved carve_saved(Carve &cv, const llama_config *c, int batch, int seq) {
  const size_t n = (size_t)batch * seq, d = c->dim, hid = c->hidden;
  TrainSaved t{};
  t.q = cv.take<float>(n * d);
  t.k = cv.take<float>(n * d);
  t.v = cv.take<float>(n * d);
  t.a = cv.take<float>(n * d);
  t.h = cv.take<float>(n * d);
  t.gate = cv.take<float>(n * hid);
  t.up = cv.take<float>(n * hid);
  t.lse = cv.take<float>((size_t)batch * c->n_heads * seq);
  return t;
}

// Backward workspace: recomputed norms and SiLU(gate)*up, gradient buffers.
struct BwdWs {
  float *z1, *z2, *u, *du, *dup, *dz, *dh, *da, *dq, *dk, *dv, *delta, *rstd, *kv_part;
};
BwdWs carve_backward(Carve &cv, const llama_config *c, int batch, int seq) {
  const size_t n = (size_t)batch * seq, d = c->dim, hid = c->hidden;
  BwdWs w{};
  w.z1 = cv.take<float>(n * d);
  w.z2 = cv.take<float>(n * d);
  w.u = cv.take<float>(n * hid);
  w.du = cv.take<float>(n * hid);
  w.dup = cv.take<float>(n * hid);
  w.dz = cv.take<float>(n * d);
  w.dh = cv.take<float>(n * d);
  w.da = cv.take<float>(n * d);
  w.dq = cv.take<float>(n * d);
  w.dk = cv.take<float>(n * d);
  w.dv = cv.take<float>(n * d);
  w.delta = cv.take<float>((size_t)batch * c->n_heads * seq);
  w.rstd = cv.take<float>(n);
  w.kv_part = cv.take<float>((size_t)kAttnBwdKvRanges * 2 * n * d);
  return w;
}

// fp32 pre-norm blocks with one K/V head per query head.
int check_train_cfg(const llama_config *c, int batch, int seq) {
  const int st = check_block_cfg(c, batch, seq);
  if (st) return st;
  if (c->dtype != LLAMA_F32 || c->norm_placement != LLAMA_NORM_PRE || kv_heads(c) != c->n_heads)
    return LLAMA_ERR_UNSUPPORTED;
  return LLAMA_OK;
}

size_t ws_bytes_of(const llama_config *c, int op, int batch, int seq) {
  Carve cv(nullptr);
  const int64_t n = (int64_t)batch * seq;
  switch (op) {
    case LLAMA_OP_CAUSAL_ATTN: {
      const int d = c->dim;
      if (c->dtype == LLAMA_BF16) {
        for (int i = 0; i < 4; ++i) cv.take<uint16_t>(n * d);
        const size_t vt = (size_t)batch * d * vt_stride_of(seq);
        cv.take<uint16_t>(vt);
        cv.take<uint16_t>(vt);
      } else {
        cv.take<float>(n * d);
      }
      break;
    }
    case LLAMA_OP_SWIGLU_FFN:
      if (c->dtype == LLAMA_BF16) {
        cv.take<uint16_t>(n * c->hidden);
        cv.take<uint16_t>(n * c->hidden);
      } else {
        cv.take<float>(n * c->hidden);
        cv.take<float>(n * c->hidden);
      }
      break;
    case LLAMA_OP_BLOCK_FORWARD:
      carve_block(cv, c, batch, seq);
      break;
    case LLAMA_OP_MODEL_FORWARD:
      cv.take<float>(n * c->dim);
      cv.take<float>(n * c->dim);
      carve_block(cv, c, batch, seq, c->max_seq);
      break;
    case LLAMA_OP_MODEL_DECODE:
      carve_decode(cv, c, std::min(batch, kDecChunk));   // chunks of kDecChunk sequences reuse it
      break;
    case LLAMA_OP_CAUSAL_ATTN_BACKWARD:
      cv.take<float>(n * c->dim);                                 // recomputed output
      cv.take<float>((size_t)batch * c->n_heads * seq);           // log-sum-exp
      cv.take<float>((size_t)batch * c->n_heads * seq);           // rowsum(dout * out)
      cv.take<float>((size_t)kAttnBwdKvRanges * 2 * n * c->dim);  // split key/value-gradient sums
      break;
    case LLAMA_OP_BLOCK_BACKWARD:
      carve_backward(cv, c, batch, seq);
      break;
    default:
      return 0;
  }
  return cv.off + 256;
}

// ------------------------------------------------------------------ decode weight pack
// Per layer: Wq|Wk|Wv (3d rows, K = d), Wo (d, d), W_gate/W_up interleaved by
// 32 rows (2h, d), W_down (d, h); then the output head (vocab, d). Each matrix
// holds ceil(rows/32)*32 rows in tile order.
size_t tile_elems(int rows, int K) { return (size_t)((rows + 31) / 32) * 32 * K; }

struct PackLayout {
  size_t qkv, o, gu, down, layer, head_off, total;   // element offsets / sizes (u16)
};

PackLayout pack_layout(const llama_config *c) {
  PackLayout p{};
  const int d = c->dim, h = c->hidden;
  p.qkv = 0;
  p.o = tile_elems(d + 2 * kv_dim(c), d);
  p.gu = p.o + tile_elems(d, d);
  p.down = p.gu + tile_elems(2 * h, d);
  p.layer = p.down + tile_elems(d, h);
  p.head_off = p.layer * c->n_layers;
  p.total = p.head_off + tile_elems(c->vocab, d);
  return p;
}

// ------------------------------------------------------------------ block launch sequences
// make_rope: build the (cos, sin) table in b.rope_tab first (a stack of blocks
// over the same positions builds it once).
// start_pos (device [batch], or nullptr): the sequences continue a cached
// prefix (model prefill); k and v^T then hold kv_rows positions per sequence.
int block_bf16(const llama_config *c, const llama_block_weights *w, int x_dtype, const void *x, float *y,
               int batch, int seq, const BlockWs &b, uint16_t *kcache, uint16_t *vcache, int max_seq,
               hipStream_t s, bool make_rope = true, const int32_t *start_pos = nullptr, int kv_rows = 0) {
  const int d = c->dim, H = c->n_heads, hd = d / H, M = batch * seq;
  const uint32_t num = numerics_of(c);
  const bool qkv_pair = num & LLAMA_NUM_QKV_A_PAIR, ffn_pair = num & LLAMA_NUM_FFN_A_PAIR;
  const bool opair = num & LLAMA_NUM_O_A_PAIR, dpair = num & LLAMA_NUM_DOWN_A_PAIR;
  const bool af16 = num & LLAMA_NUM_ATTN_F16;
  // fp16 activation operands, per projection
  const int qf16 = (num & LLAMA_NUM_QKV_A_F16) ? 1 : 0, of16 = (num & LLAMA_NUM_O_A_F16) ? 1 : 0;
  const int ff16 = (num & LLAMA_NUM_FFN_A_F16) ? 1 : 0, df16 = (num & LLAMA_NUM_DOWN_A_F16) ? 1 : 0;
  // GEMM mode of an fp16 operand: weights converted in registers (1) or supplied as fp16 (2)
  const int wf = (num & LLAMA_NUM_W_F16) ? 2 : 1;
  if (!start_pos) kv_rows = seq;
  const int vts = vt_stride_of(kv_rows);
  // Pre-norm (LLaMA) folds RMSNorm into the next projection; post-norm and
  // no-norm feed the branches the trunk itself (operand x; the row multiplier
  // then only undoes the fp16 operand's power-of-two scale).
  const bool pre = c->norm_placement == LLAMA_NORM_PRE, post = c->norm_placement == LLAMA_NORM_POST;

  // z = RMSNorm(x; g1): statistic + gained operand; the rstd multiply happens
  // in the QKV epilogue. The same launch builds the RoPE table when asked.
  RopeRows rope;
  if (make_rope) rope = RopeRows{b.rope_tab, seq, hd, (double)c->rope_theta};
  HIP_TRY(norm_prep_launch(x_dtype == LLAMA_F32, x, pre ? (const uint16_t *)w->attn_norm : nullptr, M, d,
                           c->norm_eps, b.rstd1, b.xg_hi, qkv_pair ? b.xg_lo : nullptr, s, nullptr, 0, nullptr,
                           qf16, rope),
          "attention norm");

  GemmArgs q{};
  q.M = M;
  const int kvd = kv_dim(c), nkv = kv_heads(c);
  q.N = d + 2 * kvd;
  q.K = d;
  q.A = b.xg_hi;
  q.A_lo = qkv_pair ? b.xg_lo : nullptr;
  q.lda = d;
  q.rstd = b.rstd1;
  q.b_mode = BMODE_CONCAT3;
  q.B0 = (const uint16_t *)w->wq;
  q.B1 = (const uint16_t *)w->wk;
  q.B2 = (const uint16_t *)w->wv;
  q.n_seg = d;
  q.qh = b.qh;
  q.ql = b.ql;
  q.kh = b.kh;
  q.kl = b.kl;
  q.vth = b.vth;
  q.vtl = b.vtl;
  q.rope_tab = b.rope_tab;
  q.attn_f16 = af16;
  // fp16 attention operands: q leaves the epilogue already scaled by the
  // attention's log2(e)/sqrt(hd), one fp16 rounding of the scaled value
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  q.q_mul = af16 ? scale_log2 : 0.f;
  q.seq = seq;
  q.n_heads = H;
  q.head_dim = hd;
  q.dim = d;
  q.n_seg_kv = kvd;
  q.kv_dim = kvd;
  q.n_kv_heads = nkv;
  q.vt_stride = vts;
  q.kcache = kcache;
  q.vcache = vcache;
  q.max_seq = max_seq;
  q.start_pos = start_pos;
  q.kv_rows = kv_rows;
  ColPart qp[2];
  const int nqp = plan_qkv(M, d, kvd, qp);
  for (int i = 0; i < nqp; ++i) {
    q.n_base = qp[i].n_base;
    q.n_end = qp[i].n_end;
    HIP_TRY(gemm_launch(GemmKey{qp[i].bn, qkv_pair, EPI_QKV, qf16 * wf}, q, s), "qkv projection");
  }
  // earlier positions of every sequence come from the cache
  if (start_pos)
    HIP_TRY(kv_prefix_launch(kcache, vcache, start_pos, batch, nkv, hd, max_seq, seq, b.kh,
                             (num & LLAMA_NUM_QK_PAIR) ? b.kl : nullptr, b.vth, (num & LLAMA_NUM_V_PAIR) ? b.vtl : nullptr,
                             kv_rows, vts, af16, s),
            "cached prefix");

  AttnArgs at{};
  at.qh = b.qh;
  at.ql = b.ql;
  at.kh = b.kh;
  at.kl = b.kl;
  at.vth = b.vth;
  at.vtl = b.vtl;
  at.o = b.a_hi;
  at.o_lo = opair ? b.a_lo : nullptr;
  at.o_f32 = 0;
  at.o_f16 = of16;
  at.batch = batch;
  at.seq = seq;
  at.n_heads = H;
  at.head_dim = hd;
  at.dim = d;
  at.kv_dim = kvd;
  at.n_kv_heads = nkv;
  at.vt_stride = vts;
  at.scale_log2 = scale_log2;
  at.q_scaled = af16;
  at.start_pos = start_pos;
  at.kv_rows = kv_rows;
  at.max_seq = max_seq;
  HIP_TRY(attn_prefill_launch(at, (num & LLAMA_NUM_QK_PAIR) ? 1 : 0, (num & LLAMA_NUM_V_PAIR) ? 1 : 0, af16, s),
          "attention");

  // h = x + attn Wo^T. With a split K the two partial products go to the
  // q/k buffers (dead after attention) and the ffn norm prep forms h.
  ResidCfg oc = choose_resid(M, d, d, opair);
  if (post) oc.splits = 1;   // the trunk norm below reads x + attn Wo^T whole
  GemmArgs o{};
  o.M = M;
  o.N = d;
  o.K = d;
  o.A = b.a_hi;
  o.A_lo = opair ? b.a_lo : nullptr;
  o.lda = d;
  o.b_mode = BMODE_PLAIN;
  o.B0 = (const uint16_t *)w->wo;
  o.C = b.h;
  o.ldc = d;
  o.R = x;
  o.r_f32 = x_dtype == LLAMA_F32;
  o.k_splits = oc.splits;
  o.part = b.part;
  HIP_TRY(gemm_launch(GemmKey{oc.bn, opair, oc.splits > 1 ? EPI_PARTIAL : EPI_RESID, of16 * wf}, o, s),
          "output projection");

  // post-norm: h = RMSNorm(x + attn Wo^T; g1) in place, fp32
  if (post) HIP_TRY(rmsnorm_launch(1, 1, b.h, w->attn_norm, b.h, M, d, c->norm_eps, s, 0), "attention norm");
  // the down projection's tiling, and whether its two K ranges add the
  // residual themselves (the ffn norm prep then clears their tile flags)
  const ResidCfg dc = choose_resid(M, d, c->hidden, dpair);
  GemmArgs dn{};
  dn.M = M;
  dn.N = d;
  dn.K = c->hidden;
  dn.A = b.u_hi;
  dn.A_lo = dpair ? b.u_lo : nullptr;
  dn.lda = c->hidden;
  dn.b_mode = BMODE_PLAIN;
  dn.B0 = (const uint16_t *)w->w_down;
  dn.C = y;
  dn.ldc = d;
  dn.R = b.h;
  dn.r_f32 = 1;
  dn.k_splits = dc.splits;
  dn.part = b.part;
  const bool fuse_down = dc.splits == 2 && gemm_fused_split_ok(dn);
  if (fuse_down) dn.tile_flags = b.tile_flags;
  const int n_flags = fuse_down ? tile_flag_count(M, d) : 0;
  // z2 = RMSNorm(h; g2), operand reuses the x*g1 buffers
  const uint16_t *g2 = pre ? (const uint16_t *)w->ffn_norm : nullptr;
  if (oc.splits > 1)
    HIP_TRY(norm_prep_launch(x_dtype == LLAMA_F32, x, g2, M, d, c->norm_eps, b.rstd2, b.xg_hi,
                             ffn_pair ? b.xg_lo : nullptr, s, b.part, oc.splits, b.h, ff16, RopeRows{},
                             b.tile_flags, n_flags),
            "ffn norm");
  else
    HIP_TRY(norm_prep_launch(1, b.h, g2, M, d, c->norm_eps, b.rstd2, b.xg_hi, ffn_pair ? b.xg_lo : nullptr, s,
                             nullptr, 0, nullptr, ff16, RopeRows{}, b.tile_flags, n_flags),
            "ffn norm");
  GemmArgs f{};
  f.M = M;
  f.N = 2 * c->hidden;
  f.K = d;
  f.A = b.xg_hi;
  f.A_lo = ffn_pair ? b.xg_lo : nullptr;
  f.lda = d;
  f.rstd = b.rstd2;
  f.b_mode = BMODE_GATEUP;
  f.B0 = (const uint16_t *)w->w_gate;
  f.B1 = (const uint16_t *)w->w_up;
  f.C = b.u_hi;
  f.C_lo = dpair ? b.u_lo : nullptr;
  f.c_f16 = df16;   // u in the format the down projection takes
  f.ldc = c->hidden;
  FfnPart fp[2];
  const int nfp = plan_ffn(M, f.N, ffn_pair, fp);
  for (int i = 0; i < nfp; ++i) {
    f.n_base = fp[i].n_base;
    f.n_end = fp[i].n_end;
    GemmKey fk{256, ffn_pair, EPI_SILU, ff16 * wf};
    fk.bm = fp[i].bm;
    HIP_TRY(gemm_launch(fk, f, s), "gate/up projection");
  }

  HIP_TRY(gemm_launch(GemmKey{dc.bn, dpair, dc.splits > 1 ? EPI_PARTIAL : EPI_RESID, df16 * wf}, dn, s),
          "down projection");
  if (dc.splits > 1 && !fuse_down)
    HIP_TRY(resid_sum_launch(b.h, b.part, dc.splits, (int64_t)M * d, y, s), "down residual");
  if (post) HIP_TRY(rmsnorm_launch(1, 1, y, w->ffn_norm, y, M, d, c->norm_eps, s, 0), "ffn norm");
  return LLAMA_OK;
}

int block_f32(const llama_config *c, const llama_block_weights *w, const float *x, float *y, int batch,
              int seq, const BlockWs &b, hipStream_t s) {
  const int d = c->dim, H = c->n_heads, hd = d / H, M = batch * seq, hid = c->hidden;
  const int np = c->norm_placement;
  // attention branch input: RMSNorm(x; g1) before it (pre-norm) or x itself
  const float *za = x;
  if (np == LLAMA_NORM_PRE) {
    HIP_TRY(rmsnorm_launch(1, 1, x, w->attn_norm, b.z, M, d, c->norm_eps, s), "rmsnorm");
    za = b.z;
  }
  HIP_TRY(gemm_f32_launch(za, (const float *)w->wq, b.q, nullptr, M, d, d, s), "q projection");
  HIP_TRY(gemm_f32_launch(za, (const float *)w->wk, b.k, nullptr, M, d, d, s), "k projection");
  HIP_TRY(gemm_f32_launch(za, (const float *)w->wv, b.v, nullptr, M, d, d, s), "v projection");
  HIP_TRY(rope_launch(1, b.q, b.q, nullptr, M, H, hd, c->rope_theta, seq, s), "rope q");
  HIP_TRY(rope_launch(1, b.k, b.k, nullptr, M, H, hd, c->rope_theta, seq, s), "rope k");
  HIP_TRY(attn_f32_launch(b.q, b.k, b.v, b.att, batch, seq, H, hd, s), "attention");
  HIP_TRY(gemm_f32_launch(b.att, (const float *)w->wo, b.h, x, M, d, d, s), "output projection");
  // post-norm: the trunk itself is normalised, h = RMSNorm(x + attn; g1)
  if (np == LLAMA_NORM_POST) HIP_TRY(rmsnorm_launch(1, 1, b.h, w->attn_norm, b.h, M, d, c->norm_eps, s), "rmsnorm");
  const float *zf = b.h;
  if (np == LLAMA_NORM_PRE) {
    HIP_TRY(rmsnorm_launch(1, 1, b.h, w->ffn_norm, b.z, M, d, c->norm_eps, s), "rmsnorm");
    zf = b.z;
  }
  HIP_TRY(gemm_f32_launch(zf, (const float *)w->w_gate, b.gate, nullptr, M, hid, d, s), "gate");
  HIP_TRY(gemm_f32_launch(zf, (const float *)w->w_up, b.up, nullptr, M, hid, d, s), "up");
  HIP_TRY(silu_mul_f32_launch(b.gate, b.up, b.gate, (int64_t)M * hid, s), "silu");
  HIP_TRY(gemm_f32_launch(b.gate, (const float *)w->w_down, y, b.h, M, d, hid, s), "down projection");
  if (np == LLAMA_NORM_POST) HIP_TRY(rmsnorm_launch(1, 1, y, w->ffn_norm, y, M, d, c->norm_eps, s), "rmsnorm");
  return LLAMA_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

int llama_hidden_dim(int dim, int multiple_of) {
  if (dim <= 0 || multiple_of <= 0) return -1;
  const long long hidden = (2LL * 4 * dim) / 3;
  return (int)(multiple_of * ((hidden + multiple_of - 1) / multiple_of));
}

const char *llama_status_string(int st) {
  switch (st) {
    case LLAMA_OK: return "ok";
    case LLAMA_ERR_NULL: return "null pointer argument";
    case LLAMA_ERR_SHAPE: return "invalid or inconsistent size";
    case LLAMA_ERR_DTYPE: return "unsupported dtype";
    case LLAMA_ERR_WORKSPACE: return "workspace missing or too small";
    case LLAMA_ERR_POSITION: return "position or sequence length exceeds max_seq";
    case LLAMA_ERR_UNSUPPORTED: return "shape or mode not implemented by this build";
    case LLAMA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *llama_last_error(void) { return g_last_error.c_str(); }

int llama_causal_attn_backward(int dtype, const void *q, const void *k, const void *v, const void *dout,
                               void *dq, void *dk, void *dv, int batch, int seq, int n_heads, int head_dim,
                               void *ws, size_t ws_bytes, void *stream) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return LLAMA_ERR_NULL;
  if (!dtype_ok(dtype)) return LLAMA_ERR_DTYPE;
  if (batch <= 0 || seq <= 0 || n_heads <= 0 || head_dim <= 0) return LLAMA_ERR_SHAPE;
  if (dtype != LLAMA_F32 || (head_dim != 64 && head_dim != 128)) return LLAMA_ERR_UNSUPPORTED;
  if ((int64_t)batch * seq > (1 << 24)) return LLAMA_ERR_SHAPE;
  llama_config c{};
  c.dim = n_heads * head_dim;
  c.n_heads = n_heads;
  c.dtype = dtype;
  if (!ws || ws_bytes < ws_bytes_of(&c, LLAMA_OP_CAUSAL_ATTN_BACKWARD, batch, seq)) return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Carve cv(ws);
  const int64_t n = (int64_t)batch * seq;
  float *o = cv.take<float>(n * c.dim);
  float *lse = cv.take<float>((size_t)batch * n_heads * seq);
  float *delta = cv.take<float>((size_t)batch * n_heads * seq);
  float *kv_part = cv.take<float>((size_t)kAttnBwdKvRanges * 2 * n * c.dim);
  const float *qf = (const float *)q, *kf = (const float *)k, *vf = (const float *)v;
  HIP_TRY(attn_f32_launch(qf, kf, vf, o, batch, seq, n_heads, head_dim, s, lse), "attention (recomputed)");
  HIP_TRY(attn_bwd_launch(qf, kf, vf, o, (const float *)dout, lse, delta, (float *)dq, (float *)dk, (float *)dv,
                          batch, seq, n_heads, head_dim, s, kv_part),
          "attention backward");
  return LLAMA_OK;
}

int llama_block_train_saved_size(const llama_config *c, int batch, int seq, size_t *bytes) {
  if (!c || !bytes) return LLAMA_ERR_NULL;
  const int st = check_train_cfg(c, batch, seq);
  if (st) return st;
  Carve cv(nullptr);
  carve_saved(cv, c, batch, seq);
  *bytes = cv.off + 256;
  return LLAMA_OK;
}

int llama_block_train_forward(const llama_config *c, const llama_block_weights *w, const float *x, float *y,
                              void *saved, size_t saved_bytes, int batch, int seq, void *ws, size_t ws_bytes,
                              void *stream) {
  int st = check_train_cfg(c, batch, seq);
  if (st) return st;
  if ((st = check_block_w(w))) return st;
  if (!x || !y || !saved) return LLAMA_ERR_NULL;
  size_t need_saved = 0;
  llama_block_train_saved_size(c, batch, seq, &need_saved);
  if (saved_bytes < need_saved || !ws || ws_bytes < ws_bytes_of(c, LLAMA_OP_BLOCK_BACKWARD, batch, seq))
    return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int d = c->dim, H = c->n_heads, hd = d / H, M = batch * seq, hid = c->hidden;
  Carve cs(saved), cw(ws);
  const TrainSaved t = carve_saved(cs, c, batch, seq);
  const BwdWs b = carve_backward(cw, c, batch, seq);
  HIP_TRY(rmsnorm_launch(1, 1, x, w->attn_norm, b.z1, M, d, c->norm_eps, s), "rmsnorm");
  HIP_TRY(gemm_f32_launch(b.z1, (const float *)w->wq, t.q, nullptr, M, d, d, s), "q projection");
  HIP_TRY(gemm_f32_launch(b.z1, (const float *)w->wk, t.k, nullptr, M, d, d, s), "k projection");
  HIP_TRY(gemm_f32_launch(b.z1, (const float *)w->wv, t.v, nullptr, M, d, d, s), "v projection");
  HIP_TRY(rope_launch(1, t.q, t.q, nullptr, M, H, hd, c->rope_theta, seq, s), "rope q");
  HIP_TRY(rope_launch(1, t.k, t.k, nullptr, M, H, hd, c->rope_theta, seq, s), "rope k");
  HIP_TRY(attn_f32_launch(t.q, t.k, t.v, t.a, batch, seq, H, hd, s, t.lse), "attention");
  HIP_TRY(gemm_f32_launch(t.a, (const float *)w->wo, t.h, x, M, d, d, s), "output projection");
  HIP_TRY(rmsnorm_launch(1, 1, t.h, w->ffn_norm, b.z2, M, d, c->norm_eps, s), "rmsnorm");
  HIP_TRY(gemm_f32_launch(b.z2, (const float *)w->w_gate, t.gate, nullptr, M, hid, d, s), "gate");
  HIP_TRY(gemm_f32_launch(b.z2, (const float *)w->w_up, t.up, nullptr, M, hid, d, s), "up");
  HIP_TRY(silu_mul_f32_launch(t.gate, t.up, b.u, (int64_t)M * hid, s), "silu");
  HIP_TRY(gemm_f32_launch(b.u, (const float *)w->w_down, y, t.h, M, d, hid, s), "down projection");
  return LLAMA_OK;
}

int llama_block_backward(const llama_config *c, const llama_block_weights *w, const float *x, const void *saved,
                         size_t saved_bytes, const float *dy, float *dx, const llama_block_weights *grads,
                         int batch, int seq, void *ws, size_t ws_bytes, void *stream) {
  int st = check_train_cfg(c, batch, seq);
  if (st) return st;
  if ((st = check_block_w(w)) || (st = check_block_w(grads))) return st;
  if (!x || !saved || !dy || !dx) return LLAMA_ERR_NULL;
  size_t need_saved = 0;
  llama_block_train_saved_size(c, batch, seq, &need_saved);
  if (saved_bytes < need_saved || !ws || ws_bytes < ws_bytes_of(c, LLAMA_OP_BLOCK_BACKWARD, batch, seq))
    return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int d = c->dim, H = c->n_heads, hd = d / H, M = batch * seq, hid = c->hidden;
  Carve cs((void *)saved), cw(ws);
  const TrainSaved t = carve_saved(cs, c, batch, seq);
  const BwdWs b = carve_backward(cw, c, batch, seq);
  auto W = [](const void *p) { return (const float *)p; };
  auto G = [](const void *p) { return (float *)p; };
  // C = A B with A [m, k] and B [k, n] row-major
  auto nn = [&](const float *A, const float *B, float *C, int m, int n, int k, int acc) {
    return gemm_f32_strided_launch(A, k, 1, B, n, 1, C, m, n, k, acc, s);
  };
  // C [n_out, k_in] = X^T Y with X [tokens, n_out], Y [tokens, k_in] row-major (a weight gradient)
  auto tn = [&](const float *X, const float *Y, float *C, int n_out, int k_in) {
    return gemm_f32_strided_launch(X, 1, n_out, Y, k_in, 1, C, n_out, k_in, M, 0, s);
  };
  // recomputed: the two norm outputs and SiLU(gate) * up
  HIP_TRY(rmsnorm_launch(1, 1, x, w->attn_norm, b.z1, M, d, c->norm_eps, s), "rmsnorm");
  HIP_TRY(rmsnorm_launch(1, 1, t.h, w->ffn_norm, b.z2, M, d, c->norm_eps, s), "rmsnorm");
  HIP_TRY(silu_mul_f32_launch(t.gate, t.up, b.u, (int64_t)M * hid, s), "silu");
  // y = h + u Wd^T
  HIP_TRY(tn(dy, b.u, G(grads->w_down), d, hid), "down weight gradient");
  HIP_TRY(nn(dy, W(w->w_down), b.du, M, hid, d, 0), "down input gradient");
  HIP_TRY(swiglu_bwd_launch(t.gate, t.up, b.du, b.du, b.dup, (int64_t)M * hid, s), "silu backward");
  HIP_TRY(tn(b.du, b.z2, G(grads->w_gate), hid, d), "gate weight gradient");
  HIP_TRY(tn(b.dup, b.z2, G(grads->w_up), hid, d), "up weight gradient");
  HIP_TRY(nn(b.du, W(w->w_gate), b.dz, M, d, hid, 0), "gate input gradient");
  HIP_TRY(nn(b.dup, W(w->w_up), b.dz, M, d, hid, 1), "up input gradient");
  // z2 = RMSNorm(h; g2); dh = dy + its gradient
  HIP_TRY(rmsnorm_bwd_launch(t.h, W(w->ffn_norm), b.dz, dy, b.dh, G(grads->ffn_norm), b.rstd, M, d, c->norm_eps, s),
          "ffn norm backward");
  // h = x + a Wo^T
  HIP_TRY(tn(b.dh, t.a, G(grads->wo), d, d), "output weight gradient");
  HIP_TRY(nn(b.dh, W(w->wo), b.da, M, d, d, 0), "output input gradient");
  HIP_TRY(attn_bwd_launch(t.q, t.k, t.v, t.a, b.da, t.lse, b.delta, b.dq, b.dk, b.dv, batch, seq, H, hd, s,
                          b.kv_part),
          "attention backward");
  HIP_TRY(rope_launch(1, b.dq, b.dq, nullptr, M, H, hd, c->rope_theta, seq, s, 1), "rope backward");
  HIP_TRY(rope_launch(1, b.dk, b.dk, nullptr, M, H, hd, c->rope_theta, seq, s, 1), "rope backward");
  HIP_TRY(tn(b.dq, b.z1, G(grads->wq), d, d), "q weight gradient");
  HIP_TRY(tn(b.dk, b.z1, G(grads->wk), d, d), "k weight gradient");
  HIP_TRY(tn(b.dv, b.z1, G(grads->wv), d, d), "v weight gradient");
  HIP_TRY(nn(b.dq, W(w->wq), b.dz, M, d, d, 0), "q input gradient");
  HIP_TRY(nn(b.dk, W(w->wk), b.dz, M, d, d, 1), "k input gradient");
  HIP_TRY(nn(b.dv, W(w->wv), b.dz, M, d, d, 1), "v input gradient");
  // z1 = RMSNorm(x; g1); dx = dh + its gradient
  HIP_TRY(rmsnorm_bwd_launch(x, W(w->attn_norm), b.dz, b.dh, dx, G(grads->attn_norm), b.rstd, M, d, c->norm_eps, s),
          "attention norm backward");
  return LLAMA_OK;
}

int llama_axpby(float *z, const float *x, const float *y, float a, float b, int64_t n, void *stream) {
  if (!z || !x || !y) return LLAMA_ERR_NULL;
  if (n < 0) return LLAMA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(axpby_launch(z, x, y, a, b, n, s), "axpby");
  return LLAMA_OK;
}

int llama_convert_weights_f16(const void *src, void *dst, int64_t n, void *stream) {
  if (n < 0) return LLAMA_ERR_SHAPE;
  if (n == 0) return LLAMA_OK;
  if (!src || !dst) return LLAMA_ERR_NULL;
  const char *a = (const char *)src, *b = (const char *)dst;
  const int64_t bytes = n * (int64_t)sizeof(uint16_t);
  if (a != b && a < b + bytes && b < a + bytes) return LLAMA_ERR_SHAPE;   // partial overlap
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(bf16_to_f16_launch((const uint16_t *)src, (uint16_t *)dst, n, s), "convert weights");
  return LLAMA_OK;
}

int llama_trace_begin(void *const *events, int capacity) {
  if (!events && capacity > 0) return LLAMA_ERR_NULL;
  if (capacity < 0) return LLAMA_ERR_SHAPE;
  g_trace_ev = (hipEvent_t const *)events;
  g_trace_cap = capacity;
  g_trace_n = 0;
  g_trace_labels.clear();
  return LLAMA_OK;
}

int llama_argmax(const float *logits, int64_t rows, int vocab, int32_t *out, void *stream) {
  if (!logits || !out) return LLAMA_ERR_NULL;
  if (rows < 0 || vocab <= 0 || rows > INT32_MAX) return LLAMA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(argmax_launch(logits, rows, vocab, out, s), "argmax");
  return LLAMA_OK;
}

const char *llama_trace_label(int i) {
  return i >= 0 && i < (int)g_trace_labels.size() ? g_trace_labels[i] : nullptr;
}

int llama_trace_end(void) {
  const int n = g_trace_n;
  g_trace_ev = nullptr;
  g_trace_cap = 0;
  g_trace_n = 0;
  return n;
}

int llama_workspace_size(const llama_config *c, int op, int batch, int seq, size_t *bytes) {
  if (!c || !bytes) return LLAMA_ERR_NULL;
  int st = LLAMA_OK;
  switch (op) {
    case LLAMA_OP_CAUSAL_ATTN:
    case LLAMA_OP_SWIGLU_FFN:
      if (!dtype_ok(c->dtype)) return LLAMA_ERR_DTYPE;
      if (c->dim <= 0 || batch <= 0 || seq <= 0 || (op == LLAMA_OP_SWIGLU_FFN && c->hidden <= 0))
        return LLAMA_ERR_SHAPE;
      break;
    case LLAMA_OP_BLOCK_FORWARD:
      st = check_block_cfg(c, batch, seq);
      break;
    case LLAMA_OP_MODEL_FORWARD:
      st = check_model_cfg(c, batch, seq);
      if (!st && seq > c->max_seq) st = LLAMA_ERR_POSITION;
      break;
    case LLAMA_OP_MODEL_DECODE:
      st = check_model_cfg(c, batch, 1);
      if (!st && c->max_seq > kDecMaxSeq) st = LLAMA_ERR_UNSUPPORTED;
      break;
    case LLAMA_OP_CAUSAL_ATTN_BACKWARD:
      if (!dtype_ok(c->dtype)) return LLAMA_ERR_DTYPE;
      if (c->dim <= 0 || c->n_heads <= 0 || c->dim % c->n_heads || batch <= 0 || seq <= 0) return LLAMA_ERR_SHAPE;
      if (c->dtype != LLAMA_F32) return LLAMA_ERR_UNSUPPORTED;
      break;
    case LLAMA_OP_BLOCK_BACKWARD:
      st = check_train_cfg(c, batch, seq);
      break;
    default:
      return LLAMA_ERR_UNSUPPORTED;
  }
  if (st) return st;
  *bytes = ws_bytes_of(c, op, batch, seq);
  return LLAMA_OK;
}

int llama_rmsnorm(int in_dtype, int out_dtype, const void *x, const void *g, void *y, int64_t rows, int dim,
                  float eps, void *stream) {
  if (!x || !y) return LLAMA_ERR_NULL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return LLAMA_ERR_DTYPE;
  if (rows < 0 || dim <= 0) return LLAMA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(rmsnorm_launch(in_dtype == LLAMA_F32, out_dtype == LLAMA_F32, x, g, y, rows, dim, eps, s),
          "llama_rmsnorm");
  return LLAMA_OK;
}

int llama_rope(int dtype, const void *x, void *y, const int32_t *positions, int64_t tokens, int n_heads,
               int head_dim, float theta, void *stream) {
  if (!x || !y || !positions) return LLAMA_ERR_NULL;
  if (!dtype_ok(dtype)) return LLAMA_ERR_DTYPE;
  if (tokens < 0 || n_heads <= 0 || head_dim <= 0 || (head_dim & 1) || !(theta > 0.f)) return LLAMA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(rope_launch(dtype == LLAMA_F32, x, y, positions, tokens, n_heads, head_dim, theta, 0, s), "llama_rope");
  return LLAMA_OK;
}

int llama_linear(int x_dtype, int w_dtype, int y_dtype, const void *x, const void *w, void *y, int64_t rows,
                 int n, int k, void *stream) {
  if (!x || !w || !y) return LLAMA_ERR_NULL;
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype) || !dtype_ok(y_dtype)) return LLAMA_ERR_DTYPE;
  if (rows <= 0 || n <= 0 || k <= 0 || rows > (1 << 24)) return LLAMA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (w_dtype == LLAMA_F32) {
    if (x_dtype != LLAMA_F32 || y_dtype != LLAMA_F32) return LLAMA_ERR_DTYPE;
    HIP_TRY(gemm_f32_launch((const float *)x, (const float *)w, (float *)y, nullptr, (int)rows, n, k, s),
            "llama_linear");
    return LLAMA_OK;
  }
  if (x_dtype != LLAMA_BF16) return LLAMA_ERR_DTYPE;
  if (k % 64) return LLAMA_ERR_SHAPE;
  GemmArgs a{};
  a.M = (int)rows;
  a.N = n;
  a.K = k;
  a.A = (const uint16_t *)x;
  a.lda = k;
  a.b_mode = BMODE_PLAIN;
  a.B0 = (const uint16_t *)w;
  a.C = y;
  a.c_f32 = y_dtype == LLAMA_F32;
  a.ldc = n;
  HIP_TRY(gemm_launch(GemmKey{128, 0, EPI_STORE}, a, s), "llama_linear");
  return LLAMA_OK;
}

int llama_causal_attn(int in_dtype, int out_dtype, const void *q, const void *k, const void *v, void *o,
                      int batch, int seq, int n_heads, int head_dim, void *ws, size_t ws_bytes,
                      void *stream) {
  if (!q || !k || !v || !o) return LLAMA_ERR_NULL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return LLAMA_ERR_DTYPE;
  if (batch <= 0 || seq <= 0 || n_heads <= 0 || head_dim <= 0) return LLAMA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return LLAMA_ERR_UNSUPPORTED;
  if ((int64_t)batch * seq > (1 << 24)) return LLAMA_ERR_SHAPE;
  llama_config c{};
  c.dim = n_heads * head_dim;
  c.n_heads = n_heads;
  c.dtype = in_dtype;
  const size_t need = ws_bytes_of(&c, LLAMA_OP_CAUSAL_ATTN, batch, seq);
  if (!ws || ws_bytes < need) return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Carve cv(ws);
  const int64_t n = (int64_t)batch * seq;
  const int d = c.dim;
  if (in_dtype == LLAMA_F32) {
    float *of = out_dtype == LLAMA_F32 ? (float *)o : cv.take<float>(n * d);
    HIP_TRY(attn_f32_launch((const float *)q, (const float *)k, (const float *)v, of, batch, seq, n_heads,
                            head_dim, s),
            "llama_causal_attn");
    if (out_dtype != LLAMA_F32) HIP_TRY(convert_launch(1, 0, of, o, n * d, s), "llama_causal_attn");
    return LLAMA_OK;
  }
  uint16_t *qh = cv.take<uint16_t>(n * d), *ql = cv.take<uint16_t>(n * d);
  uint16_t *kh = cv.take<uint16_t>(n * d), *kl = cv.take<uint16_t>(n * d);
  const int vts = vt_stride_of(seq);
  const size_t vt = (size_t)batch * d * vts;
  uint16_t *vth = cv.take<uint16_t>(vt), *vtl = cv.take<uint16_t>(vt);
  HIP_TRY(attn_pack_launch(0, q, k, v, qh, ql, kh, kl, vth, vtl, batch, seq, n_heads, head_dim, vts, s),
          "llama_causal_attn");
  AttnArgs at{};
  at.qh = qh;
  at.ql = ql;
  at.kh = kh;
  at.kl = kl;
  at.vth = vth;
  at.vtl = vtl;
  at.o = o;
  at.o_f32 = out_dtype == LLAMA_F32;
  at.batch = batch;
  at.seq = seq;
  at.n_heads = n_heads;
  at.head_dim = head_dim;
  at.dim = d;
  at.kv_dim = d;
  at.n_kv_heads = n_heads;
  at.vt_stride = vts;
  at.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  // bf16 inputs are exact, so their lo parts are zero: one pass each.
  HIP_TRY(attn_prefill_launch(at, 0, 0, 0, s), "llama_causal_attn");
  return LLAMA_OK;
}

int llama_swiglu_ffn(int in_dtype, int out_dtype, const void *z, const void *w_gate, const void *w_up,
                     const void *w_down, void *y, int64_t tokens, int dim, int hidden, void *ws,
                     size_t ws_bytes, void *stream) {
  if (!z || !w_gate || !w_up || !w_down || !y) return LLAMA_ERR_NULL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return LLAMA_ERR_DTYPE;
  if (tokens <= 0 || dim <= 0 || hidden <= 0 || tokens > (1 << 24)) return LLAMA_ERR_SHAPE;
  llama_config c{};
  c.dim = dim;
  c.hidden = hidden;
  c.dtype = in_dtype;
  const size_t need = ws_bytes_of(&c, LLAMA_OP_SWIGLU_FFN, (int)tokens, 1);
  if (!ws || ws_bytes < need) return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Carve cv(ws);
  const int M = (int)tokens;
  if (in_dtype == LLAMA_F32) {
    if (out_dtype != LLAMA_F32) return LLAMA_ERR_DTYPE;
    float *g = cv.take<float>((size_t)M * hidden), *u = cv.take<float>((size_t)M * hidden);
    HIP_TRY(gemm_f32_launch((const float *)z, (const float *)w_gate, g, nullptr, M, hidden, dim, s), "gate");
    HIP_TRY(gemm_f32_launch((const float *)z, (const float *)w_up, u, nullptr, M, hidden, dim, s), "up");
    HIP_TRY(silu_mul_f32_launch(g, u, g, (int64_t)M * hidden, s), "silu");
    HIP_TRY(gemm_f32_launch(g, (const float *)w_down, (float *)y, nullptr, M, dim, hidden, s), "down");
    return LLAMA_OK;
  }
  if (dim % 64 || hidden % 128) return LLAMA_ERR_UNSUPPORTED;
  uint16_t *uh = cv.take<uint16_t>((size_t)M * hidden), *ul = cv.take<uint16_t>((size_t)M * hidden);
  GemmArgs f{};
  f.M = M;
  f.N = 2 * hidden;
  f.K = dim;
  f.A = (const uint16_t *)z;
  f.lda = dim;
  f.b_mode = BMODE_GATEUP;
  f.B0 = (const uint16_t *)w_gate;
  f.B1 = (const uint16_t *)w_up;
  f.C = uh;
  f.C_lo = ul;
  f.ldc = hidden;
  FfnPart fp[2];
  const int nfp = plan_ffn(M, f.N, false, fp);
  for (int i = 0; i < nfp; ++i) {
    f.n_base = fp[i].n_base;
    f.n_end = fp[i].n_end;
    GemmKey fk{256, 0, EPI_SILU};
    fk.bm = fp[i].bm;
    HIP_TRY(gemm_launch(fk, f, s), "gate/up projection");
  }
  GemmArgs dn{};
  dn.M = M;
  dn.N = dim;
  dn.K = hidden;
  dn.A = uh;
  dn.A_lo = ul;
  dn.lda = hidden;
  dn.b_mode = BMODE_PLAIN;
  dn.B0 = (const uint16_t *)w_down;
  dn.C = y;
  dn.c_f32 = out_dtype == LLAMA_F32;
  dn.ldc = dim;
  HIP_TRY(gemm_launch(GemmKey{128, 1, EPI_STORE}, dn, s), "down projection");
  return LLAMA_OK;
}

int llama_block_forward(const llama_config *c, const llama_block_weights *w, int x_dtype, const void *x,
                        float *y, int batch, int seq, void *ws, size_t ws_bytes, void *stream) {
  int st = check_block_cfg(c, batch, seq);
  if (st) return st;
  if ((st = check_block_w(w))) return st;
  if (!x || !y) return LLAMA_ERR_NULL;
  if (!dtype_ok(x_dtype)) return LLAMA_ERR_DTYPE;
  if (c->dtype == LLAMA_F32 && x_dtype != LLAMA_F32) return LLAMA_ERR_DTYPE;
  const size_t need = ws_bytes_of(c, LLAMA_OP_BLOCK_FORWARD, batch, seq);
  if (!ws || ws_bytes < need) return LLAMA_ERR_WORKSPACE;
  Carve cv(ws);
  const BlockWs b = carve_block(cv, c, batch, seq);
  hipStream_t s = (hipStream_t)stream;
  if (c->dtype == LLAMA_F32) return block_f32(c, w, (const float *)x, y, batch, seq, b, s);
  return block_bf16(c, w, x_dtype, x, y, batch, seq, b, nullptr, nullptr, 0, s);
}

int llama_model_forward(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                        const int32_t *start_pos, int batch, int seq, void *k_cache, void *v_cache, float *logits,
                        void *ws, size_t ws_bytes, void *stream) {
  int st = check_model_cfg(c, batch, seq);
  if (st) return st;
  if ((st = check_model_w(c, w))) return st;
  if (!tokens || !k_cache || !v_cache || !logits) return LLAMA_ERR_NULL;
  if (seq > c->max_seq) return LLAMA_ERR_POSITION;
  const size_t need = ws_bytes_of(c, LLAMA_OP_MODEL_FORWARD, batch, seq);
  if (!ws || ws_bytes < need) return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)batch * seq;
  const int d = c->dim, hd = d / c->n_heads;
  Carve cv(ws);
  float *xa = cv.take<float>(n * d), *xb = cv.take<float>(n * d);
  const BlockWs b = carve_block(cv, c, batch, seq, c->max_seq);
  HIP_TRY(embed_launch(0, w->tok_embeddings, tokens, n, d, c->vocab, xa, s), "embedding");
  const size_t layer_elems = (size_t)batch * kv_heads(c) * c->max_seq * hd;
  // shared by every layer; positions up to max_seq when continuing a prefix
  HIP_TRY(rope_table_launch(b.rope_tab, start_pos ? c->max_seq : seq, hd, c->rope_theta, s), "rope table");
  for (int l = 0; l < c->n_layers; ++l) {
    st = block_bf16(c, &w->layers[l], LLAMA_F32, xa, xb, batch, seq, b,
                    (uint16_t *)k_cache + l * layer_elems, (uint16_t *)v_cache + l * layer_elems, c->max_seq, s,
                    false, start_pos, c->max_seq);
    if (st) return st;
    std::swap(xa, xb);
  }
  // the head's operand RMSNorm(x)*g_f is carried like the QKV projection's
  // (fp16, a bf16 pair or bf16, by the numerics bits of that projection)
  const uint32_t num = numerics_of(c);
  const bool hpair = num & LLAMA_NUM_QKV_A_PAIR;
  const int hf16 = (num & LLAMA_NUM_QKV_A_F16) ? 1 : 0;
  HIP_TRY(norm_prep_launch(1, xa, (const uint16_t *)w->final_norm, n, d, c->norm_eps, b.rstd1, b.xg_hi,
                           hpair ? b.xg_lo : nullptr, s, nullptr, 0, nullptr, hf16),
          "final norm");
  GemmArgs hd_{};
  hd_.M = (int)n;
  hd_.N = c->vocab;
  hd_.K = d;
  hd_.A = b.xg_hi;
  hd_.A_lo = hpair ? b.xg_lo : nullptr;
  hd_.lda = d;
  hd_.rstd = b.rstd1;
  hd_.b_mode = BMODE_PLAIN;
  hd_.B0 = (const uint16_t *)w->output;
  hd_.C = logits;
  hd_.c_f32 = 1;
  hd_.ldc = c->vocab;
  HIP_TRY(gemm_launch(GemmKey{256, hpair, EPI_STORE, hf16 * ((num & LLAMA_NUM_W_F16) ? 2 : 1)}, hd_, s), "output head");
  if (start_pos)
    HIP_TRY(nan_unplaced_rows_launch(start_pos, batch, seq, c->max_seq, logits, c->vocab, s), "unplaced sequences");
  return LLAMA_OK;
}

// One decode step over `batch` <= kDecChunk sequences whose layer-0 caches
// start at k_cache / v_cache; layer l's are layer_elems further on (the
// stride of the caller's whole batch).
static int model_decode_chunk(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                              const int32_t *pos, int batch, uint16_t *k_cache, uint16_t *v_cache,
                              size_t layer_elems, float *logits, void *ws, hipStream_t s) {
  const int d = c->dim, hd = d / c->n_heads;
  Carve cv(ws);
  const DecodeWs dw = carve_decode(cv, c, batch);
  DecodeArgs da{};
  da.batch = batch;
  da.dim = d;
  da.n_heads = c->n_heads;
  da.n_kv_heads = kv_heads(c);
  da.head_dim = hd;
  da.hidden = c->hidden;
  da.max_seq = c->max_seq;
  da.vocab = c->vocab;
  da.eps = c->norm_eps;
  da.pos = pos;
  da.rope_tab = dw.rope_tab;

  HIP_TRY(rope_table_pos_launch(dw.rope_tab, pos, batch, hd, c->rope_theta, c->max_seq, s), "rope table");
  HIP_TRY(dec_embed_norm_launch(da, (const uint16_t *)w->tok_embeddings, tokens,
                                (const uint16_t *)w->layers[0].attn_norm, dw.x, dw.rstd, dw.ag_hi, dw.ag_lo, s),
          "embedding");
  const uint16_t *pack = (const uint16_t *)w->decode_pack;
  const PackLayout pl = pack_layout(c);
  const uint16_t *packed_mat = nullptr;   // set before each projection when the pack is present
  auto gemv = [&](int N, int K, int mode, const void *b0, const void *b1, const void *b2, int &splits) {
    GemvArgs g{};
    g.packed = packed_mat;
    int kc;
    gemv_split(N, K, splits, kc);
    g.M = batch;
    g.N = N;
    g.K = K;
    g.k_chunk = kc;
    g.splits = splits;
    g.A_hi = dw.ag_hi;
    g.A_lo = dw.ag_lo;
    g.b_mode = mode;
    g.B0 = (const uint16_t *)b0;
    g.B1 = (const uint16_t *)b1;
    g.B2 = (const uint16_t *)b2;
    g.n_seg = d;
    g.n_seg_kv = kv_dim(c);
    g.part = dw.part;
    return gemv_launch(g, s);
  };
  for (int l = 0; l < c->n_layers; ++l) {
    const llama_block_weights &L = w->layers[l];
    uint16_t *kc = k_cache + l * layer_elems, *vc = v_cache + l * layer_elems;
    int sp;
    const uint16_t *lp = pack ? pack + (size_t)l * pl.layer : nullptr;
    packed_mat = lp ? lp + pl.qkv : nullptr;
    HIP_TRY(gemv(d + 2 * kv_dim(c), d, BMODE_CONCAT3, L.wq, L.wk, L.wv, sp), "qkv projection");
    HIP_TRY(dec_attn_launch(da, dw.part, sp, dw.rstd, kc, vc, dw.ag_hi, dw.ag_lo, dw.attn_part, s), "attention");
    packed_mat = lp ? lp + pl.o : nullptr;
    HIP_TRY(gemv(d, d, BMODE_PLAIN, L.wo, nullptr, nullptr, sp), "output projection");
    HIP_TRY(dec_resid_norm_launch(da, dw.x, dw.part, sp, (const uint16_t *)L.ffn_norm, dw.h, dw.rstd, dw.ag_hi,
                                  dw.ag_lo, s),
            "attention residual");
    packed_mat = lp ? lp + pl.gu : nullptr;
    HIP_TRY(gemv(2 * c->hidden, d, BMODE_GATEUP, L.w_gate, L.w_up, nullptr, sp), "gate/up projection");
    HIP_TRY(dec_gateup_combine_launch(da, dw.part, sp, dw.rstd, dw.ag_hi, dw.ag_lo, s), "silu");
    packed_mat = lp ? lp + pl.down : nullptr;
    HIP_TRY(gemv(d, c->hidden, BMODE_PLAIN, L.w_down, nullptr, nullptr, sp), "down projection");
    const void *gnext = l + 1 < c->n_layers ? w->layers[l + 1].attn_norm : w->final_norm;
    HIP_TRY(dec_resid_norm_launch(da, dw.h, dw.part, sp, (const uint16_t *)gnext, dw.x, dw.rstd, dw.ag_hi,
                                  dw.ag_lo, s),
            "ffn residual");
  }
  int sp;
  packed_mat = pack ? pack + pl.head_off : nullptr;
  HIP_TRY(gemv(c->vocab, d, BMODE_PLAIN, w->output, nullptr, nullptr, sp), "output head");
  HIP_TRY(dec_head_combine_launch(da, dw.part, sp, dw.rstd, logits, s), "head combine");
  return LLAMA_OK;
}

int llama_model_decode(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                       const int32_t *pos, int batch, void *k_cache, void *v_cache, float *logits, void *ws,
                       size_t ws_bytes, void *stream) {
  int st = check_model_cfg(c, batch, 1);
  if (st) return st;
  if (c->max_seq > kDecMaxSeq) return LLAMA_ERR_UNSUPPORTED;
  if ((st = check_model_w(c, w))) return st;
  // without a pack the skinny GEMMs read the projections themselves, as bf16
  if (c->dtype == LLAMA_BF16 && (numerics_of(c) & LLAMA_NUM_W_F16) && !w->decode_pack) return LLAMA_ERR_UNSUPPORTED;
  if (!tokens || !pos || !k_cache || !v_cache || !logits) return LLAMA_ERR_NULL;
  const size_t need = ws_bytes_of(c, LLAMA_OP_MODEL_DECODE, batch, 1);
  if (!ws || ws_bytes < need) return LLAMA_ERR_WORKSPACE;
  const size_t seq_elems = (size_t)kv_heads(c) * c->max_seq * (c->dim / c->n_heads);   // one sequence, one layer
  const size_t layer_elems = (size_t)batch * seq_elems;
  for (int b0 = 0; b0 < batch; b0 += kDecChunk) {
    const int nb = std::min(kDecChunk, batch - b0);
    st = model_decode_chunk(c, w, tokens + b0, pos + b0, nb, (uint16_t *)k_cache + b0 * seq_elems,
                            (uint16_t *)v_cache + b0 * seq_elems, layer_elems, logits + (size_t)b0 * c->vocab, ws,
                            (hipStream_t)stream);
    if (st) return st;
  }
  return LLAMA_OK;
}

int llama_model_decode_static(const llama_config *c, const llama_model_weights *w, const int32_t *tokens,
                              const int32_t *pos, int batch, void *k_cache, void *v_cache, float *logits,
                              void *stream) {
  const int st = check_model_cfg(c, batch, 1);
  if (st) return st;
  const size_t need = ws_bytes_of(c, LLAMA_OP_MODEL_DECODE, batch, 1);
  if (need > kStaticScratchBytes) {
    g_last_error = "llama_model_decode_static: the step needs " + std::to_string(need) +
                   " bytes of scratch; the library's static scratch holds " + std::to_string(kStaticScratchBytes);
    return LLAMA_ERR_WORKSPACE;
  }
  void *ws = nullptr;
  const int sst = static_scratch_of_current_device(&ws);
  if (sst) return sst;
  return llama_model_decode(c, w, tokens, pos, batch, k_cache, v_cache, logits, ws, kStaticScratchBytes, stream);
}

int llama_decode_pack_max_read(const llama_config *c, size_t *bytes) {
  if (!c || !bytes) return LLAMA_ERR_NULL;
  const int st = check_model_cfg(c, 1, 1);
  if (st) return st;
  // every skinny GEMM launch of a decode step, with the block addressing of
  // gemv_kernel: workgroup x, wavefront w, tile j of NTW; split y streams
  // steps it < nit of its K chunk, pieces q < 4, lanes < 64 (16 bytes each)
  const PackLayout pl = pack_layout(c);
  const int d = c->dim, h = c->hidden;
  struct Mat { size_t off; int N, K; };
  const Mat mats[5] = {{pl.qkv, d + 2 * kv_dim(c), d}, {pl.o, d, d}, {pl.gu, 2 * h, d}, {pl.down, d, h},
                       {pl.head_off, c->vocab, d}};
  size_t end = 0;
  for (int m = 0; m < 5; ++m) {
    const Mat &mt = mats[m];
    // every layer's matrices share the first layer's offsets plus whole layers
    const size_t layer_base = m < 4 ? (size_t)(c->n_layers - 1) * pl.layer : 0;
    int splits, kc;
    gemv_split(mt.N, mt.K, splits, kc);
    const int ntw = gemv_shape(mt.N, mt.K).ntw, n_tiles = (mt.N + 31) / 32, per_wg = 128 * ntw;
    const int n_wg = (mt.N + per_wg - 1) / per_wg;
    for (int y = 0; y < splits; ++y) {
      const int ks = y * kc, ke = std::min(mt.K, ks + kc), nit = (ke - ks) / 64;
      for (int x = 0; x < n_wg; ++x)
        for (int w = 0; w < 4; ++w)
          for (int j = 0; j < ntw; ++j) {
            const int t = std::min((x * 4 + w) * ntw + j, n_tiles - 1);
            const size_t last = (size_t)pack_block(t, ks / 64, n_tiles, mt.K / 64, kc / 64) * 2048 +
                                63 * 8 + 2048 * (size_t)(nit - 1) + 512 * 3 + 8;   // one past the last element
            end = std::max(end, mt.off + layer_base + last);
          }
    }
  }
  *bytes = end * sizeof(uint16_t);
  return LLAMA_OK;
}

int llama_decode_pack_size(const llama_config *c, size_t *bytes) {
  if (!c || !bytes) return LLAMA_ERR_NULL;
  const int st = check_model_cfg(c, 1, 1);
  if (st) return st;
  *bytes = pack_layout(c).total * sizeof(uint16_t);
  return LLAMA_OK;
}

int llama_pack_decode_weights(const llama_config *c, const llama_model_weights *w, void *dst, size_t dst_bytes,
                              void *stream) {
  int st = check_model_cfg(c, 1, 1);
  if (st) return st;
  if ((st = check_model_w(c, w))) return st;
  if (numerics_of(c) & LLAMA_NUM_W_F16) return LLAMA_ERR_UNSUPPORTED;   // the pack is built from bf16 weights
  if (!dst) return LLAMA_ERR_NULL;
  const PackLayout pl = pack_layout(c);
  if (dst_bytes < pl.total * sizeof(uint16_t)) return LLAMA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int d = c->dim, h = c->hidden;
  uint16_t *out = (uint16_t *)dst;
  auto kc_of = [](int N, int K) {   // the K chunk the skinny GEMM runs with for this shape
    int sp, kc;
    gemv_split(N, K, sp, kc);
    return kc;
  };
  const int kvd = kv_dim(c), nqkv = d + 2 * kvd;
  for (int l = 0; l < c->n_layers; ++l) {
    const llama_block_weights &L = w->layers[l];
    uint16_t *lp = out + (size_t)l * pl.layer;
    HIP_TRY(pack_tiles_launch(BMODE_CONCAT3, (const uint16_t *)L.wq, (const uint16_t *)L.wk, (const uint16_t *)L.wv,
                              d, kvd, nqkv, d, kc_of(nqkv, d), lp + pl.qkv, s),
            "pack qkv");
    HIP_TRY(pack_tiles_launch(BMODE_PLAIN, (const uint16_t *)L.wo, nullptr, nullptr, d, 0, d, d, kc_of(d, d),
                              lp + pl.o, s),
            "pack o");
    HIP_TRY(pack_tiles_launch(BMODE_GATEUP, (const uint16_t *)L.w_gate, (const uint16_t *)L.w_up, nullptr, d, 0,
                              2 * h, d, kc_of(2 * h, d), lp + pl.gu, s),
            "pack gate/up");
    HIP_TRY(pack_tiles_launch(BMODE_PLAIN, (const uint16_t *)L.w_down, nullptr, nullptr, d, 0, d, h, kc_of(d, h),
                              lp + pl.down, s),
            "pack down");
  }
  HIP_TRY(pack_tiles_launch(BMODE_PLAIN, (const uint16_t *)w->output, nullptr, nullptr, d, 0, c->vocab, d,
                            kc_of(c->vocab, d), out + pl.head_off, s),
          "pack head");
  return LLAMA_OK;
}

}  // extern "C"
