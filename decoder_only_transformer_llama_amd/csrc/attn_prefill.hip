// Causal flash-style attention for prefill on gfx950 matrix cores.
//
// Per (sequence, head, 128-query tile) one workgroup of 4 wavefronts; each
// wavefront owns 32 queries. Keys/values stream through LDS in tiles of 32.
// The product is formed transposed — S^T = K Q^T and O^T = V^T P^T — so that in
// the 32x32 accumulator layout every lane holds values of ONE query (its lane
// index mod 32): the running max, the running sum and the rescaling of O stay
// in that lane's registers, and the only cross-lane step is one exchange
// between the two 32-lane halves. Keys are read from LDS in a permuted order
// (bits 2 and 3 of the key index swapped) so that the probabilities a lane
// holds after the S^T product are exactly the eight consecutive keys it must
// supply as the P^T operand of the next product: no register shuffles.
//
// Softmax is online in fp32 with exp2 and a log2(e)/sqrt(hd) prescale (with
// fp16 operands folded into q by the QKV epilogue); masked
// keys get exactly zero weight; tiles entirely above the diagonal are never
// loaded and fully masked 32-key halves are skipped per wavefront. Operands are
// either bf16 (q/k and v optionally as hi/lo pairs: 3 and 2 matrix-core
// passes) or IEEE fp16 (F16: q, k, v and the probabilities, one pass each;
// 11 significant bits instead of 8, range up to 65504).
//
// Attention itself is the 2017 scaled-dot-product attention with a causal mask
// (paperfordummies.in LLaMA page, "LLaMA is a pull request against the 2017
// transformer": the attention is untouched; RoPE is applied to q and k before).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace llama {

DEV int perm23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// LDS chunk swizzles (gfx950 serves a 16-byte read 16 lanes per pass over a
// 256-byte bank window): K rows of 256 bytes XOR the chunk with row mod 16,
// K rows of 128 bytes with (row / 2) mod 8, v^T rows of 64 bytes with
// (row / 4) mod 4, so any 16 consecutive rows read at one logical chunk hit 16
// distinct 16-byte slots.
template <int CHUNKS>
DEV int rswz(int row) { return CHUNKS == 16 ? (row & 15) : ((row >> 1) & 7); }
DEV int vswz(int row) { return (row >> 2) & 3; }

#define ATT_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#define ATT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// (sequence*head, query tile) of workgroup `k`. Causal work grows with the
// query tile, so when the tile count is even the first half of the grid takes
// the long tiles nqt-1-i, longest first, and the second half the short tile i:
// when the dispatcher fills CUs round-robin, workgroups k and k + total/2 share
// a CU and every CU gets about the same number of key tiles.
DEV void attn_tile_of(int k, int nqt, int bh_count, int &bh, int &qt) {
  if ((nqt & 1) == 0) {
    const int halfn = (nqt >> 1) * bh_count;
    const int half = k / halfn, j = k % halfn;
    bh = j / (nqt >> 1);
    const int i = j % (nqt >> 1);
    qt = half == 0 ? nqt - 1 - i : i;
  } else {
    bh = k / nqt;
    qt = nqt - 1 - k % nqt;
  }
}

template <int HD, bool QKPAIR, bool VPAIR, bool F16>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(const AttnArgs a) {
  static_assert(!F16 || (!QKPAIR && !VPAIR), "fp16 operands are single");
  constexpr int KT = 32;                         // keys per tile
  constexpr int KCH = HD / 8;                    // 16-byte chunks per K row
  constexpr int NKK = HD / 16;                   // k-steps of the score product
  constexpr int NEB = HD / 32;                   // 32-wide blocks of the head dimension
  constexpr int KTILE = KT * KCH;                // u32x4 per K tile
  constexpr int VTILE = HD * 4;                  // u32x4 per v^T tile (4 chunks of 8 keys)
  constexpr int STAGE1 = KTILE * (QKPAIR ? 2 : 1) + VTILE * (VPAIR ? 2 : 1);   // one 32-key tile
  // Tiles per step (SUB): with fp16 operands two 32-key tiles share one
  // barrier and one softmax update (f16_step below), so each step carries two
  // independent score chains; the longest workgroups (the last query tiles,
  // 2048 keys) then take half as many dependent steps.
  constexpr int SUB = F16 ? 2 : 1;
  constexpr int STAGE = SUB * STAGE1;
  // LDS ring depth 2 (64 KB at hd 128), so that two workgroups share a
  // compute unit. (A third slot measured slower: loads are not what the
  // steps wait on.)
  constexpr int NST = 2;
  constexpr float kLazyRescale = 8.0f;   // log2 units a running maximum may lag the true one
  constexpr int KBLK = KTILE / 64, VBLK = VTILE / 64;       // 1 KB blocks per tile
  constexpr int NBLK = KBLK * (QKPAIR ? 2 : 1) + VBLK * (VPAIR ? 2 : 1);
  static_assert(NBLK % 4 == 0, "blocks split evenly over 4 wavefronts");
  __shared__ u32x4 smem[NST * STAGE];

  const int S = a.seq;
  const int nqt = (S + 127) / 128;
  int bh, qt;
  attn_tile_of(blockIdx.x, nqt, a.batch * a.n_heads, bh, qt);
  const int b = bh / a.n_heads, h = bh % a.n_heads;
  // the wavefront index as a scalar: the block each wavefront loads and its
  // diagonal tests then branch on scalars, without per-lane masks
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int q0 = qt * 128;
  const int qi = q0 + 32 * w + l32;          // this lane's query
  const int qwave_max = q0 + 32 * w + 31;
  const int64_t tok0 = (int64_t)b * S;
  // Continuing a cached prefix: queries are positions p0 .. p0+S-1 and the
  // keys positions 0 .. p0+S-1 (k rows by position, kv_rows per sequence).
  const int p0 = max(chunk_start(a.start_pos, b, S, a.max_seq), 0);
  const int nkeys = p0 + S;
  const int64_t ktok0 = a.start_pos ? (int64_t)b * a.kv_rows : tok0;
  // key/value head of this query head: consecutive groups of n_heads / n_kv_heads
  const int n_kv = a.n_kv_heads > 0 ? a.n_kv_heads : a.n_heads;
  const int kvd = a.kv_dim > 0 ? a.kv_dim : a.dim;
  const int hk = h / (a.n_heads / n_kv);
  const int64_t vbase = ((int64_t)b * n_kv + hk) * HD * a.vt_stride;

  const int kend = min(nkeys, p0 + q0 + 128);
  const int n_kt = (kend + KT - 1) / KT;        // 32-key tiles
  const int n_st = (n_kt + SUB - 1) / SUB;      // steps of SUB tiles

  // ---- direct-to-LDS tile loads: block q of this wavefront, lane i -> LDS slot i.
  // Ring slot st % NST holds tiles SUB*st .. SUB*st + SUB-1; tiles past the
  // last reload the last tile (their keys are masked, or the slot is never
  // read) so that every step waits on the same number of loads.
  // Per block this wavefront loads: K or v^T (wavefront-uniform), the lane's
  // fixed part of the source address, and the block's place in a stage.
  // Loads go out as buffer loads to LDS: a uniform base per block (this
  // sequence and head's K rows, or v^T row block) and per-lane byte offsets.
  constexpr int NQB = NBLK / 4;
  bool isk[NQB];
  const u16 *lbase[NQB];
  uint32_t loff[NQB];
  int lrow[NQB], ldst[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int blk = w * NQB + qb;
    isk[qb] = blk < KBLK * (QKPAIR ? 2 : 1);
    if (isk[qb]) {
      const int part = blk / KBLK, kb = blk % KBLK;
      const int row = kb * (64 / KCH) + lane / KCH;
      const int c = (lane % KCH) ^ rswz<KCH>(row);
      lrow[qb] = row;
      lbase[qb] = (part ? a.kl : a.kh) + ktok0 * kvd + hk * HD;
      loff[qb] = (uint32_t)(8 * c * 2);
      ldst[qb] = part * KTILE + kb * 64;
    } else {
      const int vblk = blk - KBLK * (QKPAIR ? 2 : 1);
      const int part = vblk / VBLK, vb = vblk % VBLK;
      const int e = vb * 16 + (lane >> 2);
      const int c = (lane & 3) ^ vswz(e);
      lrow[qb] = 0;
      lbase[qb] = (part ? a.vtl : a.vth) + vbase;
      loff[qb] = (uint32_t)((e * a.vt_stride + 8 * c) * 2);
      ldst[qb] = KTILE * (QKPAIR ? 2 : 1) + part * VTILE + vb * 64;
    }
  }
  // fp16 operands: a block's source offset is a lane part that stays fixed
  // plus a scalar part per 32-key tile (K rows step kvd elements per key, v^T
  // columns one), so a tile's loads take no vector arithmetic and no branch
  // per block. Otherwise, and for a tile that runs past the last key, the
  // offset is formed per lane, and K rows past the last key load that key
  // instead (masked later).
  uint32_t lvo[NQB], sst[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    lvo[qb] = loff[qb] + (isk[qb] ? (uint32_t)(lrow[qb] * kvd * 2) : 0u);
    sst[qb] = isk[qb] ? (uint32_t)(KT * kvd * 2) : (uint32_t)(KT * 2);
  }
  auto issue = [&](int st_slot) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      u32x4 *st = smem + (st_slot % NST) * STAGE + u * STAGE1;
      const int kt = min(st_slot * SUB + u, n_kt - 1);
      if (F16 && kt * KT + KT <= nkeys) {   // (the bf16 pair forms lack the registers)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) buf_load_lds16(lbase[qb], lvo[qb], (uint32_t)kt * sst[qb], st + ldst[qb]);
      } else {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          if (isk[qb])
            buf_load_lds16(lbase[qb], loff[qb] + (uint32_t)(min(kt * KT + lrow[qb], nkeys - 1) * kvd * 2), 0,
                           st + ldst[qb]);
          else
            buf_load_lds16(lbase[qb], loff[qb], (uint32_t)(kt * KT * 2), st + ldst[qb]);
        }
      }
    }
  };

  issue(0);

  // q fragments (B operand of S^T = K Q^T): q[qi][16kk + 8g .. +7]
  u32x4 qh[NKK], ql[QKPAIR ? NKK : 1];
  {
    const int64_t base = (tok0 + min(qi, S - 1)) * a.dim + h * HD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qh[kk] = *(const u32x4 *)(a.qh + base + 16 * kk);
      if (QKPAIR) ql[kk] = *(const u32x4 *)(a.ql + base + 16 * kk);
    }
  }

  const float c = a.scale_log2;
  // fp16 operands: q arrives multiplied by c = log2(e)/sqrt(hd) (the QKV
  // epilogue folds it in before its one fp16 rounding), so the score products
  // come out in log2 units, and the running maximum (same units) is taken
  // off by starting the score accumulators at -m: a key's exponent is then
  // its accumulator as it stands.
  f32x16 negm;
  if constexpr (F16) {
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = 0.f;
  }
  f32x16 acc_o[NEB];
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[e][r] = 0.f;
  // running maximum: of s*c with fp16 operands, of s with bf16 operands
  float m_run = -INFINITY, l_run = 0.f;
  const int krow = perm23(l32);   // key (within the tile) this lane supplies as A-operand row
  for (int st = 1; st < NST - 1; ++st) issue(st);   // after the q fragments: they complete first

  // One step of the fp16 path: SUB = 2 tiles of 32 keys in ring slot `stg`,
  // keys s0 .. s0 + 63. Ordered so that latencies overlap inside the
  // wavefront: every K fragment read is issued before the first product, the
  // two tiles' score chains alternate on the matrix cores, the v^T fragments
  // are read while the softmax runs, and the second tile's exponentials are
  // computed while the first tile's P^T products run.
  auto f16_step = [&](const u32x4 *stg, int s0) __attribute__((always_inline)) {
    u32x4 kf[SUB][NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int so = krow * KCH + ((2 * kk + g) ^ rswz<KCH>(krow));
#pragma unroll
      for (int u = 0; u < SUB; ++u) kf[u][kk] = stg[u * STAGE1 + so];
    }
    // scores s*c - m (log2 units, relative to the running maximum)
    f32x16 sc[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) sc[u] = mfma32h(as_f16x8(kf[u][0]), as_f16x8(qh[0]), negm);
#pragma unroll
    for (int kk = 1; kk < NKK; ++kk)
#pragma unroll
      for (int u = 0; u < SUB; ++u) sc[u] = mfma32h(as_f16x8(kf[u][kk]), as_f16x8(qh[kk]), sc[u]);
    // every K fragment read ahead of the first product (left alone, the
    // compiler reuses two register quads and waits on each read in turn)
    __builtin_amdgcn_sched_group_barrier(0x100, SUB * NKK, 0);   // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, SUB * NKK, 0);   // matrix-core products
    u32x4 vf[SUB][2][NEB];
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < NEB; ++e) {
          const int row = 32 * e + l32;
          vf[u][s2][e] = stg[u * STAGE1 + KTILE + row * 4 + ((2 * s2 + g) ^ vswz(row))];
        }
    // masked maximum of each tile (independent chains), then over both
    // 32-lane halves of the wavefront (lanes l and l ^ 32 hold the same query)
    float mxu[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int kt0 = s0 + u * KT;
      float m = -INFINITY;
      if (kt0 + KT - 1 > p0 + q0 + 32 * w || kt0 + KT > nkeys) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + 16 * ((r >> 2) >> 1) + 8 * g + 4 * ((r >> 2) & 1) + (r & 3);
          const bool ok = key <= p0 + qi && key < nkeys;
          sc[u][r] = ok ? sc[u][r] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[u][r]);
      mxu[u] = m;
    }
    float mx = mxu[0];
#pragma unroll
    for (int u = 1; u < SUB; ++u) mx = fmaxf(mx, mxu[u]);
    {
      // v_permlane32_swap: lanes l and l ^ 32 exchange values, no LDS round trip
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // lazy rescaling, as below for bf16 operands; mx is already relative to
    // the maximum the accumulators started from (0 while m_run = -inf, which
    // always takes the update)
    if (!__all(m_run > -INFINITY && mx <= kLazyRescale)) {
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      const float m_new = fmaxf(m_run, mx + m_use);
      const float m_new_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new_use);   // -inf -> 0
      const float d = m_use - m_new_use;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < NEB; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[e][r] *= alpha;
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[u][r] += d;   // masked keys stay -inf
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[r] = -m_new_use;
    }
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(sc[u][r]);   // exp2(-inf) = 0 for masked keys
        ps[r & 3] += pr[r];
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4 pf = pack8h(pr + 8 * s2);
#pragma unroll
        for (int e = 0; e < NEB; ++e) acc_o[e] = mfma32h(as_f16x8(vf[u][s2][e]), as_f16x8(pf), acc_o[e]);
      }
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // Waits for this wavefront's loads of `step` (and the q fragments), then
  // for everyone's at the barrier (everyone is then done with the previous
  // step), and issues the loads of a later step.
  auto step_begin = [&](int step) __attribute__((always_inline)) {
    ATT_WAIT_VMCNT((NST - 2) * SUB * (NBLK / 4));
    __builtin_amdgcn_s_barrier();
    if (NST == 2) {
      if (step + 1 < n_st) issue(step + 1);   // overwrites the buffer of the previous step
    } else {
      issue(step + NST - 1);
    }
  };
  if constexpr (F16) {
    // Steps in pairs, so that each one's ring slot is a constant and the
    // fragment reads take it as an instruction offset (no address arithmetic).
    static_assert(NST == 2, "the step pairs alternate two ring slots");
    auto f16_iter = [&](auto slot, int step) __attribute__((always_inline)) {
      step_begin(step);
      const int s0 = step * SUB * KT;
      if (s0 > p0 + qwave_max) return;   // whole step above this wavefront's diagonal
      f16_step(smem + decltype(slot)::value * STAGE, s0);
    };
    for (int step = 0; step < n_st; step += 2) {
      f16_iter(std::integral_constant<int, 0>{}, step);
      if (step + 1 < n_st) f16_iter(std::integral_constant<int, 1>{}, step + 1);
    }
  }
  for (int step = 0; !F16 && step < n_st; ++step) {
    step_begin(step);
    const int s0 = step * SUB * KT;
    if (s0 > p0 + qwave_max) continue;   // whole step above this wavefront's diagonal
    // ---- bf16 operands, one tile per step. Scores S^T (32 keys x 32
    // queries): two accumulators (even and odd k-steps) so that two dependent
    // matrix-core chains of half the length run interleaved.
    constexpr int NACC = 2;
    f32x16 sc[SUB];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const u32x4 *sk = smem + (step % NST) * STAGE + u * STAGE1;
      const u32x4 *skl = sk + KTILE;
      f32x16 sacc[NACC];
#pragma unroll
      for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int so = krow * KCH + ((2 * kk + g) ^ rswz<KCH>(krow));
        f32x16 &acc = sacc[kk % NACC];
        const bf16x8 kf = as_bf16x8(sk[so]);
        acc = mfma32(kf, as_bf16x8(qh[kk]), acc);
        if (QKPAIR) {
          acc = mfma32(as_bf16x8(skl[so]), as_bf16x8(qh[kk]), acc);
          acc = mfma32(kf, as_bf16x8(ql[kk]), acc);
        }
      }
      sc[u] = sacc[0] + sacc[1];
    }

    // ---- online softmax (fp32); lane holds 16 keys of query qi per tile.
    // Only tiles crossing this wavefront's diagonal or the sequence end need
    // the mask (a wavefront-uniform test).
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int kt0 = s0 + u * KT;
      if (kt0 + KT - 1 > p0 + q0 + 32 * w || kt0 + KT > nkeys) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + 16 * ((r >> 2) >> 1) + 8 * g + 4 * ((r >> 2) & 1) + (r & 3);
          const bool ok = key <= p0 + qi && key < nkeys;
          sc[u][r] = ok ? sc[u][r] : -INFINITY;
          mx = fmaxf(mx, sc[u][r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[u][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescaling: the reference maximum m_run moves (and O, l are
    // rescaled) only when some lane's new maximum exceeds it by more than
    // kLazyRescale in log2 units; otherwise probabilities up to 2^kLazyRescale
    // enter P (exact in fp32, within fp16 range) and the final 1/l cancels the
    // common factor. m_run = -inf (no visible key yet) always takes the update.
    if (!__all((mx - m_run) * c <= kLazyRescale)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);   // -inf -> 0
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < NEB; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[e][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    const float mc = -m_use * c;   // exponent (s - m) c as one fma: s c - m c
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][r], c, mc));   // exp2(-inf) = 0 for masked keys
        sc[u][r] = pr;
        psum += pr;
      }
    l_run += psum;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const u32x4 *sv = smem + (step % NST) * STAGE + u * STAGE1 + KTILE * (QKPAIR ? 2 : 1);
      const u32x4 *svl = sv + VTILE;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = sc[u][8 * s2 + i];
        const u32x4 pf = pack8(pv);
        const int ch = 2 * s2 + g;
#pragma unroll
        for (int e = 0; e < NEB; ++e) {
          const int row = 32 * e + l32;
          const int so = row * 4 + (ch ^ vswz(row));
          acc_o[e] = mfma32(as_bf16x8(sv[so]), as_bf16x8(pf), acc_o[e]);
          if (VPAIR) acc_o[e] = mfma32(as_bf16x8(svl[so]), as_bf16x8(pf), acc_o[e]);
        }
      }
    }
  }

  // ---- normalise and store o[qi][h*HD + e]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qi >= S) return;
  const int64_t obase = (tok0 + qi) * a.dim + h * HD;
#pragma unroll
  for (int e = 0; e < NEB; ++e) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int e0 = 32 * e + 8 * rq + 4 * g;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc_o[e][4 * rq + i] * inv;
      if (a.o_f32) {
        *(f32x4 *)((float *)a.o + obase + e0) = f32x4{v[0], v[1], v[2], v[3]};
      } else if (a.o_f16) {   // the fp16 operand of an fp16 output projection
        *(u32x2 *)((u16 *)a.o + obase + e0) = u32x2{pack2h(v[0], v[1]), pack2h(v[2], v[3])};
      } else {
        u16 hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_pair(v[i], hi[i], lo[i]);
        *(u32x2 *)((u16 *)a.o + obase + e0) =
            u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
        if (a.o_lo)
          *(u32x2 *)(a.o_lo + obase + e0) =
              u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
      }
    }
  }
}

// Zero v^T columns [seq, vt_stride) so partial key tiles multiply finite zeros.
__global__ void vt_pad_zero_kernel(u16 *vth, u16 *vtl, int64_t rows, int seq, int vt_stride) {
  const int pad = vt_stride - seq;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * pad) return;
  const int64_t o = (idx / pad) * vt_stride + seq + idx % pad;
  vth[o] = 0;
  if (vtl) vtl[o] = 0;
}

// Cached prefix of a prefill chunk into the attention operands. One thread
// per (sequence, key/value head, 8 positions, 8 channels): an 8 x 8 block of
// the bf16 cache goes to 8 k rows (16-byte stores) and to 8 v^T rows (16-byte
// stores when all 8 positions are prefix, else element by element).
template <bool F16>
__global__ void kv_prefix_kernel(const u16 *__restrict__ kc, const u16 *__restrict__ vc, const int32_t *start_pos,
                                 int batch, int n_kv, int hd, int max_seq, int seq, u16 *kh, u16 *kl, u16 *vth,
                                 u16 *vtl, int kv_rows, int vt_stride) {
  const int npos8 = (max_seq + 7) / 8, nch8 = hd / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * n_kv * npos8 * nch8) return;
  const int e0 = 8 * (int)(idx % nch8);
  const int64_t r = idx / nch8;
  const int j0 = 8 * (int)(r % npos8);
  const int bh = (int)(r / npos8), b = bh / n_kv, hk = bh % n_kv;
  const int p0 = max(chunk_start(start_pos, b, seq, max_seq), 0);
  const int pad_end = min((p0 + seq + 31) / 32 * 32, vt_stride);
  if (j0 >= p0 && (j0 + 8 <= p0 + seq || j0 >= pad_end)) return;   // nothing of this block to write
  auto cvt = [](u16 v) -> u16 { return F16 ? f2h(bf2f(v)) : v; };   // bf16 -> fp16 is exact in fp16's range
  const int kvd = n_kv * hd;
  u16 vt[8][8];   // [channel][position]
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int j = j0 + jj;
    u16 vals[8];
    if (j < p0) {
      const int64_t src = (((int64_t)b * n_kv + hk) * max_seq + j) * hd + e0;
      const u32x4 kq = *(const u32x4 *)(kc + src), vq = *(const u32x4 *)(vc + src);
      const u16 *kk = (const u16 *)&kq, *vv = (const u16 *)&vq;
      u32x4 ko;
      u16 *ko16 = (u16 *)&ko;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ko16[i] = cvt(kk[i]);
        vals[i] = cvt(vv[i]);
      }
      const int64_t dst = ((int64_t)b * kv_rows + j) * kvd + hk * hd + e0;
      *(u32x4 *)(kh + dst) = ko;
      if (kl) *(u32x4 *)(kl + dst) = u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) vals[i] = 0;   // +0 in bf16 and fp16
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) vt[i][jj] = vals[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t o = (((int64_t)b * n_kv + hk) * hd + e0 + i) * vt_stride + j0;
    if (j0 + 8 <= p0) {
      *(u32x4 *)(vth + o) = *(const u32x4 *)vt[i];
      if (vtl) *(u32x4 *)(vtl + o) = u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        if (j < p0 || (j >= p0 + seq && j < pad_end)) {
          vth[o + jj] = vt[i][jj];
          if (vtl) vtl[o + jj] = 0;
        }
      }
    }
  }
}

hipError_t kv_prefix_launch(const uint16_t *kcache, const uint16_t *vcache, const int32_t *start_pos, int batch,
                            int n_kv, int head_dim, int max_seq, int seq, uint16_t *kh, uint16_t *kl, uint16_t *vth,
                            uint16_t *vtl, int kv_rows, int vt_stride, int f16, hipStream_t s) {
  if (batch == 0 || seq == 0) return hipSuccess;
  if (head_dim % 8 || kv_rows < max_seq || vt_stride < kv_rows || vt_stride % 8) return hipErrorInvalidValue;
  if (f16 && (kl || vtl)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)batch * n_kv * ((max_seq + 7) / 8) * (head_dim / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(kv_prefix_kernel<true>, grid, dim3(256), 0, s, kcache, vcache, start_pos, batch, n_kv, head_dim,
                       max_seq, seq, kh, kl, vth, vtl, kv_rows, vt_stride);
  else
    hipLaunchKernelGGL(kv_prefix_kernel<false>, grid, dim3(256), 0, s, kcache, vcache, start_pos, batch, n_kv,
                       head_dim, max_seq, seq, kh, kl, vth, vtl, kv_rows, vt_stride);
  return hipGetLastError();
}

template <int HD, bool QKPAIR, bool VPAIR, bool F16 = false>
static hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
  const int nqt = (a.seq + 127) / 128;
  hipLaunchKernelGGL((attn_prefill_kernel<HD, QKPAIR, VPAIR, F16>), dim3(nqt * a.batch * a.n_heads), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t attn_prefill_launch(const AttnArgs &a, int qk_pair, int v_pair, int f16, hipStream_t s) {
  if (f16 && (qk_pair || v_pair || !a.q_scaled)) return hipErrorInvalidValue;
  if (a.batch * a.seq == 0) return hipSuccess;
  if (a.start_pos && (a.kv_rows < a.seq || a.max_seq > a.kv_rows || a.vt_stride < a.kv_rows))
    return hipErrorInvalidValue;
  if (a.seq % 32 && !a.start_pos) {   // with start_pos the prefix copy zeroes the pad
    const int64_t rows = (int64_t)a.batch * (a.n_kv_heads > 0 ? a.n_kv_heads : a.n_heads) * a.head_dim;
    const int64_t n = rows * (a.vt_stride - a.seq);
    // all-zero bits are +0 in bf16 and in fp16
    hipLaunchKernelGGL(vt_pad_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (u16 *)a.vth, v_pair ? (u16 *)a.vtl : (u16 *)nullptr, rows, a.seq, a.vt_stride);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (f16) {
    if (a.head_dim == 128) return launch_t<128, false, false, true>(a, s);
    if (a.head_dim == 64) return launch_t<64, false, false, true>(a, s);
    return hipErrorInvalidValue;
  }
#define ATTN_CASE(HD_, QK_, V_) \
  if (a.head_dim == HD_ && !!qk_pair == QK_ && !!v_pair == V_) return launch_t<HD_, QK_, V_>(a, s);
  ATTN_CASE(128, true, true)
  ATTN_CASE(128, true, false)
  ATTN_CASE(128, false, true)
  ATTN_CASE(128, false, false)
  ATTN_CASE(64, true, true)
  ATTN_CASE(64, true, false)
  ATTN_CASE(64, false, true)
  ATTN_CASE(64, false, false)
#undef ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace llama
