// Matrix-core GEMM for gfx950 over bf16 weights: C[M, N] = A[M, K] * B[N, K]^T,
// fp32 accumulate.
//
// One workgroup = 8 wavefronts (2 x 4, two per SIMD so one wavefront's LDS and
// barrier waits overlap the other's matrix-core work) computing a 256 x BN tile
// with v_mfma_f32_32x32x16_{bf16,f16} (each wavefront 128 x BN/4). A and B move
// HBM -> LDS with global_load_lds_dwordx4 (no register staging): every
// wavefront instruction drops 64 lanes x 16 bytes into one contiguous 1 KB
// block of LDS, and the row/chunk each lane fetches is chosen so the block
// lands already XOR-swizzled. K is consumed in steps of 64 (32 when A is a
// hi/lo pair) with a ring of STAGES LDS buffers (STAGES-1 steps of loads in
// flight); operand reads of the next 16-deep substep are interleaved with the
// current substep's MFMAs; one barrier per step with explicit vmcnt/lgkmcnt
// waits. The 64-deep step halves the barriers per MFMA: on the 7B block the
// QKV, gate/up and down GEMMs run 2.5-5% faster than with 32-deep steps.
//
// A is bf16, a bf16 hi/lo pair (A_lo non-null: both parts are multiplied into
// the same accumulator, which carries an fp32 activation at ~2^-16 relative
// accuracy through bf16 matrix cores), or IEEE fp16 (F16 1: the bf16 weights
// are converted to fp16 in registers, exactly in fp16's normal range, and the
// fp16 matrix cores run at the bf16 rate with 11-bit activations; F16 2: the
// weights arrive already converted, by the same conversion, and go to the
// matrix cores as loaded).
//
// Epilogues (elementwise work of the block fused into the producing GEMM):
//  - every epilogue first scales row r by rstd[r] when rstd is given: the
//    RMSNorm statistic, so the product is RMSNorm(x; g) W^T with the operand
//    x * g prepared by the norm-prep kernel (diag(rstd) commutes with the
//    product; RMSNorm with gain as on the chenyuan1125.github.io LLaMA page).
//  - EPI_QKV: RoPE of q and k after a per-wavefront LDS transpose (a lane
//    owns 16 consecutive columns of one row), stored as fp16 or a bf16 hi/lo
//    pair; v is written transposed per head ([b][h][e][s]) via an LDS
//    transpose so the stores stay 16-byte vectors; optional bf16 KV-cache copy.
//  - EPI_SILU: B rows interleave W_gate and W_up in blocks of 32, so a lane
//    holds gate and up of the same output; u = SiLU(gate) * up (bf16, hi/lo
//    pair or fp16).
//  - EPI_RESID: C = R + acc (the pre-norm skip connection), fp32 out.
//  - EPI_PARTIAL: split-K partial product of range blockIdx.y, fp32, into
//    part[blockIdx.y]; the consumer adds the ranges in order (no atomics).
//  - EPI_STORE: plain fp32 or bf16 (hi/lo) store.
//  RESID, PARTIAL and STORE leave through an LDS transpose as whole 128-byte
//  row segments when the output allows (N % 32 == 0, 16-byte aligned rows).
#pragma once

#include "common.h"
#include "internal.h"

namespace llama {

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in [15:14]).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

#ifndef GEMM_BK
#define GEMM_BK 64
#endif
template <int BN, bool APAIR>
struct GemmCfg {
  // K step: GEMM_BK (32 or 64) for single operands; hi/lo pairs keep 32 (a
  // 64-deep stage with A_lo would not fit two stages in LDS)
  static constexpr int BM = 256, BK = APAIR ? 32 : GEMM_BK;
  static constexpr int CH = BK / 8;                // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CH;              // rows per 1 KB wavefront load
#ifndef GEMM_NW
#define GEMM_NW 8
#endif
  static constexpr int NW = GEMM_NW;               // wavefronts: 2 (M) x NW/2 (N)
  static constexpr int WM = BM / 2, WN = BN / (NW / 2);
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_TILE = BM * CH;           // u32x4 per A tile
  static constexpr int B_TILE = BN * CH;
  static constexpr int STAGE = A_TILE * (APAIR ? 2 : 1) + B_TILE;
  static constexpr int STAGE_BYTES = STAGE * 16;
  static constexpr int STAGES = STAGE_BYTES * 5 <= 160 * 1024   ? 5
                                : STAGE_BYTES * 4 <= 160 * 1024 ? 4
                                : STAGE_BYTES * 3 <= 160 * 1024 ? 3
                                                                : 2;
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS ring exceeds 160 KB");
  static constexpr int A_LD = BM / RPL / NW;       // 1 KB loads per wavefront per A tile
  static constexpr int B_LD = BN / RPL / NW;
  static constexpr int LPS = A_LD * (APAIR ? 2 : 1) + B_LD;  // loads per stage per wavefront
};

// Swizzle of the CH chunks of an LDS row (CH * 16 bytes). gfx950 LDS serves a
// 16-byte read 16 lanes per pass across 64 four-byte banks (256 bytes): the 16
// rows read together (same logical chunk) must land on 16 distinct 16-byte
// slots of the 256-byte bank window: distinct (row mod 4, chunk) pairs for
// 64-byte rows, distinct (row mod 2, chunk) pairs for 128-byte rows.
template <int CH>
DEV int swz(int row) { return CH == 4 ? (row >> 2) & 3 : (row >> 1) & 7; }

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (compile-time indices).
template <int I, int N, class F>
DEV void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Scheduling hint: alternate one MFMA with one LDS read, then the remainder.
template <int NMF, int NRD, int ID>
DEV void interleave() {
  constexpr int P = NMF < NRD ? NMF : NRD;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, ID);  // one LDS read
  }
  if (NMF > P) __builtin_amdgcn_sched_group_barrier(0x008, NMF - P, ID);
  if (NRD > P) __builtin_amdgcn_sched_group_barrier(0x100, NRD - P, ID);
}

// F16 0: bf16 A (or pair) and bf16 B. F16 1: the A operand holds IEEE fp16
// and the bf16 B fragments are converted to fp16 in registers (exactly, for
// weights in fp16's normal range) before fp16 matrix-core products: 11-bit
// activations at the bf16 rate. F16 2: A and B both hold fp16 (B converted
// once, ahead of time, by the same rule), so the products see the same bits
// as with F16 1 without the 3 VALU instructions per two weights.
template <int BN, bool APAIR, int EPI, int F16 = 0>
__global__ __launch_bounds__(GEMM_NW * 64, 1) void gemm_bf16_kernel(const GemmArgs a) {
  static_assert(!(F16 && APAIR), "fp16 operands are single");
  using G = GemmCfg<BN, APAIR>;
  constexpr int BM = G::BM, BK = G::BK, CH = G::CH, STAGES = G::STAGES;
  __shared__ u32x4 smem[STAGES * G::STAGE];

  // the wavefront index as a scalar: LDS destinations of the direct loads are then scalar sums
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (G::NW / 2), wn = wave % (G::NW / 2);
  const int g = lane >> 5, l32 = lane & 31;

  const int tiles_m = (a.M + BM - 1) / BM;
  const int n_end = a.n_end > 0 ? a.n_end : a.N;
  const int tiles_n = (n_end - a.n_base + BN - 1) / BN;
  // Tiles in groups of up to 8 row tiles, column-major inside a group, so
  // that the 32 workgroups one XCD runs at a time cover 8 row tiles x 4
  // column tiles of C (12 operand strips through that XCD's L2) whatever M
  // is, instead of one column of up to M/256 row tiles.
  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  constexpr int GM = 8;
  const int grp = t / (GM * tiles_n), first = grp * GM;
  const int gm = min(tiles_m - first, GM), r_in = t - first * tiles_n;
  const int tm = first + r_in % gm, tn = r_in / gm;
  const int m0 = tm * BM, n0 = a.n_base + tn * BN;

  // ---- global source of each lane's 16-byte piece, fixed over K
  // A block q of this wavefront covers tile rows RPL * (wave * A_LD + q) + lane / CH.
  const u16 *asrc[G::A_LD], *alsrc[APAIR ? G::A_LD : 1];
#pragma unroll
  for (int q = 0; q < G::A_LD; ++q) {
    const int r = G::RPL * (wave * G::A_LD + q) + lane / G::CH;
    const int c = (lane % G::CH) ^ swz<G::CH>(r);
    const int row = min(m0 + r, a.M - 1);  // rows past M load a valid row; never stored
    asrc[q] = (const u16 *)a.A + (int64_t)row * a.lda + 8 * c;
    if (APAIR) alsrc[q] = a.A_lo + (int64_t)row * a.lda + 8 * c;
  }
  const u16 *bsrc[G::B_LD];
#pragma unroll
  for (int q = 0; q < G::B_LD; ++q) {
    const int r = G::RPL * (wave * G::B_LD + q) + lane / G::CH;
    const int c = (lane % G::CH) ^ swz<G::CH>(r);
    const u16 *ptr;
    if (a.b_mode == BMODE_GATEUP) {
      const int blk = r >> 5;
      const int row = (n0 >> 1) + (blk >> 1) * 32 + (r & 31);
      ptr = ((blk & 1) ? a.B1 : a.B0) + (int64_t)row * a.K;
    } else if (a.b_mode == BMODE_CONCAT3) {
      ptr = concat3_row(a.B0, a.B1, a.B2, a.n_seg, a.n_seg_kv > 0 ? a.n_seg_kv : a.n_seg, min(n0 + r, a.N - 1),
                        a.K);
    } else {
      ptr = a.B0 + (int64_t)min(n0 + r, a.N - 1) * a.K;
    }
    bsrc[q] = ptr + 8 * c;
  }

  // K range of this workgroup: split blockIdx.y of k_splits equal ranges
  const int nk = a.K / BK / max(a.k_splits, 1);
  const int kb0 = blockIdx.y * nk * BK;
  auto issue = [&](int kt) {
    const int k0 = kb0 + min(kt, nk - 1) * BK;   // past the end: reload the last step (never read)
    u32x4 *st = smem + (kt % STAGES) * G::STAGE;
#pragma unroll
    for (int q = 0; q < G::A_LD; ++q)
      __builtin_amdgcn_global_load_lds((const void *)(asrc[q] + k0), LDS_PTR(st + (wave * G::A_LD + q) * 64), 16,
                                       0, 0);
    if (APAIR) {
#pragma unroll
      for (int q = 0; q < G::A_LD; ++q)
        __builtin_amdgcn_global_load_lds((const void *)(alsrc[q] + k0),
                                         LDS_PTR(st + G::A_TILE + (wave * G::A_LD + q) * 64), 16, 0, 0);
    }
    u32x4 *sb = st + G::A_TILE * (APAIR ? 2 : 1);
#pragma unroll
    for (int q = 0; q < G::B_LD; ++q)
      __builtin_amdgcn_global_load_lds((const void *)(bsrc[q] + k0), LDS_PTR(sb + (wave * G::B_LD + q) * 64), 16,
                                       0, 0);
  };

  f32x16 acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand fragments of one 16-deep k-substep: A (and its lo part) for the
  // wavefront's 4 row tiles, B for its TN column tiles.
  struct Frag {
    u32x4 a[G::TM], al[APAIR ? G::TM : 1], b[G::TN];   // raw bits: bf16, or fp16 per F16
  };
  auto read_frag = [&](Frag &f, int kt, int ks) {
    const u32x4 *sa = smem + (kt % STAGES) * G::STAGE;
    const u32x4 *sal = sa + G::A_TILE;
    const u32x4 *sb = sa + G::A_TILE * (APAIR ? 2 : 1);
    const int c = ks * 2 + g;
#pragma unroll
    for (int j = 0; j < G::TN; ++j) {
      const int r = wn * G::WN + j * 32 + l32;
      f.b[j] = sb[r * CH + (c ^ swz<CH>(r))];   // converted at use (F16 1), not here: the
                                                  // LDS wait then stays next to the MFMAs
    }
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int r = wm * G::WM + i * 32 + l32;
      const int off = r * CH + (c ^ swz<CH>(r));
      f.a[i] = sa[off];
      if (APAIR) f.al[i] = sal[off];
    }
  };
  auto mma = [&](const Frag &f) {
    u32x4 bh[G::TN];
#pragma unroll
    for (int j = 0; j < G::TN; ++j) bh[j] = F16 == 1 ? bf16x8_to_f16x8(f.b[j]) : f.b[j];
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
        acc[i][j] = F16 ? mfma32h(as_f16x8(f.a[i]), as_f16x8(bh[j]), acc[i][j])
                        : mfma32(as_bf16x8(f.a[i]), as_bf16x8(bh[j]), acc[i][j]);
      if (APAIR) {
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma32(as_bf16x8(f.al[i]), as_bf16x8(f.b[j]), acc[i][j]);
      }
    }
  };

  // Pipeline per K step kt (NS = BK/16 substeps, fragments alternating in
  // f[0] / f[1]), one barrier:
  //   issue loads of stage kt+S-1 | for each substep but the last:
  //   [mma f(ss) interleaved with reads of f(ss+1)]
  //   wait own stage-(kt+1) loads, drain own LDS reads, barrier
  //   [mma of the last substep interleaved with reads of f[0] of step kt+1]
  // The buffer refilled at step kt held stage kt-1; every wavefront drained its
  // reads of it before the previous barrier. Loads past the last step re-read
  // the last step into buffers nobody reads, so the body has no branches.
  constexpr int NS = BK / 16;
  static_assert(NS % 2 == 0, "the last substep's fragments are f[1]");
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  WAIT_VMCNT((STAGES - 2) * G::LPS);
  __builtin_amdgcn_s_barrier();
  Frag f[2];
  read_frag(f[0], 0, 0);
  constexpr int NMF = G::TM * G::TN * (APAIR ? 2 : 1);     // MFMAs per substep
  constexpr int NRD = G::TM * (APAIR ? 2 : 1) + G::TN;      // LDS reads per substep
  auto inner = [&](int kt) {   // substeps 0 .. NS-2 of step kt
    static_for<0, NS - 1>([&](auto ic) {
      constexpr int ss = decltype(ic)::value;
      read_frag(f[(ss + 1) & 1], kt, ss + 1);
      mma(f[ss & 1]);
      interleave<NMF, NRD, ss>();
    });
  };
  for (int kt = 0; kt < nk - 1; ++kt) {
    issue(kt + STAGES - 1);
    // the substeps before the barrier at raised wave priority: when both
    // wavefronts of a SIMD are ready, the one in its MFMA stretch issues
    // first (~1.5% on the 7B block)
    __builtin_amdgcn_s_setprio(1);
    inner(kt);
    __builtin_amdgcn_s_setprio(0);
    WAIT_VMCNT((STAGES - 2) * G::LPS);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    read_frag(f[0], kt + 1, 0);
    mma(f[1]);
    interleave<NMF, NRD, NS - 1>();
  }
  inner(nk - 1);
  mma(f[1]);
  WAIT_VMCNT(0);   // drain the reloads past the end before LDS is reused

  // ---------------------------------------------------------------- epilogue
  if (EPI == EPI_QKV) {
    // segment of this workgroup's columns: q [0, dim), k [dim, dim + kvd),
    // v [dim + kvd, dim + 2 kvd) (uniform: dim and kvd are multiples of BN)
    const int kvd = a.kv_dim > 0 ? a.kv_dim : a.dim;
    const int n_kv = a.n_kv_heads > 0 ? a.n_kv_heads : a.n_heads;
    const int seg = n0 < a.dim ? 0 : (n0 < a.dim + kvd ? 1 : 2);
    const int seg_base = seg == 0 ? 0 : (seg == 1 ? a.dim : a.dim + kvd);
    const int hd_shift = a.head_dim == 128 ? 7 : 6;
    if (seg == 2) {
      // v: transpose each 32x32 accumulator tile through LDS, store rows of v^T
      __builtin_amdgcn_s_barrier();  // all waves are done with the K-loop buffers
      constexpr int TS = 40;         // padded row length (u16) of the transpose tile
      u16 *tr = (u16 *)smem + wave * (2 * 32 * TS);
#pragma unroll
      for (int i = 0; i < G::TM; ++i) {
        const int mb = m0 + wm * G::WM + i * 32;  // first row of the tile
        const int bq = mb / a.seq, s0 = mb - bq * a.seq;
        const bool fast = mb + 32 <= a.M && s0 + 32 <= a.seq && (s0 & 7) == 0;
        float sc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mb + 8 * (r >> 2) + 4 * g + (r & 3);
          sc[r] = (a.rstd && row < a.M) ? a.rstd[row] : 1.0f;
        }
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
          const int cd0 = n0 + wn * G::WN + j * 32 - seg_base;
          if (fast) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              u16 hi[4], lo[4];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const float x = acc[i][j][4 * rq + rr] * sc[4 * rq + rr];
                if (a.attn_f16) {
                  hi[rr] = f2h(x);
                  lo[rr] = 0;
                } else {
                  split_pair(x, hi[rr], lo[rr]);
                }
              }
              const int o = l32 * TS + 8 * rq + 4 * g;
              *(u32x2 *)(tr + o) = u32x2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
              *(u32x2 *)(tr + 32 * TS + o) = u32x2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane -> (column e of the tile, half of its 32 rows)
            const int ce = lane >> 1, half = lane & 1;
            const int cd = cd0 + ce;
            const int hh = cd >> hd_shift, e = cd & (a.head_dim - 1);
            const int64_t o = (((int64_t)bq * n_kv + hh) * a.head_dim + e) * a.vt_stride + s0 + 16 * half;
            const u32x4 *srch = (const u32x4 *)(tr + ce * TS + 16 * half);
            const u32x4 *srcl = (const u32x4 *)(tr + 32 * TS + ce * TS + 16 * half);
            const u32x4 h0 = srch[0], h1 = srch[1], q0 = srcl[0], q1 = srcl[1];
            *(u32x4 *)(a.vth + o) = h0;
            *(u32x4 *)(a.vth + o + 8) = h1;
            if (!a.attn_f16) {
              *(u32x4 *)(a.vtl + o) = q0;
              *(u32x4 *)(a.vtl + o + 8) = q1;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          }
          // element-wise stores: v^T where the fast path does not apply, and
          // the cache copy
          if (!fast || a.vcache) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = 8 * (r >> 2) + 4 * g + (r & 3);
              const int row = mb + off;
              if (row >= a.M) continue;
              // (sequence, position) of the row from those of the tile's first
              // row, without a division per element
              int b = bq, s = s0 + off;
              while (s >= a.seq) {
                s -= a.seq;
                ++b;
              }
              const int cd = cd0 + l32;
              const int hh = cd >> hd_shift, e = cd & (a.head_dim - 1);
              const float x = acc[i][j][r] * sc[r];
              if (!fast) {
                const int64_t o = (((int64_t)b * n_kv + hh) * a.head_dim + e) * a.vt_stride + s;
                if (a.attn_f16) {
                  a.vth[o] = f2h(x);
                } else {
                  u16 hi, lo;
                  split_pair(x, hi, lo);
                  a.vth[o] = hi;
                  a.vtl[o] = lo;
                }
              }
              if (a.vcache) a.vcache[(((int64_t)b * n_kv + hh) * a.max_seq + s) * a.head_dim + e] = f2bf(x);
            }
          }
        }
      }
      return;
    }
    // q, k: each 32 x 32 accumulator block goes through a per-wavefront LDS
    // tile, so that a lane then owns 16 consecutive columns of one row: one
    // rstd and position per lane, the (cos, sin) of its 8 pairs as 16-byte
    // loads, and 16-byte stores of the rotated hi/lo parts.
    u16 *dh = seg == 0 ? a.qh : a.kh;
    u16 *dl = seg == 0 ? a.ql : a.kl;
    __builtin_amdgcn_s_barrier();  // all waves are done with the K-loop buffers
    constexpr int TQ = 36;         // row stride (floats) of the transpose tile, 16-byte aligned
    float *tq = (float *)smem + wave * (32 * TQ);
    const int rr = lane >> 1, c0 = 16 * (lane & 1);
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int row = m0 + wm * G::WM + i * 32 + rr;
      const bool ok = row < a.M;
      const int b = ok ? row / a.seq : 0, s = ok ? row - b * a.seq : 0;
      const float sc = (a.rstd && ok) ? a.rstd[row] : 1.0f;
      const float2 *tab = a.rope_tab + (int64_t)s * (a.head_dim >> 1);
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tq[(8 * (r >> 2) + 4 * g + (r & 3)) * TQ + l32] = acc[i][j][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 t4 = *(const f32x4 *)(tq + rr * TQ + c0 + 4 * q);
#pragma unroll
          for (int k = 0; k < 4; ++k) v[4 * q + k] = t4[k] * sc;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();   // the tile is rewritten for the next block
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (!ok) continue;
        const int cd = n0 + wn * G::WN + j * 32 + c0 - seg_base;   // first of 16 columns
        const int e0 = cd & (a.head_dim - 1);                        // even: 8 whole pairs
        float rot[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 cs2 = *(const f32x4 *)(tab + (e0 >> 1) + 2 * q);   // (cos, sin) of 2 pairs
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float x0 = v[4 * q + 2 * h], x1 = v[4 * q + 2 * h + 1];
            const float cs = cs2[2 * h], sn = cs2[2 * h + 1];
            rot[4 * q + 2 * h] = x0 * cs - x1 * sn;
            rot[4 * q + 2 * h + 1] = x0 * sn + x1 * cs;
          }
        }
        u32x4 hi0, lo0, hi1, lo1;
        const int64_t o = (int64_t)row * (seg == 0 ? a.dim : kvd) + cd;
        if (a.attn_f16) {
          *(u32x4 *)(dh + o) = pack8h(rot);
          *(u32x4 *)(dh + o + 8) = pack8h(rot + 8);
          hi0 = pack8(rot);   // the cache holds bf16
          hi1 = pack8(rot + 8);
        } else {
          pack8_pair(rot, hi0, lo0);
          pack8_pair(rot + 8, hi1, lo1);
          *(u32x4 *)(dh + o) = hi0;
          *(u32x4 *)(dh + o + 8) = hi1;
          *(u32x4 *)(dl + o) = lo0;
          *(u32x4 *)(dl + o + 8) = lo1;
        }
        if (seg == 1 && a.kcache) {
          const int hh = cd >> hd_shift;
          u16 *kp = a.kcache + (((int64_t)b * n_kv + hh) * a.max_seq + s) * a.head_dim + e0;
          *(u32x4 *)kp = hi0;
          *(u32x4 *)(kp + 8) = hi1;
        }
      }
    }
    return;
  }

  // Row-contiguous stores (RESID, PARTIAL, STORE): each 32 x 32 accumulator
  // block goes through a per-wavefront LDS tile and comes back as 8 rows per
  // instruction, 8 lanes per row, 4 consecutive columns per lane: every
  // residual load and output store then covers whole 128-byte row segments
  // with 16-byte (fp32) or 8-byte (bf16) vectors, instead of one column per
  // lane.
  const uintptr_t base_bits = (uintptr_t)a.C | (uintptr_t)a.C_lo | (uintptr_t)a.R | (uintptr_t)a.part;
  if (EPI != EPI_SILU && a.N % 32 == 0 && a.ldc % 16 == 0 && base_bits % 16 == 0) {
    __builtin_amdgcn_s_barrier();  // all waves are done with the K-loop buffers
    constexpr int TQ = 40;         // row stride (floats): the two half-waves write disjoint banks
    float *tq = (float *)smem + wave * (32 * TQ);
    const int r8 = lane >> 3, c4 = 4 * (lane & 7);
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int rb = m0 + wm * G::WM + i * 32;   // first row of the block
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) tq[(8 * (r >> 2) + 4 * g + (r & 3)) * TQ + l32] = acc[i][j][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = *(const f32x4 *)(tq + (8 * q + r8) * TQ + c4);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();   // the tile is rewritten for the next block
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int col = n0 + wn * G::WN + j * 32 + c4;   // N % 32 == 0: the block is inside or outside
        if (col >= a.N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = rb + 8 * q + r8;
          if (row >= a.M) continue;
          f32x4 x = v[q];
          if (a.rstd) x *= a.rstd[row];
          if (EPI == EPI_PARTIAL) {
            *(f32x4 *)(a.part + (int64_t)blockIdx.y * a.M * a.N + (int64_t)row * a.N + col) = x;
            continue;
          }
          const int64_t o = (int64_t)row * a.ldc + col;
          if (EPI == EPI_RESID) {
            if (a.r_f32) {
              x += *(const f32x4 *)((const float *)a.R + o);
            } else {
              const u32x2 r2 = *(const u32x2 *)((const u16 *)a.R + o);
              x += f32x4{__uint_as_float(r2[0] << 16), __uint_as_float(r2[0] & 0xffff0000u),
                         __uint_as_float(r2[1] << 16), __uint_as_float(r2[1] & 0xffff0000u)};
            }
          }
          if (EPI == EPI_RESID || a.c_f32) {
            *(f32x4 *)((float *)a.C + o) = x;
          } else {
            u16 h[4], l[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) split_pair(x[k], h[k], l[k]);
            *(u32x2 *)((u16 *)a.C + o) = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
            if (a.C_lo) *(u32x2 *)(a.C_lo + o) = u32x2{l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16)};
          }
        }
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * G::WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (row >= a.M) continue;
      const float sc = a.rstd ? a.rstd[row] : 1.0f;
      if (EPI == EPI_PARTIAL) {
        float *out = a.part + (int64_t)blockIdx.y * a.M * a.N + (int64_t)row * a.N;
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
          const int col = n0 + wn * G::WN + j * 32 + l32;
          if (col < a.N) out[col] = acc[i][j][r] * sc;
        }
      } else if (EPI == EPI_SILU) {
#pragma unroll
        for (int j = 0; j < G::TN; j += 2) {
          const float u = silu(acc[i][j][r] * sc) * (acc[i][j + 1][r] * sc);
          const float un = lane_swap1(u);   // the next column's value (even lanes use it)
          if (l32 & 1) continue;
          const int col = (n0 >> 1) + wn * (G::WN / 2) + (j >> 1) * 32 + l32;
          const int64_t o = (int64_t)row * a.ldc + col;   // even: two columns as one 4-byte word
          if (a.c_f16) {
            *(uint32_t *)((u16 *)a.C + o) = pack2h(u, un);
            continue;
          }
          u16 h0, l0, h1, l1;
          split_pair(u, h0, l0);
          split_pair(un, h1, l1);
          *(uint32_t *)((u16 *)a.C + o) = (uint32_t)h0 | ((uint32_t)h1 << 16);
          if (a.C_lo) *(uint32_t *)(a.C_lo + o) = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
          const int col = n0 + wn * G::WN + j * 32 + l32;
          if (col >= a.N) continue;
          float v = acc[i][j][r] * sc;
          const int64_t o = (int64_t)row * a.ldc + col;
          if (EPI == EPI_RESID) {
            v += a.r_f32 ? ((const float *)a.R)[o] : bf2f(((const u16 *)a.R)[o]);
            ((float *)a.C)[o] = v;
          } else if (a.c_f32) {
            ((float *)a.C)[o] = v;
          } else {
            const u16 hi = f2bf(v);
            ((u16 *)a.C)[o] = hi;
            if (a.C_lo) a.C_lo[o] = f2bf(v - bf2f(hi));
          }
        }
      }
    }
  }
}

template <int BN, bool APAIR, int EPI, int F16 = 0>
hipError_t gemm_launch_t(const GemmArgs &a, hipStream_t s) {
  using G = GemmCfg<BN, APAIR>;
  const int n_end = a.n_end > 0 ? a.n_end : a.N;
  if (a.n_base < 0 || a.n_base % BN || n_end > a.N || n_end <= a.n_base) return hipErrorInvalidValue;
  const int nb = ((a.M + G::BM - 1) / G::BM) * ((n_end - a.n_base + BN - 1) / BN);
  if (nb == 0) return hipSuccess;
  const int ks = a.k_splits > 1 ? a.k_splits : 1;
  if (a.K % (G::BK * ks)) return hipErrorInvalidValue;
  if (ks > 1 && EPI != EPI_PARTIAL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BN, APAIR, EPI, F16>), dim3(nb, ks), dim3(G::NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace llama

#define GEMM_CASE(BN_, APAIR_, EPI_)                                                       \
  if (key.bn == BN_ && key.apair == APAIR_ && key.epi == EPI_ && !key.f16)                  \
    return gemm_launch_t<BN_, APAIR_, EPI_>(a, s);
#define GEMM_CASE_F16(BN_, EPI_)                                                           \
  if (key.bn == BN_ && !key.apair && key.epi == EPI_ && key.f16 == 1)                       \
    return gemm_launch_t<BN_, false, EPI_, 1>(a, s);                                       \
  if (key.bn == BN_ && !key.apair && key.epi == EPI_ && key.f16 == 2)                       \
    return gemm_launch_t<BN_, false, EPI_, 2>(a, s);
