// bf16 matrix-core GEMM for gfx950: C[M, N] = A[M, K] * B[N, K]^T, fp32 accumulate.
//
// One workgroup = 4 wavefronts (2 x 2) computing a 256 x BN tile with
// v_mfma_f32_32x32x16_bf16. A and B tiles go global -> registers -> LDS,
// double-buffered in LDS so the next tile's global loads are in flight while
// the matrix cores work on the current one (one barrier per K step). LDS rows
// are XOR-swizzled in 16-byte chunks so the 64 lanes of an operand read hit
// distinct banks.
//
// Fused prologue/epilogue (the block's elementwise work never makes its own
// pass over HBM):
//  - norm fold (NORM): the A operand is x * g and each thread accumulates the
//    sum of squares of the raw rows it stages; the epilogue multiplies the
//    fp32 accumulator by rstd = 1/sqrt(mean(x^2) + eps). Since diag(rstd)
//    commutes with the product this is RMSNorm(x; g) W^T exactly (up to
//    rounding order) — RMSNorm with gain as in the chenyuan1125.github.io
//    LLaMA page ("An Architecture Recipe ..." equation).
//  - APAIR: the A operand is carried as bf16 hi + lo (two matrix-core passes
//    into the same accumulator), exact to ~2^-16 relative.
//  - EPI_QKV: RoPE of q and k in registers (pair partner in the neighbouring
//    lane), hi/lo split, v stored transposed per head for the attention kernel.
//  - EPI_SILU: B rows interleave W_gate and W_up in blocks of 32, so one lane
//    holds gate and up of the same output; u = SiLU(gate) * up.
//  - EPI_RESID: C = R + acc (the pre-norm skip connection).
#pragma once

#include "common.h"
#include "internal.h"

namespace llama {

template <int BN, int ASRC, bool APAIR, bool NORM, int EPI>
struct GemmCfg {
  static constexpr int BM = 256;
  static constexpr int BK = APAIR ? 32 : 64;
  static constexpr int CH = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int RPW = 128 / (BK * 2);   // rows per 128-byte bank window
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_VEC = BM * CH / 256;  // 16-byte A vectors per thread per tile
  static constexpr int B_VEC = BN * CH / 256;
  static constexpr int ROWSTEP = 256 / CH;     // row distance between a thread's vectors
  static constexpr int A_TILE = BM * CH;       // in 16-byte units
  static constexpr int B_TILE = BN * CH;
  static constexpr int STAGE = A_TILE * (APAIR ? 2 : 1) + B_TILE;
};

DEV int swz_chunk(int row, int c, int ch, int rpw) { return c ^ ((row / rpw) % ch); }

template <int BN, int ASRC, bool APAIR, bool NORM, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const GemmArgs a) {
  using G = GemmCfg<BN, ASRC, APAIR, NORM, EPI>;
  constexpr int BM = G::BM, BK = G::BK, CH = G::CH, RPW = G::RPW;
  __shared__ u32x4 smem[2 * G::STAGE];
  __shared__ float rstd_s[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;

  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const int nb = tiles_m * tiles_n;
  const int t = xcd_remap(blockIdx.x, nb);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- per-thread staging coordinates
  const int v_c = tid % CH;          // chunk within the tile row
  const int v_r = tid / CH;          // first row; further rows every ROWSTEP
  // B row pointers (fixed over K)
  const u16 *brow[G::B_VEC];
  bool bvalid[G::B_VEC];
#pragma unroll
  for (int p = 0; p < G::B_VEC; ++p) {
    const int r = v_r + p * G::ROWSTEP;
    const u16 *ptr;
    bvalid[p] = n0 + r < a.N;
    if (a.b_mode == BMODE_GATEUP) {
      const int blk = r >> 5;
      const int row = (n0 >> 1) + (blk >> 1) * 32 + (r & 31);
      ptr = ((blk & 1) ? a.B1 : a.B0) + (int64_t)row * a.K;
    } else if (a.b_mode == BMODE_CONCAT3) {
      const int n = n0 + r, seg = n / a.n_seg;
      const u16 *base = seg == 0 ? a.B0 : (seg == 1 ? a.B1 : a.B2);
      ptr = base + (int64_t)(n - seg * a.n_seg) * a.K;
    } else {
      ptr = a.B0 + (int64_t)(bvalid[p] ? n0 + r : 0) * a.K;
    }
    brow[p] = ptr + v_c * 8;
  }

  float ss[G::A_VEC];
#pragma unroll
  for (int p = 0; p < G::A_VEC; ++p) ss[p] = 0.f;

  // raw staging registers
  constexpr int AW = (ASRC == ASRC_F32) ? 2 : 1;  // u32x4 per A vector
  u32x4 ra[G::A_VEC][AW];
  u32x4 ra_lo[ASRC == ASRC_BF16PAIR ? G::A_VEC : 1];
  u32x4 rb[G::B_VEC];
  u32x4 rg;  // gain chunk

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int p = 0; p < G::A_VEC; ++p) {
      const int row = m0 + v_r + p * G::ROWSTEP;
      const int k = k0 + v_c * 8;
      if (row < a.M) {
        if (ASRC == ASRC_F32) {
          const u32x4 *src = (const u32x4 *)((const float *)a.A + row * a.lda + k);
          ra[p][0] = src[0];
          ra[p][AW - 1] = src[1];
        } else {
          ra[p][0] = *(const u32x4 *)((const u16 *)a.A + row * a.lda + k);
          if (ASRC == ASRC_BF16PAIR) ra_lo[p] = *(const u32x4 *)(a.A_lo + row * a.lda + k);
        }
      } else {
#pragma unroll
        for (int w = 0; w < AW; ++w) ra[p][w] = u32x4{0, 0, 0, 0};
        if (ASRC == ASRC_BF16PAIR) ra_lo[p] = u32x4{0, 0, 0, 0};
      }
    }
    if (NORM) rg = *(const u32x4 *)(a.gain + k0 + v_c * 8);
#pragma unroll
    for (int p = 0; p < G::B_VEC; ++p)
      rb[p] = bvalid[p] ? *(const u32x4 *)(brow[p] + k0) : u32x4{0, 0, 0, 0};
  };

  auto store_tile = [&](int buf) {
    u32x4 *sa = smem + buf * G::STAGE;
    u32x4 *sa_lo = sa + G::A_TILE;
    u32x4 *sb = sa + G::A_TILE * (APAIR ? 2 : 1);
    float gf[8];
    if (NORM) unpack8(rg, gf);
#pragma unroll
    for (int p = 0; p < G::A_VEC; ++p) {
      const int r = v_r + p * G::ROWSTEP;
      const int off = r * CH + swz_chunk(r, v_c, CH, RPW);
      if (ASRC == ASRC_BF16PAIR) {
        sa[off] = ra[p][0];
        sa_lo[off] = ra_lo[p];
        continue;
      }
      if (ASRC == ASRC_BF16 && !NORM && !APAIR) {
        sa[off] = ra[p][0];
        continue;
      }
      float f[8];
      if (ASRC == ASRC_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = __uint_as_float(ra[p][0][i]);
          f[4 + i] = __uint_as_float(ra[p][AW - 1][i]);
        }
      } else {
        unpack8(ra[p][0], f);
      }
      if (NORM) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += f[i] * f[i];
        ss[p] += s;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] *= gf[i];
      }
      if (APAIR) {
        u32x4 hi, lo;
        pack8_pair(f, hi, lo);
        sa[off] = hi;
        sa_lo[off] = lo;
      } else {
        sa[off] = pack8(f);
      }
    }
#pragma unroll
    for (int p = 0; p < G::B_VEC; ++p) {
      const int r = v_r + p * G::ROWSTEP;
      sb[r * CH + swz_chunk(r, v_c, CH, RPW)] = rb[p];
    }
  };

  f32x16 acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int buf) {
    const u32x4 *sa = smem + buf * G::STAGE;
    const u32x4 *sa_lo = sa + G::A_TILE;
    const u32x4 *sb = sa + G::A_TILE * (APAIR ? 2 : 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + g;
      bf16x8 bfr[G::TN];
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int r = wn * G::WN + j * 32 + l32;
        bfr[j] = as_bf16x8(sb[r * CH + swz_chunk(r, c, CH, RPW)]);
      }
#pragma unroll
      for (int i = 0; i < G::TM; ++i) {
        const int r = wm * G::WM + i * 32 + l32;
        const int off = r * CH + swz_chunk(r, c, CH, RPW);
        const bf16x8 af = as_bf16x8(sa[off]);
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma32(af, bfr[j], acc[i][j]);
        if (APAIR) {
          const bf16x8 al = as_bf16x8(sa_lo[off]);
#pragma unroll
          for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma32(al, bfr[j], acc[i][j]);
        }
      }
    }
  };

  const int nk = a.K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
    compute(kt & 1);
    if (kt + 1 < nk) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // ---- row statistics of the norm fold
  if (NORM) {
#pragma unroll
    for (int p = 0; p < G::A_VEC; ++p) {
      float s = ss[p];
#pragma unroll
      for (int o = 1; o < CH; o <<= 1) s += __shfl_xor(s, o, 64);
      if (v_c == 0) rstd_s[v_r + p * G::ROWSTEP] = rstd_of(s, a.K, a.eps);
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = rq * 4 + rr;
        const int lrow = wm * G::WM + i * 32 + 8 * rq + 4 * g + rr;
        const int row = m0 + lrow;
        const float sc = NORM ? rstd_s[lrow] : 1.0f;
        if (EPI == EPI_SILU) {
#pragma unroll
          for (int j = 0; j < G::TN; j += 2) {
            const float gt = acc[i][j][r] * sc, up = acc[i][j + 1][r] * sc;
            const float u = silu(gt) * up;
            const int col = (n0 >> 1) + wn * (G::WN / 2) + (j >> 1) * 32 + l32;
            if (row < a.M) {
              u16 hi = f2bf(u);
              ((u16 *)a.C)[(int64_t)row * a.ldc + col] = hi;
              if (a.C_lo) a.C_lo[(int64_t)row * a.ldc + col] = f2bf(u - bf2f(hi));
            }
          }
        } else if (EPI == EPI_QKV) {
          const int seg = n0 / a.dim;  // uniform per workgroup (dim % BN == 0)
#pragma unroll
          for (int j = 0; j < G::TN; ++j) {
            const int col = n0 + wn * G::WN + j * 32 + l32;
            const int cd = col - seg * a.dim;
            const int hh = cd / a.head_dim, e = cd - hh * a.head_dim;
            float v = acc[i][j][r] * sc;
            const int b = row / a.seq, s = row - b * a.seq;
            if (seg < 2) {
              const float partner = __shfl_xor(v, 1, 64);
              if (row < a.M) {
                const float2 cs = a.rope_tab[s * (a.head_dim >> 1) + (e >> 1)];
                v = (e & 1) ? partner * cs.y + v * cs.x : v * cs.x - partner * cs.y;
              }
            }
            if (row < a.M) {
              u16 hi, lo;
              split_pair(v, hi, lo);
              if (seg < 2) {
                const int64_t o = (int64_t)row * a.dim + cd;
                (seg == 0 ? a.qh : a.kh)[o] = hi;
                (seg == 0 ? a.ql : a.kl)[o] = lo;
              } else {
                const int64_t o = (((int64_t)b * a.n_heads + hh) * a.head_dim + e) * a.vt_stride + s;
                a.vth[o] = hi;
                a.vtl[o] = lo;
              }
              if (seg > 0 && a.kcache) {
                const int64_t o = (((int64_t)b * a.n_heads + hh) * a.max_seq + s) * a.head_dim + e;
                (seg == 1 ? a.kcache : a.vcache)[o] = hi;
              }
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < G::TN; ++j) {
            const int col = n0 + wn * G::WN + j * 32 + l32;
            if (row >= a.M || col >= a.N) continue;
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
}

template <int BN, int ASRC, bool APAIR, bool NORM, int EPI>
hipError_t gemm_launch_t(const GemmArgs &a, hipStream_t s) {
  using G = GemmCfg<BN, ASRC, APAIR, NORM, EPI>;
  const int nb = ((a.M + G::BM - 1) / G::BM) * ((a.N + BN - 1) / BN);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BN, ASRC, APAIR, NORM, EPI>), dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace llama

#define GEMM_CASE(BN_, ASRC_, APAIR_, NORM_, EPI_)                                                \
  if (key.bn == BN_ && key.asrc == ASRC_ && key.apair == APAIR_ && key.norm == NORM_ &&          \
      key.epi == EPI_)                                                                            \
    return gemm_launch_t<BN_, ASRC_, APAIR_, NORM_, EPI_>(a, s);
