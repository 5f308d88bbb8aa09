// Causal flash-style attention for prefill on gfx950 matrix cores.
//
// Per (sequence, head, 128-query tile) one workgroup of 4 wavefronts; each
// wavefront owns 32 queries. Keys/values stream through LDS in tiles of 64.
// The product is formed transposed — S^T = K Q^T and O^T = V^T P^T — so that in
// the 32x32 accumulator layout every lane holds values of ONE query (its lane
// index mod 32): the running max, the running sum and the rescaling of O stay
// in that lane's registers, and the only cross-lane step is one exchange
// between the two 32-lane halves. Keys are read from LDS in a permuted order
// (bits 2 and 3 of the key index swapped) so that the probabilities a lane
// holds after the S^T product are exactly the eight consecutive keys it must
// supply as the P^T operand of the next product: no register shuffles.
//
// Softmax is online in fp32 with exp2 and a log2(e)/sqrt(hd) prescale; masked
// keys get exactly zero weight; tiles entirely above the diagonal are never
// loaded and fully masked 32-key halves are skipped per wavefront. q/k and v
// can be carried as bf16 hi/lo pairs (3 and 2 matrix-core passes).
//
// Attention itself is the 2017 scaled-dot-product attention with a causal mask
// (paperfordummies.in LLaMA page, "LLaMA is a pull request against the 2017
// transformer": the attention is untouched; RoPE is applied to q and k before).
#include "common.h"
#include "internal.h"

namespace llama {

DEV int perm23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// LDS chunk swizzles (gfx950 serves a 16-byte read 16 lanes per pass over a
// 256-byte bank window): rows of 256 bytes XOR the chunk with row mod 16, rows
// of 128 bytes with (row / 2) mod 8, so any 16 consecutive rows read at one
// logical chunk hit 16 distinct 16-byte slots.
template <int CHUNKS>
DEV int rswz(int row) { return CHUNKS == 16 ? (row & 15) : ((row >> 1) & 7); }

template <int HD, bool QKPAIR, bool VPAIR>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(const AttnArgs a) {
  constexpr int KT = 64;            // keys per tile
  constexpr int KCH = HD / 8;       // 16-byte chunks per K row
  constexpr int NKK = HD / 16;      // k-steps of the score product
  constexpr int NEB = HD / 32;      // 32-wide blocks of the head dimension
  constexpr int KTILE = KT * KCH;   // u32x4 per K tile
  constexpr int VTILE = HD * 8;     // u32x4 per V^T tile (8 chunks of 8 keys)
  __shared__ u32x4 sk[KTILE], skl[QKPAIR ? KTILE : 1], sv[VTILE], svl[VPAIR ? VTILE : 1];

  const int S = a.seq;
  const int nqt = (S + 127) / 128;
  const int qt = nqt - 1 - blockIdx.x;  // longest (most keys) first
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int q0 = qt * 128;
  const int qi = q0 + 32 * w + l32;          // this lane's query
  const int qwave_max = q0 + 32 * w + 31;
  const int64_t tok0 = (int64_t)b * S;

  // q fragments (B operand of S^T = K Q^T): q[qi][16kk + 8g .. +7]
  bf16x8 qh[NKK], ql[QKPAIR ? NKK : 1];
  {
    const int64_t base = (tok0 + qi) * a.dim + h * HD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
      if (qi < S) {
        v = *(const u32x4 *)(a.qh + base + 16 * kk);
        if (QKPAIR) vl = *(const u32x4 *)(a.ql + base + 16 * kk);
      }
      qh[kk] = as_bf16x8(v);
      if (QKPAIR) ql[kk] = as_bf16x8(vl);
    }
  }

  f32x16 acc_o[NEB];
#pragma unroll
  for (int e = 0; e < NEB; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[e][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  const int kend = min(S, q0 + 128);
  const int n_kt = (kend + KT - 1) / KT;
  const int64_t vbase = ((int64_t)b * a.n_heads + h) * HD * a.vt_stride;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int kt0 = kt * KT;
    __syncthreads();
    // ---- stage K (and lo) rows and V^T (and lo) rows of this key tile
#pragma unroll
    for (int p = 0; p < KTILE / 256; ++p) {
      const int idx = tid + p * 256;
      const int row = idx / KCH, ch = idx % KCH;
      const int key = kt0 + row;
      u32x4 v = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
      if (key < S) {
        const int64_t o = (tok0 + key) * a.dim + h * HD + ch * 8;
        v = *(const u32x4 *)(a.kh + o);
        if (QKPAIR) vl = *(const u32x4 *)(a.kl + o);
      }
      const int so = row * KCH + (ch ^ rswz<KCH>(row));
      sk[so] = v;
      if (QKPAIR) skl[so] = vl;
    }
#pragma unroll
    for (int p = 0; p < VTILE / 256; ++p) {
      const int idx = tid + p * 256;
      const int e = idx >> 3, ch = idx & 7;
      const int key = kt0 + ch * 8;
      u32x4 v = {0, 0, 0, 0}, vl = {0, 0, 0, 0};
      const int64_t o = vbase + (int64_t)e * a.vt_stride + key;
      if (key + 8 <= S) {
        v = *(const u32x4 *)(a.vth + o);
        if (VPAIR) vl = *(const u32x4 *)(a.vtl + o);
      } else if (key < S) {
        uint32_t hv[8], lv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hv[i] = key + i < S ? a.vth[o + i] : 0;
          lv[i] = (VPAIR && key + i < S) ? a.vtl[o + i] : 0;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = hv[2 * i] | (hv[2 * i + 1] << 16);
          vl[i] = lv[2 * i] | (lv[2 * i + 1] << 16);
        }
      }
      const int so = e * 8 + (ch ^ rswz<8>(e));
      sv[so] = v;
      if (VPAIR) svl[so] = vl;
    }
    __syncthreads();

    // ---- scores S^T for the two 32-key halves
    f32x16 s[2];
    bool live[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      live[t] = kt0 + 32 * t <= qwave_max && kt0 + 32 * t < S;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
      if (!live[t]) continue;
      const int krow = 32 * t + perm23(l32);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int so = krow * KCH + ((2 * kk + g) ^ rswz<KCH>(krow));
        const bf16x8 kf = as_bf16x8(sk[so]);
        s[t] = mfma32(kf, qh[kk], s[t]);
        if (QKPAIR) {
          s[t] = mfma32(as_bf16x8(skl[so]), qh[kk], s[t]);
          s[t] = mfma32(kf, ql[kk], s[t]);
        }
      }
    }

    // ---- online softmax (fp32); lane holds keys of query qi
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + 32 * t + 16 * ((r >> 2) >> 1) + 8 * g + 4 * ((r >> 2) & 1) + (r & 3);
        const bool ok = live[t] && key <= qi && key < S;
        s[t][r] = ok ? s[t][r] : -INFINITY;
        mx = fmaxf(mx, s[t][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f((m_run - m_use) * c);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f((s[t][r] - m_use) * c);   // exp2(-inf) = 0 for masked keys
        s[t][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int e = 0; e < NEB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[e][r] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (!live[t]) continue;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = s[t][8 * s2 + i];
        const bf16x8 pf = as_bf16x8(pack8(pv));
        const int ch = 4 * t + 2 * s2 + g;
#pragma unroll
        for (int e = 0; e < NEB; ++e) {
          const int row = 32 * e + l32;
          const int so = row * 8 + (ch ^ rswz<8>(row));
          acc_o[e] = mfma32(as_bf16x8(sv[so]), pf, acc_o[e]);
          if (VPAIR) acc_o[e] = mfma32(as_bf16x8(svl[so]), pf, acc_o[e]);
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

template <int HD, bool QKPAIR, bool VPAIR>
static hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
  dim3 grid((a.seq + 127) / 128, a.n_heads, a.batch);
  hipLaunchKernelGGL((attn_prefill_kernel<HD, QKPAIR, VPAIR>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t attn_prefill_launch(const AttnArgs &a, int qk_pair, int v_pair, hipStream_t s) {
  if (a.batch * a.seq == 0) return hipSuccess;
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
