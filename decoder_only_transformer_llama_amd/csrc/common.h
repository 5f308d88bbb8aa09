// Device-side helpers shared by the gfx950 kernels: bf16 conversions, the
// hi/lo pair split, vector types of the matrix-core builtins and wavefront
// reductions. Wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

DEV float bf2f(u16 h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
DEV u16 f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(u16, b);
}

// f = hi + lo + O(2^-16 |f|): hi = bf16(f), lo = bf16(f - hi).
DEV void split_pair(float f, u16 &hi, u16 &lo) {
  hi = f2bf(f);
  lo = f2bf(f - bf2f(hi));
}

// Two packed bf16 (low half = first element) from two floats.
DEV uint32_t pack2(float a, float b) { return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16); }

DEV void unpack8(const u32x4 &v, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

DEV u32x4 pack8(const float *f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack2(f[2 * i], f[2 * i + 1]);
  return r;
}

DEV void pack8_pair(const float *f, u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u16 h0, l0, h1, l1;
    split_pair(f[2 * i], h0, l0);
    split_pair(f[2 * i + 1], h1, l1);
    hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
}

DEV bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }
DEV f16x8 as_f16x8(const u32x4 &v) { return __builtin_bit_cast(f16x8, v); }

DEV f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
DEV f32x16 mfma32h(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Eight bf16 values (16 bytes) as eight IEEE fp16 values. Exact for zero and
// for magnitudes in [2^-14, 65504] (fp16 has 3 more significand bits and the
// exponent fits); smaller magnitudes become fp16 subnormals cut to a
// multiple of 2^-24, larger ones +-inf. The conversion truncates, which is
// exact wherever the value is representable.
DEV u32x4 bf16x8_to_f16x8(const u32x4 &v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xffff0000u);
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return r;
}

// fp32 -> IEEE fp16, round to nearest even (overflow gives +-inf).
DEV u16 f2h(float f) { return __builtin_bit_cast(u16, (_Float16)f); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two floats as two packed fp16 (low half = first), the same rounding as
// f2h; one v_cvt_pk_f16_f32 on gfx950.
DEV uint32_t pack2h(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
DEV u32x4 pack8h(const float *f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack2h(f[2 * i], f[2 * i + 1]);
  return r;
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 1 / sqrt(mean + eps) in IEEE fp32 (correctly rounded sqrt and divide).
DEV float rstd_of(float sumsq, int n, float eps) {
  return 1.0f / __fsqrt_rn(sumsq / (float)n + eps);
}

// SiLU(t) = t / (1 + e^-t); e^-t overflows to +inf for very negative t and
// the quotient is then -0, never NaN.
DEV float silu(float t) { return t / (1.0f + expf(-t)); }

// The same function from the hardware exponential and reciprocal
// (v_exp_f32 of -t log2(e), v_rcp_f32; about 3e-7 relative error against the
// correctly rounded quotient), for the GEMM epilogue whose result is rounded
// to fp16 or bf16 right after. Very negative t: 2^(+big) = +inf, 1/inf = 0,
// t * 0 = -0; very positive t: 2^(-big) = 0, t * 1 = t.
DEV float silu_fast(float t) {
  return t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t * -1.4426950408889634f));
}

// Value of the neighbouring lane (lane ^ 1) by a DPP quad permutation [1,0,3,2]
// (no LDS traffic, unlike a generic shuffle).
DEV float lane_swap1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
}

// Round a workgroup count up and remap a linear workgroup id so that ids the
// hardware sends to one XCD (id % 8) get a contiguous range of tiles.
DEV int xcd_remap(int bid, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int x = bid % 8, i = bid / 8;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// 16 bytes per lane from base + voff + soff (bytes) into LDS at lds + 16 * lane:
// buffer_load_dwordx4 ... lds (the LDS address comes from M0, the lane slot
// from the lane index). Offsets are 32-bit: callers keep them small (below a
// tile or one sequence's rows). Used instead of the global form of the same
// load, which the compiler also counts as an outstanding LDS access: every
// LDS operand read would then wait for all loads in flight (lgkmcnt(0)).
DEV void buf_load_lds16(const void *base, uint32_t voff, uint32_t soff, void *lds) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// v, which must already be the same in every lane of the wavefront, as a
// value the compiler knows to be uniform (it is read from the first active
// lane). A buffer load whose base the compiler cannot prove uniform is
// wrapped in a loop over the distinct lane values.
// (The builtin returns a signed int: each half goes back through uint32_t so
// that the low half is zero-extended, not sign-extended, into 64 bits.)
DEV int64_t wave_uniform(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}
template <typename T>
DEV T *wave_uniform(T *p) {
  return (T *)wave_uniform((int64_t)p);
}
