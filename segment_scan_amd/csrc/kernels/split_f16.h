// split_f16.h -- fp32 values as sums of fp16 terms for the matrix cores, and
// the split-operand products (shared by the dense chain kernel and the fused
// composition of the delta build).
//
// An fp32 operand enters a 16-bit MFMA as N fp16 terms: each term the nearest
// fp16 of what the earlier terms leave, after scaling the block by a power of
// two.  Two terms carry about 2^-22 of the value; the products keep the term
// pairs i + j < N (the rest is below the fp32 accumulation's own rounding).
#pragma once

#include "common.h"

namespace hypic {

// power-of-two exponent that maps a block maximum m into [2^14, 2^15)
__device__ __forceinline__ int split_exp(float m) {
  if (!(m > 0.f)) return 0;
  int e;
  frexpf(m, &e);
  return e - 15;
}

// NT fp16 terms of an operand fragment
template <int N>
struct HFrag {
  f16x8 t[N];
};

// 8 values (already scaled) as N fp16 terms, each the nearest fp16 of the
// remaining residual (the residuals are exact in fp32)
template <int N>
__device__ __forceinline__ HFrag<N> split8h(const float (&x)[8]) {
  HFrag<N> f;
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = x[j];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16_t t = (f16_t)r[j];
      f.t[i][j] = t;
      if (i + 1 < N) r[j] -= (float)t;
    }
  }
  return f;
}

// x s rounded to fp32 and hidden from the optimiser.  The leading fp16 term of
// a split is the fp16 rounding of this value, and the residual is taken from the
// exact product with one fused multiply-add; left visible, the product may be
// fused into one use of the term (an fp16 conversion of the exact product) and
// not into another (fp16 of the fp32 product), and where the two roundings
// differ the stored term and the residual disagree by an fp16 ulp.
__device__ __forceinline__ float mul_opaque(float x, float s) {
  float p = x * s;
  asm volatile("" : "+v"(p));
  return p;
}

// The same for x s with s a power of two, exponent within fp32's normal range:
// t0 = fp16(x s) and every residual exact in fp32 (each step one fused
// multiply-add with an fp16 operand)
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
// fp16 of two products x s, one conversion instruction for the pair
__device__ __forceinline__ f16x2_t cvt2h_scaled(float x0, float x1, float s) {
  return __builtin_convertvector((f32x2_t){mul_opaque(x0, s), mul_opaque(x1, s)}, f16x2_t);
}

template <int N>
__device__ __forceinline__ HFrag<N> split8h_scaled(const float (&x)[8], float s) {
  HFrag<N> f;
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const f16x2_t t = cvt2h_scaled(x[j], x[j + 1], s);
    f.t[0][j] = t[0];
    f.t[0][j + 1] = t[1];
    if (N > 1) {
      r[j] = __builtin_fmaf(x[j], s, -(float)t[0]);
      r[j + 1] = __builtin_fmaf(x[j + 1], s, -(float)t[1]);
    }
  }
#pragma unroll
  for (int i = 1; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16_t t = (f16_t)r[j];
      f.t[i][j] = t;
      if (i + 1 < N) r[j] -= (float)t;
    }
  }
  return f;
}

// 2^-e as a float, e clamped so that the factor stays a normal number (values
// this far from 1 lose low bits in fp16 instead of overflowing the factor)
__device__ __forceinline__ float pow2_neg(int e) { return ldexpf(1.f, -min(max(e, -100), 100)); }

__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// acc += A B on 32x32x16 fp16 MFMA, term pairs i + j < max(NA, NB), small first
template <int NA, int NB>
__device__ __forceinline__ void mmah(f32x16& acc, const HFrag<NA>& a, const HFrag<NB>& b) {
  constexpr int N = NA > NB ? NA : NB;
#pragma unroll
  for (int s = N - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int j = s - i;
      if (j >= 0 && j < NB) acc = mfma32h(a.t[i], b.t[j], acc);
    }
  }
}

// the same on 16x16x32 fp16 MFMA
template <int NA, int NB>
__device__ __forceinline__ void mmah16(f32x4& acc, const HFrag<NA>& a, const HFrag<NB>& b) {
  constexpr int N = NA > NB ? NA : NB;
#pragma unroll
  for (int s = N - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int j = s - i;
      if (j >= 0 && j < NB) acc = mfma16h(a.t[i], b.t[j], acc);
    }
  }
}

// position of k offset o (0..15) inside its 16-wide block: bits 2 and 3 swapped
__device__ __forceinline__ constexpr int kperm(int o) { return (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1); }

template <int N>
struct H4 {
  f16x4 t[N];
};
// 4 values times s (a power of two) as N fp16 terms, as split8h_scaled
template <int N>
__device__ __forceinline__ H4<N> split4h_scaled(const f32x4& x, float s) {
  H4<N> f;
  float r[4];
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    const f16x2_t t = cvt2h_scaled(x[j], x[j + 1], s);
    f.t[0][j] = t[0];
    f.t[0][j + 1] = t[1];
    if (N > 1) {
      r[j] = __builtin_fmaf(x[j], s, -(float)t[0]);
      r[j + 1] = __builtin_fmaf(x[j + 1], s, -(float)t[1]);
    }
  }
#pragma unroll
  for (int i = 1; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16_t t = (f16_t)r[j];
      f.t[i][j] = t;
      if (i + 1 < N) r[j] -= (float)t;
    }
  return f;
}

__device__ __forceinline__ void buffer_store4(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}

}  // namespace hypic
