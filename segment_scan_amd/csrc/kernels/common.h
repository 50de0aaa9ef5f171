// common.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix products run on the CDNA4 matrix cores with
// v_mfma_f32_32x32x16_bf16 (wave64; A 32x16, B 16x32, fp32 accumulate 32x32).
// fp32 operands are fed as sums of bf16 terms ("split-bf16"): x = t0 + t1 (+ t2),
// each term the round-to-nearest-even bf16 of the remaining residual.  A
// product of an NA-term by an NB-term operand keeps the term pairs with
// i + j < max(NA, NB), which drops only products below the last kept term's
// precision: 1 term ~ 2^-9, 2 terms ~ 2^-17, 3 terms ~ 2^-25 relative.
//
// Register layout of one 32x32 fp32 accumulator tile (f32x16 per lane):
//   lane l holds column (l & 31); element r holds row
//   8*(r >> 2) + 4*(l >> 5) + (r & 3).
// Operand layout of one MFMA step (8 bf16 per lane):
//   A (32 rows x 16 k): lane l holds row (l & 31), k = 8*(l >> 5) + j, j = 0..7
//   B (16 k x 32 cols): lane l holds col (l & 31), k = 8*(l >> 5) + j.
// The k order only has to agree between A and B, which lets an accumulator
// tile be reused as a B operand without moving data: elements 8m .. 8m+7 of a
// tile hold, for lane half h = l >> 5, the tile rows
//   16m + 8*(j >> 2) + 4h + (j & 3),  j = 0..7,
// so the matching A operand reads those k indices (two runs of 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hypic {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef _Float16 f16_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A copy of `x` the optimiser cannot see through.  Per-lane indices are taken
// through this at the top of a long loop so that values derived from them
// (addresses, masks) are recomputed where used instead of being hoisted out of
// the loop and kept live -- in the kernels that hold a large state in
// registers that hoisting costs more registers than it saves instructions.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
// The wave index as a wave-uniform (scalar) value, for branches and addresses
// the compiler must know to be uniform.
__device__ __forceinline__ int wave_id_uniform() { return __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6; }

// Raw buffer resource over `bytes` bytes from `p` (gfx9 word 3: 32-bit data
// format, no swizzle, no index stride).  A buffer load whose offset lies at or
// past `bytes` returns zeros and touches no memory, so ragged tails need no
// branch or clamp.  Offsets are 32-bit: voffset per lane plus soffset per wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t buffer_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Compiler-only fence: memory operations are not moved across it.  Used inside
// unrolled MFMA loops to bound how far ahead LDS fragments are loaded (and so
// how many registers they hold).
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of accumulator element r for this lane (column is lane & 31).
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// NT-term bf16 operand fragment.
template <int NT>
struct Frag {
  bf16x8 t[NT];
};

// Split 8 fp32 values into NT bf16 terms.
template <int NT>
__device__ __forceinline__ Frag<NT> split8(const float (&x)[8]) {
  Frag<NT> f;
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = x[j];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16_t h = (bf16_t)r[j];
      f.t[i][j] = h;
      if (i + 1 < NT) r[j] -= (float)h;
    }
  }
  return f;
}

// Elements 8m .. 8m+7 of an accumulator tile as an NT-term B fragment.
template <int NT>
__device__ __forceinline__ Frag<NT> acc_as_b(const f32x16& acc, int m, float scale = 1.f) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = acc[8 * m + j] * scale;
  return split8<NT>(x);
}

// acc += A * B with split operands (small products first).
template <int NA, int NB>
__device__ __forceinline__ void mma(f32x16& acc, const Frag<NA>& a, const Frag<NB>& b) {
  constexpr int N = NA > NB ? NA : NB;
#pragma unroll
  for (int s = N - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int j = s - i;
      if (j >= 0 && j < NB) acc = mfma32(a.t[i], b.t[j], acc);
    }
  }
}

// bf16 bit patterns <-> float.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Load 8 consecutive input elements (bf16 or fp32) as floats.
template <bool IN_F32>
__device__ __forceinline__ void load8(const void* base, size_t idx, float (&x)[8]) {
  if constexpr (IN_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + idx);
    f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}

template <bool IN_F32>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  if constexpr (IN_F32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  }
}

// Maximum across the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// The same with DPP moves inside each 16-lane row (swap neighbours, swap
// pairs, mirror within 8, mirror within 16) and the four row maxima read into
// scalar registers: no LDS traffic.  The result is wave-uniform.
// x of lane + N within the lane's row of 16 (0 where that is past the row)
template <int N>
__device__ __forceinline__ float dpp_row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}

__device__ __forceinline__ float dpp_max_step(float x, int ctrl_sel) {
  int y;
  const int xi = __builtin_bit_cast(int, x);
  switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: y = __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    case 2: y = __builtin_amdgcn_mov_dpp(xi, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_mov_dpp(xi, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return fmaxf(x, __builtin_bit_cast(float, y));
}
__device__ __forceinline__ float wave_max_uniform(float x) {
  x = dpp_max_step(x, 0);
  x = dpp_max_step(x, 1);
  x = dpp_max_step(x, 2);
  x = dpp_max_step(x, 3);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Power-of-two scaling of an fp16 operand block whose largest magnitude is m:
// returns the exponent e such that the block is converted as x * 2^-e.  Blocks
// already inside [2^-6, 2^12] are left unscaled (e = 0): there every value that
// matters to the block's norm is a normal fp16 number with headroom for the
// products it feeds; otherwise the largest magnitude is mapped into [2^11, 2^12).
__device__ __forceinline__ int f16_scale_exp(float m) {
  if (!(m > 0.f) || (m >= 0x1p-6f && m <= 0x1p12f)) return 0;
  int e;
  frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
  return e - 12;
}

// Two 8-byte LDS reads (k = off .. off+3 and off+8 .. off+11) joined into one
// A fragment: the k order that matches an accumulator tile used as B (see the
// layout notes at the top).  `p` already holds the lane's row and 4*(lane >> 5) offset, so
// every address is a base register plus an immediate.
template <int NT>
__device__ __forceinline__ Frag<NT> lds_a_perm(const bf16_t* p, int term_stride, int off) {
  Frag<NT> f;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + i * term_stride + off);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + i * term_stride + off + 8);
    f.t[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  return f;
}

// Standard-order fragment: 8 consecutive k starting at `off` (two 8-byte reads).
template <int NT>
__device__ __forceinline__ Frag<NT> lds_frag(const bf16_t* p, int term_stride, int off) {
  Frag<NT> f;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + i * term_stride + off);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + i * term_stride + off + 4);
    f.t[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  return f;
}

__device__ __forceinline__ void st8(bf16_t* p, const bf16x8& v) {
  *reinterpret_cast<bf16x4*>(p) = __builtin_shufflevector(v, v, 0, 1, 2, 3);
  *reinterpret_cast<bf16x4*>(p + 4) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}

// ---- (I + M)^-1 of the two 32 x 32 diagonal blocks of a 64 x 64 array -----------
// M strictly lower triangular in sM (fp32, pitch P floats, P % 4 == 0, rows
// 16-byte aligned); on return the two diagonal 32 x 32 blocks hold N_bb =
// (I + M_bb)^-1 in full (ones on the diagonal, zeros above), the rest of sM
// untouched.  Run by one whole wave, with no workgroup barrier inside (the
// caller orders it against other waves).  Each 32-block is split in two:
//   the four 16 x 16 diagonal blocks by forward substitution, lane 16 q + c
//   owning column c of block q (rows of M read as LDS broadcasts, only entries
//   below the diagonal);
//   the off-diagonal 16 x 16 block of each 32-block, N_10 = -N_11 (M_10 N_00),
//   as two 16x16x16 bf16 MFMA products with both operands split into two
//   terms (about 2^-16 relative), the first product's result feeding the
//   second from registers.
// (16x16x16 layout: lane l holds A[l % 16][4 (l / 16) + j], B[4 (l / 16) + j][l % 16]
// and D[4 (l / 16) + j][l % 16], j = 0..3.)
__device__ __forceinline__ void bf16_split4(const float (&x)[4], bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[j] = (bf16_t)x[j];
    lo[j] = (bf16_t)(x[j] - (float)hi[j]);
  }
}
__device__ __forceinline__ f32x4 mma16_split(const float (&a)[4], const float (&b)[4], f32x4 c) {
  bf16x4 ah, al, bh, bl;
  bf16_split4(a, ah, al);
  bf16_split4(b, bh, bl);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
}
// The wave's LDS operations issued so far have completed (lgkmcnt(0) alone:
// the gfx9 s_waitcnt field layout, vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void inv_diag32_blocks(float* sM, int P, int lane) {
  {  // 16 x 16 diagonal blocks
    const int q = lane >> 4, c = lane & 15;
    const float* Mb = sM + 16 * q * P + 16 * q;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc0 = 0.f, acc1 = 0.f;
      const float* Mr = Mb + r * P;
#pragma unroll
      for (int k4 = 0; k4 < r / 4; ++k4) {
        const f32x4 m4 = *reinterpret_cast<const f32x4*>(Mr + 4 * k4);
        acc0 = fmaf(m4[0], x[4 * k4], acc0);
        acc1 = fmaf(m4[1], x[4 * k4 + 1], acc1);
        acc0 = fmaf(m4[2], x[4 * k4 + 2], acc0);
        acc1 = fmaf(m4[3], x[4 * k4 + 3], acc1);
      }
#pragma unroll
      for (int k = r & ~3; k < r; ++k) acc0 = fmaf(Mr[k], x[k], acc0);
      x[r] = (r < c) ? 0.f : ((r == c) ? 1.f : -(acc0 + acc1));
    }
    wave_lds_sync();  // every lane has read its block of M
    float* Nb = sM + 16 * q * P + 16 * q;
#pragma unroll
    for (int r = 0; r < 16; ++r) Nb[r * P + c] = x[r];
    // the upper-right 16 x 16 block of each 32-block is zero: lane 32 b + 16 h + c
    // clears rows 32 b + 8 h .. + 7, column 32 b + 16 + c
    const int b = lane >> 5, h = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 8; ++r) sM[(32 * b + 8 * h + r) * P + 32 * b + 16 + c] = 0.f;
  }
  wave_lds_sync();
  const int i16 = lane & 15, k4 = 4 * (lane >> 4);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int o = 32 * b;
    float a[4], bb[4], p[4];
    const f32x4 m10 = *reinterpret_cast<const f32x4*>(sM + (o + 16 + i16) * P + o + k4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = m10[j];
      bb[j] = sM[(o + k4 + j) * P + o + i16];  // N_00
    }
    const f32x4 P10 = mma16_split(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});  // M_10 N_00
    const f32x4 n11 = *reinterpret_cast<const f32x4*>(sM + (o + 16 + i16) * P + o + 16 + k4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = n11[j];
      p[j] = P10[j];
    }
    const f32x4 Q = mma16_split(a, p, f32x4{0.f, 0.f, 0.f, 0.f});  // N_11 (M_10 N_00)
    wave_lds_sync();  // every lane has read M_10
#pragma unroll
    for (int j = 0; j < 4; ++j) sM[(o + 16 + k4 + j) * P + o + i16] = -Q[j];
  }
  wave_lds_sync();
}

// LDS tile of bf16 with 64 columns (128 B rows), 16-byte column chunks
// XOR-swizzled by (row & 7) ^ ((row >> 3) & 7): 8 consecutive rows read at the
// same logical chunk hit distinct banks, and so do rows 8 apart (a transposed
// write of one channel from 8 channel blocks).
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * 64 + ((chunk ^ (row & 7) ^ ((row >> 3) & 7)) << 3);
}

}  // namespace hypic
