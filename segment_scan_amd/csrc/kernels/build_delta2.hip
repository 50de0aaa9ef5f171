// build_delta2.hip -- delta-rule segment build (DeltaNet, GDN), bf16 tokens,
// d = 128, in two kernels: a per-chunk WY preparation and a per-unit state pass.
//
// [youleyou, linear-layer paragraph] T_C is the ordered product of the
// segment's per-token transitions a_t (I - beta_t k_t k_t^T), kept as exp(g) U,
// and S(C|0) is its final state from a zero start.  The segment is processed in
// 64-token chunks joined by the composition law of the same paragraph; a
// chunk's 64 rank-1 factors are applied in the compact WY/UT form
//   A0 = (I + strict_lower(diag(b) K K^T))^-1 diag(b)
//   U <- U - K^T (A0 (K U))
//   S <- exp(G_C) S + K^T (A0 (diag(exp(G_C - G)) V - exp(G_C) K S))
// (G: inclusive gate prefix within the chunk, G_C its total).  The S update is
// the ungated rule on values exp(-G_t) v_t in the frame scaled by exp(-G),
// moved back by exp(G_C): both halves share A0, and every factor is <= 1.
//
// Nothing in A0 depends on the running state, so the per-chunk factors are a
// separate, fully parallel job:
//  - delta_prep: one wave per (segment, chunk, chain) builds the Gram matrix on
//    MFMA, inverts (I + M) in 32 x 32 blocks (each diagonal block from four
//    16 x 16 forward substitutions in fp32 and 16x16 MFMA products, the
//    off-diagonal block by two MFMA products), and writes A0 (fp16, each row
//    scaled by a power of two) with the gate prefix G to a workspace;
//  - delta_state: one workgroup per (segment, chain) keeps [U | S] in MFMA
//    accumulators (8 waves x 32 columns) and, per chunk, stages K (row-major
//    and transposed), V and A0 in LDS and runs the three products.
// The workspace makes the state pass a plain stream (two barriers per chunk,
// around the staging) and lets the latency-bound inverse hide behind other
// workgroups.
//
// Operands enter the matrix cores as fp16 (fp32 accumulate).  bf16 keys are
// exact in fp16 within its normal range (normalised delta-rule keys are);
// derived operands are rounded once, each block scaled by a power of two
// chosen from its largest magnitude (f16_scale_exp in common.h; A0 per row, the
// state pass's operands per column),
// so only rounding error remains: about 2^-12 per product, near 4e-4 relative
// on 512-token GDN segments.  Longer segments use build_delta.hip.
#include "common.h"
#include "split_f16.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int D = 128;
constexpr int C = 64;
constexpr int KP = D + 4;  // 16-bit pitch of K [t][d] (fp16) and V [t][d] (bf16)
constexpr int TP = C + 4;  // 16-bit pitch of K^T [d][t] and of A [t][t'] (fp16)

// Workspace record of one (chunk, chain): A0 (fp16, scaled rows), the row
// scales (2^e as float) and the inclusive gate prefix G.
constexpr int REC_A = 0;
constexpr int REC_RS = C * C * 2;
constexpr int REC_G = REC_RS + C * 4;
constexpr int REC_BYTES = REC_G + C * 4;


__device__ __forceinline__ uint32_t pk_f16_from_bf16x2(uint32_t w) {
  // exact conversion of two bf16 values, so the packing rounding mode is irrelevant
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)));
}

// A fragment in the accumulator-as-B k order (see common.h): k = off + {0..3}, off + 8 + {0..3}.
__device__ __forceinline__ f16x8 lds_a_perm_h(const f16_t* p, int off) {
  const f16x4 lo = *reinterpret_cast<const f16x4*>(p + off);
  const f16x4 hi = *reinterpret_cast<const f16x4*>(p + off + 8);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Elements 8m .. 8m+7 of an accumulator tile, times s, as an fp16 B fragment
// (s is the power-of-two scale of the lane's column: lanes l and l ^ 32 agree).
__device__ __forceinline__ f16x8 acc_as_b_h(const f32x16& acc, int m, float s) {
  f16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (f16_t)(acc[8 * m + j] * s);
  return f;
}
// The same for s = 1 (NEG: s = -1): the conversion alone, the sign a source
// modifier.  Blocks whose power-of-two scale is 1 -- the usual case -- take it.
template <bool NEG>
__device__ __forceinline__ f16x8 acc_as_b_unit(const f32x16& acc, int m) {
  f16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (f16_t)(NEG ? -acc[8 * m + j] : acc[8 * m + j]);
  return f;
}

// Largest magnitude over the accumulator column that lanes l and l ^ 32 hold
// together (as a B operand a column spans both halves of the wave, so its two
// lanes must agree on one scale).  m >= 0: bit patterns order like the values.
// xaddr = 4 (lane ^ 32).
__device__ __forceinline__ float pair_max(float m, int xaddr) {
  const unsigned a = __float_as_uint(m);
  const unsigned b = (unsigned)__builtin_amdgcn_ds_bpermute(xaddr, (int)a);
  return __uint_as_float(a > b ? a : b);
}
__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// =====================================================================================
// delta_prep: per (chunk, chain) A0 = (I + strict_lower(diag(b) K K^T))^-1 diag(b)
// =====================================================================================

// One wave per (chunk, chain): no barriers between its phases, and several
// independent waves per SIMD to hide each one's latencies.
constexpr int MP = C + 4;  // fp32 pitch of the M / A0 work array (16-byte rows)

__global__ __launch_bounds__(64, 2) void delta_prep_kernel(const BuildArgs a, const ChunkTable cks, unsigned char* ws) {
  __shared__ __attribute__((aligned(16))) float sM[C * MP];
  __shared__ float sBeta[C];

  // workgroup -> (chunk of the launch, chain): consecutive workgroups take the
  // chains of one chunk, which share the rows of the token-major inputs
  const int n_chain = a.n_chain;
  const int gchunk = blockIdx.x / n_chain, chain = blockIdx.x % n_chain;
  int lo = 0, hi = a.seg.n_seg;  // segment: last s with base[s] <= gchunk (uniform search)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cks.base[mid] <= gchunk) lo = mid; else hi = mid;
  }
  const int c0 = a.seg.beg[lo] + (gchunk - cks.base[lo]) * C;
  const int nv = min(C, a.seg.end[lo] - c0);
  const int lane = threadIdx.x;
  const int h = lane >> 5, l32 = lane & 31;

  // ---- the chunk's keys (bf16 rows, into LDS in the space M takes later), and
  // weight and gate of token lane: all loads issued before any is waited on.
  // Instruction i loads rows 4i .. 4i + 3 whole (lane l: row 4i + l / 16, channels
  // 8 (l % 16) ..); buffer loads over the chunk's valid tokens read zeros past them.
  constexpr int KSP = D + 8;  // 16-bit pitch of the staged rows (272 bytes)
  static_assert(C * KSP * 2 <= C * MP * 4, "key staging fits in the M array");
  bf16_t* sKs = reinterpret_cast<bf16_t*>(sM);
  const size_t e0 = (size_t)c0 * n_chain + chain;  // element (token c0, chain)
  uint4 kr[C / 4];
  {
    const uint32_t row_bytes = (uint32_t)n_chain * D * 2;
    const __amdgpu_buffer_rsrc_t rk =
        buffer_rsrc(reinterpret_cast<const char*>(a.k) + e0 * D * 2, (uint32_t)(nv - 1) * row_bytes + D * 2);
    const uint32_t vo = (uint32_t)(lane >> 4) * row_bytes + (lane & 15) * 16;
#pragma unroll
    for (int i = 0; i < C / 4; ++i) kr[i] = buffer_load16(rk, vo, 4 * i * row_bytes);
  }
  const uint32_t sb = (uint32_t)(nv - 1) * n_chain * 2 + 2, so = (uint32_t)lane * n_chain * 2;
  const float beta =
      __uint_as_float((uint32_t)buffer_load2(buffer_rsrc(reinterpret_cast<const char*>(a.beta) + e0 * 2, sb), so, 0)
                      << 16);
  const float lg =
      a.lg ? __uint_as_float((uint32_t)buffer_load2(buffer_rsrc(reinterpret_cast<const char*>(a.lg) + e0 * 2, sb), so, 0)
                             << 16)
           : 0.f;
  // ---- per-token scalars: lane t holds token t; gate prefix by a wave scan --------
  const float G = wave_incl_scan(lg);
  sBeta[lane] = beta;
#pragma unroll
  for (int i = 0; i < C / 4; ++i)
    *reinterpret_cast<uint4*>(sKs + (4 * i + (lane >> 4)) * KSP + 8 * (lane & 15)) = kr[i];
  __syncthreads();

  // ---- Gram K K^T on bf16 MFMA (exact products) ------------------------------------
  // A and B fragments of a 32-token block are the same registers: lane l holds
  // token 32 tb + (l & 31), channels 16 ks + 8h .. +7.
  f32x16 g00 = zero16(), g10 = zero16(), g11 = zero16();
  {
    const bf16_t* r0 = sKs + l32 * KSP + 8 * h;
    const bf16_t* r1 = sKs + (32 + l32) * KSP + 8 * h;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 f0 = *reinterpret_cast<const bf16x8*>(r0 + 16 * ks);
      const bf16x8 f1 = *reinterpret_cast<const bf16x8*>(r1 + 16 * ks);
      g00 = mfma32(f0, f0, g00);
      g10 = mfma32(f1, f0, g10);
      g11 = mfma32(f1, f1, g11);
    }
  }
  // A0 = (I + B L)^-1 B with B = diag(beta), L = strict_lower(K K^T), formed as
  // B (I + L B)^-1 (the two are equal: B (I + L B) = (I + B L) B), so that the
  // weights scale columns of the Gram here (one factor per lane) and rows of
  // the inverse at the end (one factor per row, folded into its fp16 scale).
  // M = L B into LDS (row-major; upper part unused)
  __syncthreads();
  {
    const float b0 = sBeta[l32], b1 = sBeta[32 + l32];  // the lane's columns
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(r, lane);
      sM[row * MP + l32] = (row > l32) ? b0 * g00[r] : 0.f;
      sM[(32 + row) * MP + l32] = b0 * g10[r];
      sM[(32 + row) * MP + 32 + l32] = (row > l32) ? b1 * g11[r] : 0.f;
    }
  }
  __syncthreads();

  // ---- N = (I + M)^-1 in 32 x 32 blocks ---------------------------------------------
  // The diagonal blocks in 16-blocks (common.h), then the upper-right block of
  // N, which is zero.
  inv_diag32_blocks(sM, MP, lane);
#pragma unroll
  for (int r = 0; r < 16; ++r) sM[(16 * (lane >> 5) + r) * MP + 32 + l32] = 0.f;  // rows 0..31
  __syncthreads();
  // Off-diagonal block N_10 = -N_11 (M_10 N_00): two 32 x 32 x 32 products on
  // bf16 MFMA with both operands split into two terms (about 2^-16 relative).
  auto prod = [&](const float* Ab, const float* Bb) {
    // Ab, Bb: 32 x 32 blocks of sM (pitch MP); returns Ab Bb in accumulator layout
    f32x16 P = zero16();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float xa[8], xb[8];
      const float* ar = Ab + l32 * MP + 16 * ks + 8 * h;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(ar);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(ar + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xa[j] = a0[j];
        xa[4 + j] = a1[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[j] = Bb[(16 * ks + 8 * h + j) * MP + l32];
      mma<2, 2>(P, split8<2>(xa), split8<2>(xb));
    }
    return P;
  };
  {
    const f32x16 P = prod(sM + 32 * MP, sM);  // M_10 N_00
    __syncthreads();                          // M_10 is read; its block now holds P
#pragma unroll
    for (int r = 0; r < 16; ++r) sM[(32 + acc_row(r, lane)) * MP + l32] = P[r];
  }
  __syncthreads();
  {
    const f32x16 Q = prod(sM + 32 * MP + 32, sM + 32 * MP);  // N_11 P
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) sM[(32 + acc_row(r, lane)) * MP + l32] = -Q[r];
  }
  __syncthreads();

  // ---- A0 = diag(beta) N (row t scaled by beta_t); rows to fp16 with row scales -----
  unsigned char* rec = ws + (size_t)blockIdx.x * REC_BYTES;
  {
    const int t = lane;  // row of A0
    const float* Ar = sM + t * MP;
    float m = 0.f;
#pragma unroll
    for (int j4 = 0; j4 < C / 4; ++j4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(Ar + 4 * j4);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
    const float bt = sBeta[t];
    // a row whose largest entry is already inside fp16's working range keeps
    // scale 1 (the usual case), so the state pass can skip the row factors
    const int e = f16_scale_exp(m * fabsf(bt));
    const float s = bt * ldexpf(1.f, -e);
    f16x8* dst = reinterpret_cast<f16x8*>(rec + REC_A + t * C * 2);
#pragma unroll
    for (int j8 = 0; j8 < C / 8; ++j8) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(Ar + 8 * j8);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(Ar + 8 * j8 + 4);
      f16x8 hv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hv[j] = (f16_t)(v0[j] * s);
        hv[4 + j] = (f16_t)(v1[j] * s);
      }
      dst[j8] = hv;
    }
    reinterpret_cast<float*>(rec + REC_RS)[t] = ldexpf(1.f, e);
    reinterpret_cast<float*>(rec + REC_G)[t] = G;
  }
}

// =====================================================================================
// delta_state: per unit, [U | S] in registers, three MFMA products per chunk
// =====================================================================================

template <bool KDA>
struct StateLdsT {  // one staging buffer
  static constexpr int O_K = 0;
  static constexpr int O_KT = O_K + C * KP * 2;
  static constexpr int O_V = O_KT + D * TP * 2;
  static constexpr int O_A0 = O_V + D * TP * 2;
  static constexpr int O_SM = O_A0 + C * TP * 2;  // eW[64] = exp(G_C - G_t), rs[64], exp(G_C)
  static constexpr int O_RF = O_SM + (2 * C + 4) * 4;  // KDA: row factors of S [128], of U [128]
  static constexpr int BUF = O_RF + (KDA ? 2 * D * 4 : 0);
};

// ---- the fused composition (hypic_seg_build_compose, fused schedule) -----------------
// Node k of the tree over P leaves: its leftmost leaf, and the node that holds its
// pair (a node whose right subtree is empty stands for its left child).
__device__ __forceinline__ int fuse_leftmost(int k, int P) {
  while (k < P) k *= 2;
  return k - P;
}
__device__ __forceinline__ int fuse_resolve(int k, int P, int n_seg) {
  while (k < P && fuse_leftmost(2 * k + 1, P) >= n_seg) k *= 2;
  return k;
}

// LDS of the node composition: U of the right child split into two fp16 terms
// (A operand, k bits 2 and 3 swapped inside 16-blocks so that a fragment is one
// 16-byte read), then the exponents of its 16-row blocks.
constexpr int FUSE_UP = D + 8;
constexpr int FUSE_OFF_E = 2 * D * FUSE_UP * 2;
constexpr int FUSE_LDS = FUSE_OFF_E + 64;

// Pair (g, U, S) of node k's children, composed in order: g = g_L + g_R,
// U = U_R U_L, S = exp(g_R) U_R S_L + S_R ([youleyou, linear-layer paragraph]:
// S(C1.C2) = T(C2) S(C1) + S(C2), T = exp(g) U).  Eight waves: wave w computes
// columns 32 (w & 3) .. of U (w < 4) or S (w >= 4) with the left child's columns
// as the B operand and U_R as A, both in two fp16 terms (fp32-class products,
// as in the dense chain kernel); row tiles one at a time, each stored as it is
// finished.  (Not inlined: the state pass around it keeps its own register
// allocation.)
// (The arguments are the values it needs, not the kernel's argument block, which
// would then be copied to scratch memory.)
__device__ __noinline__ void fuse_compose(const FuseArgs f, const float* pg, const float* pU, const float* pS,
                                          int n_chain, int k, int chain, unsigned char* smem) {
  const int P = f.P;
  const int L = fuse_resolve(2 * k, P, f.n_seg), R = fuse_resolve(2 * k + 1, P, f.n_seg);
  auto unit = [&](int r) { return (size_t)(r >= P ? r - P : r) * n_chain + chain; };
  const float* gsrc_L = L >= P ? pg : f.g;
  const float* gsrc_R = R >= P ? pg : f.g;
  const float* U_L = (L >= P ? pU : f.U) + unit(L) * D * D;
  const float* S_L = (L >= P ? pS : f.S) + unit(L) * D * D;
  const float* U_R = (R >= P ? pU : f.U) + unit(R) * D * D;
  const float* S_R = (R >= P ? pS : f.S) + unit(R) * D * D;
  const float gL = gsrc_L[unit(L)], gR = gsrc_R[unit(R)];
  const bool root = k == 1;
  float* U_o = root ? f.U_tot : f.U + unit(k) * D * D;
  float* S_o = root ? f.S_out + (size_t)chain * D * D : f.S + unit(k) * D * D;
  if (root && U_o) U_o += (size_t)chain * D * D;

  const int wave = threadIdx.x >> 6;
  const int lane = opaque((int)threadIdx.x) & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const bool uh = wave < 4;  // U columns (else S columns)
  const int cb = (wave & 3) * 32;
  f16_t* sU = reinterpret_cast<f16_t*>(smem);
  int* sE = reinterpret_cast<int*>(smem + FUSE_OFF_E);

  // U_R split: wave w rows 16 w .. 16 w + 15, lane rows 16 w + 2 i + h, columns 4 l32 ..
  {
    f32x4 ur[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ur[i] = *reinterpret_cast<const f32x4*>(U_R + (size_t)(16 * wave + 2 * i + h) * D + 4 * l32);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(ur[i][j]));
    const int eu = min(max(split_exp(wave_max_uniform(m)), -100), 100);
    if (lane == 0) sE[wave] = eu;
    const float su = ldexpf(1.f, -eu);
    f16_t* dst = sU + (16 * wave + h) * FUSE_UP + 16 * (l32 >> 2) + kperm(4 * (l32 & 3));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const H4<2> t = split4h_scaled<2>(ur[i], su);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) *reinterpret_cast<f16x4*>(dst + (tt * D + 2 * i) * FUSE_UP) = t.t[tt];
    }
  }
  // the left child's columns (B operand), in the accumulator layout
  f32x16 Z[4];
  {
    const float* src = (uh ? U_L : S_L) + cb + l32;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) Z[rt][r] = src[(size_t)(32 * rt + acc_row(r, lane)) * D];
  }
  __syncthreads();  // the split is in LDS
  const float fs = uh ? 1.f : expf(gR);
  float m = 0.f;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(Z[rt][r]));
  m = fmaxf(m, __shfl_xor(m, 32, 64));  // the partner lane holds the column's other rows
  const int ec = min(max(split_exp(m * fs), -100), 100);
  const float sc = fs * ldexpf(1.f, -ec);
  const f16_t* pa = sU + l32 * FUSE_UP + 8 * h;
  float* dst = uh ? U_o : S_o;
#pragma unroll 1
  for (int rt = 0; rt < 4; ++rt) {
    f32x16 T = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = Z[ks >> 1][8 * (ks & 1) + j];
      const HFrag<2> fb = split8h_scaled<2>(x, sc);
      HFrag<2> fa;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        fa.t[tt] = *reinterpret_cast<const f16x8*>(pa + (tt * D + 32 * rt) * FUSE_UP + 16 * ks);
      mmah<2, 2>(T, fa, fb);
    }
    const int e0 = sE[2 * rt] + ec, e1 = sE[2 * rt + 1] + ec;  // rows 32 rt + 0..15, + 16..31
    if (dst) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const size_t o = (size_t)(32 * rt + acc_row(r, lane)) * D + cb + l32;
        float y = ldexpf(T[r], r < 8 ? e0 : e1);
        if (!uh) y += S_R[o];
        dst[o] = y;
      }
    }
  }
  float* g_o = root ? (f.g_tot ? f.g_tot + chain : nullptr) : f.g + unit(k);
  if (threadIdx.x == 0 && g_o) *g_o = gL + gR;
}

// Per chunk, in the frame scaled by the chunk's gate (the gated delta rule is
// the ungated one on values v_t exp(-G_t), then scaled by exp(G_C)):
//   U <- U + K^T (-A0 (K U))
//   S <- exp(G_C) S + K^T (A0 (diag(exp(G_C - G)) V - exp(G_C) K S))
// so both halves share A0 and every gate factor is at most 1.
// KDA mode: the same three products over the records of the KDA factor pass,
// with the decayed keys Kb (for K Z) and Kd (for K^T X) in place of K, the value
// weights exp(mu_C - mu_t), exp(mu_C) in place of exp(G_C - G_t), exp(G_C), and
// per-row factors exp(G_C) (S) and exp(G_C - mu_C) (U) in place of the scalar
// exp(G_C) in step 3; g accumulates mu_C.
// 8 waves: wave w keeps the 32 state columns 32 (w & 3) .. of U (w < 4) or S
// (w >= 4) in accumulators.  One staging buffer: chunk c+1 is loaded after chunk
// c's products and stored over the buffer after a barrier (two per chunk); at
// about 60 KB of LDS and at most 128 registers two workgroups share a CU and
// cover each other's waits.
// FUSE (delta mode): the fused composition follows the unit's pair (a separate
// instantiation, so the plain build carries none of its code).
template <bool KDA, bool FUSE = false>
__global__ __launch_bounds__(512, 4) void delta_state_kernel(const BuildArgs a, const ChunkTable cks,
                                                             const unsigned char* ws) {
  using StateLds = StateLdsT<KDA>;
  constexpr int RB = KDA ? KREC_BYTES : REC_BYTES;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int wave = threadIdx.x >> 6;
  const bool s_wave = wave >= 4;
  const int col0 = (wave & 3) * 32;
  const int n_chain = a.n_chain;
  const int s_local = blockIdx.x / n_chain;  // slot: longest segments first
  const int chain = blockIdx.x % n_chain;
  const int t_begin = a.seg.beg[s_local], t_end = a.seg.end[s_local];
  const int n_ck = (t_end - t_begin + C - 1) / C;
  const size_t unit = (size_t)a.seg.out[s_local] * n_chain + chain;

  f32x16 Z[4];
  {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Z[rt][r] = (!s_wave && 32 * rt + acc_row(r, lane) == col0 + (lane & 31)) ? 1.f : 0.f;
  }
  double g_acc = 0.0;
  // threads < 64: G_t, G_C and the row scale of A0 row t (KDA: the value weight,
  // mu_C, the row scale; threads < 128 the two row factors; thread 0 exp(mu_C))
  float fin[KDA ? 6 : 3];

  // ---- staging of one chunk: loads into registers, then conversion into LDS ---------
  // threads 0..255: a 4-token x 8-channel block of K; 256..511: of V; every
  // thread 8 entries of A0, and the first 64 the factors of token tid
  uint4 raw[KDA ? 7 : 5];
  auto load_chunk = [&](int c) {
    const int tid = opaque(threadIdx.x);
    const int c0 = t_begin + c * C;
    const int nv = min(C, t_end - c0);
    const unsigned char* rec = ws + ((size_t)(cks.base[s_local] + c) * n_chain + chain) * RB;
    const int id = tid & 255, tb = id & 15, db = id >> 4;
    if (KDA && tid < 256) {  // decayed keys Kb, rows of fp16 (zero past the end)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        raw[r] = *reinterpret_cast<const uint4*>(rec + KREC_KB + ((tb * 4 + r) * D + db * 8) * 2);
    } else {
      // K (waves 0-3) or V (waves 4-7) over the chunk's valid tokens only: a
      // buffer load past them returns zeros, which tokens past the end must be
      const uint32_t row_bytes = (uint32_t)n_chain * D * 2;
      const char* src = reinterpret_cast<const char*>(wave_id_uniform() >= 4 ? a.v : a.k) +
                        ((size_t)c0 * n_chain + chain) * D * 2;
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (uint32_t)(nv - 1) * row_bytes + D * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) raw[r] = buffer_load16(rs, (uint32_t)(tb * 4) * row_bytes + db * 16, r * row_bytes);
    }
    // A0 (X) row tid / 8, entries 8 (tid % 8) ..
    raw[4] = *reinterpret_cast<const uint4*>(rec + (KDA ? KREC_X : REC_A) + tid * 16);
    if constexpr (KDA) {  // Kd: 16-byte pieces 2 tid, 2 tid + 1 of the [128][64] fp16 rows
      raw[5] = *reinterpret_cast<const uint4*>(rec + KREC_KD + (2 * tid) * 16);
      raw[6] = *reinterpret_cast<const uint4*>(rec + KREC_KD + (2 * tid + 1) * 16);
    }
#pragma unroll
    for (int i = 0; i < (KDA ? 6 : 3); ++i) fin[i] = 0.f;
    if constexpr (KDA) {
      if (tid < C) {
        fin[0] = reinterpret_cast<const float*>(rec + KREC_VF)[tid];
        fin[1] = reinterpret_cast<const float*>(rec + KREC_M)[0];
        fin[2] = reinterpret_cast<const float*>(rec + KREC_XS)[tid];
        fin[5] = reinterpret_cast<const float*>(rec + KREC_M)[1];
      }
      if (tid < D) {
        fin[3] = reinterpret_cast<const float*>(rec + KREC_RS)[tid];
        fin[4] = reinterpret_cast<const float*>(rec + KREC_RU)[tid];
      }
    } else if (tid < C) {
      const float* G = reinterpret_cast<const float*>(rec + REC_G);
      fin[0] = G[tid];
      fin[1] = G[C - 1];
      fin[2] = reinterpret_cast<const float*>(rec + REC_RS)[tid];
    }
  };
  auto store_chunk = [&] {
    const int tid = opaque(threadIdx.x);
    unsigned char* base = smem;
    const int id = tid & 255, tb = id & 15, db = id >> 4;
    if (tid < 256) {  // keys: exact bf16 -> fp16 (KDA: Kb, already fp16), row-major
      f16_t* sK = reinterpret_cast<f16_t*>(base + StateLds::O_K);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (!KDA)
          raw[r] = make_uint4(pk_f16_from_bf16x2(raw[r].x), pk_f16_from_bf16x2(raw[r].y),
                              pk_f16_from_bf16x2(raw[r].z), pk_f16_from_bf16x2(raw[r].w));
        f16_t* row = sK + (tb * 4 + r) * KP + db * 8;
        *reinterpret_cast<uint2*>(row) = make_uint2(raw[r].x, raw[r].y);
        *reinterpret_cast<uint2*>(row + 4) = make_uint2(raw[r].z, raw[r].w);
      }
    }
    // keys (fp16) or values (bf16) transposed: channel cc of the block holds its
    // 4 tokens as two dwords (element cc of rows 0, 1 and of rows 2, 3).  KDA:
    // only the values; the transposed keys are Kd, copied as they are.
    if (!KDA || tid >= 256) {
      uint16_t* sT = reinterpret_cast<uint16_t*>(base + (tid < 256 ? StateLds::O_KT : StateLds::O_V));
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
        auto w = [&](int r) {
          const uint4 q = raw[r];
          return (cc >> 1) == 0 ? q.x : (cc >> 1) == 1 ? q.y : (cc >> 1) == 2 ? q.z : q.w;
        };
        *reinterpret_cast<uint2*>(sT + (db * 8 + cc) * TP + tb * 4) =
            make_uint2(__builtin_amdgcn_perm(w(1), w(0), sel), __builtin_amdgcn_perm(w(3), w(2), sel));
      }
    }
    if constexpr (KDA) {
      f16_t* sKt = reinterpret_cast<f16_t*>(base + StateLds::O_KT);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int piece = 2 * tid + i, row = piece >> 3, col8 = piece & 7;
        f16_t* dst = sKt + row * TP + col8 * 8;
        *reinterpret_cast<uint2*>(dst) = make_uint2(raw[5 + i].x, raw[5 + i].y);
        *reinterpret_cast<uint2*>(dst + 4) = make_uint2(raw[5 + i].z, raw[5 + i].w);
      }
    }
    {
      f16_t* sA = reinterpret_cast<f16_t*>(base + StateLds::O_A0) + (tid >> 3) * TP + (tid & 7) * 8;
      *reinterpret_cast<uint2*>(sA) = make_uint2(raw[4].x, raw[4].y);
      *reinterpret_cast<uint2*>(sA + 4) = make_uint2(raw[4].z, raw[4].w);
    }
    if (tid < C) {
      float* sF = reinterpret_cast<float*>(base + StateLds::O_SM);
      sF[tid] = KDA ? fin[0] : __expf(fin[1] - fin[0]);  // value weight to the chunk end
      sF[C + tid] = fin[2];                               // row scale of A0
      // (threads < C are wave 0: one vote) every row scale of the chunk is 1
      const bool unit_rows = __ballot(fin[2] != 1.f) == 0;
      if (tid == 0) {
        sF[2 * C] = KDA ? fin[5] : __expf(fin[1]);
        sF[2 * C + 1] = unit_rows ? 1.f : 0.f;
        g_acc += (double)fin[1];
      }
    }
    if constexpr (KDA) {
      if (tid < D) {
        float* sR = reinterpret_cast<float*>(base + StateLds::O_RF);
        sR[tid] = fin[3];
        sR[D + tid] = fin[4];
      }
    }
  };

  load_chunk(0);
  store_chunk();
  __syncthreads();

  for (int c = 0; c < n_ck; ++c) {
    // (the next chunk's loads are issued after the products, so no staging
    // registers live across them; the other workgroup on the CU runs meanwhile)
    {
      const unsigned char* base = smem;
      const f16_t* sK = reinterpret_cast<const f16_t*>(base + StateLds::O_K);
      const f16_t* sKt = reinterpret_cast<const f16_t*>(base + StateLds::O_KT);
      const bf16_t* sVt = reinterpret_cast<const bf16_t*>(base + StateLds::O_V);
      const f16_t* sA0 = reinterpret_cast<const f16_t*>(base + StateLds::O_A0);
      const float* sF = reinterpret_cast<const float*>(base + StateLds::O_SM);
      const int lane = opaque(threadIdx.x) & 63;
      const int h = lane >> 5, l32 = lane & 31;
      const int xaddr = (lane ^ 32) << 2;
      // the scale of an operand column: over the two lanes that hold it
      auto col_max = [&](float m) { return pair_max(m, xaddr); };
      const float eGC = sF[2 * C];
      float fez;   // delta mode: W = K Z / fez after step 1
      float f_er;  // W holds X' / f_er after step 2
      f32x16 W[2];
      // Every operand scale below is per column (lanes l and l ^ 32 agree on it),
      // and the products of a column carry its factor to where it is used.
      // ---- step 1: Y = K Z.  Delta mode, S waves: S <- exp(G_C) S first, so that
      // step 1 and step 3 use the decayed state alike (KDA: the factor folded into
      // Z's conversion; its per-row factors come in step 3) -------------------------
      {
        if (!KDA && s_wave) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) Z[rt][r] *= eGC;
        }
        float m = 0.f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(Z[rt][r]));
        const float gz = (KDA && s_wave) ? eGC : 1.f;
        const int ez = f16_scale_exp(col_max(m) * gz);
        // delta mode, U waves: -Z, so that X' comes out with its sign (U <- U - K^T A0 K U)
        const float sz = KDA ? gz * ldexpf(1.f, -ez) : (s_wave ? 1.f : -1.f) * ldexpf(1.f, -ez);
        fez = KDA ? 1.f : ldexpf(1.f, ez);
        const f16_t* pK = sK + l32 * KP + 4 * h;
        W[0] = zero16();
        W[1] = zero16();
        auto product = [&](auto conv) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              const f16x8 fb = conv(Z[rt], mm);
#pragma unroll
              for (int tt = 0; tt < 2; ++tt)
                W[tt] = mfma32h(lds_a_perm_h(pK, 32 * tt * KP + 32 * rt + 16 * mm), fb, W[tt]);
            }
        };
        // (delta mode, every column at scale 1: the conversion alone, the sign a modifier)
        if (!KDA && !wave_any(ez != 0)) {
          if (s_wave) product([](const f32x16& z, int mm) { return acc_as_b_unit<false>(z, mm); });
          else product([](const f32x16& z, int mm) { return acc_as_b_unit<true>(z, mm); });
        } else {
          product([&](const f32x16& z, int mm) { return acc_as_b_h(z, mm, sz); });
        }
        if (KDA && wave_any(ez != 0)) {
          const float f = ldexpf(1.f, ez);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r) W[tt][r] *= f;
        }
        // (delta mode: W = K Z 2^-ez; the factor 2^ez is applied where W is used)
      }
      // ---- step 2: R = diag(eW) V - exp(G_C) Y (S) or Y (U);  X' = (-)diag(rs) A0 R -----
      {
        // S waves: R = diag(eW) V - W 2^ez; U waves: R = W, its factor 2^ez carried on
        if (s_wave) {
          // elements 4q .. 4q+3 of tile tt are tokens 32 tt + 8q + 4h + 0..3 of the lane's column
          const bf16_t* pV = sVt + (col0 + l32) * TP + 4 * h;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint2 vv = *reinterpret_cast<const uint2*>(pV + 32 * tt + 8 * q);
              const f32x4 ew = *reinterpret_cast<const f32x4*>(sF + 32 * tt + 8 * q + 4 * h);
              const float v4[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                                   __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
#pragma unroll
              for (int j = 0; j < 4; ++j) W[tt][4 * q + j] = fmaf(W[tt][4 * q + j], -fez, ew[j] * v4[j]);  // (W carries exp(G_C))
            }
        }
        float m = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(W[tt][r]));
        const int er = f16_scale_exp(col_max(m));
        const f16_t* pA = sA0 + l32 * TP + 4 * h;
        if (!KDA && wave_any(er != 0)) {  // (delta mode: R converted once, scaled in place where needed)
          const float sr = ldexpf(1.f, -er);
#pragma unroll
          for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int r = 0; r < 16; ++r) W[tp][r] *= sr;
        }
        f16x8 fb[2][2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) fb[tp][mm] = KDA ? acc_as_b_h(W[tp], mm, ldexpf(1.f, -er)) : acc_as_b_unit<false>(W[tp], mm);
        W[0] = zero16();
        W[1] = zero16();
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int tt = tp; tt < 2; ++tt)
              W[tt] = mfma32h(lds_a_perm_h(pA, 32 * tt * TP + 32 * tp + 16 * mm), fb[tp][mm], W[tt]);
        // X' = W f_er (times the row scales of A0 unless all are 1)
        if constexpr (KDA) f_er = (s_wave ? 1.f : -1.f) * ldexpf(1.f, er);
        else f_er = ldexpf(1.f, er) * (s_wave ? 1.f : fez);
        if (KDA || sF[2 * C + 1] == 0.f) {
          const float* fac = sF + C + 4 * h;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 f4 = *reinterpret_cast<const f32x4*>(fac + 32 * tt + 8 * q) * f_er;
#pragma unroll
              for (int j = 0; j < 4; ++j) W[tt][4 * q + j] *= f4[j];
            }
          f_er = 1.f;
        }
      }
      // ---- step 3: Z = Z (delta; S waves decayed in step 1) or diag(row factors) Z
      // (KDA) + K^T X' ---------------------------------------------------------------
      {
        float m = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(W[tt][r]));
        const int ex = f16_scale_exp(col_max(m) * fabsf(f_er));
        const bool any_ex = wave_any(ex != 0);
        if constexpr (KDA) {  // per-row factors exp(G_C) (S) or exp(G_C - mu_C) (U)
          const float sc = ldexpf(1.f, -ex);
          const float* rf = reinterpret_cast<const float*>(base + StateLds::O_RF) + (s_wave ? 0 : D) + 4 * h;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 f4 = *reinterpret_cast<const f32x4*>(rf + 32 * rt + 8 * q) * sc;
#pragma unroll
              for (int j = 0; j < 4; ++j) Z[rt][4 * q + j] *= f4[j];
            }
        } else if (any_ex) {
          const float pre = ldexpf(1.f, -ex);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) Z[rt][r] *= pre;
        }
        const f16_t* pKt = sKt + l32 * TP + 4 * h;
        const float sx = f_er * ldexpf(1.f, -ex);
        if (!KDA && wave_any(sx != 1.f)) {  // (delta mode: X' converted once, scaled in place where needed)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r) W[tt][r] *= sx;
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const f16x8 fb = KDA ? acc_as_b_h(W[tt], mm, sx) : acc_as_b_unit<false>(W[tt], mm);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
              Z[rt] = mfma32h(lds_a_perm_h(pKt, 32 * rt * TP + 32 * tt + 16 * mm), fb, Z[rt]);
          }
        if (any_ex) {
          const float f = ldexpf(1.f, ex);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) Z[rt][r] *= f;
        }
      }
    }
    if (c + 1 < n_ck) {  // (one branch, so the staging registers die with it)
      load_chunk(c + 1);
      __syncthreads();  // every wave is done with the buffer
      store_chunk();
      __syncthreads();
    }
  }

  const int lane = threadIdx.x & 63;
  float* dst = (s_wave ? a.S : a.U) + unit * D * D;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(size_t)(32 * rt + acc_row(r, lane)) * D + col0 + (lane & 31)] = Z[rt][r];
  if (threadIdx.x == 0) a.g[unit] = (float)g_acc;

  // ---- fused composition: count this pair's arrival at its parent; the last
  // arrival at a node composes it and goes on to the node's parent ----------------
  if constexpr (FUSE && !KDA) {
    {
      __shared__ int s_last;
      const FuseArgs f = a.fuse;
      for (int k = (f.P + a.seg.out[s_local]) >> 1; k >= 1; k >>= 1) {
        // release at device scope: this workgroup's pair (or node) written back
        // to where every CU sees it, by every thread, before the count
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (threadIdx.x == 0) {
          const int need = fuse_leftmost(2 * k + 1, f.P) < f.n_seg ? 2 : 1;
          s_last = atomicAdd(f.cnt + (size_t)k * n_chain + chain, 1) + 1 == need;
        }
        __syncthreads();
        if (!s_last) break;
        // acquire (the last arrival only): the siblings' pairs, not stale copies
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (fuse_leftmost(2 * k + 1, f.P) < f.n_seg) fuse_compose(f, a.g, a.U, a.S, n_chain, k, chain, smem);
      }
    }
  }
}

}  // namespace

namespace {
__global__ void zero_ints_kernel(int* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
}  // namespace

hipError_t launch_zero_ints(int* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

size_t delta2_workspace_bytes(const SegTable& seg, int n_chain) {
  return (size_t)chunk_table(seg, nullptr) * n_chain * REC_BYTES;
}

namespace {
template <bool KDA, bool FUSE>
hipError_t launch_state_t(const BuildArgs& a, const ChunkTable& ct, const unsigned char* w, hipStream_t stream) {
  // (the fused composition splits a 128 x 128 operand into the same LDS)
  constexpr int lds = (FUSE && FUSE_LDS > StateLdsT<KDA>::BUF) ? FUSE_LDS : StateLdsT<KDA>::BUF;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&delta_state_kernel<KDA, FUSE>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((delta_state_kernel<KDA, FUSE>), dim3(a.seg.n_seg * a.n_chain), dim3(512), lds, stream, a, ct,
                     w);
  return hipGetLastError();
}
template <bool KDA>
hipError_t launch_state(const BuildArgs& a, const ChunkTable& ct, const unsigned char* w, hipStream_t stream) {
  if constexpr (!KDA) {
    if (a.fuse.cnt) return launch_state_t<false, true>(a, ct, w, stream);
  }
  return launch_state_t<KDA, false>(a, ct, w, stream);
}
}  // namespace

hipError_t launch_build_delta2(const BuildArgs& a, void* ws, hipStream_t stream) {
  ChunkTable ct;
  const int n_chunks = chunk_table(a.seg, &ct);
  unsigned char* w = reinterpret_cast<unsigned char*>(ws);
  hipLaunchKernelGGL(delta_prep_kernel, dim3(n_chunks * a.n_chain), dim3(64), 0, stream, a, ct, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_state<false>(a, ct, w, stream);
}

hipError_t launch_kda_state(const BuildArgs& a, const ChunkTable& ct, const void* ws, hipStream_t stream) {
  return launch_state<true>(a, ct, reinterpret_cast<const unsigned char*>(ws), stream);
}

}  // namespace hypic
