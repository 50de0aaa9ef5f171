// build_kda.hip -- segment build for the KDA family (the delta rule with one
// gate per key channel): emits T_C = exp(g) U and S(C|0) of every
// (segment, chain).
//
// [youleyou, linear-layer paragraph] T_C is the product of the segment's
// per-token transitions, here A_t = (I - beta_t k_t k_t^T) diag(alpha_t), and
// S(C|0) the final state from a zero start.  The channel gates do not commute
// with the erase factors, so T_C is a dense product; g is a scale that keeps U
// in range: the sum over tokens of each token's largest channel gate, which
// bounds the decay of every product of the factors.
//
// Chunk form (64 tokens; within the chunk the per-channel inclusive gate
// prefixes G [C][d], the summed largest gates mu_t, and H = G - mu, which is
// <= 0 and non-increasing along t in every channel; G_C, H_C, mu_C the last
// rows): in the frame diag(exp(-mu_t)) the chunk's product of rank-1 factors
// is a generalised WY product whose two sides carry the keys decayed in
// opposite directions:
//   M[i,j] = b_i sum_c k_ic k_jc exp(H_ic - H_jc)   (i > j),  X = (I + M)^-1 diag(b)
//   (formed as X = diag(b) (I + L diag(b))^-1 with L the Gram without the
//   weights: the two are equal, and the weights then scale the Gram's columns
//   and the inverse's rows)
//   Kb = K o exp(H),  Kd = (K o exp(H_C - H))^T
//   U <- diag(exp(G_C - mu_C)) U - Kd X (Kb U),   g += mu_C
//   S <- diag(exp(G_C)) S + Kd X (diag(exp(mu_C - mu)) V - exp(mu_C) Kb S)
// Every factor is at most 1 whatever the gates, and the result equals running
// the tokens one by one (the tests check this algebra against the token-by-
// token oracle).  The Gram terms exp(H_ic - H_jc) are formed without overflow:
// block pairs of 32, 16, 8 and 4 tokens go through keys decayed against a
// reference token between the two blocks (both factors <= 1), and the sixteen
// 4-token diagonal blocks are summed term by term.
//
// Two forms.  For d = 128 with bf16 tokens and segments of at most 2048 tokens
// the chunks' factors come from a parallel factor pass (kda_prep_kernel, one
// workgroup per chunk and chain) that writes a record per chunk (layout in
// launch.h), and the delta state kernel of build_delta2.hip runs the three
// products on the records.  Otherwise one workgroup of 4 waves per unit does
// both (build_kda_kernel): the state [U | S] (d x 2d fp32) lives in MFMA
// accumulators for the whole segment, waves 0-1 holding U and waves 2-3 S, d/2
// columns each, and per chunk the keys, gate prefixes, the decayed key copies
// (split into bf16 terms) and X sit in LDS.  In both, the off-diagonal Gram
// blocks run on bf16 MFMA with operands decayed on the fly, and the 64 x 64
// inverse takes its 32 x 32 diagonal blocks by forward substitution and the
// off-diagonal block by two MFMA products.
#include <type_traits>

#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int C = 64;  // tokens per chunk

template <int D, bool IN_F32>
struct KdaCfg {
  static constexpr int NTK = IN_F32 ? 3 : 2;  // bf16 terms of the decayed keys and Gram operands
  static constexpr int NTD = IN_F32 ? 3 : 2;  // bf16 terms of X and of accumulators used as B
  static constexpr int NRT = D / 32;          // row tiles of the state
  static constexpr int CT = D / 64;           // 32-column tiles per wave (d/2 columns)
  static constexpr int CPW = D / 2;
  static constexpr int FP = D + 8;            // bf16 / fp32 pitch of the staged keys [t][d]
                                              // (rows 16-byte aligned for vector reads)
  static constexpr int GP = D + 4;            // fp32 pitch of the gate prefixes [t][d]
  static constexpr int KP = D + 4;            // bf16 pitch of Kb [t][d]
  static constexpr int TP = C + 4;            // bf16 pitch of Kd [d][t] and of X [t][t']
  static constexpr int NP = C + 4;            // fp32 pitch of the Gram / inverse array (16-byte rows)
  using KT = typename std::conditional<IN_F32, float, bf16_t>::type;  // staged keys (exact)
  static constexpr int KF_BYTES = (C * FP * (int)sizeof(KT) + 15) / 16 * 16;
  static constexpr int VP = D + 8;            // pitch of the staged values [t][d]
  static constexpr int V_BYTES = (C * VP * (int)sizeof(KT) + 15) / 16 * 16;
  static constexpr int G_BYTES = C * GP * 4;
  static constexpr int KB_BYTES = NTK * C * KP * 2;
  static constexpr int KD_BYTES = NTK * D * TP * 2;
  static constexpr int A_BYTES_BF = NTD * C * TP * 2;
  static constexpr int N_BYTES = C * NP * 4;  // the fp32 Gram / inverse (aliases X)
  static constexpr int A_BYTES = ((A_BYTES_BF > N_BYTES ? A_BYTES_BF : N_BYTES) + 15) / 16 * 16;
  static constexpr int OFF_KF = 0;
  static constexpr int OFF_V = OFF_KF + KF_BYTES;
  static constexpr int OFF_G = OFF_V + V_BYTES;
  static constexpr int OFF_KB = OFF_G + G_BYTES;
  static constexpr int OFF_KD = OFF_KB + KB_BYTES;
  static constexpr int OFF_A = OFF_KD + KD_BYTES;
  static constexpr int OFF_SMALL = OFF_A + A_BYTES;
  // beta, token max gate, mu, exp(mu_C - mu), G_C, exp(G_C), exp(G_C - mu_C), misc
  static constexpr int SMALL_BYTES = (4 * C + 3 * D + 4) * 4;
  static constexpr int LDS = OFF_SMALL + SMALL_BYTES;
  static_assert(LDS <= 160 * 1024, "one workgroup's LDS");
};

// Key channels c0 .. c0+7 of token t decayed against token `ref` in the
// shifted prefixes H: k * exp(H_t - H_ref) (toward = true) or
// k * exp(H_ref - H_t), split into NT terms.
// Eight consecutive staged keys as floats (one 16-byte LDS read for bf16).
__device__ __forceinline__ void lds_keys8(const bf16_t* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
}
__device__ __forceinline__ void lds_keys8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}
__device__ __forceinline__ void lds_f8(const float* p, float (&x)[8]) { lds_keys8(p, x); }

// Eight floats into LDS as one 16-byte row piece (bf16) or two (fp32).
__device__ __forceinline__ void st_row8(bf16_t* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16_t)x[j];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void st_row8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

template <int NT, typename KT>
__device__ __forceinline__ Frag<NT> decayed_frag(const KT* sKf, const float* sH, int FP, int GP, int t, int ref,
                                                 int c0, bool toward) {
  float k[8], ht[8], hr[8], x[8];
  lds_keys8(sKf + t * FP + c0, k);
  lds_f8(sH + t * GP + c0, ht);
  lds_f8(sH + ref * GP + c0, hr);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = k[j] * __expf(toward ? ht[j] - hr[j] : hr[j] - ht[j]);
  return split8<NT>(x);
}

// The same eight decayed keys as one fp16 fragment (every value is at most |k|
// in magnitude, so fp16 holds it with 11 significant bits).
template <typename KT>
__device__ __forceinline__ f16x8 decayed_frag_h(const KT* sKf, const float* sH, int FP, int GP, int t, int ref, int c0,
                                               bool toward) {
  float k[8], ht[8], hr[8];
  lds_keys8(sKf + t * FP + c0, k);
  lds_f8(sH + t * GP + c0, ht);
  lds_f8(sH + ref * GP + c0, hr);
  f16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (f16_t)(k[j] * __expf(toward ? ht[j] - hr[j] : hr[j] - ht[j]));
  return f;
}

template <int NT>
__device__ __forceinline__ void split4_store(bf16_t* p, int term_stride, const float (&x)[4]) {
  float r[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    bf16x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16_t hb = (bf16_t)r[j];
      v[j] = hb;
      if (i + 1 < NT) r[j] -= (float)hb;
    }
    *reinterpret_cast<bf16x4*>(p + i * term_stride) = v;
  }
}

// The factor phases of one 64-token chunk, shared by the single-kernel build and
// the factor pass: stage the chunk's keys (and values), gates and weights;
// per-channel prefixes in place as H = G - mu; the strictly lower Gram
// L diag(b), L = (K o e^H)(K o e^-H)^T, formed without overflow; and
// N = (I + L diag(b))^-1, left in sN (X = diag(b) N).  Every thread of the 256-thread workgroup calls it (it holds
// barriers).  early() runs in every thread once H, sMu, sGC and sMisc ([0] =
// mu_C, [1] = exp(mu_C)) are valid, before the Gram.  GRAM_F16: the Gram's
// decayed keys enter the MFMA as one fp16 term each (bf16 tokens: the Gram then
// carries about 2^-11 relative error, the class of the fp16 X it feeds)
// instead of bf16 terms.  N_ON_G: sN shares the
// memory of sG, so sG is valid only until the Gram (early() is its last
// reader); otherwise sKf, sG, sN, sBeta, sMu, sGC and sMisc are all valid on
// return.
template <int D, bool IN_F32, bool WITH_V, bool N_ON_G, typename KT, typename Early, bool GRAM_F16 = false>
__device__ __forceinline__ void kda_chunk_factors(const BuildArgs& a, int c0, int nv, int chain, KT* sKf, KT* sV,
                                                  float* sG, float* sN, float* sBeta, float* sMax, float* sMu,
                                                  float* sGC, float* sMisc, Early early) {
  using Cfg = KdaCfg<D, IN_F32>;
  constexpr int NTK = Cfg::NTK, NTD = Cfg::NTD, FP = Cfg::FP, GP = Cfg::GP, VP = Cfg::VP, NP = Cfg::NP;
  const int n_chain = a.n_chain;
  const int tid = opaque(threadIdx.x);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wave = tid >> 6;
  (void)VP;
  // ---- stage keys, values and per-channel log gates (zero past the segment
  // end) and each token's largest gate (its D/8 channel groups are consecutive
  // lanes); every load of the chunk is issued before the first store
  constexpr int NIT = C * (D / 8) / 256;
  static_assert(NIT * 256 == C * (D / 8), "every lane runs every staging step");
  // (the weights' load joins the others: one memory round trip before the stores)
  const float beta = (tid < C && tid < nv) ? load1<IN_F32>(a.beta, (size_t)(c0 + tid) * n_chain + chain) : 0.f;
  {
    float x[NIT][8], lg[NIT][8], vx[NIT][8];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int it = tid + 256 * k;
      const int t = it / (D / 8), db = it % (D / 8);
      if (t < nv) {
        const size_t idx = ((size_t)(c0 + t) * n_chain + chain) * D + db * 8;
        load8<IN_F32>(a.k, idx, x[k]);
        load8<IN_F32>(a.lg, idx, lg[k]);
        if constexpr (WITH_V) load8<IN_F32>(a.v, idx, vx[k]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[k][j] = lg[k][j] = vx[k][j] = 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int it = tid + 256 * k;
      const int t = it / (D / 8), db = it % (D / 8);
      float mx = lg[k][0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, lg[k][j]);
      st_row8(sKf + t * FP + db * 8, x[k]);
      if constexpr (WITH_V) st_row8(sV + t * VP + db * 8, vx[k]);
      st_row8(sG + t * GP + db * 8, lg[k]);
      // maximum over the token's D/8 lanes (aligned groups of 8 or 16 lanes)
      mx = dpp_max_step(mx, 0);
      mx = dpp_max_step(mx, 1);
      mx = dpp_max_step(mx, 2);
      if constexpr (D / 8 == 16) mx = dpp_max_step(mx, 3);
      if (db == 0) sMax[t] = mx;
    }
  }
  if (tid < C) sBeta[tid] = beta;
  __syncthreads();

  // ---- per-channel prefixes: G_C, and in place of the gates H_t = G_t - mu_t.
  // Thread c < D takes channel c over the first half of the chunk, thread D + c
  // the same channel over the second half (local prefixes, then the first
  // half's totals added after the barrier).  mu_t is the same in every thread
  // of a half (the same sums in the same order); threads 0 and D record it.
  constexpr int HC = C / 2;
  const int part = tid / D, ch = tid % D;
  float gl[HC], ml[HC];
  if (tid < 2 * D) {
    float acc = 0.f, mu = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < HC / 4; ++t4) {
      const f32x4 m4 = *reinterpret_cast<const f32x4*>(sMax + part * HC + 4 * t4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * t4 + j;
        acc += sG[(part * HC + t) * GP + ch];
        mu += m4[j];
        gl[t] = acc;
        ml[t] = mu;
      }
    }
    if (part == 0) {
#pragma unroll
      for (int t = 0; t < HC; ++t) sG[t * GP + ch] = gl[t] - ml[t];
      if (ch == 0)
#pragma unroll
        for (int t = 0; t < HC; ++t) sMu[t] = ml[t];
      sGC[ch] = acc;  // G at the half's end
      if (ch == 0) sMisc[2] = mu;
    }
  }
  __syncthreads();
  if (part == 1) {
    const float g0 = sGC[ch], m0 = sMisc[2];
#pragma unroll
    for (int t = 0; t < HC; ++t) sG[(HC + t) * GP + ch] = (g0 + gl[t]) - (m0 + ml[t]);
    sGC[ch] = g0 + gl[HC - 1];  // (this thread's own entry)
    if (ch == 0) {
#pragma unroll
      for (int t = 0; t < HC; ++t) sMu[HC + t] = m0 + ml[t];
      const float muC = m0 + ml[HC - 1];
      sMisc[0] = muC;
      sMisc[1] = __expf(muC);
    }
  }
  __syncthreads();
  early();

  // ---- Gram L[i][j] b_j = b_j sum_c k_ic k_jc exp(H_ic - H_jc), i > j ---------
  // Each wave forms one 32 x 32 MFMA tile of products of decayed keys, both
  // factors decayed against a reference token between the row and the column
  // tokens (so both are <= |k|); parts of a tile whose row and column refer to
  // different references are discarded (their factors are <= |k| as well):
  //   wave 0: rows 32..63 x columns 0..31, reference 31
  //   wave 1: rows 32a+16..32a+31 x columns 32a..32a+15 (a = 0, 1), references 32a+15
  //   wave 2: rows 16a+8..16a+15 x columns 16a..16a+7 (a = 0..3), references 16a+7
  //   wave 3: rows 8a+4..8a+7 x columns 8a..8a+3 (a = 0..7), references 8a+3
  // which leaves the sixteen 4 x 4 diagonal blocks, summed term by term.
  const int sh = 5 - wave;  // log2 of the row group size in the tile: 16, 8, 4 (wave 0: one group of 32)
  int ra, rb, ref;
  if (wave == 0) {
    ra = 32 + l32;
    rb = l32;
    ref = 31;
  } else {
    const int ga = l32 >> sh, w = l32 & ((1 << sh) - 1);  // group, position in the group
    ra = (ga << (sh + 1)) + (1 << sh) + w;
    rb = (ga << (sh + 1)) + w;
    ref = (ga << (sh + 1)) + (1 << sh) - 1;
  }
  f32x16 acc = zero16();
#pragma unroll 2
  for (int ks = 0; ks < D / 16; ++ks) {
    const int cc = 16 * ks + 8 * h;
    if constexpr (GRAM_F16) {
      acc = mfma32h(decayed_frag_h(sKf, sG, FP, GP, ra, ref, cc, true),
                    decayed_frag_h(sKf, sG, FP, GP, rb, ref, cc, false), acc);
    } else {
      const Frag<NTK> fa = decayed_frag<NTK>(sKf, sG, FP, GP, ra, ref, cc, true);
      const Frag<NTK> fb = decayed_frag<NTK>(sKf, sG, FP, GP, rb, ref, cc, false);
      mma<NTK, NTK>(acc, fa, fb);
    }
  }
  // The sixteen 4-token diagonal blocks term by term: the 16 threads of block
  // b = tid / 16 take 8 channels each (at d = 64 the second 8 idle) and form
  // the block's six pairs (1,0), (2,0), (2,1), (3,0), (3,1), (3,2), summed over
  // the 16 lanes.
  const int dblk = tid >> 4, dsub = tid & 15;
  const int b0 = 4 * dblk;
  float dacc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (8 * dsub < D) {
    float kk[4][8], hh[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lds_keys8(sKf + (b0 + r) * FP + 8 * dsub, kk[r]);
      lds_f8(sG + (b0 + r) * GP + 8 * dsub, hh[r]);
    }
    int p = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < i; ++j, ++p) {
        float term = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) term = fmaf(kk[i][e] * kk[j][e], __expf(hh[i][e] - hh[j][e]), term);
        dacc[p] = term;
      }
  }
#pragma unroll
  for (int p = 0; p < 6; ++p)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dacc[p] += __shfl_xor(dacc[p], o, 64);
  if constexpr (N_ON_G) __syncthreads();  // every reader of sG is done: sN takes its memory
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rho = acc_row(r, lane);
    int i;
    bool keep;
    if (wave == 0) {
      i = 32 + rho;
      keep = true;
    } else {
      const int ga = rho >> sh;
      i = (ga << (sh + 1)) + (1 << sh) + (rho & ((1 << sh) - 1));
      keep = ga == (l32 >> sh);
    }
    if (keep) sN[i * NP + rb] = sBeta[rb] * acc[r];
  }
  if (dsub == 0) {
    int p = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < i; ++j, ++p) sN[(b0 + i) * NP + b0 + j] = sBeta[b0 + j] * dacc[p];
  }
  __syncthreads();

  // ---- N = (I + M)^-1 in 32 x 32 blocks, by wave 0 (the others wait) ---------
  // The diagonal blocks in 16-blocks (common.h); then N_10 = -N_11 (M_10 N_00)
  // as two 32 x 32 x 32 products on MFMA with both operands split into bf16
  // terms.
  if (wave == 0) inv_diag32_blocks(sN, NP, lane);
  __syncthreads();
  {
    auto prod = [&](const float* Ab, const float* Bb) {  // 32 x 32 blocks of sN; Ab Bb
      f32x16 P = zero16();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float xa[8], xb[8];
        const float* ar = Ab + l32 * NP + 16 * ks + 8 * h;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(ar);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(ar + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xa[j] = a0[j];
          xa[4 + j] = a1[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xb[j] = Bb[(16 * ks + 8 * h + j) * NP + l32];
        mma<NTD, NTD>(P, split8<NTD>(xa), split8<NTD>(xb));
      }
      return P;
    };
    if (wave == 0) {
      const f32x16 P = prod(sN + 32 * NP, sN);  // M_10 N_00
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) sN[(32 + acc_row(r, lane)) * NP + l32] = P[r];
    }
    __syncthreads();
    if (wave == 0) {
      const f32x16 Q = prod(sN + 32 * NP + 32, sN + 32 * NP);  // N_11 P
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) sN[(32 + acc_row(r, lane)) * NP + l32] = -Q[r];
    }
  }
  __syncthreads();
}

// ORDERED: workgroup rows read their segment from the launch's slot table
// (ragged launches); a contiguous launch of equal lengths computes it.
template <int D, bool IN_F32, bool ORDERED>
__global__ __launch_bounds__(256, 1) void build_kda_kernel(const BuildArgs a) {
  using Cfg = KdaCfg<D, IN_F32>;
  using KT = typename Cfg::KT;
  constexpr int NTK = Cfg::NTK, NTD = Cfg::NTD, NRT = Cfg::NRT, CT = Cfg::CT, CPW = Cfg::CPW;
  constexpr int FP = Cfg::FP, GP = Cfg::GP, KP = Cfg::KP, TP = Cfg::TP, NP = Cfg::NP, VP = Cfg::VP;
  constexpr int KBS = C * KP;  // term stride (elements) of Kb
  constexpr int KDS = D * TP;  // term stride of Kd
  constexpr int ATS = C * TP;  // term stride of X

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  KT* sKf = reinterpret_cast<KT*>(smem + Cfg::OFF_KF);
  KT* sV = reinterpret_cast<KT*>(smem + Cfg::OFF_V);
  float* sG = reinterpret_cast<float*>(smem + Cfg::OFF_G);
  bf16_t* sKb = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KB);
  bf16_t* sKd = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KD);
  bf16_t* sA = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_A);
  float* sN = reinterpret_cast<float*>(smem + Cfg::OFF_A);  // aliases sA
  float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_SMALL);
  float* sMax = sBeta + C;  // largest channel gate of each token
  float* sMu = sMax + C;    // mu_t: inclusive prefix of sMax
  float* sVf = sMu + C;     // exp(mu_C - mu_t): value factors
  float* sGC = sVf + C;     // G_C per channel
  float* sRS = sGC + D;     // exp(G_C): row factors of S
  float* sRU = sRS + D;     // exp(G_C - mu_C): row factors of U
  float* sMisc = sRU + D;   // [0] = mu_C, [1] = exp(mu_C)

  const int lane0 = lane_id();
  const int wave = wave_id();
  const int n_chain = a.n_chain;
  const int slot = (int)blockIdx.x / n_chain;
  const int chain = blockIdx.x % n_chain;
  const int len0 = a.seg.end[0] - a.seg.beg[0];
  const int t_begin = ORDERED ? a.seg.beg[slot] : a.seg.beg[0] + slot * len0;
  const int t_end = ORDERED ? a.seg.end[slot] : t_begin + len0;
  const size_t unit = (size_t)(ORDERED ? a.seg.out[slot] : a.seg.out[0] + slot) * n_chain + chain;
  const bool s_wave = wave >= 2;
  const int col0 = (wave & 1) * CPW;

  // ---- running state: U = I (waves 0-1), S = 0 (waves 2-3) -------------------
  f32x16 Z[NRT][CT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rt + acc_row(r, lane0);
        const int col = col0 + 32 * ct + (lane0 & 31);
        Z[rt][ct][r] = (!s_wave && row == col) ? 1.f : 0.f;
      }
  double g_acc = 0.0;

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int nv = min(C, t_end - c0);
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    kda_chunk_factors<D, IN_F32, true, false>(a, c0, nv, chain, sKf, sV, sG, sN, sBeta, sMax, sMu, sGC, sMisc,
                                              [] {});
    if (wave == 0) g_acc += (double)sMisc[0];  // mu_C; every lane of wave 0 keeps the same sum

    // ---- X = diag(beta) N split to bf16 terms; decayed key copies ------------
    {
      const int t = tid >> 2;
      const int cb = (tid & 3) * 16;
      float nv16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tp = cb + j;
        nv16[j] = (tp <= t) ? sN[t * NP + tp] : 0.f;
      }
      __syncthreads();  // sN is overwritten below
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float x0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x0[j] = nv16[8 * half + j] * sBeta[t];
        const Frag<NTD> f0 = split8<NTD>(x0);
#pragma unroll
        for (int i = 0; i < NTD; ++i) st8(sA + i * ATS + t * TP + cb + 8 * half, f0.t[i]);
      }
    }
    if (tid < 16 * (D / 8)) {
      // tokens 4*tq .. 4*tq+3, channels 8*db .. 8*db+7
      const int tq = tid & 15, db = tid >> 4;
      float hC[8];
      lds_f8(sG + (C - 1) * GP + 8 * db, hC);
      float kd[8][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tq + r;
        float kv[8], hv[8], kb[8];
        lds_keys8(sKf + t * FP + 8 * db, kv);
        lds_f8(sG + t * GP + 8 * db, hv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kb[j] = kv[j] * __expf(hv[j]);
          kd[j][r] = kv[j] * __expf(hC[j] - hv[j]);
        }
        const Frag<NTK> f = split8<NTK>(kb);
#pragma unroll
        for (int i = 0; i < NTK; ++i) st8(sKb + i * KBS + t * KP + 8 * db, f.t[i]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) split4_store<NTK>(sKd + (8 * db + j) * TP + 4 * tq, KDS, kd[j]);
    }
    if (tid < D) {
      sRS[tid] = __expf(sGC[tid]);
      sRU[tid] = __expf(sGC[tid] - sMisc[0]);
    }
    if (tid < C) sVf[tid] = __expf(sMisc[0] - sMu[tid]);
    __syncthreads();

    // ---- per wave: Y = Kb Z, W = X R, Z = diag(row factor) Z + Kd W -------------
    {
      const bf16_t* pKb = sKb + l32 * KP + 4 * h;
      const bf16_t* pKd = sKd + l32 * TP + 4 * h;
      const bf16_t* pA = sA + l32 * TP + 4 * h;
      const float* rowf = s_wave ? sRS : sRU;
      const float emuC = sMisc[1];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int gcol = col0 + 32 * ct + l32;
        // Y[tt] = Kb[tt rows] * Z[:, ct]
        f32x16 Y[2] = {zero16(), zero16()};
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const Frag<NTD> fb = acc_as_b<NTD>(Z[rt][ct], m);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const Frag<NTK> fa = lds_a_perm<NTK>(pKb, KBS, 32 * tt * KP + 32 * rt + 16 * m);
              mma<NTK, NTD>(Y[tt], fa, fb);
            }
          }
        if (s_wave) {  // R = diag(exp(mu_C - mu)) V - exp(mu_C) Kb S;  U waves: R = -Kb U
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              Y[tt][r] = sVf[32 * tt + acc_row(r, lane)] * (float)sV[(32 * tt + acc_row(r, lane)) * VP + gcol] -
                         emuC * Y[tt][r];
        }
        // W[tt] = sum_{tp <= tt} X[tt, tp] Y[tp]  (X lower triangular)
        f32x16 W[2] = {zero16(), zero16()};
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const Frag<NTD> fb = acc_as_b<NTD>(Y[tp], m, s_wave ? 1.f : -1.f);
#pragma unroll
            for (int tt = tp; tt < 2; ++tt) {
              const Frag<NTD> fa = lds_a_perm<NTD>(pA, ATS, 32 * tt * TP + 32 * tp + 16 * m);
              mma<NTD, NTD>(W[tt], fa, fb);
            }
          }
        // Z = diag(row factor) Z + Kd W
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r) Z[rt][ct][r] *= rowf[32 * rt + acc_row(r, lane)];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const Frag<NTD> fb = acc_as_b<NTD>(W[tt], m);
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
              const Frag<NTK> fa = lds_a_perm<NTK>(pKd, KDS, 32 * rt * TP + 32 * tt + 16 * m);
              mma<NTK, NTD>(Z[rt][ct], fa, fb);
            }
          }
      }
    }
    __syncthreads();
  }

  // ---- write U (waves 0-1) or S (waves 2-3), and g -----------------------------
  float* dst = (s_wave ? a.S : a.U) + unit * D * D;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(size_t)(32 * rt + acc_row(r, lane0)) * D + col0 + 32 * ct + (lane0 & 31)] = Z[rt][ct][r];
  if (wave == 0 && lane0 == 0) a.g[unit] = (float)g_acc;
}

template <int D, bool F32, bool ORDERED>
hipError_t launch_o(const BuildArgs& a, int n_blocks, hipStream_t stream) {
  constexpr int lds = KdaCfg<D, F32>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&build_kda_kernel<D, F32, ORDERED>), hipFuncAttributeMaxDynamicSharedMemorySize,
      lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((build_kda_kernel<D, F32, ORDERED>), dim3(n_blocks), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_t(const BuildArgs& a, int n_blocks, hipStream_t stream) {
  return seg_uniform(a.seg) ? launch_o<D, F32, false>(a, n_blocks, stream) : launch_o<D, F32, true>(a, n_blocks, stream);
}

// ---------------------------------------------------------------------------------
// Factor pass of the two-kernel build (d = 128, bf16 tokens): one 256-thread
// workgroup per (chunk, chain), all independent, so the latency of the scans,
// the Gram and the inverse hides behind other workgroups.  It writes the
// chunk's record (layout in launch.h): the decayed keys as fp16 (every factor
// <= 1, so no scaling) and the gate factors as soon as H is known, then X with
// a power-of-two scale per row (row maximum into [2^13, 2^14)); the state pass
// runs the delta state kernel's three products on them.  The Gram / inverse
// array takes the memory of the gate prefixes once the Gram has read them
// (51 KB of LDS: three workgroups per CU).
struct KdaPrepLds {
  using Cfg = KdaCfg<128, false>;
  static constexpr int OFF_KF = 0;
  static constexpr int OFF_G = OFF_KF + Cfg::KF_BYTES;
  static constexpr int OFF_N = OFF_G;  // after the Gram
  static constexpr int OFF_SMALL = OFF_G + Cfg::G_BYTES;
  // beta, token max gate, mu, G_C, misc
  static constexpr int LDS = OFF_SMALL + (3 * C + 128 + 4) * 4;
  static_assert(C * Cfg::NP * 4 <= Cfg::G_BYTES, "the Gram fits in the gate prefixes' memory");
  static_assert(3 * LDS <= 160 * 1024 - 3 * 1024, "three workgroups per CU");
  static_assert(KREC_BYTES % 16 == 0 && KREC_KD % 16 == 0 && KREC_X % 16 == 0, "16-byte record pieces");
};

__global__ __launch_bounds__(256, 3) void kda_prep_kernel(const BuildArgs a, const ChunkTable cks, unsigned char* ws) {
  constexpr int D = 128;
  using Cfg = KdaCfg<D, false>;
  constexpr int FP = Cfg::FP, GP = Cfg::GP, NP = Cfg::NP;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sKf = reinterpret_cast<bf16_t*>(smem + KdaPrepLds::OFF_KF);
  float* sG = reinterpret_cast<float*>(smem + KdaPrepLds::OFF_G);
  float* sN = reinterpret_cast<float*>(smem + KdaPrepLds::OFF_N);
  float* sBeta = reinterpret_cast<float*>(smem + KdaPrepLds::OFF_SMALL);
  float* sMax = sBeta + C;
  float* sMu = sMax + C;
  float* sGC = sMu + C;
  float* sMisc = sGC + D;

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
  const int tid = threadIdx.x;
  unsigned char* rec = ws + (size_t)blockIdx.x * KREC_BYTES;

  // decayed keys (tokens 4 tq .. 4 tq + 3, channels 8 db .. 8 db + 7) and the
  // gate factors, written while H is still in LDS
  auto early = [&] {
    const int tq = tid & 15, db = tid >> 4;
    float hC[8];
    lds_f8(sG + (C - 1) * GP + 8 * db, hC);
    float kd[8][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tq + r;
      float kv[8], hv[8];
      lds_keys8(sKf + t * FP + 8 * db, kv);
      lds_f8(sG + t * GP + 8 * db, hv);
      f16x8 kb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kb[j] = (f16_t)(kv[j] * __expf(hv[j]));
        kd[j][r] = kv[j] * __expf(hC[j] - hv[j]);
      }
      *reinterpret_cast<f16x8*>(rec + KREC_KB + (t * D + 8 * db) * 2) = kb;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (f16_t)kd[j][r];
      *reinterpret_cast<f16x4*>(rec + KREC_KD + ((8 * db + j) * C + 4 * tq) * 2) = v;
    }
    const float muC = sMisc[0];
    if (tid < C) reinterpret_cast<float*>(rec + KREC_VF)[tid] = __expf(muC - sMu[tid]);
    if (tid < D) {
      reinterpret_cast<float*>(rec + KREC_RS)[tid] = __expf(sGC[tid]);
      reinterpret_cast<float*>(rec + KREC_RU)[tid] = __expf(sGC[tid] - muC);
    }
    if (tid == 0) {
      reinterpret_cast<float*>(rec + KREC_M)[0] = muC;
      reinterpret_cast<float*>(rec + KREC_M)[1] = sMisc[1];
    }
  };
  kda_chunk_factors<D, false, false, true, bf16_t, decltype(early), true>(a, c0, nv, chain, sKf, (bf16_t*)nullptr, sG,
                                                                        sN, sBeta, sMax, sMu, sGC, sMisc, early);

  {  // X = diag(b) N, row t by the four threads 4t .. 4t+3 (16 entries each)
    const int t = tid >> 2, cb = (tid & 3) * 16;
    float x[16];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int tp = cb + j;
      x[j] = (tp <= t) ? sN[t * NP + tp] : 0.f;
      m = fmaxf(m, fabsf(x[j]));
    }
    m = dpp_max_step(m, 0);  // the row's four lanes: a quad
    m = dpp_max_step(m, 1);
    const float bt = sBeta[t];
    m *= fabsf(bt);
    int e = 0;
    if (m > 0.f) {
      frexpf(m, &e);
      e -= 14;  // row maximum into [2^13, 2^14)
    }
    const float sc = bt * ldexpf(1.f, -e);
    f16x8 lo8, hi8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo8[j] = (f16_t)(x[j] * sc);
      hi8[j] = (f16_t)(x[8 + j] * sc);
    }
    f16x8* dst = reinterpret_cast<f16x8*>(rec + KREC_X + (t * C + cb) * 2);
    dst[0] = lo8;
    dst[1] = hi8;
    if ((tid & 3) == 0) reinterpret_cast<float*>(rec + KREC_XS)[t] = ldexpf(1.f, e);
  }
}

}  // namespace

bool kda_build_supported(int d, bool in_f32) { return d == 64 || (d == 128 && !in_f32); }

namespace {
bool use_two_pass(int d, bool in_f32, const SegTable& seg) {
  if (d != 128 || in_f32) return false;
  for (int s = 0; s < seg.n_seg; ++s)
    if (seg_len(seg, s) > kDelta2MaxSegLen) return false;
  return true;
}
}  // namespace

size_t kda_workspace_bytes(int d, bool in_f32, const SegTable& seg, int n_chain) {
  return use_two_pass(d, in_f32, seg) ? (size_t)chunk_table(seg, nullptr) * n_chain * KREC_BYTES : 0;
}

hipError_t launch_build_kda(int d, bool in_f32, const BuildArgs& a, int n_blocks, void* ws, hipStream_t stream) {
  if (ws && use_two_pass(d, in_f32, a.seg)) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_prep_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, KdaPrepLds::LDS);
    if (attr != hipSuccess) return attr;
    ChunkTable ct;
    const int n_chunks = chunk_table(a.seg, &ct);
    hipLaunchKernelGGL(kda_prep_kernel, dim3(n_chunks * a.n_chain), dim3(256), KdaPrepLds::LDS, stream, a, ct,
                       reinterpret_cast<unsigned char*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_kda_state(a, ct, ws, stream);
  }
  if (d == 128 && !in_f32) return launch_t<128, false>(a, n_blocks, stream);
  if (d == 64) return in_f32 ? launch_t<64, true>(a, n_blocks, stream) : launch_t<64, false>(a, n_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace hypic
